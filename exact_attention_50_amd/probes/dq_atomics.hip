// Cost of accumulating dQ with float32 atomics, the accumulation a
// five-product backward (one kernel per key block forming dQ, dK and dV)
// needs: on the causal B1 H16 S4096 d128 backward, every (query tile of 64
// rows, key block of 128 keys) pair adds a 64 x 128 float32 block of dQ, and
// the 512 key-block workgroups (32 blocks x 16 heads) add theirs
// concurrently over the same rows, 16896 blocks (554 MB) in all.  The probe
// runs exactly that pattern of adds (the value 1.0, 256 threads per
// workgroup, one 32-bit atomic add per element, no return value) and, as a
// reference, the same pattern with plain stores; it checks every element of
// the atomic result (row r of a head is added once per key block kb with
// 2 kb <= r / 64) and prints the times.
//
// Build and run (one GPU):
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         exact_attention_50_amd/probes/dq_atomics.hip -o /tmp/dq_atomics
//   /tmp/dq_atomics
// Every index stays inside the 32 MiB buffer: head < 16, row < 4096, column < 128.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

constexpr int kHeads = 16, kS = 4096, kD = 128, kQT = 64, kKB = 128;
constexpr int kNQT = kS / kQT, kNKB = kS / kKB;

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

// workgroup = (key block kb, head h); it walks the query tiles qt = 2 kb ..
// 63 the causal mask leaves it and adds one 64 x 128 block per tile
template <bool ATOMIC>
__global__ __launch_bounds__(256) void add_blocks(float* dq) {
  const int kb = blockIdx.x / kHeads, h = blockIdx.x % kHeads;
  float* head = dq + (size_t)h * kS * kD;
  for (int qt = 2 * kb; qt < kNQT; ++qt) {
    float* tile = head + (size_t)qt * kQT * kD;
#pragma unroll 4
    for (int e = threadIdx.x; e < kQT * kD; e += 256) {
      if constexpr (ATOMIC) {
        atomicAdd(tile + e, 1.0f);   // return value unused: the no-return form
      } else {
        tile[e] = 1.0f;
      }
    }
  }
}

int main() {
  const size_t n = (size_t)kHeads * kS * kD;
  float* dq = nullptr;
  CHECK(hipMalloc(&dq, n * sizeof(float)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  long long blocks = 0;
  for (int kb = 0; kb < kNKB; ++kb) blocks += (long long)(kNQT - 2 * kb) * kHeads;
  const double bytes = (double)blocks * kQT * kD * sizeof(float);
  const dim3 grid(kNKB * kHeads), block(256);

  for (int atomic = 1; atomic >= 0; --atomic) {
    float best = 1e30f;
    for (int rep = 0; rep < 5; ++rep) {
      CHECK(hipMemset(dq, 0, n * sizeof(float)));
      CHECK(hipEventRecord(e0));
      if (atomic) hipLaunchKernelGGL(add_blocks<true>, grid, block, 0, 0, dq);
      else hipLaunchKernelGGL(add_blocks<false>, grid, block, 0, 0, dq);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0.0f;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      if (ms < best) best = ms;
    }
    if (atomic) {
      std::vector<float> h(n);
      CHECK(hipMemcpy(h.data(), dq, n * sizeof(float), hipMemcpyDeviceToHost));
      long long bad = 0;
      for (int hd = 0; hd < kHeads; ++hd)
        for (int r = 0; r < kS; ++r) {
          const float want = (float)((r / kQT) / 2 + 1);   // key blocks kb with 2 kb <= r / 64
          for (int c = 0; c < kD; ++c) bad += h[((size_t)hd * kS + r) * kD + c] != want;
        }
      printf("float32 atomic adds: %lld blocks of 64 x 128, %.1f MB, best of 5: %.1f us (%.0f GB/s); %lld wrong elements\n",
             blocks, bytes / 1e6, best * 1e3, bytes / (best * 1e-3) / 1e9, bad);
      if (bad) return 2;
    } else {
      printf("plain stores, same pattern: %.1f MB, best of 5: %.1f us (%.0f GB/s)\n", bytes / 1e6, best * 1e3,
             bytes / (best * 1e-3) / 1e9);
    }
  }
  CHECK(hipFree(dq));
  return 0;
}
