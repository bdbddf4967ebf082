// Unit rates of one MI355X (gfx950) SIMD for the per-tile roofline of the
// attention kernels: cycles per wavefront instruction of the matrix core
// (v_mfma_f32_32x32x16_bf16, v_mfma_f32_16x16x32_bf16), of the VALU
// instructions the softmax issues (fp32 FMA, v_max3_f32, v_cvt_pk_bf16_f32,
// v_exp_f32), with 4 to 32 independent dependency chains per wave (latency
// against issue rate), two VALU wavefronts sharing a SIMD (the SIMD's issue
// rate), a VALU wavefront beside an MFMA wavefront (overlap), and LDS operand
// reads (ds_read_b128, ds_read_b64_tr_b16) with 4 and 8 wavefronts per CU.
//
// Build and run (one GPU):
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         exact_attention_50_amd/probes/unit_rates.hip -o /tmp/unit_rates
//   /tmp/unit_rates
// Times are shader-clock cycles (clock64 = s_memtime) per instruction of one
// wavefront, averaged over 256 workgroups (one per CU).  Every buffer index
// stays inside its allocation; the LDS reads stay inside the workgroup's
// 64 KiB array.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlocks = 256;

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

// kinds of VALU work
enum { kFma = 0, kExp = 1, kMax3 = 2, kCvt = 3 };

template <int K>
__device__ __forceinline__ void valu(float& r, float c) {
  if (K == kFma) asm volatile("v_fma_f32 %0, %0, %1, %1" : "+v"(r) : "v"(c));
  if (K == kExp) asm volatile("v_exp_f32 %0, %0" : "+v"(r));
  if (K == kMax3) asm volatile("v_max3_f32 %0, %0, %1, %1" : "+v"(r) : "v"(c));
  if (K == kCvt) asm volatile("v_cvt_pk_bf16_f32 %0, %0, %1" : "+v"(r) : "v"(c));
}

// Role of a wavefront: 0 idle, 1 VALU chains of kind K (N chains), 2 MFMA
// 32x32x16 chain, 3 MFMA 16x16x32 chain.  ROLE_LO for waves 0-3, ROLE_HI for
// waves 4-7 (waves w and w + 4 share SIMD w).
template <int ROLE_LO, int ROLE_HI, int K, int N>
__global__ __launch_bounds__(512) void rate_kernel(const float* in, float* out, long long* cyc, int iters) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int role = w < 4 ? ROLE_LO : ROLE_HI;
  const float c0 = in[l] * 1e-3f;
  float r[N];
#pragma unroll
  for (int i = 0; i < N; ++i) r[i] = c0 * (float)(i + 1);
  long long t0 = 0, t1 = 0;
  __syncthreads();
  if (role == 1) {
    t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < N; ++i) valu<K>(r[i], c0);
    }
    t1 = clock64();
  } else if (role == 2 || role == 3) {
    const unsigned u = __builtin_bit_cast(unsigned, c0);
    const bf16x8 a = __builtin_bit_cast(bf16x8, (uint4){u, u ^ 1u, u, u ^ 2u});
    f32x16 acc = {};
    f32x4 acc4 = {};
    t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (role == 2) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, %0" : "+v"(acc) : "v"(a));
        else asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %1, %0" : "+v"(acc4) : "v"(a));
      }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc), "+v"(acc4));
    t1 = clock64();
    for (int i = 0; i < 16; ++i) r[0] += acc[i];
    for (int i = 0; i < 4; ++i) r[0] += acc4[i];
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) s += r[i];
  out[blockIdx.x * 512 + threadIdx.x] = s;
  if (l == 0) cyc[blockIdx.x * 8 + w] = t1 - t0;
}

// LDS operand reads: NW wavefronts, each reads 16-byte (b128) or 2 x 8-byte
// transposed (tr16, one MFMA A operand) fragments round a 64 KiB array.
template <bool TR, int NW>
__global__ __launch_bounds__(NW * 64) void lds_kernel(float* out, long long* cyc, int iters) {
  __shared__ __attribute__((aligned(16))) char buf[65536];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 65536 / 4; i += NW * 64) reinterpret_cast<float*>(buf)[i] = (float)i;
  __syncthreads();
  f32x4 accv = {};
  const unsigned base = (unsigned)(w * 8192 + l * 16);   // < 64 KiB for w < 8
  long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // the address moves every iteration, so no read can be hoisted
      const unsigned off = (base + (unsigned)j * 1024u + (unsigned)it * 64u) & 65535u;
      if (TR) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(buf + (off & ~7u)));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(buf + ((off + 512u) & 65535u & ~7u)));
        accv[0] += (float)lo[0] + (float)hi[1];
      } else {
        const f32x4 v = *reinterpret_cast<const f32x4*>(buf + off);
        accv += v;
      }
    }
  }
  long long t1 = clock64();
  out[blockIdx.x * NW * 64 + threadIdx.x] = accv[0] + accv[1] + accv[2] + accv[3];
  if (l == 0) cyc[blockIdx.x * 8 + w] = t1 - t0;
}

struct Bufs {
  float* in;
  float* out;
  long long* cyc;
};

// average cycles per instruction of the waves with role R (lo: waves 0-3, hi: 4-7)
template <int LO, int HI, int K, int N>
int rate(const Bufs& b, const char* what, int iters = 256) {
  for (int rep = 0; rep < 2; ++rep) {
    hipLaunchKernelGGL((rate_kernel<LO, HI, K, N>), dim3(kBlocks), dim3(512), 0, 0, b.in, b.out, b.cyc, iters);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }
  std::vector<long long> c(kBlocks * 8);
  CHECK(hipMemcpy(c.data(), b.cyc, c.size() * 8, hipMemcpyDeviceToHost));
  double lo = 0, hi = 0;
  for (int blk = 0; blk < kBlocks; ++blk)
    for (int w = 0; w < 8; ++w) (w < 4 ? lo : hi) += (double)c[blk * 8 + w];
  const double per = (double)kBlocks * 4.0 * iters * N;
  printf("%-64s", what);
  if (LO) printf("  waves 0-3: %6.2f", lo / per);
  if (HI) printf("  waves 4-7: %6.2f", hi / per);
  printf("  cycles/instr\n");
  return 0;
}

template <bool TR, int NW>
int lds_rate(const Bufs& b, const char* what, int iters = 512) {
  for (int rep = 0; rep < 2; ++rep) {
    hipLaunchKernelGGL((lds_kernel<TR, NW>), dim3(kBlocks), dim3(NW * 64), 0, 0, b.out, b.cyc, iters);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }
  std::vector<long long> c(kBlocks * 8);
  CHECK(hipMemcpy(c.data(), b.cyc, c.size() * 8, hipMemcpyDeviceToHost));
  double t = 0;
  for (int blk = 0; blk < kBlocks; ++blk)
    for (int w = 0; w < NW; ++w) t += (double)c[blk * 8 + w];
  t /= (double)kBlocks * NW;
  const double bytes = (double)NW * iters * 8 * 64 * 16;   // per CU
  printf("%-64s  %6.1f bytes/cycle per CU\n", what, bytes / t);
  return 0;
}

int main() {
  Bufs b;
  CHECK(hipMalloc(&b.in, 64 * sizeof(float)));
  CHECK(hipMalloc(&b.out, kBlocks * 512 * sizeof(float)));
  CHECK(hipMalloc(&b.cyc, kBlocks * 8 * sizeof(long long)));
  std::vector<float> h(64, 0.5f);
  CHECK(hipMemcpy(b.in, h.data(), 64 * sizeof(float), hipMemcpyHostToDevice));
  int e = 0;
  e |= rate<2, 0, kFma, 8>(b, "MFMA 32x32x16 bf16, one wave per SIMD");
  e |= rate<3, 0, kFma, 8>(b, "MFMA 16x16x32 bf16, one wave per SIMD");
  e |= rate<1, 0, kFma, 4>(b, "v_fma_f32, 4 chains, one wave per SIMD");
  e |= rate<1, 0, kFma, 8>(b, "v_fma_f32, 8 chains, one wave per SIMD");
  e |= rate<1, 0, kFma, 32>(b, "v_fma_f32, 32 chains, one wave per SIMD");
  e |= rate<1, 0, kMax3, 32>(b, "v_max3_f32, 32 chains, one wave per SIMD");
  e |= rate<1, 0, kCvt, 32>(b, "v_cvt_pk_bf16_f32, 32 chains, one wave per SIMD");
  e |= rate<1, 0, kExp, 8>(b, "v_exp_f32, 8 chains, one wave per SIMD");
  e |= rate<1, 0, kExp, 32>(b, "v_exp_f32, 32 chains, one wave per SIMD");
  e |= rate<1, 1, kFma, 32>(b, "v_fma_f32, 32 chains, two waves per SIMD");
  e |= rate<1, 1, kExp, 32>(b, "v_exp_f32, 32 chains, two waves per SIMD");
  e |= rate<2, 1, kFma, 32>(b, "MFMA 32x32x16 wave + v_fma_f32 wave (32 chains) per SIMD");
  e |= rate<2, 1, kExp, 32>(b, "MFMA 32x32x16 wave + v_exp_f32 wave (32 chains) per SIMD");
  e |= lds_rate<false, 4>(b, "ds_read_b128, 4 waves per CU");
  e |= lds_rate<false, 8>(b, "ds_read_b128, 8 waves per CU");
  e |= lds_rate<true, 4>(b, "ds_read_b64_tr_b16 (pairs), 4 waves per CU");
  e |= lds_rate<true, 8>(b, "ds_read_b64_tr_b16 (pairs), 8 waves per CU");
  return e;
}
