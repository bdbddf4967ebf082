// Backward kernels (placeholder until the backward lands).
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
size_t bwd_workspace_bytes(int B, int H, int Sq, int Sk, int d, bool deterministic) {
  (void)Sk; (void)deterministic;
  return (size_t)B * H * Sq * (d + 1) * sizeof(float);
}
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fa
