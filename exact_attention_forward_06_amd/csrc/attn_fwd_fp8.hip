// FP8 attention forward (placeholder until the kernel lands): reports unsupported.
#include "kernels.h"
namespace attn {
hipError_t launch_attn_fwd_fp8(const Fp8FwdArgs&, hipStream_t, bool* supported) {
  *supported = false;
  return hipSuccess;
}
}  // namespace attn
