// Exact-attention forward for gfx950: the kernel for each dtype and head
// dimension.
//  * fp16 / bf16, d = 64 and 128: attn_fwd_pp.hip, the ping-pong schedule
//    with one wave per 32 query rows;
//  * fp16 / bf16, d = 256: attn_fwd_pair.hip, the same schedule with a pair
//    of waves per 32 query rows (S split by keys, O by d);
//  * fp32: attn_fwd_f32.hip.
#include "kernels.h"

namespace attn {

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t s, bool* ok);
hipError_t launch_attn_fwd16_pp(const FwdArgs& a, hipStream_t s, bool* ok);
hipError_t launch_attn_fwd16_pair(const FwdArgs& a, hipStream_t s, bool* ok);

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream, bool* supported) {
  switch (a.dtype) {
    case Dtype::BF16:
    case Dtype::F16:
      return a.d == 256 ? launch_attn_fwd16_pair(a, stream, supported) : launch_attn_fwd16_pp(a, stream, supported);
    case Dtype::F32: return launch_attn_fwd_f32(a, stream, supported);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace attn
