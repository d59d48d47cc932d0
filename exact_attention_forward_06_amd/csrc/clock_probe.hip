// Shader-clock probe: one wave counts shader cycles (s_memtime) against the
// 100 MHz real-time counter (s_memrealtime) over a fixed real-time interval,
// so cycles / ticks * 100 MHz is the clock of the compute unit it runs on.
// Launched on a second stream while the attention kernels run, the wave
// shares a compute unit with them (it needs a handful of registers), which
// gives the clock those kernels actually run at -- it varies with power
// draw, well below the 2.4 GHz peak under dense MFMA work.
#include "kernels.h"

namespace attn {
namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out, long long spin_ticks) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  unsigned long long r1 = r0;
  // bounded wait: the real-time counter always advances, the iteration cap
  // only guards against a counter that does not
  for (long long it = 0; it < (1ll << 26) && (long long)(r1 - r0) < spin_ticks; ++it) {
    __builtin_amdgcn_s_sleep(1);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = t1 - t0;
    out[1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_clock_probe(unsigned long long* out, long long spin_ticks, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, spin_ticks);
  return hipGetLastError();
}

}  // namespace attn
