// Device helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int V>
using ic = std::integral_constant<int, V>;

// Workgroup barrier between the phases of the ping-pong kernels.  s_barrier
// alone is not a memory operation to the compiler, which could then move LDS
// accesses across it; the empty asm statements with a memory clobber pin
// every memory access to its side of the barrier.  No wait is implied.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS accesses have completed
// (simm16 = vmcnt 63 | expcnt 7 << 4 | lgkmcnt 0 << 8).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Cross-half reductions: lanes l and l ^ 32 hold the two halves of a row.
// v_permlane32_swap returns both register images; one of them carries the
// partner lane's value and the other the lane's own, so a symmetric combine
// of the pair is exact whichever image is which.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroup id -> logical work item such that consecutive logical items run
// on the same XCD (the dispatcher hands workgroup w to XCD w % 8).  A
// bijection of [0, total).
__device__ __forceinline__ int xcd_logical_id(int w, int total) {
  const int qd = total >> 3, rem = total & 7, x = w & 7, s = w >> 3;
  return x * qd + min(x, rem) + s;
}

}  // namespace attn
