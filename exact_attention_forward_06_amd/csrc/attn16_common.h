// Pieces shared by the attention kernels (the 16-bit forward kernels of
// attn_fwd_pp.hip and attn_fwd_pair.hip, the backward attn_bwd.hip and the
// fp32 forward attn_fwd_f32.hip): kernel parameters,
// the MFMA / rounding wrappers, the key permutation of the S^T accumulator,
// the LDS swizzle and the global -> LDS tile copy.  Private to those
// translation units.
#pragma once

#include "device_common.h"

namespace attn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

constexpr float kTau = 8.f;   // lazy-rescale threshold (log2 units)
// 2^kTau: a lane's sum of P over a tile above this may hide a P above 2^kTau
constexpr float kRescaleSum = 256.f;

// s_waitcnt vmcnt(0): this wave's global -> LDS copies have landed
// (simm16 = vmcnt 0 | expcnt 7 << 4 | lgkmcnt 15 << 8).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

struct Params {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int64_t sb, sh, sn;   // element strides of q, k, v
  int H, N, nmb, total;
  float scale_log2;     // softmax_scale * log2(e)
  // split-KV only: key range s covers keys [s * chunk, (s + 1) * chunk)
  float* o_part;        // fp32 [nsplit, B, H, N, d], each range's normalised O
  float* lse_part;      // fp32 [nsplit, B, H, N], each range's LSE (-inf if empty)
  int nsplit, chunk, bh_count;
  int nwg;              // workgroups launched (a persistent grid takes several items each)
};

template <typename T>
struct Ops;

template <>
struct Ops<__bf16> {
  using frag = bf16x8_t;
  static __device__ __forceinline__ f32x16_t mfma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float a, float b) {   // one v_cvt_pk_bf16_f32
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
  }
};

template <>
struct Ops<_Float16> {
  using frag = f16x8_t;
  static __device__ __forceinline__ f32x16_t mfma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float a, float b) {   // one v_cvt_pk_f16_f32
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2_t));
  }
};

// S^T accumulator row r of a 32-key block -> key (bits 2 and 3 swapped).
__device__ __forceinline__ int key_of_row(int r) { return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Register i (0..15) of lane group g holds key 16*(i/8) + 8*g + i%8 of the block.
__device__ __forceinline__ int key_of_reg(int i, int g) { return 16 * (i >> 3) + 8 * g + (i & 7); }

// XOR swizzle of the 16-byte chunks of an LDS row (depends on row & 15).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else return ((row & 3) << 2) | ((row >> 2) & 3);
}

// Copy one tile (TILE = LOADS * NT * 16 bytes) global -> LDS at `dst`.  DMA
// instruction t of a wave writes LDS bytes [(t * NT + wave * 64) * 16, + 1024),
// lane l's 16 bytes at + 16 l; off[t] is that lane's source offset relative
// to the tile's first row and `base` (wave-uniform, the buffer's scalar
// offset) that row's offset.  (A free function: lambdas inside the kernel
// must not capture buffer descriptors, or the host pass drops the kernel.)
// Debug builds with ATTN_LDS_POISON fill every 16 bytes a copy is about to
// land in with NaN first (and wait for those writes), so a read of a stage
// before its copy has landed -- a missing wait or barrier -- turns into NaN
// in the output instead of stale but plausible values.
template <int LOADS, int NT, bool OPAQUE_WAVE = false>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, char* dst, int wave, int base, const int* off) {
#ifdef ATTN_LDS_POISON
#pragma unroll
  for (int t = 0; t < LOADS; ++t)
    *(__attribute__((address_space(3))) u32x4_t*)(dst + (t * NT + wave * 64 + (int)(threadIdx.x & 63)) * 16) =
        u32x4_t{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the NaN writes have landed
#endif
  // With OPAQUE_WAVE the wave's LDS offset is made opaque at each copy, so
  // the M0 value of each instruction is one scalar add from it; otherwise the
  // compiler keeps every (stage, t) address live across the tile loop, and in
  // the forward kernels those SGPRs spill to VGPR lanes that each copy
  // instruction reads back.
  int wofs = wave * 64 * 16;
  if constexpr (OPAQUE_WAVE) asm volatile("" : "+s"(wofs));
#pragma unroll
  for (int t = 0; t < LOADS; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + t * NT * 16 + wofs), 16, off[t], base, 0, 0);
}

}  // namespace
}  // namespace attn
