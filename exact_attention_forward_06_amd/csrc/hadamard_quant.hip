// FP8 pre-pass for gfx950: incoherent processing + per-block E4M3 (or E5M2)
// codes.
//
// For each row x of one (b, h): x~ = H D x over the head dimension (D the
// random +-1 diagonal, H the Sylvester Hadamard matrix), then per block of
// 128 rows: amax = max |x~|, code = E4M3(x~ * 448 / amax), stored scale =
// amax / (448 sqrt(d)).  The transform is left unnormalised in the kernel:
// the codes do not depend on a common factor of the block, so the 1/sqrt(d)
// of the orthonormal rotation only enters the stored scale.
// Sources: the "FlashAttention-3" page, section "FP8 路径与低精度误差"
// (x~ = H D x on Q and K; the Hadamard transform costs O(d log d) and is
// bandwidth-bound) and the "FlashAttention-2/3" page, FlashAttention-3
// 特性三 (one quantisation scale per block).
//
// gfx950 mapping (HBM-bound: one read of x, one byte written per element)
//  * One workgroup (4 wave64) per (b, h, 128-row block); four lanes per row,
//    each holding d/4 CONSECUTIVE elements loaded with 16-byte loads.  Of the
//    log2(d) butterfly stages all but two are inside a lane; the last two
//    (partners at lane distance 1 and 2) are one v_fmac_f32 each with a DPP
//    quad_perm source -- no LDS, and the lane's resulting sign is taken
//    back by the quantisation multiply.
//  * The whole block stays in registers until its amax is known (wave
//    reduction through DPP, then 4 values through LDS), so HBM sees exactly
//    one read and one write.
//  * E4M3 codes come from v_cvt_pk_fp8_f32 (round to nearest even, OCP E4M3
//    on gfx950) after clamping to +-448; the value rounded is the quotient
//    (x~ * 448) / amax with an FMA remainder correction, not x~ times a
//    rounded 448 / amax, so exact rounding ties stay exact.
//  * E5M2 (FMT = 1, the other FP8 format of the "FlashAttention-2/3" page,
//    特性二): the same rule with 57344 (its largest finite value) in place of
//    448, codes from v_cvt_pk_bf8_f32 (OCP E5M2 on gfx950).  448 and 57344
//    share the significand 1.75, so the quotient stays exact alike.
//  * transpose_out writes [d][n] (the layout the FP8 attention kernel wants
//    for V): codes are transposed through LDS so global stores stay 16-byte.
//  * Per-head scales (the coarser granularity the per-block scheme is
//    compared with: one scale per (b, h) instead of per 128 rows) run in
//    three launches: block amaxes into the scale slots, their maximum per
//    head into every slot, then the codes with the head's amax; x is read
//    twice, and the [B, H, N/128] scale array the attention kernel reads
//    holds the head's scale in every slot.
//  * RoPE (ROPE = 1: pairs (2i, 2i+1); ROPE = 2: pairs (i, i + d/2)) runs on
//    the loaded fp32 values before D and H, so the producer pass that the
//    "FlashAttention-3" page suggests (Hadamard fused with a bandwidth-bound
//    pre-processing stage such as RoPE, section "为什么 Hadamard 适合放到内核里")
//    still reads x once and writes the codes once.  RoPE itself is the
//    published rotary embedding (RoFormer): pair i at position n turns by
//    n * theta_i, theta_i = base^(-2i/d).  The theta_i come from the host in
//    double; n * theta_i is formed and reduced by pi/2 in fp64 (an fp32
//    angle near n = 8192 would be off by up to 5e-4 rad), then sin and cos of
//    the reduced angle by their Taylor series in fp32.  Interleaved pairs sit in one lane; split-half
//    pairs are lanes l and l ^ 2, exchanged by the same DPP swap as the
//    butterflies (each of the two lanes evaluates half of the shared angles).
//    The angles do not depend on the head, so at d <= 128 a workgroup walks
//    several heads at the same positions (as many as keep about two
//    workgroups per CU), evaluates its lanes' sines and cosines once into
//    registers, and has the next head's rows in flight while it transforms
//    the current one.
#include "kernels.h"

#include <math.h>

#include <algorithm>

namespace attn {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int ROWS = 128;       // rows per scale block
constexpr int NT = 256;         // threads per workgroup
constexpr int LPR = 4;          // lanes per row
constexpr int RPP = NT / LPR;   // rows per pass
constexpr int PASSES = ROWS / RPP;

struct QParams {
  const char* x;
  int64_t sb, sh, sn;
  const int8_t* signs;
  uint8_t* x8;
  float* scales;
  int H, N, nblk;
  int BH;             // B * H
  int G;              // heads per workgroup (RoPE with the angle cache)
  float scale_norm;   // 1/sqrt(d) for the rotated path, 1 otherwise
};

// RoPE angle table (ROPE != 0 only): theta_i = base^(-2i/d), i < d/2
struct RopeTab {
  double theta[128];
  int pos_offset;
};
struct NoRope {
  int unused;
};
template <int ROPE>
struct RopeArg {
  using type = RopeTab;
};
template <>
struct RopeArg<0> {
  using type = NoRope;
};

// theta of one of NC equally spaced table entries, picked per lane: every
// index is a compile-time constant (scalar loads from the kernel arguments;
// a per-lane index would copy the table to scratch)
template <int NC, int STRIDE>
__device__ __forceinline__ double pick_theta(const RopeTab& rt, int k, int sel) {
  double t = rt.theta[k];
#pragma unroll
  for (int c = 1; c < NC; ++c)
    if (sel == c) t = rt.theta[c * STRIDE + k];
  return t;
}

// sin and cos of a non-negative angle (pos * theta, below 2^31 since
// theta <= 1): reduction by pi/2 in fp64 to t in [-pi/4, pi/4] and the
// quadrant q, then the Taylor series of sin t (to t^9) and cos t (to t^10) in
// fp32 -- the first omitted terms are below 2e-9 on that interval -- and a
// quarter-turn rotation by q.
__device__ __forceinline__ void rope_sincos(double ang, float* sn, float* cs) {
  const double k = rint(ang * 0.63661977236758134);            // 2 / pi
  const float t = (float)fma(-k, 1.5707963267948966, ang);       // pi / 2
  const float t2 = t * t;
  const float st = t * fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, 1.f / 362880.f, -1.f / 5040.f), 1.f / 120.f),
                                     -1.f / 6.f), 1.f);
  const float ct = fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, -1.f / 3628800.f, 1.f / 40320.f), -1.f / 720.f),
                                           1.f / 24.f), -0.5f), 1.f);
  const int q = (int)k & 3;
  const float a = (q & 1) ? ct : st;      // sin(t + q pi/2) up to sign
  const float b = (q & 1) ? st : ct;      // cos(t + q pi/2) up to sign
  *sn = (q & 2) ? -a : a;
  *cs = ((q + 1) & 2) ? -b : b;
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 v) { return (float)v; }
template <>
__device__ __forceinline__ float to_f32<_Float16>(_Float16 v) { return (float)v; }

// value of lane ^ 1 / lane ^ 2 (DPP quad_perm [1,0,3,2] / [2,3,0,1])
__device__ __forceinline__ float xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}

// Both cross-lane butterfly stages on 8 values: v += s1 * (v of lane ^ 1),
// then v += s2 * (v of lane ^ 2), each one v_fmac_f32 with a DPP source
// operand (the compiler does not fold a DPP move into a MAC, whose
// destination is tied).  The s_nop gives the wait states a DPP read needs
// after a VALU write of its VGPR or of EXEC; inside the block, a stage-2 read
// comes 8 instructions after the stage-1 write of its VGPR.
__device__ __forceinline__ void xlane_butterfly8(float* v, float s1, float s2) {
  asm("s_nop 4\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %9 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
      : "v"(s1), "v"(s2));
}

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// RoPE angle cache: the angles n * theta_i depend on the position and the
// pair only, so a workgroup that walks p.G heads at the same 128 positions
// evaluates each lane's sines and cosines once, into registers, and reuses
// them (not at d = 256, where they would not fit: one head per workgroup).
template <int D, int ROPE>
constexpr bool rope_cache() { return ROPE != 0 && D <= 128; }

// PT: 0 = one scale per 128-row block; per-head scales in two passes around
// head_amax_kernel: 1 = write the block's amax into its scale slot and stop,
// 2 = quantise with the amax found in the slot (the head's) and overwrite
// the slot with the head's scale.
template <typename T, int D, bool ROT, bool TRANS, int FMT, int ROPE = 0, int PT = 0>
__global__ __launch_bounds__(NT) void hadamard_quant_kernel(QParams p, typename RopeArg<ROPE>::type rt) {
  static_assert(!(ROPE && TRANS), "RoPE applies to Q and K, which are not transposed");
  static_assert(!(ROPE && PT), "RoPE runs with per-block scales");
  constexpr float QMAX = FMT == 0 ? 448.f : 57344.f;   // largest finite E4M3 / E5M2 value
  constexpr int EPL = D / LPR;                  // elements per lane
  constexpr int ES = sizeof(T);
  constexpr int LOADS = EPL * ES / 16;          // 16-byte loads per lane per row
  constexpr int PER16 = 16 / ES;                // elements per 16-byte load
  constexpr bool CACHE = rope_cache<D, ROPE>();
  const int G = CACHE ? p.G : 1;                // heads of this workgroup
  constexpr int NA = ROPE ? EPL / 2 : 1;        // angles a lane evaluates per row
  static_assert(EPL * ES % 16 == 0, "lane slice must be whole 16-byte loads");

  __shared__ float red[2][NT / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[TRANS ? D * ROWS : 16];

  const int tid = threadIdx.x;
  const int lr = tid & (LPR - 1);     // lane's quarter of the row
  const int rr = tid / LPR;           // row within a pass
  const int blk = blockIdx.x;
  const int r0 = blk * ROWS;

  float sg[ROT ? EPL : 1];
  const float bsgn1 = (lr & 1) ? -1.f : 1.f, bsgn2 = (lr & 2) ? -1.f : 1.f;
  // QMAX times the sign the butterflies leave on the lane's values
  const float qmul = ROT ? QMAX * bsgn1 * bsgn2 : QMAX;
  if constexpr (ROT) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) sg[i] = (float)p.signs[lr * EPL + i];
  }
  // RoPE sines and cosines of the lane's angles at its rows, evaluated for
  // the first head and reused by the others.  Interleaved pairs (2i, 2i+1):
  // angle j of lane lr is pair lr * EPL/2 + j.  Split halves (i, i + d/2):
  // element k of lanes lr and lr ^ 2 shares pair (lr & 1) * EPL + k; lanes
  // 0, 1 evaluate k < EPL/2 and lanes 2, 3 the rest, swapped by DPP at use.
  float rsn[CACHE ? PASSES : 1][CACHE ? NA : 1], rcs[CACHE ? PASSES : 1][CACHE ? NA : 1];
  const int asel = ROPE == 1 ? lr : 2 * (lr & 1) + (lr >> 1);   // the lane's angles
  if constexpr (CACHE) {
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const double pos = (double)(rt.pos_offset + r0 + ps * RPP + rr);
#pragma unroll
      for (int j = 0; j < NA; ++j) rope_sincos(pos * pick_theta<LPR, EPL / 2>(rt, j, asel), &rsn[ps][j], &rcs[ps][j]);
    }
  }

  // the lane's raw 16-byte loads of one head's rows (zeros past N); with
  // several heads per workgroup the next head's are in flight while the
  // current one is transformed and quantised
  auto load_rows = [&](int bh, u32x4_t (&raw)[PASSES][LOADS]) __attribute__((always_inline)) {
    const int b = bh / p.H, h = bh - b * p.H;
    const char* xb = p.x + ((int64_t)b * p.sb + (int64_t)h * p.sh) * ES;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int row = r0 + ps * RPP + rr;
      const char* src = xb + (int64_t)row * p.sn * ES + lr * EPL * ES;
#pragma unroll
      for (int l = 0; l < LOADS; ++l) {
        raw[ps][l] = u32x4_t{0u, 0u, 0u, 0u};
        if (row < p.N) raw[ps][l] = *(const u32x4_t*)(src + l * 16);
      }
    }
  };
  u32x4_t raw_next[PASSES][LOADS];
  load_rows(blockIdx.y * G, raw_next);

#pragma unroll 1
  for (int gh = 0; gh < G; ++gh) {
    const int bh = blockIdx.y * G + gh;
    if (gh > 0 && bh >= p.BH) break;
    u32x4_t raw[PASSES][LOADS];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
      for (int l = 0; l < LOADS; ++l) raw[ps][l] = raw_next[ps][l];
    if (gh + 1 < G && bh + 1 < p.BH) load_rows(bh + 1, raw_next);

    float v[PASSES][EPL];
    float amax = 0.f;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int row = r0 + ps * RPP + rr;
      const bool valid = row < p.N;
#pragma unroll
      for (int l = 0; l < LOADS; ++l) {
        const T* e = reinterpret_cast<const T*>(&raw[ps][l]);
#pragma unroll
        for (int t = 0; t < PER16; ++t) v[ps][l * PER16 + t] = to_f32<T>(e[t]);
      }
      if constexpr (ROPE != 0) {
        // sine and cosine of the lane's angle j at this row: from the
        // workgroup's cache, or evaluated here when the workgroup has one head
        auto angle = [&](int j, float& sn, float& cs) __attribute__((always_inline)) {
          if constexpr (CACHE) {
            sn = rsn[ps][j];
            cs = rcs[ps][j];
          } else {
            rope_sincos((double)(rt.pos_offset + row) * pick_theta<LPR, EPL / 2>(rt, j, asel), &sn, &cs);
          }
        };
        if constexpr (ROPE == 1) {
#pragma unroll
          for (int k = 0; k < EPL / 2; ++k) {
            float sn, cs;
            angle(k, sn, cs);
            const float a = v[ps][2 * k], c = v[ps][2 * k + 1];
            v[ps][2 * k] = a * cs - c * sn;
            v[ps][2 * k + 1] = a * sn + c * cs;
          }
        } else if constexpr (ROPE == 2) {
          // lanes 0, 1 hold the first members, lanes 2, 3 (the partners at
          // lane ^ 2, same k) the second
          const bool second = lr & 2;
#pragma unroll
          for (int j = 0; j < EPL / 2; ++j) {
            float ms, mc;
            angle(j, ms, mc);
            const float os = xor2(ms), oc = xor2(mc);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int k = j + u * (EPL / 2);
              // element k < EPL/2: lanes 0, 1 evaluated the angle; else lanes 2, 3
              const bool own = (u == 0) != second;
              const float sn = own ? ms : os, cs = own ? mc : oc;
              const float o = xor2(v[ps][k]);
              v[ps][k] = second ? o * sn + v[ps][k] * cs : v[ps][k] * cs - o * sn;
            }
          }
        }
      }
      if constexpr (ROT) {
        // D: sign flip
#pragma unroll
        for (int i = 0; i < EPL; ++i) v[ps][i] *= sg[i];
        // H: in-lane butterflies (partner distance 1 .. EPL/2)
#pragma unroll
        for (int hh = 1; hh < EPL; hh <<= 1)
#pragma unroll
          for (int i = 0; i < EPL; ++i)
            if ((i & hh) == 0) {
              const float a = v[ps][i], c = v[ps][i + hh];
              v[ps][i] = a + c;
              v[ps][i + hh] = a - c;
            }
        // cross-lane butterflies (partner distance EPL and 2*EPL elements):
        // the true outputs are s v + o (s = -1 on the upper lane of each
        // pair); v + s o is that times s, one FMA on the DPP value.  The
        // partners of the second stage share the first stage's s, so the
        // lane ends with its values times s1 s2, which the quantisation
        // multiply takes back (amax is blind to it; the codes are the same)
#pragma unroll
        for (int i = 0; i < EPL; i += 8) xlane_butterfly8(&v[ps][i], bsgn1, bsgn2);
      }
      if (valid) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(v[ps][i]));
      }
    }

    // block amax (red alternates between heads: the barrier of one head's
    // reduction separates the reads of the previous use from the next writes)
    float* slot = p.scales + (int64_t)bh * p.nblk + blk;
    float head_amax = 0.f;
    if constexpr (PT == 2) head_amax = *slot;   // read before the barrier after which thread 0 rewrites it
    amax = wave_max(amax);
    if ((tid & 63) == 0) red[gh & 1][tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[gh & 1][0], red[gh & 1][1]), fmaxf(red[gh & 1][2], red[gh & 1][3]));
    if constexpr (PT == 1) {
      if (tid == 0) *slot = amax;
      return;
    }
    if constexpr (PT == 2) amax = head_amax;
    // y = (x~ * 448) / amax, formed as a product with 1/amax plus one FMA
    // remainder correction: the remainder a - y0 * amax is exact in an FMA,
    // so a quotient that is representable (e.g. an exact E4M3 rounding tie,
    // frequent for 16-bit inputs whose x * 448 is exact) comes out exactly.
    const float ramax = amax > 0.f ? 1.f / amax : 0.f;
    if (tid == 0) *slot = amax * p.scale_norm / QMAX;   // 0 for a zero block

    // codes
    uint8_t* out = p.x8 + (int64_t)bh * p.N * D;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int lrow = ps * RPP + rr;
      const int row = r0 + lrow;
      unsigned words[EPL / 4];
#pragma unroll
      for (int w = 0; w < EPL / 4; ++w) {
        float y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float a = v[ps][4 * w + t] * qmul;
          const float y0 = a * ramax;
          const float q = fmaf(fmaf(-y0, amax, a), ramax, y0);
          y[t] = fminf(fmaxf(q, -QMAX), QMAX);
        }
        if constexpr (FMT == 0) {
          unsigned lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          words[w] = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
        } else {
          unsigned lo = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
          words[w] = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], lo, true);
        }
      }
      if constexpr (!TRANS) {
        if (row < p.N) {
          uint8_t* dst = out + (int64_t)row * D + lr * EPL;
#pragma unroll
          for (int w = 0; w < EPL / 16; ++w) {
            u32x4_t q = {words[4 * w], words[4 * w + 1], words[4 * w + 2], words[4 * w + 3]};
            *(u32x4_t*)(dst + 16 * w) = q;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          tbuf[(lr * EPL + i) * ROWS + lrow] = (uint8_t)(words[i >> 2] >> (8 * (i & 3)));
      }
    }
    if constexpr (TRANS) {
      __syncthreads();
      // out is [d][N] for this head: row = d index, 128 consecutive n per block
      constexpr int CHUNKS = D * ROWS / 16;
      const int nvalid = min(ROWS, p.N - r0);   // multiple of 16 (N % 16 == 0)
#pragma unroll
      for (int c = tid; c < CHUNKS; c += NT) {
        const int dd = c / (ROWS / 16), cc = c % (ROWS / 16);
        if (cc * 16 < nvalid)
          *(u32x4_t*)(out + (int64_t)dd * p.N + r0 + cc * 16) = *(const u32x4_t*)(tbuf + dd * ROWS + cc * 16);
      }
    }
  }
}

// Per-head amax: one workgroup per (b, h) reads the head's block amaxes from
// its scale slots and writes their maximum back to every slot.
__global__ __launch_bounds__(NT) void head_amax_kernel(float* scales, int nblk) {
  __shared__ float red[NT / 64];
  float* s = scales + (int64_t)blockIdx.x * nblk;
  float m = 0.f;
  for (int i = threadIdx.x; i < nblk; i += NT) m = fmaxf(m, s[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  for (int i = threadIdx.x; i < nblk; i += NT) s[i] = m;
}

template <typename T, int D, bool ROT, bool TRANS, int FMT>
hipError_t launch_per_head(const QParams& p, int bh_count, hipStream_t s) {
  const NoRope nr{0};
  dim3 grid(p.nblk, bh_count);
  hipLaunchKernelGGL((hadamard_quant_kernel<T, D, ROT, TRANS, FMT, 0, 1>), grid, dim3(NT), 0, s, p, nr);
  hipLaunchKernelGGL(head_amax_kernel, dim3(bh_count), dim3(NT), 0, s, p.scales, p.nblk);
  hipLaunchKernelGGL((hadamard_quant_kernel<T, D, ROT, TRANS, FMT, 0, 2>), grid, dim3(NT), 0, s, p, nr);
  return hipGetLastError();
}

template <typename T, int D, int FMT>
hipError_t launch_f(const QuantArgs& a, hipStream_t s) {
  QParams p;
  p.x = static_cast<const char*>(a.x);
  p.sb = a.sb;
  p.sh = a.sh;
  p.sn = a.sn;
  p.signs = a.signs;
  p.x8 = a.x8;
  p.scales = a.scales;
  p.H = a.H;
  p.N = a.N;
  p.nblk = (a.N + ROWS - 1) / ROWS;
  p.BH = a.B * a.H;
  p.G = 1;
  p.scale_norm = a.signs ? 1.f / sqrtf((float)D) : 1.f;
  dim3 grid(p.nblk, a.B * a.H);
  if (a.per_head) {
    if (a.signs) return a.transpose_out ? launch_per_head<T, D, true, true, FMT>(p, a.B * a.H, s)
                                        : launch_per_head<T, D, true, false, FMT>(p, a.B * a.H, s);
    return a.transpose_out ? launch_per_head<T, D, false, true, FMT>(p, a.B * a.H, s)
                           : launch_per_head<T, D, false, false, FMT>(p, a.B * a.H, s);
  }
  if (a.rope_style != 0) {
    RopeTab rt;
    for (int i = 0; i < D / 2; ++i) rt.theta[i] = pow(a.rope_base, -2.0 * i / D);
    for (int i = D / 2; i < 128; ++i) rt.theta[i] = 0.0;
    rt.pos_offset = a.pos_offset;
    if (rope_cache<D, 1>()) {
      // heads per workgroup: as many as keep about two workgroups per CU
      // resident (each holds the lane angle cache beside its rows), at most 8
      const int64_t wgs = (int64_t)p.nblk * p.BH;
      p.G = (int)std::min<int64_t>(8, std::max<int64_t>(1, wgs / 512));
    }
    grid.y = (p.BH + p.G - 1) / p.G;
    if (a.rope_style == 1) {
      if (a.signs) hipLaunchKernelGGL((hadamard_quant_kernel<T, D, true, false, FMT, 1>), grid, dim3(NT), 0, s, p, rt);
      else hipLaunchKernelGGL((hadamard_quant_kernel<T, D, false, false, FMT, 1>), grid, dim3(NT), 0, s, p, rt);
    } else {
      if (a.signs) hipLaunchKernelGGL((hadamard_quant_kernel<T, D, true, false, FMT, 2>), grid, dim3(NT), 0, s, p, rt);
      else hipLaunchKernelGGL((hadamard_quant_kernel<T, D, false, false, FMT, 2>), grid, dim3(NT), 0, s, p, rt);
    }
    return hipGetLastError();
  }
  const NoRope nr{0};
  if (a.signs) {
    if (a.transpose_out) hipLaunchKernelGGL((hadamard_quant_kernel<T, D, true, true, FMT>), grid, dim3(NT), 0, s, p, nr);
    else hipLaunchKernelGGL((hadamard_quant_kernel<T, D, true, false, FMT>), grid, dim3(NT), 0, s, p, nr);
  } else {
    if (a.transpose_out) hipLaunchKernelGGL((hadamard_quant_kernel<T, D, false, true, FMT>), grid, dim3(NT), 0, s, p, nr);
    else hipLaunchKernelGGL((hadamard_quant_kernel<T, D, false, false, FMT>), grid, dim3(NT), 0, s, p, nr);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const QuantArgs& a, hipStream_t s) {
  return a.fp8_format == 0 ? launch_f<T, D, 0>(a, s) : launch_f<T, D, 1>(a, s);
}

template <typename T>
hipError_t launch_t(const QuantArgs& a, hipStream_t s, bool* ok) {
  *ok = true;
  switch (a.d) {
    case 64: return launch_d<T, 64>(a, s);
    case 128: return launch_d<T, 128>(a, s);
    case 256: return launch_d<T, 256>(a, s);
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_hadamard_rotate_quant(const QuantArgs& a, hipStream_t stream, bool* supported) {
  if (a.block_rows != ROWS || (a.fp8_format != 0 && a.fp8_format != 1) || a.rope_style < 0 || a.rope_style > 2 ||
      (a.rope_style != 0 && a.transpose_out) || (a.per_head && a.rope_style != 0)) {
    *supported = false;
    return hipSuccess;
  }
  switch (a.dtype) {
    case Dtype::BF16: return launch_t<__bf16>(a, stream, supported);
    case Dtype::F16: return launch_t<_Float16>(a, stream, supported);
    case Dtype::F32: return launch_t<float>(a, stream, supported);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace attn
