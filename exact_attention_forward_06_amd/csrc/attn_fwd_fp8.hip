// FP8 (OCP E4M3, or E5M2 for Q, K and V) attention forward for gfx950 with
// per-block scales.
//
// Inputs are the codes and block scales written by hadamard_rotate_quant:
// Q8, K8 [B,H,N,d] (rotated by the same H D), V8t [B,H,d,N] (not rotated),
// one fp32 dequantisation scale per (b, h, 128-row block) of each tensor.
// Both products run on v_mfma_f32_32x32x64_f8f6f4 with fp32 accumulation,
// as in the FP8 path of the "FlashAttention-3" page (section
// "FP8 路径与低精度误差") with per-block quantisation ("FlashAttention-2/3"
// page, FlashAttention-3 特性三); the online softmax is that of the 16-bit
// kernels (attn_fwd_pp.hip), whose layout choices it shares.
//
//  * S: one 32x32x64 MFMA per 64 of d.  128-row workgroups and 64-key tiles
//    never straddle a 128-row scale block, so sQ * sK * softmax_scale *
//    log2(e) is ONE scalar per tile.
//  * Lazy rescale of O with threshold 2^4: the running max m_run that O and
//    l are kept relative to is a whole number (log2 units, rounded up when
//    it moves), so the rescale factors are exact powers of two.
//  * P V: P is rounded to E4M3 against its own reference m_ref, the running
//    row maximum after the tile, rounded up to a whole number -- the m of
//    the tiled online softmax of the "FlashAttention-2/3" page ("技术原理"),
//    so the rounding does not depend on the lazy threshold -- after
//    multiplication by the gain 256 sV_j / sVmax (sV_j the tile's V block
//    scale, sVmax the largest V block scale of the head; an all-zero V block,
//    scale 0, takes the gain of sVmax, and its codes contribute nothing).
//    The gain enters the exp2 argument as a per-row bias and keeps
//    P' <= 256 < 448 (no saturation).  The difference between the two
//    references, 2^(m_ref - m_run) with 0 <= m_ref - m_run <= 4, is applied
//    exactly by the MFMA's per-lane E8M0 scale of the P'^T operand (lane n
//    and n + 32 hold query n).  At the end O = acc * sVmax / 256 / l.
//  * Q and K block scales of 0 (all-zero blocks, all codes 0) are used as 1:
//    the scores are 0 either way, and a zero factor would turn the -inf of
//    masked scores into NaN.
//  * Row sums l add up the E4M3-rounded P' (over the tile's gain), so O is
//    normalised by exactly the weights its second product used (rows of the
//    effective P sum to 1) and the LSE is the log of that normaliser.  The
//    ping-pong kernel (d = 64, 128) forms them with two extra MFMAs per tile
//    against an all-ones operand; the d = 256 kernel decodes the packed
//    codes back to fp32 and adds them on the VALU.
//  * The S^T rows are permuted so that each lane group holds 16 CONSECUTIVE
//    keys of a 32-key block; the 32 P^T bytes a lane feeds to one PV MFMA
//    then pair with two 16-byte LDS reads of V8t.
//  * K8 and V8t tiles go global -> LDS with buffer_load_dwordx4 ... lds,
//    double-buffered in two LDS objects, 16-byte chunks XOR-swizzled per row
//    so the operand reads are bank-conflict free.
#include "device_common.h"
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace attn {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

constexpr float kTau8 = 4.f;         // lazy-rescale threshold (log2 units)
constexpr float kPGain = 256.f;      // P' = P * kPGain * sV_j / sVmax <= 256, P relative to m_ref

struct F8Params {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8t;
  const float* qs;
  const float* ks;
  const float* vs;
  __bf16* o;
  float* lse;
  int H, N, nmb, total, nblk;
  float scale_log2;
  // Q rotated and quantised in the kernel (ping-pong kernel, QR != 0)
  const char* qx;
  const int8_t* signs;
  int64_t qsb, qsh, qsn;
};

template <typename T>
__device__ __forceinline__ float q_to_f32(T v) { return (float)v; }

// Wave-wide maximum (all 64 lanes).
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Largest block scale of a head's nblk scales: each lane loads every 64th
// one (one round of vector loads for up to 64 blocks) and the wave reduces
// them -- a loop of scalar loads would wait out one load latency per block
// before the workgroup starts.
__device__ __forceinline__ float head_max_scale(const float* s, int nblk, int lane) {
  float m = 0.f;
  for (int i = lane; i < nblk; i += 64) m = fmaxf(m, s[i]);
  return wave_max64(m);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// S^T accumulator row r of a 32-key block -> key: lane group g = bit 2 of r
// becomes bit 4 of the key, so group g holds keys 16g .. 16g+15.
__device__ __forceinline__ int key_of_row8(int r) { return (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3); }

// FA, FB: operand formats of A and B (0: FP8 E4M3, 1: BF8 E5M2); no block
// scale operands.
template <int FA, int FB>
__device__ __forceinline__ f32x16_t mfma_fp8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// The same with a per-lane E8M0 scale of the B operand (127 = 1.0): lane
// (n, g) scales the 32 K-values of column n it holds by 2^(sb - 127).
template <int FA, int FB>
__device__ __forceinline__ f32x16_t mfma_fp8_sb(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, sb);
}

// E8M0 byte of 2^(m_ref - m_run) (both whole numbers, m_ref >= m_run).
__device__ __forceinline__ int ref_scale(float m_ref, float m_run) {
  return m_ref == -INFINITY ? 127 : 127 + (int)(m_ref - m_run);
}

__device__ __forceinline__ i32x8_t cat(u32x4_t lo, u32x4_t hi) {
  i32x8_t r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// XOR swizzles of the 16-byte chunks of an LDS row of RB bytes.  Sixteen
// lanes read one chunk position from 16 rows at once; rows that share the
// same 256 bytes of banks must map that chunk to different positions.
// K rows are read in the key_of_row8 order ({0-7, 16-23} or {8-15, 24-31}
// of a 32-key block), V8t rows consecutively.
template <int RB>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (RB >= 256) return (row & 7) | (((row >> 4) & 1) << 3);
  else if constexpr (RB == 128) return ((row >> 1) & 3) | (((row >> 4) & 1) << 2);
  else return ((row >> 2) & 1) | (((row >> 4) & 1) << 1);   // RB == 64
}
template <int RB>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (RB >= 256) return row & 15;
  else if constexpr (RB == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;                                 // RB == 64
}

// Global -> LDS copy of one tile of ROWS x RB bytes (row pitch `pitch` in
// global memory) into `dst`; DMA instruction t of a wave writes LDS bytes
// [(t * NT + wave * 64) * 16, + 1024), lane l at + 16 l.
// Debug builds with ATTN_LDS_POISON fill the destination with E4M3 NaN
// codes (0x7F) first, so a read before the copy has landed shows as NaN.
template <int LOADS, int NT>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rs, char* dst, int wave, int base, const int* off) {
#ifdef ATTN_LDS_POISON
#pragma unroll
  for (int t = 0; t < LOADS; ++t)
    *(lds_u32x4_t*)(dst + (t * NT + wave * 64 + (int)(threadIdx.x & 63)) * 16) =
        u32x4_t{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the NaN writes have landed
#endif
#pragma unroll
  for (int t = 0; t < LOADS; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + (t * NT + wave * 64) * 16), 16, off[t], base,
                                             0, 0);
}

// FMT: format of the Q, K and V codes (0: E4M3, 1: E5M2); P is always E4M3.
template <int D, int BN, bool CAUSAL, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_kernel(F8Params p) {
  constexpr int NT = 256, BLOCK_M = 128;
  constexpr int NKS = D / 64;        // MFMA K-steps of S
  constexpr int NKB = BN / 32;       // 32-key blocks per tile
  constexpr int NDB = D / 32;        // d blocks of O^T
  constexpr int NPV = BN / 64;       // PV MFMAs (64 keys each) per d block
  constexpr int KRB = D;             // K8 tile row bytes (one key)
  constexpr int VRB = BN;            // V8t tile row bytes (one d)
  constexpr int K_BYTES = BN * KRB;
  constexpr int STAGE = K_BYTES + D * VRB;
  constexpr int KLOADS = K_BYTES / (NT * 16);
  constexpr int VLOADS = D * VRB / (NT * 16);
  static_assert(K_BYTES % (NT * 16) == 0 && (D * VRB) % (NT * 16) == 0, "tile split");
  static_assert(BN % 64 == 0 && 128 % BN == 0, "tile inside one K scale block");

  __shared__ __attribute__((aligned(1024))) char smem0[STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int g = lane >> 5;
  const int N = p.N;

  const int logical = xcd_logical_id(blockIdx.x, p.total);
  const int bh = logical / p.nmb;
  int mb = logical - bh * p.nmb;
  if (CAUSAL) mb = p.nmb - 1 - mb;
  const int m0 = mb * BLOCK_M;
  const int wq0 = m0 + wave * 32;
  const int q_row = wq0 + n;
  const int64_t head = (int64_t)bh * N * D;
  const float* ksc = p.ks + (int64_t)bh * p.nblk;
  const float* vsc = p.vs + (int64_t)bh * p.nblk;
  const float sq_raw = p.qs[(int64_t)bh * p.nblk + mb];
  const float sq = sq_raw > 0.f ? sq_raw : 1.f;

  float svmax = head_max_scale(p.vs + (int64_t)bh * p.nblk, p.nblk, lane);
  if (!(svmax > 0.f)) svmax = 1.f;     // every V block is zero: O = 0
  const float inv_svmax = 1.f / svmax;

  // Q8^T fragments: lane (n, g) holds Q8[q][64 ks + 32 g .. +32]
  i32x8_t qf[NKS];
  {
    const uint8_t* src = p.q8 + head + (int64_t)q_row * D + g * 32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = cat(*(const u32x4_t*)(src + ks * 64), *(const u32x4_t*)(src + ks * 64 + 16));
  }

  // DMA source offsets (tile-relative) of this lane's chunks
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k8 + head), (short)0, N * D, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v8t + head), (short)0, N * D, 0x00020000);
  int koff[KLOADS], voff[VLOADS];
#pragma unroll
  for (int t = 0; t < KLOADS; ++t) {
    const int pos = (t * NT + tid) * 16, row = pos / KRB;
    koff[t] = row * D + (((pos % KRB) / 16) ^ swz_k<KRB>(row)) * 16;
  }
#pragma unroll
  for (int t = 0; t < VLOADS; ++t) {
    const int pos = (t * NT + tid) * 16, row = pos / VRB;
    voff[t] = row * N + (((pos % VRB) / 16) ^ swz_v<VRB>(row)) * 16;
  }
  auto issue_tile = [&](int kt0, int stage) __attribute__((always_inline)) {
    char* dst = stage ? smem1 : smem0;
    dma<KLOADS, NT>(krs, dst, wave, kt0 * D, koff);
    dma<VLOADS, NT>(vrs, dst + K_BYTES, wave, kt0, voff);
  };

  // LDS read addresses: K A-operand rows kb*32 + key_of_row8(n), bytes
  // 64 ks + 32 g (+16); V8t A-operand rows db*32 + n, keys 64 t + 16 g (+32).
  const int krow = key_of_row8(n);
  int kaddr[NKS][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      kaddr[ks][hf] = krow * KRB + (((4 * ks + 2 * g + hf) ^ swz_k<KRB>(krow)) * 16);
  int vaddr[NPV][2];
#pragma unroll
  for (int t = 0; t < NPV; ++t)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      vaddr[t][hf] = K_BYTES + n * VRB + (((4 * t + 2 * hf + g) ^ swz_v<VRB>(n)) * 16);

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;   // reference of O and l
  float m_ref = -INFINITY;   // reference of P': ceil of the running row max
  float l_run = 0.f;

  const int kv_end = CAUSAL ? min(N, m0 + BLOCK_M) : N;
  const int n_tiles = kv_end / BN;     // N is a multiple of 128
  const float c0 = sq * p.scale_log2;

  auto compute_tile = [&](int kt0, const char* sb) __attribute__((always_inline)) {
    const float ks_raw = ksc[kt0 >> 7];
    const float c = c0 * (ks_raw > 0.f ? ks_raw : 1.f);
    const float sv = vsc[kt0 >> 7];
    const float fv = sv > 0.f ? sv * inv_svmax : 1.f;     // in (0, 1]

    f32x16_t sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const i32x8_t a = cat(*(const lds_u32x4_t*)(sb + kb * 32 * KRB + kaddr[ks][0]),
                              *(const lds_u32x4_t*)(sb + kb * 32 * KRB + kaddr[ks][1]));
        sacc[kb] = mfma_fp8<FMT, FMT>(a, qf[ks], sacc[kb]);
      }
    }

    if (CAUSAL && kt0 + BN - 1 > wq0) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt0 + kb * 32 + 16 * g + i;
          if (key > q_row) sacc[kb][i] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    const float m_tile = pair_max(mx) * c;
    if (__any(m_tile > m_run + kTau8)) {
      const float m_new = ceilf(fmaxf(m_run, m_tile));   // whole number (or -inf)
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)(m_run - m_new));
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      m_run = m_new;
    }
    m_ref = fmaxf(m_ref, ceilf(m_tile));
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    const int psc = ref_scale(m_ref, m_run);
    // e = P * kPGain * fv  with P = exp2(s c - m_ref)
    const float lg = __builtin_amdgcn_logf(kPGain * fv);   // v_log_f32 is log2
    const float bias = lg - m_use;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, bias));

    // P^T operands: slot s of lane group g <-> key 64 t + 32 (s / 16) + 16 g + s % 16.
    // The row sums add up the rounded P' (decoded back from the codes).
    i32x8_t pf[NPV];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int t = 0; t < NPV; ++t)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = 2 * t + (w >> 2);
        const int i0 = (w & 3) * 4;
        unsigned lo = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[kb][i0], sacc[kb][i0 + 1], 0, false);
        pf[t][w] = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[kb][i0 + 2], sacc[kb][i0 + 3], lo, true);
        const auto r01 = __builtin_amdgcn_cvt_pk_f32_fp8(pf[t][w], false);
        const auto r23 = __builtin_amdgcn_cvt_pk_f32_fp8(pf[t][w], true);
        rs0 += r01[0] + r23[0];
        rs1 += r01[1] + r23[1];
      }
    l_run += __builtin_amdgcn_ldexpf((rs0 + rs1) * (1.f / (kPGain * fv)), psc - 127);

#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < NPV; ++t) {
        const i32x8_t a = cat(*(const lds_u32x4_t*)(sb + db * 32 * VRB + vaddr[t][0]),
                              *(const lds_u32x4_t*)(sb + db * 32 * VRB + vaddr[t][1]));
        oacc[db] = mfma_fp8_sb<FMT, 0>(a, pf[t], oacc[db], psc);
      }
  };

  auto step = [&](int j, int stage) __attribute__((always_inline)) {
    const int kt0 = j * BN;
    if (j + 1 < n_tiles) issue_tile(kt0 + BN, stage ^ 1);
    const bool active = !CAUSAL || kt0 <= wq0 + 31;
    if (active) compute_tile(kt0, stage ? smem1 : smem0);
    wait_vmem();
    __syncthreads();
  };

  issue_tile(0, 0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, 0);
    if (j + 1 < n_tiles) step(j + 1, 1);
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? svmax * (1.f / kPGain) / l_tot : 0.f;
  __bf16* orow = p.o + ((int64_t)bh * N + q_row) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int d0 = db * 32 + t * 8 + g * 4;
      typedef float f32x2_t __attribute__((ext_vector_type(2)));
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const f32x2_t a = {oacc[db][4 * t] * inv, oacc[db][4 * t + 1] * inv};
      const f32x2_t b = {oacc[db][4 * t + 2] * inv, oacc[db][4 * t + 3] * inv};
      u32x2_t w = {__builtin_bit_cast(unsigned, __builtin_convertvector(a, bf16x2_t)),
                   __builtin_bit_cast(unsigned, __builtin_convertvector(b, bf16x2_t))};
      *(u32x2_t*)(orow + d0) = w;
    }
  if (g == 0 && p.lse != nullptr) p.lse[(int64_t)bh * N + q_row] = m_run * kLn2 + logf(l_tot);
}

// ---------------------------------------------------------------------------
// Ping-pong variant for d = 64 and 128 (the schedule of attn_fwd_pp.hip):
// one workgroup of 8 wave64 covers 256 query rows; waves w and w + 4 share a
// SIMD; waves 0-3 and 4-7 alternate, one phase apart, between an MFMA phase
// (S_j^T = K8_j Q8^T and O^T += V8_{j-1}^T P8_{j-1}^T) and a softmax phase
// (mask, scale, row max, lazy rescale, P' = exp2(s c + bias) rounded to
// E4M3 against m_ref), with a workgroup barrier between phases.  The MFMA phase also forms
// the row sums of the previous tile's rounded P' (ones x P'^T); the next
// softmax phase adds them, divided by that tile's gain, to l before its own
// rescale, as they are relative to the same running max.  Every wave's 32
// rows lie inside one 128-row Q scale block; a 128-key tile is one K and one
// V scale block.  K8 and V8t tiles are copied by waves 0-3 at the start of
// their MFMA phases, two phases ahead, into two stage objects each: the
// softmax phase is the longer of the two here (64 scores per lane and tile),
// and an LDS-DMA instruction holds its issuing wave until the CU's address
// unit accepts it (about 256 cycles for a 32 KiB pair), which the MFMA phase
// absorbs in its wait at the barrier.

// QR: 0 = Q8 codes and scales from the pre-pass; 1 (bf16) or 2 (fp16) =
// 16-bit Q rotated and quantised in the prologue (see the prologue).
template <int D, bool CAUSAL, int FMT, int QR>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_pp_kernel(F8Params p) {
  constexpr int BN = 128, NT = 512, NTC = 256, BLOCK_M = 256;
  constexpr int NKS = D / 64;        // MFMA K-steps of S
  constexpr int NKB = BN / 32;       // 32-key blocks per tile
  constexpr int NDB = D / 32;        // d blocks of O^T
  constexpr int NPV = BN / 64;       // PV MFMAs (64 keys each) per d block
  constexpr int NOPS = NKB * NKS;    // MFMAs per tile of S^T, and of O^T
  constexpr int LA = 2;              // LDS read-ahead, in MFMA pairs
  constexpr int KRB = D;             // K8 tile row bytes (one key)
  constexpr int VRB = BN;            // V8t tile row bytes (one d)
  constexpr int K_BYTES = BN * KRB;
  constexpr int V_BYTES = D * VRB;
  constexpr int KLOADS = K_BYTES / (NTC * 16);
  constexpr int VLOADS = V_BYTES / (NTC * 16);
  static_assert(NOPS == NDB * NPV, "S and O MFMA counts");
  static_assert(K_BYTES % (NTC * 16) == 0 && V_BYTES % (NTC * 16) == 0, "tile split");

  __shared__ __attribute__((aligned(1024))) char sk0[K_BYTES];
  __shared__ __attribute__((aligned(1024))) char sk1[K_BYTES];
  __shared__ __attribute__((aligned(1024))) char sv0[V_BYTES];
  __shared__ __attribute__((aligned(1024))) char sv1[V_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int N = p.N;

  const int logical = xcd_logical_id(blockIdx.x, p.total);
  const int bh = logical / p.nmb;
  int mb = logical - bh * p.nmb;
  if (CAUSAL) mb = p.nmb - 1 - mb;
  const int m0 = mb * BLOCK_M;
  const int wq0 = m0 + wave * 32;
  const int q_row = wq0 + n;
  const int64_t head = (int64_t)bh * N * D;
  // block scales through the constant address space: read-only for the
  // kernel's lifetime, so uniform reads become scalar loads, which wait on
  // their own counter instead of queueing behind the K/V copies
  typedef __attribute__((address_space(4))) const float cfloat_t;
  cfloat_t* ksc = (cfloat_t*)(p.ks + (int64_t)bh * p.nblk);
  cfloat_t* vsc = (cfloat_t*)(p.vs + (int64_t)bh * p.nblk);
  float svmax = head_max_scale(p.vs + (int64_t)bh * p.nblk, p.nblk, lane);
  if (!(svmax > 0.f)) svmax = 1.f;     // every V block is zero: O = 0
  const float inv_svmax = 1.f / svmax;

  // Q8^T fragments: lane (n, g) holds Q8[q][64 ks + 32 g .. +32]
  i32x8_t qf[NKS];
  float sq_raw = 1.f;
  if constexpr (QR == 0) {
    sq_raw = (wq0 < N) ? p.qs[(int64_t)bh * p.nblk + (wq0 >> 7)] : 1.f;
    const uint8_t* src = p.q8 + head + (int64_t)q_row * D + g * 32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (q_row < N) {
        lo = *(const u32x4_t*)(src + ks * 64);
        hi = *(const u32x4_t*)(src + ks * 64 + 16);
      }
      qf[ks] = cat(lo, hi);
    }
  }
  // (QR != 0) run after the first tile copy has been issued, so that the
  // copy's latency overlaps this work
  auto q_prologue = [&]() __attribute__((always_inline)) {
    // The pre-pass's work on Q, done here on the rows the kernel needs anyway
    // (the "Hadamard in the kernel" of the "FlashAttention-3" page, section
    // "为什么 Hadamard 适合放到内核里"): x~ = H D x over d for each row, then
    // per 128-row block (the four waves of a group) amax = max |x~|,
    // code = E4M3(x~ * 448 / amax), scale = amax / (448 sqrt(d)) -- the same
    // arithmetic as hadamard_quant.hip, in the lane layout of the B operand:
    // element e of lane (n, g)'s fragment ks is d index 64 ks + 32 g + e.
    // The transform is unnormalised; its butterfly stages run over the bits
    // of e in the lane, over ks across fragments and over g across lanes
    // n and n + 32.  (The stages commute, so the order of summation differs
    // from the pre-pass and the rotated values may differ in the last bit.)
    using QT = std::conditional_t<QR == 1, __bf16, _Float16>;
    constexpr float QMAX = FMT == 0 ? 448.f : 57344.f;
    const int b_ = bh / p.H, h_ = bh - b_ * p.H;
    const char* src = p.qx + ((int64_t)b_ * p.qsb + (int64_t)h_ * p.qsh + (int64_t)q_row * p.qsn) * 2 + g * 64;
    float x[NKS][32];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        u32x4_t raw = {0u, 0u, 0u, 0u};
        if (q_row < N) raw = *(const u32x4_t*)(src + ks * 128 + l * 16);
        const QT* e = reinterpret_cast<const QT*>(&raw);
        u32x2_t sraw = *(const u32x2_t*)(p.signs + ks * 64 + g * 32 + l * 8);
        const int8_t* sg = reinterpret_cast<const int8_t*>(&sraw);
#pragma unroll
        for (int t = 0; t < 8; ++t) x[ks][l * 8 + t] = q_to_f32<QT>(e[t]) * (float)sg[t];
      }
#pragma unroll
    for (int hh = 1; hh < 32; hh <<= 1)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 32; ++e)
          if ((e & hh) == 0) {
            const float a = x[ks][e], c = x[ks][e + hh];
            x[ks][e] = a + c;
            x[ks][e + hh] = a - c;
          }
    if constexpr (NKS == 2) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float a = x[0][e], c = x[1][e];
        x[0][e] = a + c;
        x[1][e] = a - c;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float o = __shfl_xor(x[ks][e], 32);
        x[ks][e] = g ? o - x[ks][e] : x[ks][e] + o;
        amax = fmaxf(amax, fabsf(x[ks][e]));
      }
    __shared__ float qred[8];
    amax = wave_max64(amax);
    if (lane == 0) qred[wave] = amax;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    phase_barrier();
    const int w0 = wave & 4;               // the group's four waves: one 128-row scale block
    amax = fmaxf(fmaxf(qred[w0], qred[w0 + 1]), fmaxf(qred[w0 + 2], qred[w0 + 3]));
    sq_raw = amax * (1.f / sqrtf((float)D)) / QMAX;   // 0 for a zero block
    const float ramax = amax > 0.f ? 1.f / amax : 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float a = x[ks][4 * w + t] * QMAX;
          const float y0 = a * ramax;
          const float q = fmaf(fmaf(-y0, amax, a), ramax, y0);
          y[t] = fminf(fmaxf(q, -QMAX), QMAX);
        }
        if constexpr (FMT == 0) {
          const unsigned lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          qf[ks][w] = (int)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
        } else {
          const unsigned lo = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
          qf[ks][w] = (int)__builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], lo, true);
        }
      }
  };

  // copies by the 256 threads of group 0
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k8 + head), (short)0, N * D, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v8t + head), (short)0, N * D, 0x00020000);
  const int tg = tid & (NTC - 1);
  int koff[KLOADS], voff[VLOADS];
#pragma unroll
  for (int t = 0; t < KLOADS; ++t) {
    const int pos = (t * NTC + tg) * 16, row = pos / KRB;
    koff[t] = row * D + (((pos % KRB) / 16) ^ swz_k<KRB>(row)) * 16;
  }
#pragma unroll
  for (int t = 0; t < VLOADS; ++t) {
    const int pos = (t * NTC + tg) * 16, row = pos / VRB;
    voff[t] = row * N + (((pos % VRB) / 16) ^ swz_v<VRB>(row)) * 16;
  }

  const int krow = key_of_row8(n);
  int kaddr[NKS][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      kaddr[ks][hf] = krow * KRB + (((4 * ks + 2 * g + hf) ^ swz_k<KRB>(krow)) * 16);
  int vaddr[NPV][2];
#pragma unroll
  for (int t = 0; t < NPV; ++t)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      vaddr[t][hf] = n * VRB + (((4 * t + 2 * hf + g) ^ swz_v<VRB>(n)) * 16);

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;   // reference of O and l
  float m_ref = -INFINITY;   // reference of P': ceil of the running row max
  float l_run = 0.f;

  const int kv_end = CAUSAL ? min(N, m0 + BLOCK_M) : N;
  const int n_tiles = kv_end / BN;     // N is a multiple of 128
  const int w_tiles = (wq0 >= N) ? 0 : (CAUSAL ? min(n_tiles, (wq0 + 31) / BN + 1) : n_tiles);
  float c0 = 0.f;   // sq * scale * log2(e), set once Q's scale is known

  f32x16_t sacc[NKB];
  i32x8_t pf[NPV];
#pragma unroll
  for (int t = 0; t < NPV; ++t)
#pragma unroll
    for (int w = 0; w < 8; ++w) pf[t][w] = 0;
  // row sums of P' by MFMA: E4M3 ones (0x38) as the A operand; every row of
  // the 32x32 result holds the column (query) sums of the P' in pf, over all
  // 64 keys of each product, so l_run is the full row sum in both lane groups
  i32x8_t ones;
#pragma unroll
  for (int w = 0; w < 8; ++w) ones[w] = 0x38383838;
  f32x16_t lacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) lacc[i] = 0.f;
  float inv_gain_prev = 0.f;     // 1 / (kPGain * fv) of the tile whose P' is in pf
  int psc_prev = 127;            // E8M0 scale 2^(m_ref - m_run) of the P' in pf

  // MFMA phase: S^T of tile j and O^T += V^T P^T of tile j-1, operands read
  // LA MFMA pairs ahead; pair i = S block i % NKB, K-step i / NKB and O block
  // i % NDB, key half i / NDB.
  auto phase_mfma = [&](const char* kst, const char* vst) __attribute__((always_inline)) {
    i32x8_t kf[NOPS], vf[NOPS];
    auto load = [&](int i) __attribute__((always_inline)) {
      const char* kb_ = kst + (i % NKB) * 32 * KRB;
      kf[i] = cat(*(const lds_u32x4_t*)(kb_ + kaddr[i / NKB][0]), *(const lds_u32x4_t*)(kb_ + kaddr[i / NKB][1]));
      const char* vb_ = vst + (i % NDB) * 32 * VRB;
      vf[i] = cat(*(const lds_u32x4_t*)(vb_ + vaddr[i / NDB][0]), *(const lds_u32x4_t*)(vb_ + vaddr[i / NDB][1]));
    };
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int i = 0; i < LA && i < NOPS; ++i) load(i);
#pragma unroll
    for (int i = 0; i < NOPS; ++i) {
      if (i + LA < NOPS) load(i + LA);
      sacc[i % NKB] = mfma_fp8<FMT, FMT>(kf[i], qf[i / NKB], sacc[i % NKB]);
      oacc[i % NDB] = mfma_fp8_sb<FMT, 0>(vf[i], pf[i / NDB], oacc[i % NDB], psc_prev);
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      f32x16_t z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.f;
      lacc = mfma_fp8_sb<0, 0>(ones, pf[0], z, psc_prev);
#pragma unroll
      for (int t = 1; t < NPV; ++t) lacc = mfma_fp8_sb<0, 0>(ones, pf[t], lacc, psc_prev);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // K and V block scales of the next softmax phase's tile, loaded a phase
  // ahead: loaded in the phase that uses them, the wave would wait out the L2
  // latency, which the K/V copies in flight raise to several hundred cycles
  float ks_next = ksc[0], vs_next = vsc[0];

  // softmax phase of tile j (this wave needs it)
  auto phase_softmax = [&](int j) __attribute__((always_inline)) {
    const int kt0 = j * BN;
    const float c = c0 * (ks_next > 0.f ? ks_next : 1.f);
    const float fv = vs_next > 0.f ? vs_next * inv_svmax : 1.f;     // in (0, 1]
    {
      const int jn = j + 1 < w_tiles ? j + 1 : j;
      ks_next = ksc[jn];
      vs_next = vsc[jn];
    }
    if (CAUSAL && kt0 + BN - 1 > wq0) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt0 + kb * 32 + 16 * g + i;
          if (key > q_row) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    const float m_tile = pair_max(mx) * c;
    l_run = fmaf(lacc[0], inv_gain_prev, l_run);   // previous tile, same m_run as its P'
    if (__any(m_tile > m_run + kTau8)) {
      const float m_new = ceilf(fmaxf(m_run, m_tile));   // whole number (or -inf)
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)(m_run - m_new));
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      m_run = m_new;
    }
    m_ref = fmaxf(m_ref, ceilf(m_tile));
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    const float bias = __builtin_amdgcn_logf(kPGain * fv) - m_use;   // v_log_f32 is log2
    inv_gain_prev = __builtin_amdgcn_rcpf(kPGain * fv);
    psc_prev = ref_scale(m_ref, m_run);
#pragma unroll
    for (int t = 0; t < NPV; ++t)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = 2 * t + (w >> 2);
        const int i0 = (w & 3) * 4;
        const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i0], c, bias));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i0 + 1], c, bias));
        const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i0 + 2], c, bias));
        const float e3 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i0 + 3], c, bias));
        const unsigned lo = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, pf[t][w], false);
        pf[t][w] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, lo, true);
      }
  };

  // pair j = K8 tile j (j < n_tiles) and V8t tile j-1 (j >= 1), into stage ST
  auto copy_pair = [&](int j, auto st_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    if (j < n_tiles) dma<KLOADS, NTC>(krs, ST ? sk1 : sk0, wave & 3, j * BN * D, koff);
    if (j >= 1) dma<VLOADS, NTC>(vrs, ST ? sv1 : sv0, wave & 3, (j - 1) * BN, voff);
  };

  // Phase t (t % 4 == TM) of group G: local phase u = t - G; even u = MFMA
  // phase A_{u/2} reading pair u/2 from stage (u/2) & 1, odd u = softmax
  // phase B_{(u-1)/2}.  Pair j is copied during phase 2j-2 (by group 0) and
  // waited for at the end of phase 2j-1.
  auto run = [&](auto g_c) __attribute__((always_inline)) {
    constexpr int G = decltype(g_c)::value;
    auto phase = [&](int t, auto tm_c) __attribute__((always_inline)) {
      constexpr int TM = decltype(tm_c)::value;
      if constexpr ((TM & 1) == 0 && G == 0) {
        const int j = t / 2 + 1;
        if (j <= n_tiles) copy_pair(j, ic<(TM == 0) ? 1 : 0>{});
      }
      const int u = t - G;
      if (u >= 0 && u <= 2 * n_tiles) {
        const int j = u >> 1;
        if constexpr (((TM - G) & 1) == 0) {
          // both products run whenever either is needed (fixed registers for
          // S and O); in the first phase P is zero and V stage 0 zero-filled
          constexpr int AST = TM >> 1;
          if (j <= w_tiles) phase_mfma(AST ? sk1 : sk0, AST ? sv1 : sv0);
        } else if (j < w_tiles) {
          phase_softmax(j);
        }
      }
      if constexpr ((TM & 1) == 1) wait_vmem();
      if (t < 2 * n_tiles + 1) phase_barrier();
    };
    for (int t = 0; t < 2 * n_tiles + 2; t += 4) {
      phase(t, ic<0>{});
      phase(t + 1, ic<1>{});
      if (t + 2 < 2 * n_tiles + 2) {
        phase(t + 2, ic<2>{});
        phase(t + 3, ic<3>{});
      }
    }
  };

  if (group == 0) copy_pair(0, ic<0>{});
#pragma unroll
  for (int c = 0; c < V_BYTES / (NT * 16); ++c) *(lds_u32x4_t*)(sv0 + (c * NT + tid) * 16) = u32x4_t{0u, 0u, 0u, 0u};
  if constexpr (QR != 0) q_prologue();
  c0 = (sq_raw > 0.f ? sq_raw : 1.f) * p.scale_log2;
  wait_vmem();
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the zero-fill has landed
  phase_barrier();
  if (group == 0) run(ic<0>{});
  else run(ic<1>{});
  l_run = fmaf(lacc[0], inv_gain_prev, l_run);   // the last tile

  const float l_tot = l_run;
  if (q_row < N) {
    const float inv = l_tot > 0.f ? svmax * (1.f / kPGain) / l_tot : 0.f;
    __bf16* orow = p.o + ((int64_t)bh * N + q_row) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int d0 = db * 32 + t * 8 + g * 4;
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const f32x2_t a = {oacc[db][4 * t] * inv, oacc[db][4 * t + 1] * inv};
        const f32x2_t b = {oacc[db][4 * t + 2] * inv, oacc[db][4 * t + 3] * inv};
        u32x2_t w = {__builtin_bit_cast(unsigned, __builtin_convertvector(a, bf16x2_t)),
                     __builtin_bit_cast(unsigned, __builtin_convertvector(b, bf16x2_t))};
        *(u32x2_t*)(orow + d0) = w;
      }
    if (g == 0 && p.lse != nullptr) p.lse[(int64_t)bh * N + q_row] = m_run * kLn2 + logf(l_tot);
  }
}

template <int D, bool CAUSAL, int FMT, int QR>
hipError_t launch_pp(const Fp8FwdArgs& a, hipStream_t s) {
  constexpr int BLOCK_M = 256;
  F8Params p;
  p.q8 = a.q8;
  p.k8 = a.k8;
  p.v8t = a.v8t;
  p.qs = a.q_scale;
  p.ks = a.k_scale;
  p.vs = a.v_scale;
  p.o = static_cast<__bf16*>(a.o);
  p.lse = a.lse;
  p.H = a.H;
  p.N = a.N;
  p.nmb = (a.N + BLOCK_M - 1) / BLOCK_M;
  p.total = a.B * a.H * p.nmb;
  p.nblk = a.N / a.block_rows;
  p.scale_log2 = a.scale * kLog2e;
  p.qx = static_cast<const char*>(a.qx);
  p.signs = a.signs;
  p.qsb = a.qsb;
  p.qsh = a.qsh;
  p.qsn = a.qsn;
  hipLaunchKernelGGL((attn_fwd_fp8_pp_kernel<D, CAUSAL, FMT, QR>), dim3(p.total), dim3(512), 0, s, p);
  return hipGetLastError();
}

template <int D, int BN, bool CAUSAL, int FMT>
hipError_t launch_one(const Fp8FwdArgs& a, hipStream_t s) {
  constexpr int BLOCK_M = 128;
  F8Params p;
  p.q8 = a.q8;
  p.k8 = a.k8;
  p.v8t = a.v8t;
  p.qs = a.q_scale;
  p.ks = a.k_scale;
  p.vs = a.v_scale;
  p.o = static_cast<__bf16*>(a.o);
  p.lse = a.lse;
  p.H = a.H;
  p.N = a.N;
  p.nmb = a.N / BLOCK_M;
  p.total = a.B * a.H * p.nmb;
  p.nblk = a.N / a.block_rows;
  p.scale_log2 = a.scale * kLog2e;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, BN, CAUSAL, FMT>), dim3(p.total), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D, int BN, int FMT>
hipError_t launch_mask(const Fp8FwdArgs& a, hipStream_t s) {
  return a.causal ? launch_one<D, BN, true, FMT>(a, s) : launch_one<D, BN, false, FMT>(a, s);
}

template <int FMT>
hipError_t launch_fmt(const Fp8FwdArgs& a, hipStream_t stream, bool* supported) {
  if (a.qx) {   // Q rotated and quantised in the ping-pong kernel's prologue
    auto go = [&](auto qr) -> hipError_t {
      constexpr int QR = decltype(qr)::value;
      switch (a.d) {
        case 64: return a.causal ? launch_pp<64, true, FMT, QR>(a, stream) : launch_pp<64, false, FMT, QR>(a, stream);
        case 128: return a.causal ? launch_pp<128, true, FMT, QR>(a, stream) : launch_pp<128, false, FMT, QR>(a, stream);
      }
      *supported = false;
      return hipSuccess;
    };
    if (a.q_dtype == Dtype::BF16) return go(ic<1>{});
    if (a.q_dtype == Dtype::F16) return go(ic<2>{});
    *supported = false;
    return hipSuccess;
  }
  switch (a.d) {
    case 64: return a.causal ? launch_pp<64, true, FMT, 0>(a, stream) : launch_pp<64, false, FMT, 0>(a, stream);
    case 128: return a.causal ? launch_pp<128, true, FMT, 0>(a, stream) : launch_pp<128, false, FMT, 0>(a, stream);
    case 256: return launch_mask<256, 64, FMT>(a, stream);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream, bool* supported) {
  *supported = true;
  if (a.block_rows != 128 || a.N % 128 != 0) {
    *supported = false;
    return hipSuccess;
  }
  switch (a.fp8_format) {
    case 0: return launch_fmt<0>(a, stream, supported);
    case 1: return launch_fmt<1>(a, stream, supported);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace attn
