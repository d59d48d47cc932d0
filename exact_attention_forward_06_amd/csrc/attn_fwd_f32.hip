// Exact-attention forward for gfx950, fp32 inputs (the 16-bit types have
// their own kernels in attn_fwd_pp.hip and attn_fwd_pair.hip): fp32 MFMA and
// accumulation, causal or non-causal, per-row logsumexp output.
//
// Method (see include/attn.h for the sources on the pages): the grid runs
// over (batch, head, block of 128 query rows) -- the "outer loop over Q
// blocks" of the FlashAttention-2 work partition ("FlashAttention-2/3" page,
// FlashAttention-2 改进二) -- and each workgroup streams the K/V blocks of its
// head through LDS, keeping the running row max m, running row sum l and the
// unnormalised output in registers; O is divided by l once after the last
// block (改进一) and LSE = m + ln l is stored.
//
// gfx950 mapping
//  * One wave64 owns 32 query rows.  It computes S^T = K Q^T with
//    v_mfma_f32_32x32x2f32 (A = one K element per lane from LDS, B = one
//    element of Q^T held in VGPRs for the whole loop), so the accumulator
//    gives each lane ONE query (lane & 31) and 16 of the tile's keys; the
//    other 16 keys of that query sit in lane ^ 32.  Row max and row sum are
//    in-lane reductions plus one v_permlane32_swap.
//  * The key order inside a 32-key block is permuted (bits 2 and 3 of the
//    A-operand row swapped, as in the 16-bit kernels), so accumulator
//    register i of lane group g holds key key_of_reg(i, g).
//  * O^T += V^T P^T takes P straight from the S^T accumulator (one element
//    per MFMA); V stays in its natural [key][d] layout in LDS.
//  * K/V tiles are double-buffered in LDS: the buffer loads of tile j+1 are
//    issued before the MFMAs of tile j and written to the other buffer after
//    them, one barrier per tile.  Row pitches are padded by 16 bytes so the
//    per-lane row reads of one MFMA operand fall in different banks.  Rows
//    at or past N read as zero (the buffer range check).
//  * Causal: K/V tiles wholly above the diagonal of the workgroup's rows are
//    never loaded; a wave whose rows all precede a tile skips its math; the
//    element mask is applied only where a tile straddles the diagonal or the
//    ragged end of the sequence.
//  * Workgroup ids are remapped so that consecutive Q blocks of a head land
//    on the same XCD, and under the causal mask the Q blocks with the most
//    K/V tiles are issued first.
#include "attn16_common.h"
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace attn {
namespace {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1, 2)))
void attn_fwd_f32_kernel(Params p) {
  constexpr int BN = 32, WAVES = 4, NT = WAVES * 64, BLOCK_M = WAVES * 32;
  constexpr int NKS = D / 2;                // K-steps of S^T = K Q^T (2 per MFMA)
  constexpr int NDB = D / 32;               // 32-wide d blocks of O^T
  constexpr int PITCH = D * 4 + 16;         // LDS row pitch of K and V
  constexpr int K_BYTES = BN * PITCH;
  constexpr int STAGE = 2 * K_BYTES;
  constexpr int CH_ROW = D * 4 / 16;        // 16-byte chunks per row
  constexpr int PER_T = BN * CH_ROW / NT;   // chunks per thread per tile (K, and V)
  static_assert((BN * CH_ROW) % NT == 0, "tile split");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;     // query column of this lane / A-operand row
  const int g = lane >> 5;     // lane group: k half of the operands
  const int N = p.N;

  const int logical = xcd_logical_id(blockIdx.x, p.total);
  const int bh = logical / p.nmb;
  int mb = logical - bh * p.nmb;
  if (CAUSAL) mb = p.nmb - 1 - mb;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int m0 = mb * BLOCK_M;
  const int wq0 = m0 + wave * 32;
  const int q_row = wq0 + n;
  const int64_t head_off = ((int64_t)b * p.sb + (int64_t)h * p.sh) * 4;
  const int rb = (int)(p.sn * 4);          // global row pitch in bytes

  // Q^T fragments (B operand): lane (n, g) holds Q[q][2 ks + g]
  float qf[NKS];
  {
    const float* src = (const float*)(p.q + head_off + (int64_t)q_row * rb);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = (q_row < N) ? src[2 * ks + g] : 0.f;
  }

  const int64_t extent = ((int64_t)(N - 1) * p.sn + D) * 4;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + head_off), (short)0, (int)extent, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + head_off), (short)0, (int)extent, 0x00020000);

  u32x4_t kreg[PER_T], vreg[PER_T];
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int t = 0; t < PER_T; ++t) {
      const int c = tid + t * NT;
      const int off = (kt0 + c / CH_ROW) * rb + (c % CH_ROW) * 16;
      kreg[t] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
      vreg[t] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
    }
  };
  auto store_tile = [&](int stage) {
    char* sK = smem + stage * STAGE;
#pragma unroll
    for (int t = 0; t < PER_T; ++t) {
      const int c = tid + t * NT;
      const int off = (c / CH_ROW) * PITCH + (c % CH_ROW) * 16;
      *(u32x4_t*)(sK + off) = kreg[t];
      *(u32x4_t*)(sK + K_BYTES + off) = vreg[t];
    }
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;   // running max of scale*log2(e)*s (possibly stale by < kTau)
  float l_run = 0.f;         // this lane's half of the running row sum

  const int kv_end = CAUSAL ? min(N, m0 + BLOCK_M) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const float c = p.scale_log2;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int stage = j & 1;
    const int kt0 = j * BN;
    const bool more = (j + 1) < n_tiles;
    if (more) load_tile(kt0 + BN);

    const bool active = (wq0 < N) && (!CAUSAL || kt0 <= wq0 + 31);
    if (active) {
      const char* sK = smem + stage * STAGE;
      const char* sV = sK + K_BYTES;

      // S^T = K Q^T
      f32x16_t sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      const float* arow = (const float*)(sK + key_of_row(n) * PITCH) + g;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(arow[2 * ks], qf[ks], sacc, 0, 0, 0);

      // mask: ragged end of the sequence, and keys after the query (causal)
      const bool need_mask = (kt0 + BN > N) || (CAUSAL && kt0 + BN - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt0 + key_of_reg(i, g);
          if ((key >= N) || (CAUSAL && key > q_row)) sacc[i] = -INFINITY;
        }
      }

      // online softmax update (log2 domain), lazy rescale: the running max
      // only moves when a row's tile max exceeds it by more than kTau; O and
      // l share the reference, so the result is unchanged
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      const float m_tile = pair_max(mx) * c;
      if (__any(m_tile > m_run + kTau)) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i], c, -m_use));
        rs += sacc[i];
      }
      l_run += rs;

      // O^T += V^T P^T, one key per MFMA
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float a = *(const float*)(sV + key_of_reg(i, g) * PITCH + (db * 32 + n) * 4);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sacc[i], oacc[db], 0, 0, 0);
        }
    }

    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // epilogue: O = O / l, LSE = m ln2 + ln l
  const float l_tot = pair_sum(l_run);
  if (q_row < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = (float*)(p.o + (((int64_t)bh * N + q_row) * D) * 4);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int d0 = db * 32 + t * 8 + g * 4;
        *(f32x4_t*)(orow + d0) = f32x4_t{oacc[db][4 * t] * inv, oacc[db][4 * t + 1] * inv,
                                         oacc[db][4 * t + 2] * inv, oacc[db][4 * t + 3] * inv};
      }
    if (g == 0 && p.lse != nullptr) p.lse[(int64_t)bh * N + q_row] = m_run * kLn2 + logf(l_tot);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  constexpr int BLOCK_M = 128;
  Params p;
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.o = static_cast<char*>(a.o);
  p.lse = a.lse;
  p.sb = a.sb;
  p.sh = a.sh;
  p.sn = a.sn;
  p.H = a.H;
  p.N = a.N;
  p.nmb = (a.N + BLOCK_M - 1) / BLOCK_M;
  p.total = a.B * a.H * p.nmb;
  p.scale_log2 = a.scale * kLog2e;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3(p.total), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// fp32 attention forward (v_mfma_f32_32x32x2f32; V in natural layout).
hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t s, bool* ok) {
  *ok = true;
  auto go = [&](auto dc) -> hipError_t {
    constexpr int D = decltype(dc)::value;
    return a.causal ? launch_one<D, true>(a, s) : launch_one<D, false>(a, s);
  };
  switch (a.d) {
    case 64: return go(std::integral_constant<int, 64>{});
    case 128: return go(std::integral_constant<int, 128>{});
    case 256: return go(std::integral_constant<int, 256>{});
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace attn
