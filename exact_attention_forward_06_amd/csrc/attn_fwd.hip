// Exact-attention forward for gfx950, fp16 / bf16 inputs with d = 256: fp32
// accumulation, causal or non-causal, per-row logsumexp output.  (d = 64 and
// 128 run the 8-wave ping-pong kernel of attn_fwd_pp.hip, which shares this
// file's operand layouts; fp32 inputs use attn_fwd_f32.hip.)
//
// Method (sources on the pages are listed in include/attn.h): the grid runs
// over (batch, head, block of 128 query rows) -- the "outer loop over Q
// blocks" of the FlashAttention-2 work partition ("FlashAttention-2/3" page,
// FlashAttention-2 改进二) -- and each workgroup streams the K/V blocks of its
// head through LDS, keeping the running row max m, the running row sum l and
// the unnormalised output in registers; O is divided by l once after the
// last block (改进一) and LSE = m + ln l is stored.
//
// gfx950 mapping
//  * 4 wave64 per workgroup, 32 query rows per wave, two workgroups per CU
//    (<= 256 VGPRs, 64 KiB LDS each) so every SIMD runs two independent waves:
//    one wave's softmax VALU work issues while the other's MFMAs run.  (d=256
//    needs more than 256 VGPRs and runs one wave per SIMD.)
//  * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16} with Q^T resident in
//    VGPRs.  A lane's accumulator holds ONE query (lane & 31) and 16 of the
//    tile's keys (the other 16 in lane ^ 32): row max / row sum are in-lane
//    plus one v_permlane32_swap -- no LDS, each wave owns its rows (the
//    page's "split Q across warps" partition, 改进三).
//  * K rows are fed to that MFMA in a permuted order (bits 2 and 3 of the
//    A-operand row swapped) so accumulator registers 8c..8c+7 hold 8
//    consecutive keys; rounded to 16 bits they are directly the P^T operand
//    of O^T += V^T P^T.  P never leaves VGPRs.
//  * K and V tiles go global -> LDS with buffer_load_dwordx4 ... lds (no
//    VGPR staging), double-buffered: the loads of tile j+1 are issued before
//    the MFMAs of tile j.  Rows past N read as zero (buffer range check).
//  * V stays in its natural [key][d] layout in LDS; the V^T operand is read
//    with ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-d block
//    and receives it transposed: one d per lane, 4 consecutive keys).
//  * LDS rows are unpadded (the LDS-DMA writes 1 KiB per instruction
//    contiguously), so 16-byte chunks are XOR-swizzled within a row; the
//    swizzle makes both the K operand reads (16 rows, one chunk) and the
//    transposed V reads (4 rows x 4 chunks) hit distinct banks.
//  * Online softmax in the log2 domain with a lazy rescale: the running max
//    only moves when a row's tile max exceeds it by more than 2^8, so
//    P <= 256 and the O rescale is skipped on almost every tile.  Row sums
//    are accumulated from the fp32 P (the LSE keeps fp32 accuracy).
//  * Causal: K/V tiles wholly above the workgroup's diagonal are never
//    loaded; a wave whose rows all precede a tile skips its math; the element
//    mask runs only where a tile straddles the diagonal or the end of the
//    sequence.
//  * Workgroup ids are remapped so that the Q blocks of a head run on one
//    XCD (the head's K/V is then re-read from that XCD's L2); under the
//    causal mask the Q blocks with the most K/V tiles are issued first.
#include "attn16_common.h"
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace attn {

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t s, bool* ok);
hipError_t launch_attn_fwd16_pp(const FwdArgs& a, hipStream_t s, bool* ok);

namespace {

template <typename T, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1, 2)))
void attn_fwd16_kernel(Params p) {
  using Op = Ops<T>;
  using frag = typename Op::frag;
  constexpr int NT = 256, BLOCK_M = 128;
  constexpr int RB = D * 2;                // LDS row bytes (K and V)
  constexpr int TILE = BN * RB;            // bytes of one K (or V) tile
  constexpr int NKS = D / 16;              // K-steps of S^T = K Q^T
  constexpr int NKB = BN / 32;             // 32-key blocks per tile
  constexpr int NDB = D / 32;              // 32-wide d blocks of O^T
  constexpr int NCC = BN / 16;             // 16-key chunks per tile (PV K-steps)
  constexpr int LOADS = TILE / (NT * 16);  // LDS-DMA instructions per thread per tile
  static_assert(TILE % (NT * 16) == 0 && RB % 16 == 0, "tile split");
  static_assert(4 * TILE <= 65536, "LDS budget: two workgroups per CU");

  // Software pipeline over K/V tiles: iteration j issues the S MFMAs of tile
  // j+1 next to the exp / pack VALU work of tile j, then the PV MFMAs of
  // tile j next to the row max of tile j+1.  K therefore runs one tile ahead
  // of V: iteration j reads K_{j+1} and V_j and copies K_{j+2}, V_{j+1} into
  // the stages those two freed at the previous barrier.  Each stage is its
  // own LDS object, so reads of one are never made to wait for the in-flight
  // copies into another.
  __shared__ __attribute__((aligned(1024))) char sk0[TILE];
  __shared__ __attribute__((aligned(1024))) char sk1[TILE];
  __shared__ __attribute__((aligned(1024))) char sv0[TILE];
  __shared__ __attribute__((aligned(1024))) char sv1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int n = lane & 31;
  const int g = lane >> 5;
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
  const int64_t head_off = ((int64_t)b * p.sb + (int64_t)h * p.sh) * 2;
  const int rbg = (int)(p.sn * 2);         // global row pitch in bytes

  // Q^T fragments (B operand): lane (n, g) holds Q[q][16 ks + 8 g .. + 8]
  frag qf[NKS];
  {
    const char* src = p.q + head_off + (int64_t)q_row * rbg + g * 16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (q_row < N) raw = *(const u32x4_t*)(src + ks * 32);
      qf[ks] = __builtin_bit_cast(frag, raw);
    }
  }

  // K/V global -> LDS.  DMA instruction t of this wave writes LDS bytes
  // [(t*NT + wave*64) * 16, +1024) of the tile; lane l's 16 bytes land at
  // row P / RB, physical chunk (P % RB) / 16, which holds logical chunk
  // physical ^ swz(row).
  const int64_t extent = ((int64_t)(N - 1) * p.sn + D) * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + head_off), (short)0, (int)extent, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + head_off), (short)0, (int)extent, 0x00020000);
  int dma_off[LOADS];          // global byte offset of this lane's chunk, tile-relative
#pragma unroll
  for (int t = 0; t < LOADS; ++t) {
    const int pos = (t * NT + tid) * 16;
    const int row = pos / RB;
    const int chunk = ((pos % RB) / 16) ^ swz<D>(row);
    dma_off[t] = row * rbg + chunk * 16;
  }
  auto copy_k = [&](int tile, int stage) __attribute__((always_inline)) {
    dma_tile<LOADS, NT>(krs, stage ? sk1 : sk0, wave, tile * BN * rbg, dma_off);
  };
  auto copy_v = [&](int tile, int stage) __attribute__((always_inline)) {
    dma_tile<LOADS, NT>(vrs, stage ? sv1 : sv0, wave, tile * BN * rbg, dma_off);
  };

  // LDS read addresses.  K A-operand for (kb, ks): row kb*32 + key_of_row(n),
  // logical chunk 2 ks + g.  V^T A-operand (tr16): 16-lane group hq covers d
  // in [16 (hq & 1), +16) of a 32-wide d block and keys 8 (hq >> 1) + 4 half
  // + e; lane j = 4 e + a of the group addresses d columns 4a .. 4a + 3.
  // Every read is a per-lane address plus a compile-time offset.
  const int krow = key_of_row(n);
  const int kswz = swz<D>(krow);
  const int hq = lane >> 4, jj = lane & 15, ta = jj & 3, te = jj >> 2;
  const int vg = hq >> 1;
  const int vcol0 = (hq & 1) * 16 + 4 * ta;
  int kaddr[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) kaddr[ks] = krow * RB + (((2 * ks + g) ^ kswz) * 16);
  int vaddr[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = vg * 8 + half * 4 + te;      // + cc*16 (does not change row & 15)
      const int col = db * 32 + vcol0;
      vaddr[db][half] = row * RB + (((col >> 3) ^ swz<D>(row)) * 16) + (col & 7) * 2;
    }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;   // whole-number running max of scale * log2(e) * s (possibly stale by < kTau)
  float l_run = 0.f;         // this lane's half of the running row sum

  const int kv_end = CAUSAL ? min(N, m0 + BLOCK_M) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  // last tile this wave needs (causal: keys up to its last row)
  const int w_tiles = (wq0 >= N) ? 0 : (CAUSAL ? min(n_tiles, (wq0 + 31) / BN + 1) : n_tiles);
  const float c = p.scale_log2;

  // S^T = K Q^T of one tile from K stage `ks_lds`
  auto qk = [&](f32x16_t (&sacc)[NKB], const char* ks_lds) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const frag a = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(ks_lds + kb * 32 * RB + kaddr[ks]));
        sacc[kb] = Op::mfma(a, qf[ks], sacc[kb]);
      }
    }
  };
  // mask keys past the end of the sequence / after the query, then the row
  // max of the tile in log2 units
  auto tile_max = [&](f32x16_t (&sacc)[NKB], int kt0) __attribute__((always_inline)) -> float {
    const bool need_mask = (kt0 + BN > N) || (CAUSAL && kt0 + BN - 1 > wq0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt0 + kb * 32 + key_of_reg(i, g);
          if ((key >= N) || (CAUSAL && key > q_row)) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    return pair_max(mx) * c;
  };
  // lazy rescale: move the running max only when the tile max exceeds it by
  // more than kTau (then P = exp2(s c - m_run) <= 2^kTau)
  auto update_max = [&](float m_tile) __attribute__((always_inline)) {
    if (__any(m_tile > m_run + kTau)) {
      // whole numbers: the rescale is an exact power of two, and P is rounded
      // to 16 bits on a grid that does not depend on where the running max
      // happened to lie (so other tilings of the keys round P identically)
      const float m_new = ceilf(fmaxf(m_run, m_tile));
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)(m_run - m_new));
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      m_run = m_new;
    }
  };
  // P of one tile rounded to 16 bits (the P^T operand); row sums of the fp32 P
  auto softmax_p = [&](f32x16_t (&sacc)[NKB], frag (&pf)[NCC]) __attribute__((always_inline)) {
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      const int kb = cc >> 1, base = (cc & 1) * 8;
      u32x4_t w;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][base + 2 * t], c, -m_use));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][base + 2 * t + 1], c, -m_use));
        w[t] = Op::pack2(e0, e1);
        rs0 += e0;
        rs1 += e1;
      }
      pf[cc] = __builtin_bit_cast(frag, w);
    }
    l_run += rs0 + rs1;
  };
  // O^T += V^T P^T from V stage `vs_lds`
  auto pv = [&](const frag (&pf)[NCC], const char* vs_lds) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vs_lds + cc * 16 * RB + vaddr[db][0]));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vs_lds + cc * 16 * RB + vaddr[db][1]));
        u32x4_t w;
        w[0] = __builtin_bit_cast(u32x2_t, lo)[0];
        w[1] = __builtin_bit_cast(u32x2_t, lo)[1];
        w[2] = __builtin_bit_cast(u32x2_t, hi)[0];
        w[3] = __builtin_bit_cast(u32x2_t, hi)[1];
        oacc[db] = Op::mfma(__builtin_bit_cast(frag, w), pf[cc], oacc[db]);
      }
  };

  f32x16_t sA[NKB], sB[NKB];
  frag pf[NCC];

  // prologue: K_0, K_1, V_0 resident; S_0 and its max
  copy_k(0, 0);
  if (n_tiles > 1) copy_k(1, 1);
  copy_v(0, 0);
  wait_vmem();
  __syncthreads();
  if (w_tiles > 0) {
    qk(sA, sk0);
    update_max(tile_max(sA, 0));
  }
  __syncthreads();   // every wave is done with K stage 0 before K_2 lands there

  // iteration j: S_j is in `cur`; K_{j+1} in K stage (j+1)&1, V_j in V stage j&1
  auto step = [&](int j, int st, f32x16_t (&cur)[NKB], f32x16_t (&nxt)[NKB]) __attribute__((always_inline)) {
    if (j + 2 < n_tiles) copy_k(j + 2, st);
    if (j + 1 < n_tiles) copy_v(j + 1, st ^ 1);
    if (j < w_tiles) {
      // S_{j+1} MFMAs next to the exp / pack of P_j (S_{j+1} past the last
      // tile reads a stale, in-bounds stage and is not used)
      qk(nxt, st ? sk0 : sk1);
      softmax_p(cur, pf);
      // PV_j next to the row max of S_{j+1}
      pv(pf, st ? sv1 : sv0);
      if (j + 1 < w_tiles) update_max(tile_max(nxt, (j + 1) * BN));
    }
    wait_vmem();
    __syncthreads();
  };
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, 0, sA, sB);
    if (j + 1 < n_tiles) step(j + 1, 1, sB, sA);
  }

  // epilogue: O = O / l, LSE = m ln2 + ln l
  const float l_tot = pair_sum(l_run);
  if (q_row < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* orow = p.o + (((int64_t)bh * N + q_row) * D) * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int d0 = db * 32 + t * 8 + g * 4;
        u32x2_t w = {Op::pack2(oacc[db][4 * t] * inv, oacc[db][4 * t + 1] * inv),
                     Op::pack2(oacc[db][4 * t + 2] * inv, oacc[db][4 * t + 3] * inv)};
        *(u32x2_t*)(orow + d0 * 2) = w;
      }
    if (g == 0 && p.lse != nullptr) p.lse[(int64_t)bh * N + q_row] = m_run * kLn2 + logf(l_tot);
  }
}

template <typename T, int D, int BN, bool CAUSAL>
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
  hipLaunchKernelGGL((attn_fwd16_kernel<T, D, BN, CAUSAL>), dim3(p.total), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, hipStream_t s, bool* ok) {
  *ok = true;
  auto go = [&](auto dc, auto bnc) -> hipError_t {
    constexpr int D = decltype(dc)::value, BN = decltype(bnc)::value;
    return a.causal ? launch_one<T, D, BN, true>(a, s) : launch_one<T, D, BN, false>(a, s);
  };
  switch (a.d) {
    case 256: return go(std::integral_constant<int, 256>{}, std::integral_constant<int, 32>{});
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream, bool* supported) {
  // d = 64 and 128 in 16-bit types: the 8-wave ping-pong kernel (attn_fwd_pp.hip)
  if ((a.dtype == Dtype::BF16 || a.dtype == Dtype::F16) && a.d <= 128) return launch_attn_fwd16_pp(a, stream, supported);
  switch (a.dtype) {
    case Dtype::BF16: return launch_t<__bf16>(a, stream, supported);
    case Dtype::F16: return launch_t<_Float16>(a, stream, supported);
    case Dtype::F32: return launch_attn_fwd_f32(a, stream, supported);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace attn
