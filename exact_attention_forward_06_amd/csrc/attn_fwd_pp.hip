// Exact-attention forward for gfx950, fp16 / bf16 inputs, d = 64 and 128:
// fp32 accumulation, causal or non-causal, per-row logsumexp output.
//
// Method (sources on the pages are listed in include/attn.h): the grid runs
// over (batch, head, block of 256 query rows) -- the "outer loop over Q
// blocks" of the FlashAttention-2 work partition ("FlashAttention-2/3" page,
// FlashAttention-2 改进二) -- and each workgroup streams the K/V blocks of its
// head through LDS, keeping the running row max m, the running row sum l and
// the unnormalised output in registers; O is divided by l once after the
// last block (改进一) and LSE = m + ln l is stored.
//
// Work inside a compute unit: the "ping-pong" schedule.
//  * One workgroup of 8 wave64 per CU covers 256 query rows (32 per wave), so
//    every K/V tile copied into LDS serves 8 waves.
//  * Waves w and w + 4 run on the same SIMD.  Waves 0-3 (group 0) and 4-7
//    (group 1) alternate between an MFMA phase -- S_j^T = K_j Q^T and
//    O^T += V_{j-1}^T P_{j-1}^T -- and a softmax phase -- row max, lazy
//    rescale and P_j = exp2(S_j c - m) -- one phase apart, with a workgroup
//    barrier between phases.  Each SIMD thus always holds one wave issuing
//    MFMAs and one issuing the VALU work of the softmax.  This is the
//    producer / consumer overlap of softmax and matrix products that the
//    "FlashAttention-3" page describes for Hopper warpgroups (section on
//    warp specialisation and ping-pong scheduling), mapped onto two wave64
//    per SIMD.
//  * In the MFMA phase the K operand (ds_read_b128) and the V^T operand
//    (ds_read_b64_tr_b16) are read a few MFMA pairs ahead of their use (the
//    order is pinned with scheduling barriers); the S and O accumulator
//    chains alternate so no MFMA waits on the previous one, and the wave
//    raises its issue priority for the phase.
//  * Each group's phase loop is compiled separately and every MFMA phase
//    runs both products, so S and O stay in fixed registers: control flow
//    that merged different phase variants made the compiler copy all of O
//    at every phase.
//  * K_j and V_{j-1} are copied global -> LDS (buffer_load ... lds, no VGPR
//    staging; rows past N read as zero through the buffer range check) two
//    phases before they are read, into one of two LDS stages; each stage is
//    its own LDS object and the phase loop is unrolled so that every access
//    names its stage at compile time.  Only group 1 issues the copies, at
//    the start of its softmax phases: an LDS-DMA instruction holds the
//    issuing wave while the CU's address unit takes its 1 KiB, which would
//    stall the MFMA phase of the other group.
//
// Operand mapping (shared with attn_fwd_pair.hip and attn_bwd.hip)
//  * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16} with Q^T resident in
//    VGPRs.  A lane's accumulator holds ONE query (lane & 31) and 16 of a
//    32-key block (the other 16 in lane ^ 32): row max / row sum are in-lane
//    plus one v_permlane32_swap -- no LDS, each wave owns its rows (the
//    page's "split Q across warps" partition, 改进三).
//  * K rows are fed to that MFMA in a permuted order (bits 2 and 3 of the
//    A-operand row swapped) so accumulator registers 8c..8c+7 hold 8
//    consecutive keys; rounded to 16 bits they are directly the P^T operand
//    of O^T += V^T P^T.  P never leaves VGPRs.
//  * V stays in its natural [key][d] layout in LDS; the V^T operand is read
//    with ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-d block
//    and receives it transposed: one d per lane, 4 consecutive keys).
//  * LDS rows are unpadded (the LDS-DMA writes 1 KiB per instruction
//    contiguously), so 16-byte chunks are XOR-swizzled within a row; the
//    swizzle makes both the K operand reads (16 rows, one chunk) and the
//    transposed V reads (4 rows x 4 chunks) hit distinct banks.
//  * Online softmax in the log2 domain with a lazy rescale: the running max
//    is a whole number and only moves when a row's tile max exceeds it by
//    more than 8, so P <= 256 and the O rescale -- an exact power of two --
//    is skipped on almost every tile.  Row sums are accumulated from the
//    fp32 P (the LSE keeps fp32 accuracy).
//  * Causal: K/V tiles wholly above the workgroup's diagonal are never
//    loaded; a wave whose rows all precede a tile skips its math; the element
//    mask runs only where a tile straddles the diagonal or the end of the
//    sequence.
//  * Workgroup ids are remapped so that the Q blocks of a head run on one
//    XCD (the head's K/V is then re-read from that XCD's L2); under the
//    causal mask the Q blocks with the most K/V tiles are issued first.
//  * Causal at d = 128 the grid is persistent, one workgroup per CU, each
//    walking its XCD's items in a snake order; this removes the gap between
//    one workgroup's end and the next one's start on a CU and evens out the
//    per-CU totals of heavy and light causal blocks.
#include "attn16_common.h"
#include "kernels.h"

#include <algorithm>
#include <climits>

#include <math.h>

#include <type_traits>

namespace attn {
namespace {

// SPLIT: the grid also runs over p.nsplit key ranges; each workgroup covers
// one range and writes that range's normalised O (fp32) and LSE to o_part
// and lse_part, which attn_merge.hip combines.
template <typename T, int D, int BN, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_pp_kernel(Params p) {
  using Op = Ops<T>;
  using frag = typename Op::frag;
  constexpr int NT = 512, BLOCK_M = 256;
  constexpr int RB = D * 2;                // LDS row bytes (K and V)
  constexpr int TILE = BN * RB;            // bytes of one K (or V) tile
  constexpr int NKS = D / 16;              // K-steps of S^T = K Q^T
  constexpr int NKB = BN / 32;             // 32-key blocks per tile
  constexpr int NDB = D / 32;              // 32-wide d blocks of O^T
  constexpr int NCC = BN / 16;             // 16-key chunks per tile (PV K-steps)
  constexpr int NOPS = NKB * NKS;          // MFMAs per tile of S^T, and of O^T
  constexpr int LA = 3;                    // LDS read-ahead, in MFMA pairs
  constexpr int NTC = NT / 2;               // threads of the copying group (group 1)
  constexpr int LOADS = TILE / (NTC * 16); // LDS-DMA instructions per copying thread per tile
  static_assert(NOPS == NDB * NCC, "S and O MFMA counts");
  static_assert(TILE % (NTC * 16) == 0 && RB % 16 == 0, "tile split");
  static_assert(4 * TILE <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) char sk0[TILE];
  __shared__ __attribute__((aligned(1024))) char sk1[TILE];
  __shared__ __attribute__((aligned(1024))) char sv0[TILE];
  __shared__ __attribute__((aligned(1024))) char sv1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int group = wave >> 2;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int N = p.N;

  // Workgroup w runs on XCD w % 8 and takes the items of that XCD's
  // contiguous share of the item list (one head's items are consecutive, so
  // they share the XCD's L2).  With one workgroup per item that is the plain
  // XCD grouping.  The causal kernel runs as a persistent grid instead (one
  // workgroup per CU, p.nwg of them): no workgroup launch between items,
  // and the XCD's items are taken in a snake order over its workgroups, so
  // that with the heaviest blocks first in each head a round of heavy items
  // is followed by a round of light ones and the workgroups' totals match
  // (at d = 128; at d = 64 the loop's registers made the kernel spill).
  constexpr bool PERSIST = CAUSAL && !SPLIT && D == 128;
  const int xw = blockIdx.x & 7, lw = blockIdx.x >> 3;
  const int n_x = (p.total >> 3) + (xw < (p.total & 7) ? 1 : 0);
  const int l0_x = xw * (p.total >> 3) + min(xw, p.total & 7);
  const int w_x = (p.nwg >> 3) + (xw < (p.nwg & 7) ? 1 : 0);
  for (int round = 0; round < (PERSIST ? INT_MAX : 1); ++round) {
    const int s_item = round * w_x + ((round & 1) ? w_x - 1 - lw : lw);
    if (s_item >= n_x) break;
    if (round > 0) phase_barrier();    // the previous item's LDS reads are done
    const int logical = l0_x + s_item;
    int bh, mb, split = 0;
    if constexpr (SPLIT) {
      bh = logical / (p.nmb * p.nsplit);
      const int rem = logical - bh * p.nmb * p.nsplit;
      split = rem / p.nmb;
      mb = rem - split * p.nmb;
    } else {
      bh = logical / p.nmb;
      mb = logical - bh * p.nmb;
    }
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

    // K/V global -> LDS: lane l of wave w, DMA instruction t, writes LDS bytes
    // (t*NT + w*64 + l) * 16 of the stage = row P / RB, physical chunk
    // (P % RB) / 16, which holds logical chunk physical ^ swz(row).
    const int64_t extent = ((int64_t)(N - 1) * p.sn + D) * 2;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + head_off), (short)0, (int)extent, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + head_off), (short)0, (int)extent, 0x00020000);
    int dma_off[LOADS];
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      const int pos = (t * NTC + (tid & (NTC - 1))) * 16;
      const int row = pos / RB;
      const int chunk = ((pos % RB) / 16) ^ swz<D>(row);
      dma_off[t] = row * rbg + chunk * 16;
    }

    // LDS read addresses: K A-operand row kb*32 +
    // key_of_row(n), logical chunk 2 ks + g; V^T A-operand via tr16 reads.
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
        const int row = vg * 8 + half * 4 + te;
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

    // keys [k_lo, kv_end) of this item, in tiles j_base .. j_base + n_tiles - 1
    const int k_lo = SPLIT ? split * p.chunk : 0;
    int kv_end = SPLIT ? min(N, k_lo + p.chunk) : N;
    if (CAUSAL) kv_end = min(kv_end, m0 + BLOCK_M);
    const int j_base = k_lo / BN;            // chunk is a multiple of 128, and BN divides 128
    const int n_tiles = kv_end > k_lo ? (kv_end - k_lo + BN - 1) / BN : 0;
    // tiles this wave needs (causal: keys up to its last row)
    const int w_tiles =
        (wq0 >= N) ? 0 : (CAUSAL ? max(0, min(n_tiles, (wq0 + 31) / BN + 1 - j_base)) : n_tiles);
    if constexpr (SPLIT) {
      if (n_tiles == 0) {   // the whole range is masked for this Q block: O = 0, LSE = -inf
        if (q_row < N) {
          float* orow = p.o_part + (((int64_t)split * p.bh_count + bh) * N + q_row) * D;
#pragma unroll
          for (int c = 0; c < D / 8; ++c) *(f32x4_t*)(orow + c * 8 + g * 4) = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (g == 0) p.lse_part[((int64_t)split * p.bh_count + bh) * N + q_row] = -INFINITY;
        }
        return;
      }
    }
    const float c = p.scale_log2;

    f32x16_t sacc[NKB];
    frag pf[NCC];

    auto mask_tile = [&](int kt0) __attribute__((always_inline)) {   // kt0: global key index
      const bool need_mask = (kt0 + BN > N) || (CAUSAL && kt0 + BN - 1 > wq0);
      if (need_mask) {
        // a key is masked where it lies past the last key the row may see
        // (min(q_row, N - 1) under the causal mask, else N - 1); measured from
        // the tile's first key and lane group g's offset, so that each
        // register's test is one compare of a constant
        const int lim = (CAUSAL ? min(q_row, N - 1) : N - 1) - kt0 - 8 * g;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * 32 + key_of_reg(i, 0) > lim) sacc[kb][i] = -INFINITY;
      }
    };
    auto tile_max = [&]() __attribute__((always_inline)) -> float {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      return pair_max(mx) * c;
    };
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
    // P_j = exp2(S_j c - m_run) into pf; returns this lane's sum of P
    auto softmax_p = [&]() __attribute__((always_inline)) -> float {
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
      return rs0 + rs1;
    };
    // Softmax phase of the tile at global key kt0.  P is first taken against
    // the running max as it stands.  A lane's sum of P bounds each of its P,
    // so while no lane's sum exceeds 2^kTau no score of the tile is more than
    // kTau above the running max and the lazy rescale would leave it where it
    // is: the tile's max is then never needed.  Otherwise (and on a wave's
    // first tile, where the running max is still -inf) the exact step runs:
    // tile max, rescale rule, P again.  The running max thus follows the same
    // sequence as with the max taken on every tile.  (One call site each for
    // update_max and for the second softmax_p: the compiler copies all of O
    // where control flow merges differently rescaled versions of it.)
    auto softmax_tile = [&](int kt0) __attribute__((always_inline)) {
      mask_tile(kt0);
      float rs = 0.f;
      bool exact = __any(m_run == -INFINITY);
      if (!exact) {
        rs = softmax_p();
        exact = __any(rs > kRescaleSum);
      }
      if (exact) {
        update_max(tile_max());
        rs = softmax_p();
      }
      l_run += rs;
    };

    // MFMA phase: S^T of tile j from K stage `kst` (DQ) and O^T += V^T P^T of
    // tile j-1 from V stage `vst` (DP).  MFMA pair i is S block i % NKB, K-step
    // i / NKB and O block i % NDB, key chunk i / NDB; its operands are read
    // from LDS LA pairs earlier.
    auto phase_mfma = [&](auto dq_c, auto dp_c, const char* kst, const char* vst) __attribute__((always_inline)) {
      constexpr bool DQ = decltype(dq_c)::value != 0, DP = decltype(dp_c)::value != 0;
      frag kf[NOPS], vf[NOPS];
      auto load = [&](int i) __attribute__((always_inline)) {
        if constexpr (DQ)
          kf[i] = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(kst + (i % NKB) * 32 * RB + kaddr[i / NKB]));
        if constexpr (DP) {
          const char* vb = vst + (i / NDB) * 16 * RB;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + vaddr[i % NDB][0]));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + vaddr[i % NDB][1]));
          u32x4_t w;
          w[0] = __builtin_bit_cast(u32x2_t, lo)[0];
          w[1] = __builtin_bit_cast(u32x2_t, lo)[1];
          w[2] = __builtin_bit_cast(u32x2_t, hi)[0];
          w[3] = __builtin_bit_cast(u32x2_t, hi)[1];
          vf[i] = __builtin_bit_cast(frag, w);
        }
      };
      __builtin_amdgcn_s_setprio(1);   // MFMA issue first when both waves of the SIMD are ready
      if constexpr (DQ) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < LA && i < NOPS; ++i) load(i);
#pragma unroll
      for (int i = 0; i < NOPS; ++i) {
        if (i + LA < NOPS) load(i + LA);
        if constexpr (DQ) sacc[i % NKB] = Op::mfma(kf[i], qf[i / NKB], sacc[i % NKB]);
        if constexpr (DP) oacc[i % NDB] = Op::mfma(vf[i], pf[i / NDB], oacc[i % NDB]);
        // keep this order: the scheduler would otherwise pull each read down
        // next to its MFMA and expose the LDS latency
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // pair j = K_j (j < n_tiles) and V_{j-1} (j >= 1), into stage ST
    auto copy_pair = [&](int j, auto st_c) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      if (j < n_tiles) dma_tile<LOADS, NTC, true>(krs, ST ? sk1 : sk0, wave & 3, (j_base + j) * BN * rbg, dma_off);
      if (j >= 1) dma_tile<LOADS, NTC, true>(vrs, ST ? sv1 : sv0, wave & 3, (j_base + j - 1) * BN * rbg, dma_off);
    };

    // Phase t (t % 4 == TM) of group G.  Local phase u = t - G: even u = MFMA
    // phase A_{u/2} (reads pair u/2), odd u = softmax phase B_{(u-1)/2}.  Pair
    // j is read in phases 2j and 2j+1, copied during phase 2j-2 into stage
    // j & 1 and waited for at the end of phase 2j-1.  The group is a template
    // parameter so that each group's loop is straight-line code.
    auto run = [&](auto g_c) __attribute__((always_inline)) {
      constexpr int G = decltype(g_c)::value;
      auto phase = [&](int t, auto tm_c) __attribute__((always_inline)) {
        constexpr int TM = decltype(tm_c)::value;
        if constexpr ((TM & 1) == 0 && G == 1) {
          const int j = t / 2 + 1;
          if (j <= n_tiles) copy_pair(j, ic<(TM == 0) ? 1 : 0>{});
        }
        const int u = t - G;
        if (u >= 0 && u <= 2 * n_tiles) {
          const int j = u >> 1;
          if constexpr (((TM - G) & 1) == 0) {
            constexpr int AST = TM >> 1;
            const char* kst = AST ? sk1 : sk0;
            const char* vst = AST ? sv1 : sv0;
            // Both products run whenever either is needed: one code path keeps
            // S and O in fixed registers (separate variants cost a copy of O
            // per phase).  The unneeded one is harmless: S_j past the wave's
            // last tile is never read, and in the first phase P is zero and V
            // stage 0 is zero-filled, so O^T gains exactly zero.
            if (j <= w_tiles) phase_mfma(ic<1>{}, ic<1>{}, kst, vst);
          } else if (j < w_tiles) {
            softmax_tile((j_base + j) * BN);
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

    if (group == 1) copy_pair(0, ic<0>{});
#pragma unroll
    for (int c = 0; c < TILE / (NT * 16); ++c) *(lds_u32x4_t*)(sv0 + (c * NT + tid) * 16) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) pf[cc] = frag{};
    wait_vmem();
    wait_lds();
    phase_barrier();
    if (group == 0) run(ic<0>{});
    else run(ic<1>{});

    // epilogue: O = O / l, LSE = m ln2 + ln l
    const float l_tot = pair_sum(l_run);
    if constexpr (SPLIT) {
      if (q_row < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* orow = p.o_part + (((int64_t)split * p.bh_count + bh) * N + q_row) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int d0 = db * 32 + t * 8 + g * 4;
            *(f32x4_t*)(orow + d0) = f32x4_t{oacc[db][4 * t] * inv, oacc[db][4 * t + 1] * inv,
                                              oacc[db][4 * t + 2] * inv, oacc[db][4 * t + 3] * inv};
          }
        if (g == 0) p.lse_part[((int64_t)split * p.bh_count + bh) * N + q_row] = m_run * kLn2 + logf(l_tot);
      }
      return;    // a split-KV grid is never persistent: one item per workgroup
    }
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
}

template <typename T, int D, int BN, bool CAUSAL, bool SPLIT>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  constexpr int BLOCK_M = 256;
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
  p.scale_log2 = a.scale * kLog2e;
  p.bh_count = a.B * a.H;
  p.nsplit = SPLIT ? a.nsplit : 1;
  p.chunk = SPLIT ? a.chunk : a.N;
  p.o_part = a.o_part;
  p.lse_part = a.lse_part;
  p.total = p.bh_count * p.nmb * p.nsplit;
  p.nwg = p.total;
  if constexpr (CAUSAL && !SPLIT && D == 128) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      // one resident workgroup per CU, and at least one per XCD share of
      // the items (workgroup w takes share w % 8)
      p.nwg = std::min(p.total, std::max(cus, 8));
  }
  hipLaunchKernelGGL((attn_fwd_pp_kernel<T, D, BN, CAUSAL, SPLIT>), dim3(p.nwg), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <typename T, bool SPLIT>
hipError_t launch_t(const FwdArgs& a, hipStream_t s, bool* ok) {
  *ok = true;
  auto go = [&](auto dc, auto bnc) -> hipError_t {
    constexpr int D = decltype(dc)::value, BN = decltype(bnc)::value;
    return a.causal ? launch_one<T, D, BN, true, SPLIT>(a, s) : launch_one<T, D, BN, false, SPLIT>(a, s);
  };
  switch (a.d) {
    case 64: return go(ic<64>{}, ic<128>{});
    case 128: return go(ic<128>{}, ic<64>{});
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

// d = 64 and 128 in bf16 / fp16; `supported` is false for anything else.
hipError_t launch_attn_fwd16_pp(const FwdArgs& a, hipStream_t stream, bool* supported) {
  switch (a.dtype) {
    case Dtype::BF16: return launch_t<__bf16, false>(a, stream, supported);
    case Dtype::F16: return launch_t<_Float16, false>(a, stream, supported);
    default: break;
  }
  *supported = false;
  return hipSuccess;
}

// Split-KV: partial O / LSE per key range (a.nsplit ranges of a.chunk keys).
hipError_t launch_attn_fwd16_pp_split(const FwdArgs& a, hipStream_t stream, bool* supported) {
  switch (a.dtype) {
    case Dtype::BF16: return launch_t<__bf16, true>(a, stream, supported);
    case Dtype::F16: return launch_t<_Float16, true>(a, stream, supported);
    default: break;
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace attn
