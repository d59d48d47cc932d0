// Exact-attention forward for gfx950, fp16 / bf16 inputs, d = 256: the
// ping-pong schedule of attn_fwd_pp.hip with each 32-row query block shared
// by a pair of waves.  Computes the FlashAttention-2 forward of the
// "FlashAttention-2/3" page (outer loop over Q blocks, online softmax, one
// division by l at the end, LSE = m + ln l).
//
// At d = 256 one wave that owns 32 query rows alone would hold Q^T (64
// registers) and the fp32 O^T accumulator (128) besides S and P: more than
// the 256 registers a wave gets when two waves share a SIMD, which the
// ping-pong schedule needs.  Here the two waves of a pair (waves 2p and
// 2p + 1, in the same ping-pong group) own the same 32 query rows and split
// the products of every 64-key tile:
//  * S^T = K Q^T: each wave takes its own 32 keys of the tile (keys
//    32 mem .. 32 mem + 31, mem = wave & 1), over the full d;
//  * O^T += V^T P^T: each wave takes its own 128 columns of d
//    (128 mem .. 128 mem + 127), over all 64 keys.
// A wave thus holds Q^T (64 registers), its half of O^T (64), S for 32 keys
// (16) and P for 64 keys (16).  The MFMA count per wave and tile (16 + 16)
// and the LDS bytes read per MFMA are those of the d = 128 kernel; the
// softmax work per wave and tile is half of it.
//
// The pair exchanges two things per tile through LDS:
//  * in the softmax phase, the row max of its half of S_j.  Both waves then
//    take the same tile max, so the whole-number running max, the lazy
//    rescale of O and l and the reference of P evolve identically in both.
//    Each wave publishes its max with the tile index beside it (one 64-bit
//    LDS write) and waits, with a bounded sleep loop, until the other's slot
//    carries the same index;
//  * its half of P_j (16-bit, in B-operand layout), written in the softmax
//    phase and read by the other wave in its next MFMA phase, on the other
//    side of the phase barrier.
// Each wave's row sum covers its own keys; the two are added once at the
// end.
//
// Everything else is as in attn_fwd_pp.hip: 8 waves, waves w and w + 4 on
// one SIMD alternating an MFMA phase and a softmax phase, K_j and V_{j-1}
// copied global -> LDS by group 1 two phases ahead into one of two stages,
// the operand layouts, key permutation and LDS swizzle, the whole-number
// running max with lazy rescale, causal skipping and the split-KV variant.
// A workgroup covers 128 query rows (4 pairs).
#include "attn16_common.h"
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

// Spin limit of the wait for the other wave's row max.  Both waves of a pair
// always publish the same tiles, so the wait ends after a few LDS round
// trips; the bound only guarantees that every wave leaves the loop.
constexpr int kMaxSpin = 1 << 20;

// The base registers of the LDS reads made per MFMA hold the read's offset
// within its stage plus the LDS address that stage 0 gets (K stages at 0 and
// 32 KiB, V stages at 64 and 96 KiB), so that every read is one register
// plus an immediate offset below 64 KiB.  The empty asm statements keep the
// compiler from folding the constant back into each read.  The addresses
// are right whatever layout the compiler chooses; only the cost of forming
// them depends on these constants.
constexpr int kBiasK = 0, kBiasV = 64 * 1024;

template <typename T, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_pair_kernel(Params p) {
  using Op = Ops<T>;
  using frag = typename Op::frag;
  constexpr int D = 256, BN = 64, NT = 512, BLOCK_M = 128;
  constexpr int RB = D * 2;                // LDS row bytes (K and V)
  constexpr int TILE = BN * RB;            // bytes of one K (or V) tile: 32 KiB
  constexpr int NKS = D / 16;              // K-steps of S^T = K Q^T
  constexpr int NDB = 4;                   // 32-wide d blocks of this wave's half of O^T
  constexpr int NOPS = 16;                 // MFMAs per tile of S^T, and of O^T
  constexpr int LA = 3;                    // LDS read-ahead, in MFMA pairs
  constexpr int NTC = NT / 2;              // threads of the copying group (group 1)
  constexpr int LOADS = TILE / (NTC * 16); // LDS-DMA instructions per copying thread per tile
  constexpr int PXW = 64 * 32;             // bytes of one wave's P half (2 fragments per lane)
  static_assert(TILE % (NTC * 16) == 0 && 4 * TILE + 8 * PXW + 8 * 32 * 12 <= 160 * 1024, "LDS budget");

  // One LDS object per stage: the compiler then knows that reads of one
  // stage do not wait for the copies in flight into the other.  Besides the
  // stages: the P halves of the 8 waves, the tagged row maxima (8 bytes per
  // wave and row) and the row sums (4 bytes per wave and row).
  __shared__ __attribute__((aligned(1024))) char sk0[TILE];
  __shared__ __attribute__((aligned(1024))) char sk1[TILE];
  __shared__ __attribute__((aligned(1024))) char sv0[TILE];
  __shared__ __attribute__((aligned(1024))) char sv1[TILE];
  __shared__ __attribute__((aligned(1024))) char spx[8 * PXW];
  __shared__ __attribute__((aligned(16))) char smx[8 * 32 * 8];
  __shared__ __attribute__((aligned(16))) char slx[8 * 32 * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int group = wave >> 2;
  const int mem = wave & 1;                // which half of the keys (S) and of d (O)
  const int pid = wave >> 1;               // pair: query rows 32 pid ..
  const int n = lane & 31;
  const int g = lane >> 5;
  const int N = p.N;

  const int logical = xcd_logical_id(blockIdx.x, p.total);
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
  const int wq0 = m0 + pid * 32;
  const int q_row = wq0 + n;
  const int64_t head_off = ((int64_t)b * p.sb + (int64_t)h * p.sh) * 2;
  const int rbg = (int)(p.sn * 2);         // global row pitch in bytes

  // Q^T fragments (B operand) over the full d: lane (n, g) holds Q[q][16 ks + 8 g .. + 8]
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

  // K A-operand: row 32 mem + key_of_row(n), logical chunk 2 ks + g.  The
  // swizzle changes only the low four bits of the chunk index, so K-steps
  // 8..15 read 256 bytes past K-steps 0..7.
  const int krow = mem * 32 + key_of_row(n);
  const int kswz = swz<D>(krow);
  int kaddr[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kaddr[ks] = krow * RB + (((2 * ks + g) ^ kswz) * 16) + kBiasK;
    asm("" : "+v"(kaddr[ks]));
  }
  // V^T A-operand (tr16 reads) of this wave's 128 columns, from the 16-key
  // chunks of its own keys (vown) and of the other wave's keys (vpart).
  const int hq = lane >> 4, jj = lane & 15, ta = jj & 3, te = jj >> 2;
  const int vg = hq >> 1;
  const int vcol0 = mem * 128 + (hq & 1) * 16 + 4 * ta;
  int vown[NDB][2], vpart[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = vg * 8 + half * 4 + te;
      const int col = db * 32 + vcol0;
      const int a = row * RB + (((col >> 3) ^ swz<D>(row)) * 16) + (col & 7) * 2;
      vown[db][half] = a + mem * 32 * RB + kBiasV;
      vpart[db][half] = a + (1 - mem) * 32 * RB + kBiasV;
      asm("" : "+v"(vown[db][half]), "+v"(vpart[db][half]));
    }
  // this wave's P half (written) and the other wave's (read), lane-major
  const int px_mine = wave * PXW + lane * 16;
  const int px_other = (wave ^ 1) * PXW + lane * 16;
  const int mx_mine = (wave * 32 + n) * 8;
  const int mx_other = ((wave ^ 1) * 32 + n) * 8;

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;   // whole-number running max of scale * log2(e) * s (possibly stale by < kTau)
  float l_run = 0.f;         // this lane's part of the running row sum over this wave's keys

  const int k_lo = SPLIT ? split * p.chunk : 0;
  int kv_end = SPLIT ? min(N, k_lo + p.chunk) : N;
  if (CAUSAL) kv_end = min(kv_end, m0 + BLOCK_M);
  const int j_base = k_lo / BN;            // chunk is a multiple of 128
  const int n_tiles = kv_end > k_lo ? (kv_end - k_lo + BN - 1) / BN : 0;
  const int w_tiles =
      (wq0 >= N) ? 0 : (CAUSAL ? max(0, min(n_tiles, (wq0 + 31) / BN + 1 - j_base)) : n_tiles);
  if constexpr (SPLIT) {
    if (n_tiles == 0) {   // the whole range is masked for this Q block: O = 0, LSE = -inf
      if (q_row < N) {
        float* orow = p.o_part + (((int64_t)split * p.bh_count + bh) * N + q_row) * D + mem * 128;
#pragma unroll
        for (int c = 0; c < 16; ++c) *(f32x4_t*)(orow + c * 8 + g * 4) = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (g == 0 && mem == 0) p.lse_part[((int64_t)split * p.bh_count + bh) * N + q_row] = -INFINITY;
      }
      return;
    }
  }
  const float c = p.scale_log2;

  f32x16_t sacc;
  frag pf[4];   // P^T B-operand chunks in MFMA order: this wave's two, then the other wave's two

  auto update_max = [&](float m_tile) __attribute__((always_inline)) {
    if (__any(m_tile > m_run + kTau)) {
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

  // Softmax phase of local tile j (global key kt0 of its first key)
  auto softmax = [&](int j, int kt0) __attribute__((always_inline)) {
    const int kb0 = kt0 + mem * 32;
    const bool need_mask = (kb0 + 32 > N) || (CAUSAL && kb0 + 31 > wq0);
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb0 + key_of_reg(i, g);
        if ((key >= N) || (CAUSAL && key > q_row)) sacc[i] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    mx = pair_max(mx);
    // publish (max, j), then take the other wave's max for the same tile
    // (volatile 64-bit LDS accesses: one ds_write_b64 / ds_read_b64 each, so
    // the value and its tag are seen together, re-read on every iteration)
    typedef volatile __attribute__((address_space(3))) u32x2_t lds_tag_t;
    if (g == 0) *(lds_tag_t*)(smx + mx_mine) = u32x2_t{__builtin_bit_cast(unsigned, mx), (unsigned)j};
    u32x2_t got;
    for (int it = 0;; ++it) {
      got = *(lds_tag_t*)(smx + mx_other);
      if (__all((int)got[1] == j) || it == kMaxSpin) break;
      __builtin_amdgcn_s_sleep(1);
    }
    const float mo = __builtin_bit_cast(float, got[0]);
    update_max(fmaxf(mx, mo) * c);

    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4_t w;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[cc * 8 + 2 * t], c, -m_use));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[cc * 8 + 2 * t + 1], c, -m_use));
        w[t] = Op::pack2(e0, e1);
        rs0 += e0;
        rs1 += e1;
      }
      pf[cc] = __builtin_bit_cast(frag, w);
      *(lds_u32x4_t*)(spx + px_mine + cc * 1024) = w;
    }
    l_run += rs0 + rs1;
    wait_lds();   // the P half is in LDS before the phase barrier
  };

  // MFMA phase: S^T of tile j (own keys) from K stage ST and this wave's
  // columns of O^T += V^T P^T of tile j-1 from V stage ST.  MFMA pair i is
  // S K-step i and O block i % NDB, key chunk i / NDB.
  auto phase_mfma = [&](auto st_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    const char* kst = (ST ? sk1 : sk0) - kBiasK;
    const char* vst = (ST ? sv1 : sv0) - kBiasV;
    frag kf[NOPS], vf[NOPS];
    pf[2] = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(spx + px_other));
    pf[3] = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(spx + px_other + 1024));
    auto load = [&](int i) __attribute__((always_inline)) {
      kf[i] = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(kst + (i >> 3) * 256 + kaddr[i & 7]));
      const int cc = i / NDB, db = i % NDB;
      const int* va = cc < 2 ? vown[db] : vpart[db];
      const char* vb = vst + (cc & 1) * 16 * RB;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + va[0]));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + va[1]));
      u32x4_t w;
      w[0] = __builtin_bit_cast(u32x2_t, lo)[0];
      w[1] = __builtin_bit_cast(u32x2_t, lo)[1];
      w[2] = __builtin_bit_cast(u32x2_t, hi)[0];
      w[3] = __builtin_bit_cast(u32x2_t, hi)[1];
      vf[i] = __builtin_bit_cast(frag, w);
    };
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int i = 0; i < LA; ++i) load(i);
#pragma unroll
    for (int i = 0; i < NOPS; ++i) {
      if (i + LA < NOPS) load(i + LA);
      sacc = Op::mfma(kf[i], qf[i], sacc);
      oacc[i % NDB] = Op::mfma(vf[i], pf[i / NDB], oacc[i % NDB]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto copy_pair = [&](int j, auto st_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    if (j < n_tiles) dma_tile<LOADS, NTC, true>(krs, ST ? sk1 : sk0, wave & 3, (j_base + j) * BN * rbg, dma_off);
    if (j >= 1) dma_tile<LOADS, NTC, true>(vrs, ST ? sv1 : sv0, wave & 3, (j_base + j - 1) * BN * rbg, dma_off);
  };

  // The phase loop of attn_fwd_pp.hip: phase t (t % 4 == TM) of group G,
  // local phase u = t - G, even u = MFMA phase of pair u / 2, odd u =
  // softmax phase of tile (u - 1) / 2.
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
          // As in attn_fwd_pp.hip both products always run: S_j past the
          // pair's last tile is never read, and in the first phase P (this
          // wave's registers and the other wave's LDS half) is zero and V
          // stage 0 is zero-filled.
          if (j <= w_tiles) phase_mfma(ic<AST>{});
        } else if (j < w_tiles) {
          softmax(j, (j_base + j) * BN);
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
  // zero V stage 0 and the P halves, and mark every max slot as "no tile yet"
#pragma unroll
  for (int k = 0; k < TILE / (NT * 16); ++k) *(lds_u32x4_t*)(sv0 + (k * NT + tid) * 16) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 8 * PXW / (NT * 16); ++k) *(lds_u32x4_t*)(spx + (k * NT + tid) * 16) = u32x4_t{0u, 0u, 0u, 0u};
  if (tid < 8 * 32) *(__attribute__((address_space(3))) u32x2_t*)(smx + tid * 8) = u32x2_t{0u, 0xFFFFFFFFu};
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) pf[cc] = frag{};
  wait_vmem();
  wait_lds();
  phase_barrier();
  if (group == 0) run(ic<0>{});
  else run(ic<1>{});

  // row sum over both waves' keys (the same sum, in the same order, in both)
  const float l_mine = pair_sum(l_run);
  if (g == 0) *(__attribute__((address_space(3))) float*)(slx + (wave * 32 + n) * 4) = l_mine;
  wait_lds();
  phase_barrier();
  const float l_other = *(__attribute__((address_space(3))) float*)(slx + ((wave ^ 1) * 32 + n) * 4);
  const float l_tot = mem == 0 ? l_mine + l_other : l_other + l_mine;
  if constexpr (SPLIT) {
    if (q_row < N) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* orow = p.o_part + (((int64_t)split * p.bh_count + bh) * N + q_row) * D + mem * 128;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int d0 = db * 32 + t * 8 + g * 4;
          *(f32x4_t*)(orow + d0) = f32x4_t{oacc[db][4 * t] * inv, oacc[db][4 * t + 1] * inv,
                                            oacc[db][4 * t + 2] * inv, oacc[db][4 * t + 3] * inv};
        }
      if (g == 0 && mem == 0)
        p.lse_part[((int64_t)split * p.bh_count + bh) * N + q_row] = m_run * kLn2 + logf(l_tot);
    }
    return;
  }
  if (q_row < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* orow = p.o + (((int64_t)bh * N + q_row) * D + mem * 128) * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int d0 = db * 32 + t * 8 + g * 4;
        u32x2_t w = {Op::pack2(oacc[db][4 * t] * inv, oacc[db][4 * t + 1] * inv),
                     Op::pack2(oacc[db][4 * t + 2] * inv, oacc[db][4 * t + 3] * inv)};
        *(u32x2_t*)(orow + d0 * 2) = w;
      }
    if (g == 0 && mem == 0 && p.lse != nullptr) p.lse[(int64_t)bh * N + q_row] = m_run * kLn2 + logf(l_tot);
  }
}

template <typename T, bool CAUSAL, bool SPLIT>
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
  p.scale_log2 = a.scale * kLog2e;
  p.bh_count = a.B * a.H;
  p.nsplit = SPLIT ? a.nsplit : 1;
  p.chunk = SPLIT ? a.chunk : a.N;
  p.o_part = a.o_part;
  p.lse_part = a.lse_part;
  p.total = p.bh_count * p.nmb * p.nsplit;
  hipLaunchKernelGGL((attn_fwd_pair_kernel<T, CAUSAL, SPLIT>), dim3(p.total), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <typename T, bool SPLIT>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  return a.causal ? launch_one<T, true, SPLIT>(a, s) : launch_one<T, false, SPLIT>(a, s);
}

template <bool SPLIT>
hipError_t launch_dt(const FwdArgs& a, hipStream_t stream, bool* supported) {
  *supported = a.d == 256;
  if (!*supported) return hipSuccess;
  switch (a.dtype) {
    case Dtype::BF16: return launch_t<__bf16, SPLIT>(a, stream);
    case Dtype::F16: return launch_t<_Float16, SPLIT>(a, stream);
    default: break;
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace

// d = 256 in bf16 / fp16; `supported` is false for anything else.
hipError_t launch_attn_fwd16_pair(const FwdArgs& a, hipStream_t stream, bool* supported) {
  return launch_dt<false>(a, stream, supported);
}

// Split-KV at d = 256: partial O / LSE per key range.
hipError_t launch_attn_fwd16_pair_split(const FwdArgs& a, hipStream_t stream, bool* supported) {
  return launch_dt<true>(a, stream, supported);
}

}  // namespace attn
