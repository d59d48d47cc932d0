// Exact-attention backward for gfx950, fp16 / bf16 inputs with d = 64, 128, 256:
// dQ, dK, dV of O = softmax(Q K^T * scale) V for an upstream gradient dO,
// with P recomputed tile by tile from the forward's stored logsumexp so that,
// as in the forward, no N x N matrix reaches device memory.
//
// Method.  The pages name the backward pass ("FlashAttention-3" page, section
// "适用范围和工程限制": fp16/bf16 forward and backward) and the role of the
// stored LSE in it ("Flash Attention V3" page, sections 2.1 and 2.2: the
// backward recomputes P from the saved softmax statistics instead of storing
// P).  Per (b, h), with c = scale * log2(e) and D_i = dO_i . O_i:
//     P_ij  = exp2(c s_ij - log2(e) LSE_i)          (0 where masked)
//     dP_ij = dO_i . V_j
//     dS_ij = P_ij (dP_ij - D_i)
//     dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K
// (the chain rule through softmax; D_i = sum_j P_ij dP_ij = dO_i . O_i).
//
// Two launches (four at d = 256, below), no atomics, deterministic:
//  * attn_bwd_dq_kernel: one workgroup per (b, h, 128 query rows); streams
//    K/V tiles like the forward.  Its prologue also computes D_i from O and
//    dO and stores it in the caller's workspace for the second launch.
//  * attn_bwd_dkdv_kernel: one workgroup per (b, h, 128 keys); streams Q/dO
//    tiles (and their LSE / D values) and accumulates dK and dV.
//
// gfx950 mapping (the forward's operand layouts, attn16_common.h)
//  * 4 wave64 per workgroup, 32 stationary rows per wave, held as the
//    B operand of v_mfma_f32_32x32x16_{bf16,f16} in VGPRs (dq: Q and dO;
//    dkdv: K and V).  The streamed 64-row tiles go global -> LDS with
//    buffer_load ... lds, double-buffered, into the XOR-swizzled row layout.
//    The dq kernel (and dkdv at d = 64) fits 256 VGPRs, so two workgroups
//    share a CU and each SIMD interleaves two waves' VALU and MFMA work.  At
//    d = 128, K, V, dK and dV of 32 keys alone take 192 registers, so dK / dV
//    run in attn_bwd_dkdv8_kernel: K and V stay in LDS, 8 waves, two per
//    SIMD, each pair splitting the query rows of every tile.
//  * dq kernel: S^T = K Q^T and dP^T = V dO^T (lane = one query, registers =
//    16 of the tile's keys, key order permuted so registers 8c..8c+7 hold 8
//    consecutive keys); dS^T rounded to 16 bits is directly the B operand of
//    dQ^T += K^T dS^T, whose A operand is read transposed from the K tile
//    with ds_read_b64_tr_b16.
//  * dkdv kernel: the mirror image: S = Q K^T and dP = dO V^T with lane = one
//    key; P and dS are the B operands of dV^T += dO^T P and dK^T += Q^T dS,
//    with dO^T and Q^T read transposed from the streamed tiles.
//  * d = 256, one wave per SIMD: the dq kernel holds Q and dO (128 VGPRs)
//    and all of dQ^T (128 registers, which the compiler places in the
//    accumulation half of the register file), so dQ takes one launch.  dK
//    and dV together would need 256 accumulator registers beside K and V, so
//    they are built in two launches over their column halves (DH = 0, 1),
//    each recomputing S and dP over the full d from 32-row streamed tiles,
//    with the 4-wave dkdv kernel (K and V in VGPRs, dK and dV halves in
//    AGPRs).
//  * Causal: the dq kernel never loads K/V tiles past its block's last
//    query; the dkdv kernel starts at the first Q tile that can see its
//    block's keys.  Element masks run only on tiles that straddle the
//    diagonal or the end of the sequence.
#include "attn16_common.h"
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace attn {
namespace {

struct BwdParams {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;
  const float* lse;
  float* delta;          // fp32 [B, H, N]: written by the dq kernel, read by dkdv
  char* dq;
  char* dk;
  char* dv;
  int64_t sb, sh, sn;    // element strides (b, h, n) of q, k and v; the rest is contiguous
  int H, N, nblk, total;
  float scale;           // softmax scale
  float scale_log2;      // softmax scale * log2(e)
};

constexpr int kBwdThreads = 256;   // 4 wave64
constexpr int kBwdBlock = 128;     // stationary rows per workgroup (32 per wave)
constexpr int kBwdTile = 64;       // streamed rows per LDS tile

// Row addresses inside an LDS tile of the swizzled [row][D] layout.
//  row(ks): the A operand "row-major" read -- lane (n, g) reads the 16 bytes
//    of logical chunk 2 ks + g of row key_of_row(n) (add kb * 32 * RB for the
//    kb-th 32-row block).
//  tr(db, half): the transposed read (ds_read_b64_tr_b16) -- lanes get one
//    column d of 4 consecutive rows; add cc * 16 * RB for the cc-th 16-row
//    chunk.
//  The swizzle touches the low 4 bits of the chunk index only, so at d = 256
//  the chunks 16..31 of a row sit 256 bytes after chunks 0..15: row(ks) of
//  ks >= 8 is row(ks - 8) + 256, an immediate offset (8 registers saved).
template <int D>
struct TileAddr {
  static constexpr int RB = D * 2;
  static constexpr int NKS = D / 16;
  static constexpr int NR = NKS < 8 ? NKS : 8;
  static constexpr int NDB = D / 32;
  int rows_[NR];
  int tr[NDB][2];
  __device__ __forceinline__ int row(int ks) const { return rows_[ks % NR] + (ks / NR) * 256; }
  __device__ __forceinline__ explicit TileAddr(int lane) {
    const int n = lane & 31, g = lane >> 5;
    const int krow = key_of_row(n);
    const int kswz = swz<D>(krow);
#pragma unroll
    for (int ks = 0; ks < NR; ++ks) rows_[ks] = krow * RB + (((2 * ks + g) ^ kswz) * 16);
    const int hq = lane >> 4, jj = lane & 15, ta = jj & 3, te = jj >> 2;
    const int vg = hq >> 1;
    const int vcol0 = (hq & 1) * 16 + 4 * ta;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int row = vg * 8 + half * 4 + te;
        const int col = db * 32 + vcol0;
        tr[db][half] = row * RB + (((col >> 3) ^ swz<D>(row)) * 16) + (col & 7) * 2;
      }
  }
};

// Transposed A operand (16-row chunk starting at `base`, d block db).
template <typename frag, int D>
__device__ __forceinline__ frag read_tr(const char* base, const TileAddr<D>& ta, int db) {
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + ta.tr[db][0]));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + ta.tr[db][1]));
  u32x4_t w;
  w[0] = __builtin_bit_cast(u32x2_t, lo)[0];
  w[1] = __builtin_bit_cast(u32x2_t, lo)[1];
  w[2] = __builtin_bit_cast(u32x2_t, hi)[0];
  w[3] = __builtin_bit_cast(u32x2_t, hi)[1];
  return __builtin_bit_cast(frag, w);
}

// acc[kb] = X Y^T for 32-row block kb of an LDS tile X (rows read permuted)
// against the resident B fragments yf (one stationary row per lane).
template <typename T, int D, int NKB>
__device__ __forceinline__ void tile_dot(f32x16_t (&acc)[NKB], const char* tile, const TileAddr<D>& ta,
                                         const typename Ops<T>::frag (&yf)[D / 16]) {
  using frag = typename Ops<T>::frag;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const frag a = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(tile + kb * 32 * TileAddr<D>::RB + ta.row(ks)));
      acc[kb] = Ops<T>::mfma(a, yf[ks], acc[kb]);
    }
  }
}

// Load one stationary row's B fragments: lane (n, g) holds
// row[16 ks + 8 g .. + 8] (zeros past the end of the sequence).
template <typename T, int D>
__device__ __forceinline__ void load_row_frags(typename Ops<T>::frag (&f)[D / 16], const char* row, bool valid, int g) {
  using frag = typename Ops<T>::frag;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *(const u32x4_t*)(row + ks * 32 + g * 16);
    f[ks] = __builtin_bit_cast(frag, raw);
  }
}

// Store a [D x 32] transposed accumulator (lane = row n of the output, its
// registers = d) times `mul` as 16-bit values of the row `dst`.
template <typename T, int D>
__device__ __forceinline__ void store_rowT(char* dst, const f32x16_t (&acc)[D / 32], float mul, int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int d0 = db * 32 + t * 8 + g * 4;
      u32x2_t w = {Ops<T>::pack2(acc[db][4 * t] * mul, acc[db][4 * t + 1] * mul),
                   Ops<T>::pack2(acc[db][4 * t + 2] * mul, acc[db][4 * t + 3] * mul)};
      *(u32x2_t*)(dst + d0 * 2) = w;
    }
}

// ---------------------------------------------------------------------------
// dQ (and D_i).  Grid: (b, h, 128-query block), XCD-grouped per head; under
// the causal mask the blocks with the most K/V tiles go first.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1, D <= 128 ? 2 : 1)))
void attn_bwd_dq_kernel(BwdParams p) {
  using Op = Ops<T>;
  using frag = typename Op::frag;
  constexpr int NT = kBwdThreads, BN = D <= 128 ? kBwdTile : 32;
  constexpr int RB = D * 2;
  constexpr int TILE = BN * RB;
  constexpr int NKS = D / 16, NKB = BN / 32, NDB = D / 32, NCC = BN / 16;
  constexpr int LOADS = TILE / (NT * 16);
  static_assert(TILE % (NT * 16) == 0, "tile split");

  __shared__ __attribute__((aligned(1024))) char sk0[TILE];
  __shared__ __attribute__((aligned(1024))) char sk1[TILE];
  __shared__ __attribute__((aligned(1024))) char sv0[TILE];
  __shared__ __attribute__((aligned(1024))) char sv1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int g = lane >> 5;
  const int N = p.N;

  const int logical = xcd_logical_id(blockIdx.x, p.total);
  const int bh = logical / p.nblk;
  int mb = logical - bh * p.nblk;
  if (CAUSAL) mb = p.nblk - 1 - mb;
  const int m0 = mb * kBwdBlock;
  const int wq0 = m0 + wave * 32;
  const int q_row = wq0 + n;
  const bool q_ok = q_row < N;
  const int64_t head = (int64_t)bh * N;      // row index of the head's first row
  const int64_t row_off = (head + q_row) * RB;   // contiguous tensors (o, dout, dq)
  const int bb = bh / p.H;
  const int64_t qkv_off = (bb * p.sb + (int64_t)(bh - bb * p.H) * p.sh) * 2;   // strided q, k, v
  const int rbg = (int)(p.sn * 2);                                                // their row pitch

  frag qf[NKS], dof[NKS];
  load_row_frags<T, D>(qf, p.q + qkv_off + (int64_t)q_row * rbg, q_ok, g);
  load_row_frags<T, D>(dof, p.dout + row_off, q_ok, g);

  // D_i = dO_i . O_i (fp32 products of the 16-bit values), stored for dkdv
  float delta;
  {
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (q_ok) raw = *(const u32x4_t*)(p.o + row_off + ks * 32 + g * 16);
      const frag of = __builtin_bit_cast(frag, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)of[e], (float)dof[ks][e], part);
    }
    delta = pair_sum(part);
    if (q_ok && g == 0) p.delta[head + q_row] = delta;
  }
  const float lse2 = q_ok ? p.lse[head + q_row] * kLog2e : 0.f;

  const int64_t extent = ((int64_t)(N - 1) * p.sn + D) * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + qkv_off), (short)0, (int)extent, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + qkv_off), (short)0, (int)extent, 0x00020000);
  const TileAddr<D> ta(lane);

  f32x16_t dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  const int kv_end = CAUSAL ? min(N, m0 + kBwdBlock) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const float c = p.scale_log2;

  auto compute = [&](int j, const char* kt, const char* vt) __attribute__((always_inline)) {
    f32x16_t sacc[NKB], pacc[NKB];
    tile_dot<T, D, NKB>(sacc, kt, ta, qf);    // S^T = K Q^T
    tile_dot<T, D, NKB>(pacc, vt, ta, dof);   // dP^T = V dO^T
    // masked scores -> -inf (P = 0, dS = 0), only on tiles that straddle
    // the diagonal or the end of the sequence
    const int kt0 = j * BN;
    if ((kt0 + BN > N) || (CAUSAL && kt0 + BN - 1 > wq0)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt0 + kb * 32 + key_of_reg(i, g);
          if ((key >= N) || (CAUSAL && key > q_row)) sacc[kb][i] = -INFINITY;
        }
    }
    frag dsf[NCC];
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      const int kb = cc >> 1, base = (cc & 1) * 8;
      u32x4_t w;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float ds2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = base + 2 * t + u;
          const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, -lse2));
          ds2[u] = pr * (pacc[kb][i] - delta);
        }
        w[t] = Op::pack2(ds2[0], ds2[1]);
      }
      dsf[cc] = __builtin_bit_cast(frag, w);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc)
        dqacc[db] = Op::mfma(read_tr<frag, D>(kt + cc * 16 * RB, ta, db), dsf[cc], dqacc[db]);
  };

  // The tile offset goes into the per-lane offset, which the buffer range
  // check always covers: rows past N read as zero.  DMA instruction t of a
  // lane covers row t * RPT + lane_row of the tile; RPT is a multiple of 16,
  // so the swizzled chunk depends on the lane alone and the offsets differ by
  // a wave-uniform term (one live register: this kernel is at its limit).
  // (At d = 256 an instruction covers 8 rows, half a swizzle period, so the
  // offsets of even and odd instructions take their own swizzle.)
  constexpr int RPT = NT * 16 / RB;
  constexpr int NOFF = RPT % 16 == 0 ? 1 : 16 / RPT;
  static_assert(RPT % 16 == 0 || 16 % RPT == 0, "swizzle period");
  const int lane_row = tid * 16 / RB;
  int lane_off[NOFF];
#pragma unroll
  for (int u = 0; u < NOFF; ++u) {
    const int row = u * RPT + lane_row;
    lane_off[u] = lane_row * rbg + ((((tid * 16) % RB) / 16) ^ swz<D>(row)) * 16;
  }
  auto copy = [&](int tile, int st) __attribute__((always_inline)) {
    int off[LOADS];
#pragma unroll
    for (int t = 0; t < LOADS; ++t) off[t] = lane_off[t % NOFF] + (tile * BN + t * RPT) * rbg;
    dma_tile<LOADS, NT>(krs, st ? sk1 : sk0, wave, 0, off);
    dma_tile<LOADS, NT>(vrs, st ? sv1 : sv0, wave, 0, off);
  };
  // Every wave runs every tile of its workgroup: a tile past a wave's last
  // query (causal) is wholly masked and adds zero.  (Skipping it per wave
  // would put the dQ accumulator under control flow, which the compiler
  // answers with a copy of the whole accumulator at every tile.)
  auto step = [&](int j, int st) __attribute__((always_inline)) {
    if (j + 1 < n_tiles) copy(j + 1, st ^ 1);
    compute(j, st ? sk1 : sk0, st ? sv1 : sv0);
    wait_vmem();
    __syncthreads();
  };
  if (n_tiles > 0) copy(0, 0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, 0);
    if (j + 1 < n_tiles) step(j + 1, 1);
  }

  if (q_ok) store_rowT<T, D>(p.dq + row_off, dqacc, p.scale, g);
}

// ---------------------------------------------------------------------------
// dK and dV.  Grid: (b, h, 128-key block), XCD-grouped per head; under the
// causal mask the low key blocks (most Q tiles) come first in natural order.
// DH (d = 256 only): this launch accumulates the columns 128 DH .. + 127 of
// dK and dV; S and dP run over the full d in both halves' launches.
template <typename T, int D, bool CAUSAL, int DH = 0>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1, D <= 64 ? 2 : 1)))
void attn_bwd_dkdv_kernel(BwdParams p) {
  using Op = Ops<T>;
  using frag = typename Op::frag;
  constexpr int NT = kBwdThreads, BN = D <= 128 ? kBwdTile : 32;
  constexpr int RB = D * 2;
  constexpr int TILE = BN * RB;
  constexpr int DO = D <= 128 ? D : 128;      // dK / dV columns of this launch
  constexpr int D0 = DH * DO;                 // ... starting here
  constexpr int NKS = D / 16, NDB = DO / 32;
  constexpr int LOADS = TILE / (NT * 16);
  static_assert(TILE % (NT * 16) == 0, "tile split");

  __shared__ __attribute__((aligned(1024))) char sq0[TILE];
  __shared__ __attribute__((aligned(1024))) char sq1[TILE];
  __shared__ __attribute__((aligned(1024))) char so0[TILE];
  __shared__ __attribute__((aligned(1024))) char so1[TILE];
  // per Q tile: LSE at [0, 64) then D at [64, 128), one float per lane of
  // the loading wave (at BN = 32 the upper 32 of each are the next tile's)
  constexpr int SD = 64;
  __shared__ __attribute__((aligned(16))) float st0[2 * SD];
  __shared__ __attribute__((aligned(16))) float st1[2 * SD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int g = lane >> 5;
  const int N = p.N;

  const int logical = xcd_logical_id(blockIdx.x, p.total);
  const int bh = logical / p.nblk;
  const int kblk = logical - bh * p.nblk;
  const int k0 = kblk * kBwdBlock;
  const int wk0 = k0 + wave * 32;
  const int key = wk0 + n;
  const bool k_ok = key < N;
  const int64_t head = (int64_t)bh * N;
  const int64_t row_off = (head + key) * RB;     // contiguous tensors (dout, dk, dv)
  const int bb = bh / p.H;
  const int64_t qkv_off = (bb * p.sb + (int64_t)(bh - bb * p.H) * p.sh) * 2;   // strided q, k, v
  const int rbg = (int)(p.sn * 2);

  frag kf[NKS], vf[NKS];
  load_row_frags<T, D>(kf, p.k + qkv_off + (int64_t)key * rbg, k_ok, g);
  load_row_frags<T, D>(vf, p.v + qkv_off + (int64_t)key * rbg, k_ok, g);

  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.q + qkv_off), (short)0, (int)(((int64_t)(N - 1) * p.sn + D) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ors =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.dout + head * RB), (short)0, (int)((int64_t)N * RB), 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.lse + head), (short)0, N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.delta + head), (short)0, N * 4, 0x00020000);
  int dma_q[LOADS], dma_o[LOADS];   // Q rows at the strided pitch, dO rows contiguous
#pragma unroll
  for (int t = 0; t < LOADS; ++t) {
    const int pos = (t * NT + tid) * 16;
    const int row = pos / RB;
    const int chunk = ((pos % RB) / 16) ^ swz<D>(row);
    dma_q[t] = row * rbg + chunk * 16;
    dma_o[t] = row * RB + chunk * 16;
  }
  const TileAddr<D> ta(lane);

  f32x16_t dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[db][i] = 0.f;
      dvacc[db][i] = 0.f;
    }

  const int n_qt = (N + BN - 1) / BN;
  const int qt_begin = CAUSAL ? k0 / BN : 0;
  const float c = p.scale_log2;

  // one 32-query block qb (queries q0 .. q0 + 31) of the tile in (qt, ot, sts)
  auto block = [&](int q0, int qb, const char* qt, const char* ot, const float* sts) __attribute__((always_inline)) {
    f32x16_t sacc[1], pacc[1];
    const char* qrows = qt + qb * 32 * RB;
    const char* orows = ot + qb * 32 * RB;
    tile_dot<T, D, 1>(sacc, qrows, ta, kf);    // S = Q K^T   (lane = key)
    tile_dot<T, D, 1>(pacc, orows, ta, vf);    // dP = dO V^T
    // masked scores -> -inf (P = 0, dS = 0), only on blocks that straddle
    // the diagonal or the end of the sequence
    if ((q0 + 32 > N) || (CAUSAL && q0 < wk0 + 31)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = q0 + key_of_reg(i, g);
        if ((qi >= N) || (CAUSAL && key > qi)) sacc[0][i] = -INFINITY;
      }
    }
    // register i holds query q0 + 16 (i >> 3) + 8 g + (i & 7); the LSE and D
    // of a chunk's 8 queries are read from LDS as the chunk needs them
    frag pf[2], dsf[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const float* sl = sts + qb * 32 + 16 * cc + 8 * g;
      const f32x4_t l0 = *(const f32x4_t*)(sl), l1 = *(const f32x4_t*)(sl + 4);
      const f32x4_t d0 = *(const f32x4_t*)(sl + SD), d1 = *(const f32x4_t*)(sl + SD + 4);
      u32x4_t wp, wd;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float pr2[2], ds2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = 2 * t + u, i = cc * 8 + e;
          const float lse = e < 4 ? l0[e] : l1[e - 4];
          const float dl = e < 4 ? d0[e] : d1[e - 4];
          const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[0][i], c, -lse * kLog2e));
          pr2[u] = pr;
          ds2[u] = pr * (pacc[0][i] - dl);
        }
        wp[t] = Op::pack2(pr2[0], pr2[1]);
        wd[t] = Op::pack2(ds2[0], ds2[1]);
      }
      pf[cc] = __builtin_bit_cast(frag, wp);
      dsf[cc] = __builtin_bit_cast(frag, wd);
    }
    // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        dvacc[db] = Op::mfma(read_tr<frag, D>(orows + cc * 16 * RB, ta, db + D0 / 32), pf[cc], dvacc[db]);
        dkacc[db] = Op::mfma(read_tr<frag, D>(qrows + cc * 16 * RB, ta, db + D0 / 32), dsf[cc], dkacc[db]);
      }
  };

  // tile offsets go into the per-lane offsets, which the buffer range check
  // always covers: rows (and LSE / D entries) past N read as zero
  auto copy = [&](int tile, int st) __attribute__((always_inline)) {
    int offq[LOADS], offo[LOADS];
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      offq[t] = dma_q[t] + tile * BN * rbg;
      offo[t] = dma_o[t] + tile * BN * RB;
    }
    dma_tile<LOADS, NT>(qrs, st ? sq1 : sq0, wave, 0, offq);
    dma_tile<LOADS, NT>(ors, st ? so1 : so0, wave, 0, offo);
    // the tile's LSE (wave 0) and D (wave 1): 64 floats, one per lane
    float* sts = st ? st1 : st0;
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (lds_void_t*)sts, 4, (tile * BN + lane) * 4, 0, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (lds_void_t*)(sts + SD), 4, (tile * BN + lane) * 4, 0, 0, 0);
  };
  // Every wave runs every block of its workgroup's tiles: a block before a
  // wave's first key (causal) or a wave past N is wholly masked or never
  // stored.  (Skipping per wave would put the dK / dV accumulators under
  // control flow, which the compiler answers with copies of them.)
  auto step = [&](int j, int st) __attribute__((always_inline)) {
    if (j + 1 < n_qt) copy(j + 1, st ^ 1);
#pragma unroll
    for (int qb = 0; qb < BN / 32; ++qb)
      block(j * BN + qb * 32, qb, st ? sq1 : sq0, st ? so1 : so0, st ? st1 : st0);
    wait_vmem();
    __syncthreads();
  };
  if (qt_begin < n_qt) copy(qt_begin, 0);
  wait_vmem();
  __syncthreads();
  for (int j = qt_begin; j < n_qt; j += 2) {
    step(j, 0);
    if (j + 1 < n_qt) step(j + 1, 1);
  }

  if (k_ok) {
    store_rowT<T, DO>(p.dk + row_off + D0 * 2, dkacc, p.scale, g);
    store_rowT<T, DO>(p.dv + row_off + D0 * 2, dvacc, 1.f, g);
  }
}

// ---------------------------------------------------------------------------
// dK and dV at d = 128 with 8 waves.  K and V of the workgroup's 128 keys
// stay in LDS and are read as B operands, so a wave holds only its dK / dV
// accumulators and one block's products (< 256 VGPRs) and two waves share
// each SIMD.  Waves w and w + 4 own the same 32 keys: wave w takes query rows
// 0..31 of every 64-row Q tile, wave w + 4 rows 32..63; at the end each pair
// adds its partial dK and dV through LDS (wave w finishes dK, wave w + 4 dV).
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv8_kernel(BwdParams p) {
  using Op = Ops<T>;
  using frag = typename Op::frag;
  constexpr int NT = 512, BN = kBwdTile;
  constexpr int RB = D * 2;
  constexpr int TILE = BN * RB;                  // one Q (or dO) tile
  constexpr int KVB = kBwdBlock * RB;            // the block's K (or V)
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int LOADS = TILE / (NT * 16);
  constexpr int KV_LOADS = KVB / (NT * 16);
  constexpr int XCH = NDB * 16 * 64 * 4;         // one wave's dK (or dV) partial, bytes
  static_assert(TILE % (NT * 16) == 0 && KVB % (NT * 16) == 0, "tile split");
  static_assert(4 * XCH <= 2 * KVB && XCH <= TILE, "exchange slots");

  __shared__ __attribute__((aligned(1024))) char skv[2 * KVB];   // K rows, then V rows
  __shared__ __attribute__((aligned(1024))) char sq0[TILE];
  __shared__ __attribute__((aligned(1024))) char sq1[TILE];
  __shared__ __attribute__((aligned(1024))) char so0[TILE];
  __shared__ __attribute__((aligned(1024))) char so1[TILE];
  __shared__ __attribute__((aligned(16))) float st0[2 * BN];
  __shared__ __attribute__((aligned(16))) float st1[2 * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3;          // key group: 32 keys
  const int qh = wave >> 2;         // query half of each tile
  const int n = lane & 31;
  const int g = lane >> 5;
  const int N = p.N;

  const int logical = xcd_logical_id(blockIdx.x, p.total);
  const int bh = logical / p.nblk;
  const int kblk = logical - bh * p.nblk;
  const int k0 = kblk * kBwdBlock;
  const int wk0 = k0 + kg * 32;
  const int key = wk0 + n;
  const int64_t head = (int64_t)bh * N;
  const int bb = bh / p.H;
  const int64_t qkv_off = (bb * p.sb + (int64_t)(bh - bb * p.H) * p.sh) * 2;   // strided q, k, v
  const int rbg = (int)(p.sn * 2);

  const int ext_qkv = (int)(((int64_t)(N - 1) * p.sn + D) * 2);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + qkv_off), (short)0, ext_qkv, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + qkv_off), (short)0, ext_qkv, 0x00020000);
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + qkv_off), (short)0, ext_qkv, 0x00020000);
  const __amdgpu_buffer_rsrc_t ors =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.dout + head * RB), (short)0, (int)((int64_t)N * RB), 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.lse + head), (short)0, N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.delta + head), (short)0, N * 4, 0x00020000);

  // the block's K and V rows (zero past N), swizzled like the tiles
  {
    int off[KV_LOADS];
#pragma unroll
    for (int t = 0; t < KV_LOADS; ++t) {
      const int pos = (t * NT + tid) * 16;
      const int row = pos / RB;
      off[t] = (k0 + row) * rbg + (((pos % RB) / 16) ^ swz<D>(row)) * 16;
    }
    dma_tile<KV_LOADS, NT>(krs, skv, wave, 0, off);
    dma_tile<KV_LOADS, NT>(vrs, skv + KVB, wave, 0, off);
  }
  int dma_q[LOADS], dma_o[LOADS];   // Q rows at the strided pitch, dO rows contiguous
#pragma unroll
  for (int t = 0; t < LOADS; ++t) {
    const int pos = (t * NT + tid) * 16;
    const int row = pos / RB;
    const int chunk = (((pos % RB) / 16) ^ swz<D>(row)) * 16;
    dma_q[t] = row * rbg + chunk;
    dma_o[t] = row * RB + chunk;
  }
  const TileAddr<D> ta(lane);
  // B operand rows of K and V: lane (n, g) reads chunk 2 ks + g of key row kg * 32 + n
  int kvaddr[NKS];
  {
    const int row = kg * 32 + n;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kvaddr[ks] = row * RB + (((2 * ks + g) ^ swz<D>(row)) * 16);
  }

  f32x16_t dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[db][i] = 0.f;
      dvacc[db][i] = 0.f;
    }

  const int n_qt = (N + BN - 1) / BN;
  const int qt_begin = CAUSAL ? k0 / BN : 0;
  const float c = p.scale_log2;

  // this wave's 32 queries q0 .. q0 + 31 of the tile in (qt, ot, sts)
  auto block = [&](int q0, const char* qt, const char* ot, const float* sts) __attribute__((always_inline)) {
    const char* qrows = qt + qh * 32 * RB;
    const char* orows = ot + qh * 32 * RB;
    f32x16_t sacc, pacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sacc[i] = 0.f;
      pacc[i] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const frag a = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(qrows + ta.row(ks)));
      const frag b = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(skv + kvaddr[ks]));
      sacc = Op::mfma(a, b, sacc);                     // S = Q K^T   (lane = key)
      const frag a2 = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(orows + ta.row(ks)));
      const frag b2 = __builtin_bit_cast(frag, *(const lds_u32x4_t*)(skv + KVB + kvaddr[ks]));
      pacc = Op::mfma(a2, b2, pacc);                   // dP = dO V^T
    }
    // masked scores -> -inf (P = 0, dS = 0) on blocks that straddle the
    // diagonal or the end of the sequence
    if ((q0 + 32 > N) || (CAUSAL && q0 < wk0 + 31)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = q0 + key_of_reg(i, g);
        if ((qi >= N) || (CAUSAL && key > qi)) sacc[i] = -INFINITY;
      }
    }
    // register i holds query q0 + 16 (i >> 3) + 8 g + (i & 7); its LSE and D
    const float* sl = sts + qh * 32 + 8 * g;
    frag pf[2], dsf[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const f32x4_t l0 = *(const f32x4_t*)(sl + 16 * cc);
      const f32x4_t l1 = *(const f32x4_t*)(sl + 16 * cc + 4);
      const f32x4_t d0 = *(const f32x4_t*)(sl + BN + 16 * cc);
      const f32x4_t d1 = *(const f32x4_t*)(sl + BN + 16 * cc + 4);
      u32x4_t wp, wd;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float pr2[2], ds2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = 2 * t + u;           // 0..7 within the chunk
          const float lse = e < 4 ? l0[e] : l1[e - 4];
          const float dl = e < 4 ? d0[e] : d1[e - 4];
          const int i = cc * 8 + e;
          const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[i], c, -lse * kLog2e));
          pr2[u] = pr;
          ds2[u] = pr * (pacc[i] - dl);
        }
        wp[t] = Op::pack2(pr2[0], pr2[1]);
        wd[t] = Op::pack2(ds2[0], ds2[1]);
      }
      pf[cc] = __builtin_bit_cast(frag, wp);
      dsf[cc] = __builtin_bit_cast(frag, wd);
    }
    // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        dvacc[db] = Op::mfma(read_tr<frag, D>(orows + cc * 16 * RB, ta, db), pf[cc], dvacc[db]);
        dkacc[db] = Op::mfma(read_tr<frag, D>(qrows + cc * 16 * RB, ta, db), dsf[cc], dkacc[db]);
      }
  };

  auto copy = [&](int tile, int st) __attribute__((always_inline)) {
    int offq[LOADS], offo[LOADS];
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      offq[t] = dma_q[t] + tile * BN * rbg;
      offo[t] = dma_o[t] + tile * BN * RB;
    }
    dma_tile<LOADS, NT>(qrs, st ? sq1 : sq0, wave, 0, offq);
    dma_tile<LOADS, NT>(ors, st ? so1 : so0, wave, 0, offo);
    float* sts = st ? st1 : st0;
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (lds_void_t*)sts, 4, (tile * BN + lane) * 4, 0, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (lds_void_t*)(sts + BN), 4, (tile * BN + lane) * 4, 0, 0, 0);
  };
  // every wave runs every tile (wholly masked blocks add zero; waves past N
  // are never stored) -- no per-wave control flow around the accumulators
  auto step = [&](int j, int st) __attribute__((always_inline)) {
    if (j + 1 < n_qt) copy(j + 1, st ^ 1);
    block(j * BN + qh * 32, st ? sq1 : sq0, st ? so1 : so0, st ? st1 : st0);
    wait_vmem();
    __syncthreads();
  };
  if (qt_begin < n_qt) copy(qt_begin, 0);
  wait_vmem();
  __syncthreads();
  for (int j = qt_begin; j < n_qt; j += 2) {
    step(j, 0);
    if (j + 1 < n_qt) step(j + 1, 1);
  }

  // pair exchange: waves 4..7 park their dK partial in skv, waves 0..3 their
  // dV partial in the tile buffers (slot = key group); layout [register][lane]
  {
    char* slot_kv = skv + kg * XCH;
    char* slot_t = kg == 0 ? sq0 : kg == 1 ? sq1 : kg == 2 ? so0 : so1;
    float* dst = (float*)(qh ? slot_kv : slot_t);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[(db * 16 + i) * 64 + lane] = qh ? dkacc[db][i] : dvacc[db][i];
    __syncthreads();
    const float* src = (const float*)(qh ? slot_t : slot_kv);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float o = src[(db * 16 + i) * 64 + lane];
        if (qh) dvacc[db][i] += o;
        else dkacc[db][i] += o;
      }
  }
  if (key < N) {
    const int64_t row_off = (head + key) * RB;
    if (qh) store_rowT<T, D>(p.dv + row_off, dvacc, 1.f, g);
    else store_rowT<T, D>(p.dk + row_off, dkacc, p.scale, g);
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const char*>(a.q);
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.o = static_cast<const char*>(a.o);
  p.dout = static_cast<const char*>(a.dout);
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = static_cast<char*>(a.dq);
  p.dk = static_cast<char*>(a.dk);
  p.dv = static_cast<char*>(a.dv);
  p.sb = a.sb;
  p.sh = a.sh;
  p.sn = a.sn;
  p.H = a.H;
  p.N = a.N;
  p.nblk = (a.N + kBwdBlock - 1) / kBwdBlock;
  p.total = a.B * a.H * p.nblk;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  if constexpr (D == 256) {
    // dQ in one launch (which writes delta, read by dK / dV), then both
    // halves of dK's and dV's columns, each launch recomputing S and dP over
    // the full d
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, CAUSAL>), dim3(p.total), dim3(kBwdThreads), 0, stream, p);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, CAUSAL, 0>), dim3(p.total), dim3(kBwdThreads), 0, stream, p);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, CAUSAL, 1>), dim3(p.total), dim3(kBwdThreads), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, CAUSAL>), dim3(p.total), dim3(kBwdThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 128)
    hipLaunchKernelGGL((attn_bwd_dkdv8_kernel<T, D, CAUSAL>), dim3(p.total), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, CAUSAL>), dim3(p.total), dim3(kBwdThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s, bool* ok) {
  *ok = true;
  switch (a.d) {
    case 64: return a.causal ? launch_bwd<T, 64, true>(a, s) : launch_bwd<T, 64, false>(a, s);
    case 128: return a.causal ? launch_bwd<T, 128, true>(a, s) : launch_bwd<T, 128, false>(a, s);
    case 256: return a.causal ? launch_bwd<T, 256, true>(a, s) : launch_bwd<T, 256, false>(a, s);
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t stream, bool* supported) {
  switch (a.dtype) {
    case Dtype::BF16: return launch_bwd_t<__bf16>(a, stream, supported);
    case Dtype::F16: return launch_bwd_t<_Float16>(a, stream, supported);
    default: break;
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace attn
