// Exact-attention forward for gfx950, fp32 inputs (the 16-bit types have
// their own kernel in attn_fwd.hip): fp32 accumulation, causal or
// non-causal, per-row logsumexp output.
//
// Method (see include/attn.h for the sources on the pages): the grid runs
// over (batch, head, block of BLOCK_M query rows) -- the "outer loop over Q
// blocks" of the FlashAttention-2 work partition ("FlashAttention-2/3" page,
// FlashAttention-2 改进二) -- and each workgroup streams the K/V blocks of its
// head through LDS, keeping the running row max m, running row sum l and the
// unnormalised output in registers; O is divided by l once after the last
// block (改进一) and LSE = m + ln l is stored.
//
// gfx950 mapping
//  * One wave64 owns 32 query rows.  It computes S^T = K Q^T with 32x32 MFMAs
//    (A = K rows from LDS, B = Q^T held in VGPRs for the whole loop), so the
//    accumulator gives each lane ONE query (lane & 31) and 16 of the tile's
//    keys; the other 16 keys of that query sit in lane ^ 32.  Row max / row
//    sum are therefore in-lane reductions plus one v_permlane32_swap -- no
//    LDS traffic, and each wave owns its rows outright (the page's
//    "split Q across warps" partition, 改进三).
//  * The key order inside a 32-key block is permuted (bits 2 and 3 of the
//    A-operand row swapped) so that the S^T accumulator registers 8c..8c+7
//    of a lane hold 8 CONSECUTIVE keys.  Rounded to 16 bits they are then
//    directly the B operand (P^T) of O^T += V^T P^T -- P never leaves VGPRs.
//  * V is stored transposed in LDS (Vt[d][key]) for the 16-bit types, so the
//    A operand V^T reads 8 consecutive keys per lane (one ds_read_b128).
//    The transpose is done in registers between the global load and the LDS
//    store.  fp32 uses 32x32x2 MFMAs whose operands are single elements, so
//    V stays in natural layout there.
//  * K/V tiles are double-buffered in LDS: the global loads of tile j+1 are
//    issued before the MFMAs of tile j and written to the other buffer after
//    them, one barrier per tile.  Row pitches are padded by 16 bytes so the
//    per-lane row reads of one MFMA operand fall in different banks.
//  * Causal: K/V tiles wholly above the diagonal of the workgroup's rows are
//    never loaded; a wave whose rows all precede a tile skips its math; the
//    element mask is applied only where a tile straddles the diagonal or the
//    ragged end of the sequence.
//  * Workgroup ids are remapped so that consecutive Q blocks of a head land
//    on the same XCD (hardware dispatch is round-robin over the 8 XCDs), and
//    K/V of a head is re-read from that XCD's L2.  Under the causal mask the
//    Q blocks with the most K/V tiles are issued first.
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.f;   // lazy-rescale threshold (log2 units)

struct KParams {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int64_t sb, sh, sn;   // element strides
  int H, N, nmb, total;
  float scale_log2;     // softmax_scale * log2(e)
};

// Row of the S^T accumulator block -> key offset inside the 32-key block
// (bits 2 and 3 swapped; an involution).
__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Accumulator register i (0..15) of lane group g of a 32x32 MFMA holds row
// (i/4)*8 + g*4 + i%4; after the permutation above that row is key
// 16*(i/8) + 8*g + i%8 of the block.
__device__ __forceinline__ int key_of_reg(int i, int g) { return 16 * (i >> 3) + 8 * g + (i & 7); }

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

template <typename T>
struct Traits;

template <>
struct Traits<__bf16> {
  static constexpr int KPACK = 8;     // elements per lane per MFMA operand
  using frag = bf16x8_t;
  static __device__ __forceinline__ f32x16_t mfma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float a, float b) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (unsigned)__builtin_bit_cast(unsigned short, x) |
           ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
  }
};

template <>
struct Traits<_Float16> {
  static constexpr int KPACK = 8;
  using frag = f16x8_t;
  static __device__ __forceinline__ f32x16_t mfma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float a, float b) {
    _Float16 x = (_Float16)a, y = (_Float16)b;
    return (unsigned)__builtin_bit_cast(unsigned short, x) |
           ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
  }
};

template <>
struct Traits<float> {
  static constexpr int KPACK = 1;
  using frag = float;
  static __device__ __forceinline__ f32x16_t mfma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <typename T, int D, int BN, int WAVES, bool CAUSAL>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1, 2)))
void attn_fwd_kernel(KParams p) {
  using Tr = Traits<T>;
  using frag = typename Tr::frag;
  constexpr int ES = sizeof(T);
  constexpr int KPACK = Tr::KPACK;
  constexpr int KSTEP = 2 * KPACK;          // MFMA K per instruction
  constexpr int NKS = D / KSTEP;            // K-steps of S = K Q^T
  constexpr int BLOCK_M = WAVES * 32;
  constexpr int NT = WAVES * 64;
  constexpr int NKB = BN / 32;              // 32-key blocks per tile
  constexpr int NDB = D / 32;               // 32-wide d blocks of O^T
  constexpr bool VT = (ES == 2);            // V transposed in LDS
  constexpr int K_PITCH = D * ES + 16;
  constexpr int V_PITCH = VT ? (BN * 2 + 16) : (D * ES + 16);
  constexpr int V_ROWS = VT ? D : BN;
  constexpr int K_BYTES = BN * K_PITCH;
  constexpr int STAGE = K_BYTES + V_ROWS * V_PITCH;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;     // query column of this lane / A-operand row
  const int g = lane >> 5;     // lane group: k half of the operands
  const int N = p.N;

  // --- workgroup -> (b, h, Q block), XCD-aware
  int logical;
  {
    const int w = blockIdx.x, tot = p.total;
    const int qd = tot >> 3, rem = tot & 7, x = w & 7, s = w >> 3;
    logical = x * qd + min(x, rem) + s;
  }
  const int bh = logical / p.nmb;
  int mb = logical - bh * p.nmb;
  if (CAUSAL) mb = p.nmb - 1 - mb;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int m0 = mb * BLOCK_M;
  const int wq0 = m0 + wave * 32;
  const int64_t head_off = ((int64_t)b * p.sb + (int64_t)h * p.sh) * ES;
  const char* qp = p.q + head_off;
  const char* kp = p.k + head_off;
  const char* vp = p.v + head_off;
  const int64_t row_bytes = p.sn * ES;

  // --- Q^T fragments (B operand), resident for the whole loop
  frag qf[NKS];
  {
    const int qrow = wq0 + n;
    const char* src = qp + (int64_t)qrow * row_bytes;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int col = ks * KSTEP + g * KPACK;
      if constexpr (KPACK == 8) {
        u32x4_t raw = {0u, 0u, 0u, 0u};
        if (qrow < N) raw = *(const u32x4_t*)(src + col * ES);
        qf[ks] = __builtin_bit_cast(frag, raw);
      } else {
        qf[ks] = (qrow < N) ? *(const float*)(src + col * ES) : 0.f;
      }
    }
  }

  // --- K/V tile staging (global -> registers -> LDS)
  constexpr int CH_ROW = D * ES / 16;              // 16-byte chunks per row
  constexpr int K_PER_T = BN * CH_ROW / NT;
  static_assert((BN * CH_ROW) % NT == 0, "K tile split");
  constexpr int DCH = D / 8;                        // 8-element d chunks (16-bit V)
  constexpr int V_PER_T = VT ? (BN / 4) * DCH / NT : K_PER_T;
  static_assert(!VT || ((BN / 4) * DCH) % NT == 0, "V tile split");
  constexpr int V_REGS = VT ? 4 : 1;

  u32x4_t kreg[K_PER_T];
  u32x4_t vreg[V_PER_T][V_REGS];

  // K/V rows come through raw buffer loads on a descriptor covering this
  // head's rows 0..N-1: rows at or past N read as zero (the hardware range
  // check), so ragged tiles need no branches and offsets stay 32-bit.
  const int64_t head_extent = ((int64_t)(N - 1) * p.sn + D) * ES;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)head_extent, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, (int)head_extent, 0x00020000);
  const int rb = (int)row_bytes;

  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int t = 0; t < K_PER_T; ++t) {
      const int c = tid + t * NT;
      const int row = c / CH_ROW, col = c % CH_ROW;
      kreg[t] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, (kt0 + row) * rb + col * 16, 0, 0));
    }
#pragma unroll
    for (int t = 0; t < V_PER_T; ++t) {
      const int u = tid + t * NT;
      if constexpr (VT) {
        const int kg = u / DCH, dc = u % DCH;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          vreg[t][kk] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, (kt0 + 4 * kg + kk) * rb + dc * 16, 0, 0));
      } else {
        const int row = u / CH_ROW, col = u % CH_ROW;
        vreg[t][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, (kt0 + row) * rb + col * 16, 0, 0));
      }
    }
  };

  auto store_tile = [&](int stage) {
    char* sK = smem + stage * STAGE;
    char* sV = sK + K_BYTES;
#pragma unroll
    for (int t = 0; t < K_PER_T; ++t) {
      const int c = tid + t * NT;
      const int row = c / CH_ROW, col = c % CH_ROW;
      *(u32x4_t*)(sK + row * K_PITCH + col * 16) = kreg[t];
    }
#pragma unroll
    for (int t = 0; t < V_PER_T; ++t) {
      const int u = tid + t * NT;
      if constexpr (VT) {
        // 4 keys x 8 d  ->  8 rows of Vt, 4 keys (8 bytes) each
        const int kg = u / DCH, dc = u % DCH;
        const u32x4_t* r = vreg[t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d0 = dc * 8 + 2 * e;
          u32x2_t even, odd;
          even[0] = (r[0][e] & 0xFFFFu) | (r[1][e] << 16);
          even[1] = (r[2][e] & 0xFFFFu) | (r[3][e] << 16);
          odd[0] = (r[0][e] >> 16) | (r[1][e] & 0xFFFF0000u);
          odd[1] = (r[2][e] >> 16) | (r[3][e] & 0xFFFF0000u);
          *(u32x2_t*)(sV + d0 * V_PITCH + kg * 8) = even;
          *(u32x2_t*)(sV + (d0 + 1) * V_PITCH + kg * 8) = odd;
        }
      } else {
        const int row = u / CH_ROW, col = u % CH_ROW;
        *(u32x4_t*)(sV + row * V_PITCH + col * 16) = vreg[t][0];
      }
    }
  };

  // --- running state
  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;   // running max of scale*log2(e)*s
  float l_run = 0.f;         // this lane's half of the running row sum

  const int kv_end = CAUSAL ? min(N, m0 + BLOCK_M) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const float c = p.scale_log2;
  const int q_row = wq0 + n;

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
      f32x16_t sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
        const char* arow = sK + (kb * 32 + swap_bits23(n)) * K_PITCH + g * KPACK * ES;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          frag a;
          if constexpr (KPACK == 8)
            a = __builtin_bit_cast(frag, *(const u32x4_t*)(arow + ks * KSTEP * ES));
          else
            a = *(const float*)(arow + ks * KSTEP * ES);
          sacc[kb] = Tr::mfma(a, qf[ks], sacc[kb]);
        }
      }

      // mask: ragged end of the sequence, and keys after the query (causal)
      const bool need_mask = (kt0 + BN > N) || (CAUSAL && kt0 + BN - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt0 + kb * 32 + key_of_reg(i, g);
            const bool masked = (key >= N) || (CAUSAL && key > q_row);
            if (masked) sacc[kb][i] = -INFINITY;
          }
      }

      // online softmax update (log2 domain).  The running max only moves
      // when a row's tile max exceeds it by more than kTau: until then
      // P = exp2(s c - m_run) <= 2^kTau, and the result is unchanged
      // (O and l share the same reference), so the O rescale is skipped on
      // almost every tile.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
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
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, -m_use));
          sacc[kb][i] = e;
          rs += e;
        }
      l_run += rs;

      // O^T += V^T P^T
      if constexpr (KPACK == 8) {
        frag pf[BN / 16];
#pragma unroll
        for (int cc = 0; cc < BN / 16; ++cc) {
          const int kb = cc >> 1, base = (cc & 1) * 8;
          u32x4_t w;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            w[t] = Tr::pack2(sacc[kb][base + 2 * t], sacc[kb][base + 2 * t + 1]);
          pf[cc] = __builtin_bit_cast(frag, w);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char* arow = sV + (db * 32 + n) * V_PITCH + g * 16;
#pragma unroll
          for (int cc = 0; cc < BN / 16; ++cc) {
            frag a = __builtin_bit_cast(frag, *(const u32x4_t*)(arow + cc * 32));
            oacc[db] = Tr::mfma(a, pf[cc], oacc[db]);
          }
        }
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kb * 32 + key_of_reg(i, g);
              const float a = *(const float*)(sV + key * V_PITCH + (db * 32 + n) * 4);
              oacc[db] = Tr::mfma(a, sacc[kb][i], oacc[db]);
            }
      }
    }

    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // --- epilogue: O = O / l, LSE = m ln2 + ln l
  const float l_tot = pair_sum(l_run);
  if (q_row < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* orow = p.o + (((int64_t)bh * N + q_row) * D) * ES;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int d0 = db * 32 + t * 8 + g * 4;
        const float v0 = oacc[db][4 * t + 0] * inv, v1 = oacc[db][4 * t + 1] * inv;
        const float v2 = oacc[db][4 * t + 2] * inv, v3 = oacc[db][4 * t + 3] * inv;
        if constexpr (ES == 2) {
          u32x2_t w = {Tr::pack2(v0, v1), Tr::pack2(v2, v3)};
          *(u32x2_t*)(orow + d0 * ES) = w;
        } else {
          f32x4_t w = {v0, v1, v2, v3};
          *(f32x4_t*)(orow + d0 * ES) = w;
        }
      }
    if (g == 0 && p.lse != nullptr) p.lse[(int64_t)bh * N + q_row] = m_run * kLn2 + logf(l_tot);
  }
}

template <typename T, int D, int BN, int WAVES, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  constexpr int BLOCK_M = WAVES * 32;
  KParams p;
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
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, WAVES, CAUSAL>), dim3(p.total), dim3(WAVES * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

// fp32 attention forward (v_mfma_f32_32x32x2f32; V in natural layout).
hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t s, bool* ok) {
  *ok = true;
  auto go = [&](auto dc) -> hipError_t {
    constexpr int D = decltype(dc)::value;
    return a.causal ? launch_one<float, D, 32, 4, true>(a, s) : launch_one<float, D, 32, 4, false>(a, s);
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
