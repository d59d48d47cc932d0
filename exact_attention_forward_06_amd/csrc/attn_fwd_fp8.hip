// FP8 (OCP E4M3) attention forward for gfx950 with per-block scales.
//
// Inputs are the codes and block scales written by hadamard_rotate_quant:
// Q8, K8 [B,H,N,d] (rotated by the same H D), V8t [B,H,d,N] (not rotated),
// one fp32 dequantisation scale per (b, h, 128-row block) of each tensor.
// Both products run on v_mfma_f32_32x32x64_f8f6f4 with fp32 accumulation,
// as in the FP8 path of the "FlashAttention-3" page (section
// "FP8 路径与低精度误差") with per-block quantisation ("FlashAttention-2/3"
// page, FlashAttention-3 特性三); the online softmax is that of the bf16
// kernel.
//
//  * S: one 32x32x64 MFMA per 64 of d.  With 128-row blocks and 128-row
//    workgroups, a K/V tile of 64 keys lies in one K block, so
//    sQ * sK * softmax_scale * log2(e) is ONE scalar per tile.
//  * P V: P is rounded to E4M3 after multiplication by 2^8 * sV_j / sVmax
//    (sV_j the tile's V block scale, sVmax the largest V block scale of the
//    head): the factor enters the exp2 argument as a per-row bias, keeps
//    P' <= 256 < 448 (no saturation) and lifts small P out of the subnormal
//    range; the row sums are kept from the unrounded P.  At the end
//    O = acc * sVmax / 256 / l.
//  * The S^T rows are permuted so that each lane group holds 16 CONSECUTIVE
//    keys of a 32-key block; the 32 P^T bytes a lane feeds to one PV MFMA
//    then pair with two 16-byte LDS reads of V8t per lane.
#include "device_common.h"
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

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
};

// S^T accumulator row r of a 32-key block -> key: lane group g = bit 2 of r
// becomes bit 4 of the key, so group g holds keys 16g .. 16g+15.
__device__ __forceinline__ int key_of_row8(int r) { return (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3); }

__device__ __forceinline__ f32x16_t mfma_fp8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  // cbsz = blgp = 0: both operands FP8 E4M3; no block scale.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8_t cat(u32x4_t lo, u32x4_t hi) {
  i32x8_t r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

template <int D, int BN, int WAVES, bool CAUSAL>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_fp8_kernel(F8Params p) {
  constexpr int BLOCK_M = WAVES * 32;
  constexpr int NT = WAVES * 64;
  constexpr int NKS = D / 64;        // MFMA K-steps of S
  constexpr int NKB = BN / 32;       // 32-key blocks per tile
  constexpr int NDB = D / 32;        // d blocks of O^T
  constexpr int NPV = BN / 64;       // PV MFMAs (64 keys each) per d block
  constexpr int K_PITCH = D + 16;    // bytes
  constexpr int V_PITCH = BN + 16;
  constexpr int K_BYTES = BN * K_PITCH;
  constexpr int STAGE = K_BYTES + D * V_PITCH;
  static_assert(BLOCK_M == 128, "one Q scale block per workgroup");
  static_assert(BN % 64 == 0 && 128 % BN == 0, "tile inside one K scale block");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int N = p.N;

  const int logical = xcd_logical_id(blockIdx.x, p.total);
  const int bh = logical / p.nmb;
  int mb = logical - bh * p.nmb;
  if (CAUSAL) mb = p.nmb - 1 - mb;
  const int m0 = mb * BLOCK_M;
  const int wq0 = m0 + wave * 32;
  const int64_t head = (int64_t)bh * N * D;
  const uint8_t* qp = p.q8 + head;
  const uint8_t* kp = p.k8 + head;
  const uint8_t* vp = p.v8t + head;   // [D][N]
  const float* ksc = p.ks + (int64_t)bh * p.nblk;
  const float* vsc = p.vs + (int64_t)bh * p.nblk;
  const float sq = p.qs[(int64_t)bh * p.nblk + mb];

  float svmax = 0.f;
  for (int i = 0; i < p.nblk; ++i) svmax = fmaxf(svmax, vsc[i]);
  const float inv_svmax = 1.f / svmax;

  // Q8^T fragments: lane (n, g) holds Q8[q][64 ks + 32 g .. +32]
  i32x8_t qf[NKS];
  {
    const uint8_t* src = qp + (int64_t)(wq0 + n) * D + g * 32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = cat(*(const u32x4_t*)(src + ks * 64), *(const u32x4_t*)(src + ks * 64 + 16));
  }

  // staging: K tile BN x D bytes, V8t tile D x BN bytes
  constexpr int KCH = BN * D / 16;
  constexpr int VCH = D * BN / 16;
  static_assert(KCH % NT == 0 && VCH % NT == 0, "tile split");
  constexpr int K_PER_T = KCH / NT, V_PER_T = VCH / NT;
  u32x4_t kreg[K_PER_T], vreg[V_PER_T];

  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int t = 0; t < K_PER_T; ++t) {
      const int c = tid + t * NT;
      const int row = c / (D / 16), col = c % (D / 16);
      kreg[t] = *(const u32x4_t*)(kp + (int64_t)(kt0 + row) * D + col * 16);
    }
#pragma unroll
    for (int t = 0; t < V_PER_T; ++t) {
      const int c = tid + t * NT;
      const int row = c / (BN / 16), col = c % (BN / 16);
      vreg[t] = *(const u32x4_t*)(vp + (int64_t)row * N + kt0 + col * 16);
    }
  };
  auto store_tile = [&](int stage) {
    char* sK = smem + stage * STAGE;
    char* sV = sK + K_BYTES;
#pragma unroll
    for (int t = 0; t < K_PER_T; ++t) {
      const int c = tid + t * NT;
      *(u32x4_t*)(sK + (c / (D / 16)) * K_PITCH + (c % (D / 16)) * 16) = kreg[t];
    }
#pragma unroll
    for (int t = 0; t < V_PER_T; ++t) {
      const int c = tid + t * NT;
      *(u32x4_t*)(sV + (c / (BN / 16)) * V_PITCH + (c % (BN / 16)) * 16) = vreg[t];
    }
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int kv_end = CAUSAL ? min(N, m0 + BLOCK_M) : N;
  const int n_tiles = kv_end / BN;     // N is a multiple of 128
  const int q_row = wq0 + n;
  const float c0 = sq * p.scale_log2;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int stage = j & 1;
    const int kt0 = j * BN;
    const bool more = (j + 1) < n_tiles;
    if (more) load_tile(kt0 + BN);

    const bool active = !CAUSAL || kt0 <= wq0 + 31;
    if (active) {
      const char* sK = smem + stage * STAGE;
      const char* sV = sK + K_BYTES;
      const float c = c0 * ksc[kt0 >> 7];
      const float fv = vsc[kt0 >> 7] * inv_svmax;     // in (0, 1]

      f32x16_t sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
        const char* arow = sK + (kb * 32 + key_of_row8(n)) * K_PITCH + g * 32;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const i32x8_t a = cat(*(const u32x4_t*)(arow + ks * 64), *(const u32x4_t*)(arow + ks * 64 + 16));
          sacc[kb] = mfma_fp8(a, qf[ks], sacc[kb]);
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
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      // e = P * 256 * fv  with P = exp2(s c - m)
      const float bias = __builtin_amdgcn_logf(256.f * fv) - m_use;   // v_log_f32 is log2
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, bias));
          sacc[kb][i] = e;
          rs += e;
        }
      l_run = l_run * alpha + rs * (1.f / (256.f * fv));
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }

      // P^T operands: slot s of lane group g <-> key 64 t + 32 (s / 16) + 16 g + s % 16
      i32x8_t pf[NPV];
#pragma unroll
      for (int t = 0; t < NPV; ++t)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int kb = 2 * t + (w >> 2);
          const int i0 = (w & 3) * 4;
          unsigned lo = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[kb][i0], sacc[kb][i0 + 1], 0, false);
          pf[t][w] = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[kb][i0 + 2], sacc[kb][i0 + 3], lo, true);
        }

#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* arow = sV + (db * 32 + n) * V_PITCH + g * 16;
#pragma unroll
        for (int t = 0; t < NPV; ++t) {
          const i32x8_t a = cat(*(const u32x4_t*)(arow + t * 64), *(const u32x4_t*)(arow + t * 64 + 32));
          oacc[db] = mfma_fp8(a, pf[t], oacc[db]);
        }
      }
    }

    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? svmax * (1.f / 256.f) / l_tot : 0.f;
  __bf16* orow = p.o + ((int64_t)bh * N + q_row) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int d0 = db * 32 + t * 8 + g * 4;
      u32x2_t w;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const __bf16 x = (__bf16)(oacc[db][4 * t + 2 * e] * inv);
        const __bf16 y = (__bf16)(oacc[db][4 * t + 2 * e + 1] * inv);
        w[e] = (unsigned)__builtin_bit_cast(unsigned short, x) |
               ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
      }
      *(u32x2_t*)(orow + d0) = w;
    }
  if (g == 0 && p.lse != nullptr) p.lse[(int64_t)bh * N + q_row] = m_run * kLn2 + logf(l_tot);
}

template <int D, int BN, bool CAUSAL>
hipError_t launch_one(const Fp8FwdArgs& a, hipStream_t s) {
  constexpr int WAVES = 4, BLOCK_M = 128;
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
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, BN, WAVES, CAUSAL>), dim3(p.total), dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}

template <int D, int BN>
hipError_t launch_mask(const Fp8FwdArgs& a, hipStream_t s) {
  return a.causal ? launch_one<D, BN, true>(a, s) : launch_one<D, BN, false>(a, s);
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream, bool* supported) {
  *supported = true;
  if (a.block_rows != 128 || a.N % 128 != 0) {
    *supported = false;
    return hipSuccess;
  }
  switch (a.d) {
    case 64: return launch_mask<64, 64>(a, stream);
    case 128: return launch_mask<128, 64>(a, stream);
    case 256: return launch_mask<256, 64>(a, stream);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace attn
