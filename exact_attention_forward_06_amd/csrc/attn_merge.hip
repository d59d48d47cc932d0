// Merge of attention partials over disjoint key ranges (split-KV).
//
// Each range s of a row carries its own normalised output O_s and logsumexp
// LSE_s = ln sum_{j in range s} exp(s_ij).  The full row is
//     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
// the identity that lets the softmax statistics of separately processed
// key blocks be combined exactly: the online softmax of the "FlashAttention-2/3"
// page (section "在线 Softmax") applied to whole ranges, with the stored
// logsumexp of the "Flash Attention V3" page (section 2.2) as each range's
// state.  Ranges with no visible key carry LSE_s = -inf and weigh 0.
//
// Bandwidth-bound: each row reads S (d + 1) fp32 values and writes d outputs
// and one LSE.  d / 4 lanes share a row (16-byte loads and stores); the
// S LSE values of a row are read by all of its lanes (one cache line).
#include "device_common.h"
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace attn {
namespace {

template <typename T>
__device__ __forceinline__ void store4(T* dst, f32x4_t v);

template <>
__device__ __forceinline__ void store4<float>(float* dst, f32x4_t v) {
  *(f32x4_t*)dst = v;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, f32x4_t v) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  *(bf16x4_t*)dst = __builtin_convertvector(v, bf16x4_t);
}
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* dst, f32x4_t v) {
  typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
  *(f16x4_t*)dst = __builtin_convertvector(v, f16x4_t);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a, int64_t rows) {
  constexpr int LPR = D / 4;                  // lanes per row
  constexpr int RPB = 256 / LPR;              // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = (threadIdx.x % LPR) * 4;
  if (row >= rows) return;
  const int64_t plane = rows;                 // rows per range (B * H * N)
  float m = -INFINITY;
  for (int s = 0; s < a.S; ++s) m = fmaxf(m, a.lse_part[s * plane + row]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < a.S; ++s) {
      const float w = expf(a.lse_part[s * plane + row] - m);   // 0 for an empty range
      const f32x4_t v = *(const f32x4_t*)(a.o_part + (s * plane + row) * D + c);
      acc += w * v;
      l += w;
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  store4<T>(static_cast<T*>(a.o) + row * D + c, acc * inv);
  if (c == 0 && a.lse != nullptr) a.lse[row] = m + logf(l);   // -inf when no range saw a key
}

template <typename T>
hipError_t launch_t(const MergeArgs& a, hipStream_t s, bool* ok) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  auto go = [&](auto dc) -> hipError_t {
    constexpr int D = decltype(dc)::value;
    constexpr int RPB = 256 / (D / 4);
    const int64_t blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((attn_merge_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a, rows);
    return hipGetLastError();
  };
  *ok = true;
  switch (a.d) {
    case 64: return go(std::integral_constant<int, 64>{});
    case 128: return go(std::integral_constant<int, 128>{});
    case 256: return go(std::integral_constant<int, 256>{});
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream, bool* supported) {
  switch (a.out_dtype) {
    case Dtype::F32: return launch_t<float>(a, stream, supported);
    case Dtype::F16: return launch_t<_Float16>(a, stream, supported);
    case Dtype::BF16: return launch_t<__bf16>(a, stream, supported);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace attn
