// C-ABI entry points of libattn: argument validation, dispatch, errors.
// Every check runs before the first HIP call, so a rejected call has no side
// effects; no C++ exception leaves this file.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) {
  switch (dtype) {
    case ATTN_F32: return 4;
    case ATTN_F16: return 2;
    case ATTN_BF16: return 2;
    default: return 0;
  }
}

// Byte interval [lo, hi) touched by a strided [B, H, N, d] tensor.
struct Span {
  uintptr_t lo, hi;
};

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Validates shape and strides of a [B, H, N, cols] tensor whose cols stride is
// 1; fills `span`.  Returns ATTN_OK or an error status (message set).
int check_strided(const char* name, const void* ptr, int B, int H, int N, int cols, int64_t sb,
                  int64_t sh, int64_t sn, int esize, Span* span) {
  if (ptr == nullptr) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  if (sb < 0 || sh < 0 || sn < 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "%s has a negative stride", name);
  if (sn < cols && N > 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s rows overlap (n stride < d)", name);
  if ((sb * esize) % 16 || (sh * esize) % 16 || (sn * esize) % 16)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "%s strides are not multiples of 16 bytes", name);
  // extent in elements, computed in 128 bits to catch overflow
  __int128 ext = (__int128)(B - 1) * sb + (__int128)(H - 1) * sh + (__int128)(N - 1) * sn + cols;
  __int128 bytes = ext * esize;
  if (bytes > ((__int128)1 << 62))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "%s extent overflows", name);
  span->lo = reinterpret_cast<uintptr_t>(ptr);
  span->hi = span->lo + (uintptr_t)bytes;
  return ATTN_OK;
}

int check_dense(const char* name, const void* ptr, int64_t bytes, Span* span, bool align16 = true) {
  if (ptr == nullptr) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (align16 && !aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  if ((reinterpret_cast<uintptr_t>(ptr) & 3u) != 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", name);
  span->lo = reinterpret_cast<uintptr_t>(ptr);
  span->hi = span->lo + (uintptr_t)bytes;
  return ATTN_OK;
}

int check_sizes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d H=%d N=%d d=%d)", B, H, N, d);
  if ((int64_t)B * H * N > INT32_MAX)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "B*H*N exceeds 2^31-1");
  if ((int64_t)B * H * N * d > ((int64_t)1 << 40))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "B*H*N*d exceeds 2^40 elements");
  if (d != 64 && d != 128 && d != 256)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d is not one of 64, 128, 256", d);
  return ATTN_OK;
}

int check_scale_causal(float softmax_scale, int causal) {
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "softmax_scale must be positive and finite");
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  return ATTN_OK;
}

void strides_or_contiguous(const int64_t* s, int H, int N, int d, int64_t* sb, int64_t* sh,
                           int64_t* sn) {
  if (s) {
    *sb = s[0];
    *sh = s[1];
    *sn = s[2];
  } else {
    *sn = d;
    *sh = (int64_t)N * d;
    *sb = (int64_t)H * N * d;
  }
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARGUMENT: return "ATTN_ERR_INVALID_ARGUMENT";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_UNKNOWN_STATUS";
  }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_fwd(int dtype, int B, int H, int N, int d, const void* q, const void* k, const void* v,
             const int64_t* qkv_strides, void* o, float* lse, float softmax_scale, int causal,
             void* stream) {
  const int es = elem_size(dtype);
  if (es == 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (int st = check_sizes(B, H, N, d)) return st;
  if (int st = check_scale_causal(softmax_scale, causal)) return st;
  int64_t sb, sh, sn;
  strides_or_contiguous(qkv_strides, H, N, d, &sb, &sh, &sn);
  Span sq, sk, sv, so, sl{0, 0};
  if (int st = check_strided("q", q, B, H, N, d, sb, sh, sn, es, &sq)) return st;
  if (int st = check_strided("k", k, B, H, N, d, sb, sh, sn, es, &sk)) return st;
  if (int st = check_strided("v", v, B, H, N, d, sb, sh, sn, es, &sv)) return st;
  if (int st = check_dense("o", o, (int64_t)B * H * N * d * es, &so)) return st;
  if (lse) {
    if (int st = check_dense("lse", lse, (int64_t)B * H * N * 4, &sl, false)) return st;
  }
  if (overlaps(so, sq) || overlaps(so, sk) || overlaps(so, sv))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "o overlaps an input");
  // the kernels address one head's K/V rows with 32-bit buffer offsets
  // (including up to one tile of rows past N, which read as zero)
  if (((int64_t)N + 256) * sn * es + (int64_t)d * es >= ((int64_t)1 << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "one head's rows span 2 GiB or more");
  if (lse && (overlaps(sl, sq) || overlaps(sl, sk) || overlaps(sl, sv) || overlaps(sl, so)))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "lse overlaps another tensor");

  attn::FwdArgs a;
  a.dtype = static_cast<attn::Dtype>(dtype);
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.q = q;
  a.k = k;
  a.v = v;
  a.sb = sb;
  a.sh = sh;
  a.sn = sn;
  a.o = o;
  a.lse = lse;
  a.scale = softmax_scale;
  a.causal = causal != 0;
  bool supported = true;
  hipError_t e = attn::launch_attn_fwd(a, static_cast<hipStream_t>(stream), &supported);
  if (!supported) return fail(ATTN_ERR_UNSUPPORTED, "no attn_fwd kernel for dtype %d d=%d", dtype, d);
  return hip_status(e, "attn_fwd launch");
}

int attn_fwd_splitkv(int dtype, int B, int H, int N, int d, const void* q, const void* k,
                     const void* v, const int64_t* qkv_strides, int num_splits, float* o_part,
                     float* lse_part, void* o, float* lse, float softmax_scale, int causal,
                     void* stream) {
  const int es = elem_size(dtype);
  if (es == 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (int st = check_sizes(B, H, N, d)) return st;
  if (int st = check_scale_causal(softmax_scale, causal)) return st;
  if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "num_splits must be in 1..%d", ATTN_MAX_SPLITS);
  if (dtype == ATTN_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_splitkv covers fp16 / bf16");
  int64_t sb, sh, sn;
  strides_or_contiguous(qkv_strides, H, N, d, &sb, &sh, &sn);
  const int64_t rows = (int64_t)B * H * N;
  Span sq, sk, sv, so, sl{0, 0}, sp, spl;
  if (int st = check_strided("q", q, B, H, N, d, sb, sh, sn, es, &sq)) return st;
  if (int st = check_strided("k", k, B, H, N, d, sb, sh, sn, es, &sk)) return st;
  if (int st = check_strided("v", v, B, H, N, d, sb, sh, sn, es, &sv)) return st;
  if (int st = check_dense("o", o, rows * d * es, &so)) return st;
  if (lse) {
    if (int st = check_dense("lse", lse, rows * 4, &sl, false)) return st;
  }
  if (int st = check_dense("o_part", o_part, (int64_t)num_splits * rows * d * 4, &sp)) return st;
  if (int st = check_dense("lse_part", lse_part, (int64_t)num_splits * rows * 4, &spl, false)) return st;
  const Span ins[3] = {sq, sk, sv};
  for (const Span& i : ins) {
    if (overlaps(so, i) || overlaps(sp, i) || overlaps(spl, i) || (lse && overlaps(sl, i)))
      return fail(ATTN_ERR_INVALID_ARGUMENT, "an output overlaps an input");
  }
  if (overlaps(so, sp) || overlaps(so, spl) || overlaps(sp, spl) ||
      (lse && (overlaps(sl, so) || overlaps(sl, sp) || overlaps(sl, spl))))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs overlap each other");
  if (((int64_t)N + 256) * sn * es + (int64_t)d * es >= ((int64_t)1 << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "one head's rows span 2 GiB or more");

  attn::FwdArgs a;
  a.dtype = static_cast<attn::Dtype>(dtype);
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.q = q;
  a.k = k;
  a.v = v;
  a.sb = sb;
  a.sh = sh;
  a.sn = sn;
  a.o = o;
  a.lse = lse;
  a.scale = softmax_scale;
  a.causal = causal != 0;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.nsplit = num_splits;
  a.chunk = attn_splitkv_chunk(N, num_splits);
  attn::MergeArgs m;
  m.out_dtype = a.dtype;
  m.S = num_splits;
  m.B = B;
  m.H = H;
  m.N = N;
  m.d = d;
  m.o_part = o_part;
  m.lse_part = lse_part;
  m.o = o;
  m.lse = lse;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  bool supported = true;
  hipError_t e = d == 256 ? attn::launch_attn_fwd16_pair_split(a, hs, &supported)
                          : attn::launch_attn_fwd16_pp_split(a, hs, &supported);
  if (!supported) return fail(ATTN_ERR_UNSUPPORTED, "no split-KV kernel for dtype %d d=%d", dtype, d);
  if (e != hipSuccess) return hip_status(e, "attn_fwd_splitkv launch");
  e = attn::launch_attn_merge(m, hs, &supported);
  return hip_status(e, "attn_fwd_splitkv merge launch");
}

int attn_merge(int out_dtype, int S, int B, int H, int N, int d, const float* o_part,
               const float* lse_part, void* o, float* lse, void* stream) {
  const int es = elem_size(out_dtype);
  if (es == 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", out_dtype);
  if (int st = check_sizes(B, H, N, d)) return st;
  if (S < 1 || S > ATTN_MAX_MERGE)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "S must be in 1..%d", ATTN_MAX_MERGE);
  const int64_t rows = (int64_t)B * H * N;
  Span sp, spl, so, sl{0, 0};
  if (int st = check_dense("o_part", o_part, (int64_t)S * rows * d * 4, &sp)) return st;
  if (int st = check_dense("lse_part", lse_part, (int64_t)S * rows * 4, &spl, false)) return st;
  if (int st = check_dense("o", o, rows * d * es, &so)) return st;
  if (lse) {
    if (int st = check_dense("lse", lse, rows * 4, &sl, false)) return st;
  }
  if (overlaps(so, sp) || overlaps(so, spl) || (lse && (overlaps(sl, sp) || overlaps(sl, spl) || overlaps(sl, so))))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "an output overlaps an input or the other output");
  attn::MergeArgs m;
  m.out_dtype = static_cast<attn::Dtype>(out_dtype);
  m.S = S;
  m.B = B;
  m.H = H;
  m.N = N;
  m.d = d;
  m.o_part = o_part;
  m.lse_part = lse_part;
  m.o = o;
  m.lse = lse;
  bool supported = true;
  hipError_t e = attn::launch_attn_merge(m, static_cast<hipStream_t>(stream), &supported);
  if (!supported) return fail(ATTN_ERR_UNSUPPORTED, "no attn_merge kernel for d=%d", d);
  return hip_status(e, "attn_merge launch");
}

}  // extern "C"

namespace {

int rotate_quant(int in_dtype, int B, int H, int N, int d, const void* x, const int64_t* x_strides,
                 const int8_t* signs, int block_rows, int fp8_format, int transpose_out, uint8_t* x8,
                 float* scales, void* stream, bool per_head) {
  const int es = elem_size(in_dtype);
  if (es == 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", in_dtype);
  if (int st = check_sizes(B, H, N, d)) return st;
  if (block_rows != 128) return fail(ATTN_ERR_INVALID_ARGUMENT, "block_rows must be 128");
  if (fp8_format != ATTN_FP8_E4M3 && fp8_format != ATTN_FP8_E5M2)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown fp8_format %d", fp8_format);
  if (transpose_out != 0 && transpose_out != 1)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "transpose_out must be 0 or 1");
  if (transpose_out && N % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "transpose_out needs N a multiple of 16");
  int64_t sb, sh, sn;
  strides_or_contiguous(x_strides, H, N, d, &sb, &sh, &sn);
  const int nblk = (N + block_rows - 1) / block_rows;
  Span sx, s8, ss, sg{0, 0};
  if (int st = check_strided("x", x, B, H, N, d, sb, sh, sn, es, &sx)) return st;
  if (int st = check_dense("x8", x8, (int64_t)B * H * N * d, &s8)) return st;
  if (int st = check_dense("scales", scales, (int64_t)B * H * nblk * 4, &ss, false)) return st;
  if (signs) {
    if (int st = check_dense("signs", signs, d, &sg, false)) return st;
  }
  if (overlaps(s8, sx) || overlaps(ss, sx) || overlaps(s8, ss) || (signs && (overlaps(sg, s8) || overlaps(sg, ss))))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs overlap inputs or each other");

  attn::QuantArgs a;
  a.dtype = static_cast<attn::Dtype>(in_dtype);
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.x = x;
  a.sb = sb;
  a.sh = sh;
  a.sn = sn;
  a.signs = signs;
  a.block_rows = block_rows;
  a.fp8_format = fp8_format;
  a.transpose_out = transpose_out != 0;
  a.x8 = x8;
  a.scales = scales;
  a.per_head = per_head;
  bool supported = true;
  hipError_t e = attn::launch_hadamard_rotate_quant(a, static_cast<hipStream_t>(stream), &supported);
  if (!supported) return fail(ATTN_ERR_UNSUPPORTED, "no hadamard_rotate_quant kernel for d=%d", d);
  return hip_status(e, "hadamard_rotate_quant launch");
}

}  // namespace

extern "C" {

int hadamard_rotate_quant(int in_dtype, int B, int H, int N, int d, const void* x,
                          const int64_t* x_strides, const int8_t* signs, int block_rows,
                          int fp8_format, int transpose_out, uint8_t* x8, float* scales,
                          void* stream) {
  return rotate_quant(in_dtype, B, H, N, d, x, x_strides, signs, block_rows, fp8_format, transpose_out, x8,
                      scales, stream, false);
}

int hadamard_rotate_quant_per_tensor(int in_dtype, int B, int H, int N, int d, const void* x,
                                     const int64_t* x_strides, const int8_t* signs, int block_rows,
                                     int fp8_format, int transpose_out, uint8_t* x8, float* scales,
                                     void* stream) {
  return rotate_quant(in_dtype, B, H, N, d, x, x_strides, signs, block_rows, fp8_format, transpose_out, x8,
                      scales, stream, true);
}

int rope_hadamard_rotate_quant(int in_dtype, int B, int H, int N, int d, const void* x,
                               const int64_t* x_strides, int rope_style, double rope_base,
                               int pos_offset, const int8_t* signs, int block_rows, int fp8_format,
                               uint8_t* x8, float* scales, void* stream) {
  const int es = elem_size(in_dtype);
  if (es == 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", in_dtype);
  if (int st = check_sizes(B, H, N, d)) return st;
  if (block_rows != 128) return fail(ATTN_ERR_INVALID_ARGUMENT, "block_rows must be 128");
  if (fp8_format != ATTN_FP8_E4M3 && fp8_format != ATTN_FP8_E5M2)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown fp8_format %d", fp8_format);
  if (rope_style != ATTN_ROPE_INTERLEAVED && rope_style != ATTN_ROPE_HALF)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown rope_style %d", rope_style);
  if (!std::isfinite(rope_base) || !(rope_base >= 1.0))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "rope_base must be finite and at least 1");
  if (pos_offset < 0 || (int64_t)pos_offset + N > INT32_MAX)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "positions pos_offset .. pos_offset + N - 1 must lie in 0 .. 2^31 - 1");
  int64_t sb, sh, sn;
  strides_or_contiguous(x_strides, H, N, d, &sb, &sh, &sn);
  const int nblk = (N + block_rows - 1) / block_rows;
  Span sx, s8, ss, sg{0, 0};
  if (int st = check_strided("x", x, B, H, N, d, sb, sh, sn, es, &sx)) return st;
  if (int st = check_dense("x8", x8, (int64_t)B * H * N * d, &s8)) return st;
  if (int st = check_dense("scales", scales, (int64_t)B * H * nblk * 4, &ss, false)) return st;
  if (signs) {
    if (int st = check_dense("signs", signs, d, &sg, false)) return st;
  }
  if (overlaps(s8, sx) || overlaps(ss, sx) || overlaps(s8, ss) || (signs && (overlaps(sg, s8) || overlaps(sg, ss))))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs overlap inputs or each other");

  attn::QuantArgs a;
  a.dtype = static_cast<attn::Dtype>(in_dtype);
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.x = x;
  a.sb = sb;
  a.sh = sh;
  a.sn = sn;
  a.signs = signs;
  a.block_rows = block_rows;
  a.fp8_format = fp8_format;
  a.transpose_out = false;
  a.x8 = x8;
  a.scales = scales;
  a.rope_style = rope_style;
  a.rope_base = rope_base;
  a.pos_offset = pos_offset;
  bool supported = true;
  hipError_t e = attn::launch_hadamard_rotate_quant(a, static_cast<hipStream_t>(stream), &supported);
  if (!supported) return fail(ATTN_ERR_UNSUPPORTED, "no rope_hadamard_rotate_quant kernel for d=%d", d);
  return hip_status(e, "rope_hadamard_rotate_quant launch");
}

int attn_fwd_fp8(int B, int H, int N, int d, const uint8_t* q8, const float* q_scale,
                 const uint8_t* k8, const float* k_scale, const uint8_t* v8t, const float* v_scale,
                 int block_rows, int fp8_format, void* o, float* lse, float softmax_scale,
                 int causal, void* stream) {
  if (int st = check_sizes(B, H, N, d)) return st;
  if (int st = check_scale_causal(softmax_scale, causal)) return st;
  if (block_rows != 128) return fail(ATTN_ERR_INVALID_ARGUMENT, "block_rows must be 128");
  if (fp8_format != ATTN_FP8_E4M3 && fp8_format != ATTN_FP8_E5M2)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown fp8_format %d", fp8_format);
  if (N % block_rows != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8 needs N a multiple of block_rows");
  if ((int64_t)N * d >= ((int64_t)1 << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "one head's codes span 2 GiB or more");
  const int64_t codes = (int64_t)B * H * N * d;
  const int64_t nsc = (int64_t)B * H * (N / block_rows) * 4;
  Span a1, a2, a3, b1, b2, b3, so, sl{0, 0};
  if (int st = check_dense("q8", q8, codes, &a1)) return st;
  if (int st = check_dense("k8", k8, codes, &a2)) return st;
  if (int st = check_dense("v8t", v8t, codes, &a3)) return st;
  if (int st = check_dense("q_scale", q_scale, nsc, &b1, false)) return st;
  if (int st = check_dense("k_scale", k_scale, nsc, &b2, false)) return st;
  if (int st = check_dense("v_scale", v_scale, nsc, &b3, false)) return st;
  if (int st = check_dense("o", o, codes * 2, &so)) return st;
  if (lse) {
    if (int st = check_dense("lse", lse, (int64_t)B * H * N * 4, &sl, false)) return st;
  }
  const Span ins[6] = {a1, a2, a3, b1, b2, b3};
  for (const Span& s : ins) {
    if (overlaps(so, s) || (lse && overlaps(sl, s)))
      return fail(ATTN_ERR_INVALID_ARGUMENT, "an output overlaps an input");
  }
  if (lse && overlaps(sl, so)) return fail(ATTN_ERR_INVALID_ARGUMENT, "lse overlaps o");

  attn::Fp8FwdArgs a;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.q8 = q8;
  a.q_scale = q_scale;
  a.k8 = k8;
  a.k_scale = k_scale;
  a.v8t = v8t;
  a.v_scale = v_scale;
  a.block_rows = block_rows;
  a.fp8_format = fp8_format;
  a.o = o;
  a.lse = lse;
  a.scale = softmax_scale;
  a.causal = causal != 0;
  bool supported = true;
  hipError_t e = attn::launch_attn_fwd_fp8(a, static_cast<hipStream_t>(stream), &supported);
  if (!supported) return fail(ATTN_ERR_UNSUPPORTED, "no attn_fwd_fp8 kernel for d=%d", d);
  return hip_status(e, "attn_fwd_fp8 launch");
}

int attn_fwd_fp8_qrot(int dtype, int B, int H, int N, int d, const void* q, const int64_t* q_strides,
                      const int8_t* signs, const uint8_t* k8, const float* k_scale, const uint8_t* v8t,
                      const float* v_scale, int block_rows, int fp8_format, void* o, float* lse,
                      float softmax_scale, int causal, void* stream) {
  if (dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(dtype == ATTN_F32 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID_ARGUMENT,
                "attn_fwd_fp8_qrot takes fp16 or bf16 q (dtype %d)", dtype);
  if (int st = check_sizes(B, H, N, d)) return st;
  if (int st = check_scale_causal(softmax_scale, causal)) return st;
  if (block_rows != 128) return fail(ATTN_ERR_INVALID_ARGUMENT, "block_rows must be 128");
  if (fp8_format != ATTN_FP8_E4M3 && fp8_format != ATTN_FP8_E5M2)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown fp8_format %d", fp8_format);
  if (d == 256) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8_qrot covers d = 64 and 128");
  if (N % block_rows != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8_qrot needs N a multiple of block_rows");
  if ((int64_t)N * d >= ((int64_t)1 << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "one head's codes span 2 GiB or more");
  int64_t sb, sh, sn;
  strides_or_contiguous(q_strides, H, N, d, &sb, &sh, &sn);
  const int64_t codes = (int64_t)B * H * N * d;
  const int64_t nsc = (int64_t)B * H * (N / block_rows) * 4;
  Span sq, ssg, a2, a3, b2, b3, so, sl{0, 0};
  if (int st = check_strided("q", q, B, H, N, d, sb, sh, sn, 2, &sq)) return st;
  if (int st = check_dense("signs", signs, d, &ssg)) return st;
  if (int st = check_dense("k8", k8, codes, &a2)) return st;
  if (int st = check_dense("v8t", v8t, codes, &a3)) return st;
  if (int st = check_dense("k_scale", k_scale, nsc, &b2, false)) return st;
  if (int st = check_dense("v_scale", v_scale, nsc, &b3, false)) return st;
  if (int st = check_dense("o", o, codes * 2, &so)) return st;
  if (lse) {
    if (int st = check_dense("lse", lse, (int64_t)B * H * N * 4, &sl, false)) return st;
  }
  const Span ins[6] = {sq, ssg, a2, a3, b2, b3};
  for (const Span& s : ins) {
    if (overlaps(so, s) || (lse && overlaps(sl, s)))
      return fail(ATTN_ERR_INVALID_ARGUMENT, "an output overlaps an input");
  }
  if (lse && overlaps(sl, so)) return fail(ATTN_ERR_INVALID_ARGUMENT, "lse overlaps o");

  attn::Fp8FwdArgs a;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.q8 = nullptr;
  a.q_scale = nullptr;
  a.k8 = k8;
  a.k_scale = k_scale;
  a.v8t = v8t;
  a.v_scale = v_scale;
  a.block_rows = block_rows;
  a.fp8_format = fp8_format;
  a.o = o;
  a.lse = lse;
  a.scale = softmax_scale;
  a.causal = causal != 0;
  a.qx = q;
  a.q_dtype = static_cast<attn::Dtype>(dtype);
  a.qsb = sb;
  a.qsh = sh;
  a.qsn = sn;
  a.signs = signs;
  bool supported = true;
  hipError_t e = attn::launch_attn_fwd_fp8(a, static_cast<hipStream_t>(stream), &supported);
  if (!supported) return fail(ATTN_ERR_UNSUPPORTED, "no attn_fwd_fp8_qrot kernel for d=%d", d);
  return hip_status(e, "attn_fwd_fp8_qrot launch");
}

}  // extern "C"

namespace {

// Validation and argument packing shared by attn_bwd and attn_bwd_noalloc.
// With scratch_delta the workspace is the library's own array (checked and
// resolved by the caller after this returns), so delta is not checked here.
int bwd_prepare(int dtype, int B, int H, int N, int d, const void* q, const void* k, const void* v,
                const int64_t* qkv_strides, const void* o, const float* lse, const void* dout, float* delta,
                bool scratch_delta, void* dq, void* dk, void* dv, float softmax_scale, int causal,
                attn::BwdArgs* a) {
  const int es = elem_size(dtype);
  if (es == 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (int st = check_sizes(B, H, N, d)) return st;
  if (int st = check_scale_causal(softmax_scale, causal)) return st;
  if (dtype == ATTN_F32) return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd covers fp16 / bf16");
  const int64_t rows = (int64_t)B * H * N;
  const int64_t tbytes = rows * d * es;
  int64_t sb, sh, sn;
  strides_or_contiguous(qkv_strides, H, N, d, &sb, &sh, &sn);
  Span sq, sk, sv, so, sl, sdo, sdl = {0, 0}, sdq, sdk, sdv;
  if (int st = check_strided("q", q, B, H, N, d, sb, sh, sn, es, &sq)) return st;
  if (int st = check_strided("k", k, B, H, N, d, sb, sh, sn, es, &sk)) return st;
  if (int st = check_strided("v", v, B, H, N, d, sb, sh, sn, es, &sv)) return st;
  if (int st = check_dense("o", o, tbytes, &so)) return st;
  if (int st = check_dense("lse", lse, rows * 4, &sl, false)) return st;
  if (int st = check_dense("dout", dout, tbytes, &sdo)) return st;
  if (!scratch_delta)
    if (int st = check_dense("delta", delta, rows * 4, &sdl, false)) return st;
  if (int st = check_dense("dq", dq, tbytes, &sdq)) return st;
  if (int st = check_dense("dk", dk, tbytes, &sdk)) return st;
  if (int st = check_dense("dv", dv, tbytes, &sdv)) return st;
  const Span ins[6] = {sq, sk, sv, so, sl, sdo};
  const Span outs[4] = {sdl, sdq, sdk, sdv};
  for (int i = 0; i < 4; ++i) {
    for (const Span& in : ins)
      if (overlaps(outs[i], in)) return fail(ATTN_ERR_INVALID_ARGUMENT, "an output overlaps an input");
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs overlap each other");
  }
  // one head's rows are addressed with 32-bit buffer offsets (including up
  // to one 128-row block past N, which reads as zero)
  if (((int64_t)N + 128) * (sn > d ? sn : d) * es + (int64_t)d * es >= ((int64_t)1 << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "one head's rows span 2 GiB or more");

  a->dtype = static_cast<attn::Dtype>(dtype);
  a->B = B;
  a->H = H;
  a->N = N;
  a->d = d;
  a->q = q;
  a->k = k;
  a->v = v;
  a->sb = sb;
  a->sh = sh;
  a->sn = sn;
  a->o = o;
  a->dout = dout;
  a->lse = lse;
  a->delta = delta;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->scale = softmax_scale;
  a->causal = causal != 0;
  return ATTN_OK;
}

int bwd_launch(const attn::BwdArgs& a, void* stream) {
  bool supported = true;
  hipError_t e = attn::launch_attn_bwd(a, static_cast<hipStream_t>(stream), &supported);
  if (!supported) return fail(ATTN_ERR_UNSUPPORTED, "no attn_bwd kernel for dtype %d d=%d", (int)a.dtype, a.d);
  return hip_status(e, "attn_bwd launch");
}

// The workspace of attn_bwd_noalloc: one array per GPU, in the library's
// device code object, alive until the process ends.  Host code must never
// pass `scratch` itself to a kernel (in host code the name is a stand-in,
// not a device address): its per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kScratchFloats = (int64_t)1 << 21;   // 8 MiB: delta of up to 2^21 rows
__device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (resolved on the first call on
// the current device).
int scratch_address(float** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED, "device %d is beyond the %d the scratch table covers", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)))
      return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd(int dtype, int B, int H, int N, int d, const void* q, const void* k,
                        const void* v, const int64_t* qkv_strides, const void* o, const float* lse,
                        const void* dout, float* delta, void* dq, void* dk, void* dv,
                        float softmax_scale, int causal, void* stream) {
  attn::BwdArgs a;
  if (int st = bwd_prepare(dtype, B, H, N, d, q, k, v, qkv_strides, o, lse, dout, delta, false, dq, dk, dv,
                           softmax_scale, causal, &a))
    return st;
  return bwd_launch(a, stream);
}

extern "C" int attn_bwd_noalloc(int dtype, int B, int H, int N, int d, const void* q, const void* k,
                                const void* v, const int64_t* qkv_strides, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, float softmax_scale,
                                int causal, void* stream) {
  attn::BwdArgs a;
  if (int st = bwd_prepare(dtype, B, H, N, d, q, k, v, qkv_strides, o, lse, dout, nullptr, true, dq, dk, dv,
                           softmax_scale, causal, &a))
    return st;
  if ((int64_t)B * H * N > kScratchFloats)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "B*H*N = %lld rows exceed the %lld of the library's scratch array",
                (long long)B * H * N, (long long)kScratchFloats);
  float* delta = nullptr;
  if (int st = scratch_address(&delta)) return st;
  a.delta = delta;
  return bwd_launch(a, stream);
}

extern "C" int attn_clock_probe(int spin_us, uint64_t* out, void* stream) {
  if (spin_us < 1 || spin_us > 100000)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "spin_us=%d is not in 1 .. 100000", spin_us);
  if (out == nullptr) return fail(ATTN_ERR_INVALID_ARGUMENT, "out is NULL");
  if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "out is not 8-byte aligned");
  hipError_t e = attn::launch_clock_probe(reinterpret_cast<unsigned long long*>(out), (long long)spin_us * 100,
                                          static_cast<hipStream_t>(stream));
  return hip_status(e, "attn_clock_probe launch");
}
