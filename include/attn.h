/*
 * attn.h -- C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * The library computes the fused exact-attention forward
 *     O = softmax(Q K^T * softmax_scale) V        (per batch b, head h)
 * with an online (running max / running sum) softmax tiled over row blocks of
 * Q and an inner loop over blocks of K and V, so the N x N score matrix never
 * reaches device memory; it also writes the per-row logsumexp (LSE).
 * Sources: the attention definition is the displayed equation of the
 * "FlashAttention-3" page (lyirs.cc), restated in its section
 * "数学对象没变，执行图变了"; the tiled loop order (outer Q blocks, inner K/V
 * blocks, running m_i and l_i, one normalisation at the end) is the
 * "FlashAttention-2/3" page (compassingai.com), sections "在线 Softmax",
 * "FlashAttention-2 的三大改进" and "技术原理"; the LSE output and the
 * skipping of fully masked causal blocks are section 2.2 of the
 * "Flash Attention V3" page (jsqmd.com).
 *
 * The FP8 variant follows the "FlashAttention-3" page, section
 * "FP8 路径与低精度误差": incoherent processing x~ = H D x (random +-1 diagonal
 * D, then a Hadamard transform over the head dimension) applied to Q and K,
 * and per-block quantisation ("FlashAttention-2/3" page, FlashAttention-3
 * 特性三).  It is two calls: hadamard_rotate_quant() per tensor, then
 * attn_fwd_fp8().
 *
 * Conventions shared by every entry point
 *  - Tensors are device pointers (hipMalloc / torch device memory).  Q, K, V
 *    are [B, H, N, d] with d contiguous; the b, h and n strides (in elements)
 *    may be passed, NULL meaning contiguous.  Outputs are contiguous.
 *  - N_q = N_k = N >= 1; d in {64, 128, 256}.  causal = 1 means query i sees
 *    keys 0..i.
 *  - The caller allocates and owns every buffer.  The library keeps no
 *    pointer to them after a call returns and allocates no device memory.
 *    Its only state is the per-thread message of attn_last_error() and the
 *    per-device scratch array of attn_bwd_noalloc (see there); calls are
 *    thread-safe except overlapping attn_bwd_noalloc calls on one device.
 *    Outputs must not overlap inputs.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and is asynchronous: completion is observed by the caller.
 *  - Arguments are validated before any HIP call, so a rejected call has no
 *    side effects.  No C++ exception crosses this interface.
 *  - Pointers must be 16-byte aligned and every row start (b, h, n strides
 *    times the element size) must be a multiple of 16 bytes.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 7

/* Status codes returned by every entry point. */
enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1, /* null pointer, size <= 0, overflow, bad stride,
                                    misaligned pointer, overlapping output, bad flag */
  ATTN_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement
                                    (e.g. d not in {64,128,256}) */
  ATTN_ERR_HIP = 3               /* a HIP runtime call failed; attn_last_error()
                                    holds the runtime's message */
};

/* Element types of Q, K, V and O. */
enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 };

/* FP8 code formats (OCP): E4M3 (largest finite 448, no infinities) and E5M2
 * (largest finite 57344) -- the two FP8 formats the "FlashAttention-2/3" page
 * names (FlashAttention-3 特性二). */
enum { ATTN_FP8_E4M3 = 0, ATTN_FP8_E5M2 = 1 };

/* ABI version of the loaded library (ATTN_ABI_VERSION it was built with). */
int attn_abi_version(void);

/* Static, human-readable name of a status code. */
const char* attn_status_string(int status);

/* Detail message of the last failing call on this thread ("" if none). */
const char* attn_last_error(void);

/*
 * attn_fwd -- exact attention forward in fp32, fp16 or bf16.
 *
 *   dtype          ATTN_F32, ATTN_F16 or ATTN_BF16: type of q, k, v and o.
 *   B, H, N, d     batch, heads, sequence length, head dimension.
 *   q, k, v        device [B, H, N, d] inputs (read only).
 *   qkv_strides    host array of 3 int64 element strides (b, h, n) shared by
 *                  q, k and v; the d stride is 1.  NULL = contiguous
 *                  (H*N*d, N*d, d).
 *   o              device output [B, H, N, d], contiguous, same dtype.
 *   lse            device output [B, H, N] fp32, LSE_i = ln sum_j exp(s_ij)
 *                  over the keys row i sees, s = softmax_scale * q.k;
 *                  may be NULL (not written).
 *   softmax_scale  positive, finite; callers pass 1/sqrt(d).
 *   causal         0 or 1.
 *   stream         hipStream_t or NULL.
 *
 * Accumulation is fp32 throughout; O is rounded to the output dtype once,
 * after the final division by the row sum.
 */
int attn_fwd(int dtype, int B, int H, int N, int d,
             const void* q, const void* k, const void* v,
             const int64_t* qkv_strides,
             void* o, float* lse,
             float softmax_scale, int causal, void* stream);

/*
 * Split-KV: the key axis cut into ranges processed by separate workgroups
 * (more parallelism than batch x heads x Q blocks gives, for few heads or
 * long sequences: the sequence-parallel direction of the "FlashAttention-2/3"
 * page, section "FlashAttention-2 的三大改进", 改进二), then merged exactly
 * through each range's logsumexp (the stored LSE of the "Flash Attention V3"
 * page, section 2.2).  The same merge combines partial results computed
 * anywhere -- the building block that ring attention over several devices
 * needs (same page as above, section "常见误读纠偏", 误读三).
 *
 * Range s of S covers keys [s * chunk, min(N, (s + 1) * chunk)) with
 * chunk = attn_splitkv_chunk(N, S), i.e. ceil(N / S) rounded up to a
 * multiple of 128; ranges past N (or fully masked for a row under the causal
 * mask) carry O = 0 and LSE = -inf for that row.
 */
#define ATTN_MAX_SPLITS 64
#define ATTN_MAX_MERGE 1024

static inline int attn_splitkv_chunk(int N, int S) {
  const int per = (N + S - 1) / S;
  return (per + 127) / 128 * 128;
}

/*
 * attn_fwd_splitkv -- attn_fwd computed as S key-range partials plus a merge.
 *
 *   dtype          ATTN_F16 or ATTN_BF16 (others: ATTN_ERR_UNSUPPORTED).
 *   B, H, N, d     as in attn_fwd; d in {64, 128, 256}.
 *   q, k, v, qkv_strides, softmax_scale, causal, stream   as in attn_fwd.
 *   num_splits     S, 1 <= S <= ATTN_MAX_SPLITS.
 *   o_part         device fp32 [S, B, H, N, d] workspace, written with each
 *                  range's normalised output (16-byte aligned).
 *   lse_part       device fp32 [S, B, H, N] workspace, each range's LSE.
 *   o, lse         outputs as in attn_fwd (lse may be NULL).
 *
 * o_part and lse_part are caller-owned scratch that the call overwrites and
 * the library does not keep; they must not overlap each other, the inputs
 * or the outputs.  Both launches go on `stream` in order.  The result equals
 * attn_fwd's up to fp32 rounding order (plus one fp32 rounding of each
 * partial output).
 */
int attn_fwd_splitkv(int dtype, int B, int H, int N, int d,
                     const void* q, const void* k, const void* v,
                     const int64_t* qkv_strides, int num_splits,
                     float* o_part, float* lse_part,
                     void* o, float* lse,
                     float softmax_scale, int causal, void* stream);

/*
 * attn_merge -- combine S attention partials over disjoint key ranges:
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 *
 *   out_dtype      ATTN_F32, ATTN_F16 or ATTN_BF16: type of o.
 *   S              number of partials, 1 <= S <= ATTN_MAX_MERGE.
 *   B, H, N, d     shape of each partial; d in {64, 128, 256}.
 *   o_part         device fp32 [S, B, H, N, d]: each partial's output,
 *                  normalised by its own row sum (16-byte aligned).
 *   lse_part       device fp32 [S, B, H, N]: each partial's LSE, -inf for a
 *                  row that saw no key in that range (weight 0).
 *   o              device [B, H, N, d] output of out_dtype (contiguous).
 *   lse            device fp32 [B, H, N] output, or NULL.
 *   stream         hipStream_t or NULL.
 *
 * A row whose partials are all -inf gets O = 0 and LSE = -inf.  Outputs must
 * not overlap the partials.
 */
int attn_merge(int out_dtype, int S, int B, int H, int N, int d,
               const float* o_part, const float* lse_part,
               void* o, float* lse, void* stream);

/*
 * hadamard_rotate_quant -- FP8 pre-pass for one tensor.
 *
 * For every row x of x[B, H, N, d]: if `signs` is given, x~ = (1/sqrt(d)) H D x
 * with D = diag(signs) and H the Sylvester-order Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)); otherwise x~ = x.  Then, per
 * (b, h, block of block_rows consecutive rows) over all d columns:
 * amax = max |x~|, scale = amax / Q (0 for an all-zero block), and
 * code = round-to-nearest-even of x~ * Q / amax in the chosen format, with
 * Q = 448 for OCP E4M3 (bias 7) and Q = 57344 for OCP E5M2 (bias 15).
 * Dequantisation is x~ = decode(code) * scale.
 *
 *   in_dtype       ATTN_F32, ATTN_F16 or ATTN_BF16 (type of x).
 *   B, H, N, d     shape of x; d in {64, 128, 256}.
 *   x              device input; x_strides as qkv_strides of attn_fwd.
 *   signs          device int8 [d] of +-1 (shared by the Q and K calls), or
 *                  NULL for no rotation (V, and the unrotated comparison).
 *   block_rows     rows per scale block; must be 128.
 *   fp8_format     ATTN_FP8_E4M3 or ATTN_FP8_E5M2.
 *   transpose_out  0: x8 is [B, H, N, d];  1: x8 is [B, H, d, N] (the layout
 *                  attn_fwd_fp8 wants for V).
 *   x8             device uint8 output codes.
 *   scales         device fp32 output [B, H, ceil(N / block_rows)].
 *   stream         hipStream_t or NULL.
 */
int hadamard_rotate_quant(int in_dtype, int B, int H, int N, int d,
                          const void* x, const int64_t* x_strides,
                          const int8_t* signs, int block_rows, int fp8_format,
                          int transpose_out, uint8_t* x8, float* scales,
                          void* stream);

/*
 * hadamard_rotate_quant_per_tensor -- the same pre-pass with one scale per
 * (b, h) instead of per block of 128 rows: the coarser granularity that
 * per-block quantisation ("FlashAttention-2/3" page, FlashAttention-3 特性三)
 * is compared with.  amax = max |x~| over all N rows of the head, and the
 * codes follow the rule of hadamard_rotate_quant with that amax.
 *
 *   Arguments as hadamard_rotate_quant (block_rows must be 128).  scales is
 *   still [B, H, ceil(N / block_rows)], every slot of a head holding the
 *   head's scale, so attn_fwd_fp8 consumes the codes unchanged.
 *
 * Three launches on `stream`: the block amaxes into the scale slots, their
 * maximum per head into every slot, then the codes (x is read twice); the
 * scale array is the only intermediate storage.
 */
int hadamard_rotate_quant_per_tensor(int in_dtype, int B, int H, int N, int d,
                                     const void* x, const int64_t* x_strides,
                                     const int8_t* signs, int block_rows, int fp8_format,
                                     int transpose_out, uint8_t* x8, float* scales,
                                     void* stream);

/*
 * attn_fwd_fp8 -- attention forward on FP8 codes with per-block scales.
 *
 *   q8, k8         device uint8 [B, H, N, d] codes (hadamard_rotate_quant
 *                  with the same signs for both), q_scale / k_scale device
 *                  fp32 [B, H, N/block_rows].
 *   v8t            device uint8 [B, H, d, N] codes (transpose_out = 1, no
 *                  rotation), v_scale device fp32 [B, H, N/block_rows].
 *   block_rows     128; N must be a multiple of block_rows.
 *   fp8_format     format of q8, k8 and v8t: ATTN_FP8_E4M3 or ATTN_FP8_E5M2
 *                  (all three the same; the MFMA reads either natively).
 *   o              device bf16 output [B, H, N, d].
 *   lse            device fp32 [B, H, N] or NULL.
 *   softmax_scale, causal, stream as in attn_fwd.
 *
 * Both products run on FP8 MFMA with fp32 accumulation: S = Q8 K8^T with
 * the two block scales and softmax_scale folded into one factor per tile,
 * and O += P V where P is rounded to E4M3 (whatever fp8_format is) after
 * multiplication by a gain of 256 * w_j / max_j sV_j (w_j = sV_j, the scale
 * of V's key block j, or max_j sV_j for an all-zero block), so that the V
 * block scales fold into P.  P is taken relative to the running row maximum
 * of the online pass after each block of B_c keys (B_c = 128 for d <= 128,
 * 64 for d = 256), rounded up to a whole number in log2 units, so the
 * rounding grid is that of 2^(s log2 e) times a power of two and the scaled
 * P is at most 256.  The row sums l are those of the rounded P (each
 * block's sum divided by its gain), so O is normalised by exactly the
 * weights its second product used, and lse is m + log(l) of that
 * normaliser: it lies within log(1 + 2^-4) of the logsumexp of the
 * dequantised scores (E4M3 keeps 3 mantissa bits) for rows whose scaled P
 * stay in the E4M3 normal range.
 */
int attn_fwd_fp8(int B, int H, int N, int d,
                 const uint8_t* q8, const float* q_scale,
                 const uint8_t* k8, const float* k_scale,
                 const uint8_t* v8t, const float* v_scale,
                 int block_rows, int fp8_format,
                 void* o, float* lse,
                 float softmax_scale, int causal, void* stream);

/*
 * attn_fwd_fp8_qrot -- attn_fwd_fp8 with Q's incoherent processing and
 * quantisation done by the attention kernel itself, on the rows it reads:
 * the "FlashAttention-3" page, section "为什么 Hadamard 适合放到内核里" (the
 * Hadamard transform placed in the kernel), with the per-block scales of the
 * "FlashAttention-2/3" page, FlashAttention-3 特性三.  The result is that of
 * hadamard_rotate_quant on q (with these signs) followed by attn_fwd_fp8:
 * each 128-row block of Q gets amax, codes and scale by the same rule.  The
 * fp32 sums of the transform run in another order than in the pre-pass, so
 * a code may differ where the rotated value lies within a few fp32 ulps of a
 * rounding midpoint.
 *
 *   dtype          ATTN_F16 or ATTN_BF16: the type of q.
 *   q              device [B, H, N, d] at element strides q_strides (b, h, n;
 *                  NULL = contiguous), d stride 1, 16-byte aligned rows.
 *   signs          device int8 [d], the +-1 diagonal D (the one K's codes
 *                  were rotated with), 16-byte aligned.
 *   k8, k_scale, v8t, v_scale, block_rows, fp8_format, o, lse,
 *   softmax_scale, causal, stream   as in attn_fwd_fp8.
 *   d              64 or 128 (256: ATTN_ERR_UNSUPPORTED).
 */
int attn_fwd_fp8_qrot(int dtype, int B, int H, int N, int d,
                      const void* q, const int64_t* q_strides, const int8_t* signs,
                      const uint8_t* k8, const float* k_scale,
                      const uint8_t* v8t, const float* v_scale,
                      int block_rows, int fp8_format,
                      void* o, float* lse,
                      float softmax_scale, int causal, void* stream);

/* Pairings of rope_hadamard_rotate_quant. */
enum { ATTN_ROPE_INTERLEAVED = 1, ATTN_ROPE_HALF = 2 };

/*
 * rope_hadamard_rotate_quant -- the FP8 pre-pass of Q or K with rotary
 * position embedding fused in front: per row x at position n,
 *     x~ = (1/sqrt(d)) H D RoPE_n(x)        (signs given; RoPE_n(x) if NULL)
 * then per-128-row-block codes and scales exactly as hadamard_rotate_quant.
 * Source: the "FlashAttention-3" page, section "为什么 Hadamard 适合放到内核里",
 * suggests fusing the Hadamard transform with a bandwidth-bound
 * pre-processing stage such as RoPE; the page gives no RoPE formula, so
 * RoPE is the published rotary embedding (RoFormer, Su et al.): pair i of
 * the row turns by the angle n * theta_i, theta_i = rope_base^(-2i/d),
 *     (a, b) -> (a cos - b sin, a sin + b cos).
 *
 *   in_dtype, B, H, N, d, x, x_strides, signs, block_rows, fp8_format, x8,
 *   scales, stream   as in hadamard_rotate_quant (codes in [B, H, N, d]
 *                  order only: V, the transposed tensor, has no RoPE).
 *   rope_style     ATTN_ROPE_INTERLEAVED: pairs (x[2i], x[2i+1]);
 *                  ATTN_ROPE_HALF: pairs (x[i], x[i + d/2]).
 *   rope_base      finite, >= 1 (10000 in common use), so theta_i <= 1.
 *   pos_offset     position of row 0 (rows of every (b, h) are positions
 *                  pos_offset .. pos_offset + N - 1); pos_offset >= 0 and
 *                  pos_offset + N <= 2^31 - 1.
 *
 * theta_i is computed in double on the host; n * theta_i is reduced by
 * pi/2 in fp64 on the device; sin, cos and the rotation run in fp32.
 */
int rope_hadamard_rotate_quant(int in_dtype, int B, int H, int N, int d,
                               const void* x, const int64_t* x_strides,
                               int rope_style, double rope_base, int pos_offset,
                               const int8_t* signs, int block_rows, int fp8_format,
                               uint8_t* x8, float* scales, void* stream);

/*
 * attn_bwd -- gradients of the exact attention of attn_fwd:
 *     dV = P^T dO,   dS = P o (dO V^T - D),   D_i = dO_i . O_i,
 *     dQ = softmax_scale dS K,   dK = softmax_scale dS^T Q,
 * with P = exp(softmax_scale Q K^T - LSE) recomputed tile by tile from the
 * forward's logsumexp, so no N x N matrix reaches device memory.  Sources:
 * the backward pass is named on the "FlashAttention-3" page (section
 * "适用范围和工程限制", fp16/bf16 forward and backward) and its recomputation
 * of P from the saved softmax statistics (the LSE) on the "Flash Attention
 * V3" page, sections 2.1 and 2.2; the formulas are the chain rule through
 * the attention definition of the "FlashAttention-3" page.
 *
 *   dtype          ATTN_F16 or ATTN_BF16 (ATTN_F32: ATTN_ERR_UNSUPPORTED):
 *                  type of q, k, v, o, dout, dq, dk, dv.
 *   B, H, N, d     as in attn_fwd; d in {64, 128, 256}.
 *   q, k, v        device [B, H, N, d] forward inputs.
 *   qkv_strides    host array of 3 int64 element strides (b, h, n) shared by
 *                  q, k and v, as in attn_fwd; NULL = contiguous.
 *   o, lse         device forward outputs of attn_fwd on the same q, k, v,
 *                  softmax_scale and causal: o [B, H, N, d] contiguous,
 *                  lse fp32 [B, H, N].
 *   dout           device [B, H, N, d] upstream gradient dO, contiguous.
 *   delta          device fp32 [B, H, N] caller-owned workspace; the call
 *                  overwrites it with D_i = dO_i . O_i (fp32 sums of the
 *                  16-bit products) and keeps no pointer to it.
 *   dq, dk, dv     device [B, H, N, d] outputs, contiguous, same dtype.
 *   softmax_scale, causal, stream   as in attn_fwd.
 *
 * Two launches on `stream` in order (dQ and D first, then dK and dV; at
 * d = 256 three: dQ in one, then dK's and dV's columns 0..127 and 128..255
 * in launches of their own, which both recompute P and dP over the full d);
 * no atomics, so the result is bitwise reproducible.  Accumulation is fp32;
 * P and dS are rounded to the input dtype as operands of the second
 * products, and each gradient is rounded to the dtype once at the end.
 * Outputs and the workspace must not overlap each other or the inputs.
 */
int attn_bwd(int dtype, int B, int H, int N, int d,
             const void* q, const void* k, const void* v,
             const int64_t* qkv_strides,
             const void* o, const float* lse, const void* dout,
             float* delta, void* dq, void* dk, void* dv,
             float softmax_scale, int causal, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and arguments without `delta`,
 * whose role (D_i = dO_i . O_i, fp32 [B, H, N]) is taken by the library's
 * own scratch array, a file-scope device array of 2^21 floats (8 MiB) per
 * GPU that lives until the process ends.
 *
 *   Arguments as attn_bwd; B * H * N must not exceed 2^21 (2,097,152 rows),
 *   or the call fails with ATTN_ERR_INVALID_ARGUMENT before any HIP call.
 *
 * The call allocates nothing (no hipMalloc, no library allocation); on the
 * first call on a device it looks up that device's scratch address
 * (hipGetSymbolAddress) and keeps it.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (two streams, or two
 * host threads) race and must be serialised by the caller.  Nothing in the
 * array needs clearing: the first launch writes every D_i the second reads.
 */
int attn_bwd_noalloc(int dtype, int B, int H, int N, int d,
                     const void* q, const void* k, const void* v,
                     const int64_t* qkv_strides,
                     const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv,
                     float softmax_scale, int causal, void* stream);

/*
 * attn_clock_probe -- measurement aid, not part of the computation: the
 * shader clock under load.  One wave counts shader cycles against the
 * 100 MHz real-time counter for spin_us microseconds of real time, so
 * MHz = out[0] / out[1] * 100.  Launched on a second stream while attention
 * kernels run, the wave shares a compute unit with them and measures the
 * clock they run at (it falls well below the 2.4 GHz peak under dense MFMA
 * work, by the chip's power management).
 *
 *   spin_us   1 .. 100000.
 *   out       device uint64 [2]: shader cycles, real-time ticks.
 *   stream    hipStream_t or NULL.
 */
int attn_clock_probe(int spin_us, uint64_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
