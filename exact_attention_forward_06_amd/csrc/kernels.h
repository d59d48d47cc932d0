// Private interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

enum class Dtype : int { F32 = 0, F16 = 1, BF16 = 2 };

struct FwdArgs {
  Dtype dtype;
  int B, H, N, d;
  const void* q;
  const void* k;
  const void* v;
  int64_t sb, sh, sn;   // element strides of q, k, v (b, h, n); d stride is 1
  void* o;              // contiguous [B, H, N, d]
  float* lse;           // [B, H, N] or nullptr
  float scale;          // softmax scale (> 0)
  bool causal;
  // split-KV only (attn_fwd_splitkv): partial outputs of nsplit key ranges
  float* o_part = nullptr;    // fp32 [nsplit, B, H, N, d]
  float* lse_part = nullptr;  // fp32 [nsplit, B, H, N]
  int nsplit = 1;
  int chunk = 0;              // keys per range, a multiple of 128
};

struct MergeArgs {
  Dtype out_dtype;
  int S, B, H, N, d;
  const float* o_part;        // fp32 [S, B, H, N, d]
  const float* lse_part;      // fp32 [S, B, H, N]
  void* o;                    // out_dtype [B, H, N, d]
  float* lse;                 // [B, H, N] or nullptr
};

struct QuantArgs {
  Dtype dtype;
  int B, H, N, d;
  const void* x;
  int64_t sb, sh, sn;
  const int8_t* signs;  // nullptr = no rotation
  int block_rows;
  int fp8_format;       // 0: E4M3, 1: E5M2
  bool transpose_out;
  uint8_t* x8;
  float* scales;
  // RoPE before the rotation: 0 none, 1 pairs (2i, 2i+1), 2 pairs (i, i + d/2)
  int rope_style = 0;
  double rope_base = 10000.0;
  int pos_offset = 0;   // position of row 0
  bool per_head = false;   // one scale per (b, h), replicated into every 128-row slot
};

struct Fp8FwdArgs {
  int B, H, N, d;
  const uint8_t* q8;
  const float* q_scale;
  const uint8_t* k8;
  const float* k_scale;
  const uint8_t* v8t;
  const float* v_scale;
  int block_rows;
  int fp8_format;       // codes of q8, k8, v8t: 0 E4M3, 1 E5M2
  void* o;              // bf16 [B, H, N, d]
  float* lse;
  float scale;
  bool causal;
  // Q rotated and quantised by the kernel (q8 and q_scale unused): 16-bit Q
  // of dtype q_dtype at element strides (qsb, qsh, qsn), D = signs
  const void* qx = nullptr;
  Dtype q_dtype = Dtype::BF16;
  int64_t qsb = 0, qsh = 0, qsn = 0;
  const int8_t* signs = nullptr;
};

struct BwdArgs {
  Dtype dtype;          // F16 or BF16
  int B, H, N, d;
  const void* q;        // [B, H, N, d], element strides sb, sh, sn (d stride 1)
  const void* k;
  const void* v;
  int64_t sb, sh, sn;
  const void* o;        // forward output, contiguous
  const void* dout;     // upstream gradient dO
  const float* lse;     // forward LSE [B, H, N]
  float* delta;         // workspace [B, H, N]: dO . O per row
  void* dq;             // outputs, contiguous [B, H, N, d], dtype of q
  void* dk;
  void* dv;
  float scale;
  bool causal;
};

// Each returns hipSuccess or the launch error.  `supported` is set false
// (and nothing launched) when no instantiation covers the request.
hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream, bool* supported);
hipError_t launch_hadamard_rotate_quant(const QuantArgs& a, hipStream_t stream, bool* supported);
hipError_t launch_attn_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream, bool* supported);
// split-KV partials (bf16 / fp16; d = 64 and 128, and d = 256) and their merge
hipError_t launch_attn_fwd16_pp_split(const FwdArgs& a, hipStream_t stream, bool* supported);
hipError_t launch_attn_fwd16_pair_split(const FwdArgs& a, hipStream_t stream, bool* supported);
hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t stream, bool* supported);
// backward: dq kernel (also writes delta) then dk/dv kernel (fp16 / bf16, d = 64, 128 and 256)
hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t stream, bool* supported);
// measurement aid: shader cycles and 100 MHz ticks over spin_ticks ticks
hipError_t launch_clock_probe(unsigned long long* out, long long spin_ticks, hipStream_t stream);

}  // namespace attn
