"""Exact-attention forward for AMD MI355X (gfx950).

Public API (thin wrappers over the C ABI of libattn.so, include/attn.h):

    attn_fwd(q, k, v, causal=False, softmax_scale=None) -> (o, lse)
    hadamard_rotate_quant(x, signs=None, block_rows=128, transpose_out=False)
        -> (codes, scales)
    attn_fwd_fp8(q8, q_scale, k8, k_scale, v8t, v_scale, causal=False)
        -> (o, lse)
    attn_fwd_fp8_e2e(q, k, v, signs, causal=False, rope=None) -> (o, lse)
    rope_hadamard_rotate_quant(x, signs=None, style="interleaved", base=10000,
                               pos_offset=0) -> (codes, scales)
    attn_fwd_splitkv(q, k, v, num_splits, causal=False)
        -> (o, lse, o_part, lse_part)
    attn_merge(o_part, lse_part, out_dtype) -> (o, lse)
    attn_bwd(q, k, v, o, lse, dout, causal=False) -> (dq, dk, dv, delta)
"""
from ._lib import (AttnError, attn_bwd, attn_bwd_noalloc, attn_fwd, attn_fwd_fp8, attn_fwd_fp8_qrot, attn_fwd_splitkv, attn_merge, hadamard_rotate_quant,
                   clock_probe, load, rope_hadamard_rotate_quant, splitkv_chunk)


def attn_fwd_fp8_e2e(q, k, v, signs, causal=False, softmax_scale=None, stream=None, fp8_format="e4m3",
                     rope=None, per_tensor=False, q_in_kernel=False):
    """The whole FP8 path: rotate+quantise Q and K with the shared signs,
    quantise V into the transposed layout, then the FP8 attention kernel
    (codes in fp8_format: "e4m3" or "e5m2").  rope = dict(style=..., base=...,
    pos_offset=...) puts RoPE in front of the rotation of Q and K (one fused
    pass each).  per_tensor=True quantises with one scale per (b, h) instead
    of per 128-row block (not with rope).  q_in_kernel=True leaves Q's
    rotation and quantisation to the attention kernel (attn_fwd_fp8_qrot:
    two pre-pass launches instead of three; d = 64 and 128, not with rope or
    per_tensor)."""
    if q_in_kernel:
        if rope is not None or per_tensor:
            raise ValueError("q_in_kernel is not combined with rope or per_tensor")
        k8, sk = hadamard_rotate_quant(k, signs, stream=stream, fp8_format=fp8_format)
        v8t, sv = hadamard_rotate_quant(v, None, transpose_out=True, stream=stream, fp8_format=fp8_format)
        return attn_fwd_fp8_qrot(q, signs, k8, sk, v8t, sv, causal=causal, softmax_scale=softmax_scale,
                                 stream=stream, fp8_format=fp8_format)
    if per_tensor:
        if rope is not None:
            raise ValueError("per_tensor scales are not combined with rope")
        q8, sq = hadamard_rotate_quant(q, signs, stream=stream, fp8_format=fp8_format, per_tensor=True)
        k8, sk = hadamard_rotate_quant(k, signs, stream=stream, fp8_format=fp8_format, per_tensor=True)
        v8t, sv = hadamard_rotate_quant(v, None, transpose_out=True, stream=stream, fp8_format=fp8_format,
                                        per_tensor=True)
        return attn_fwd_fp8(q8, sq, k8, sk, v8t, sv, causal=causal, softmax_scale=softmax_scale,
                            stream=stream, fp8_format=fp8_format)
    if rope is None:
        q8, sq = hadamard_rotate_quant(q, signs, stream=stream, fp8_format=fp8_format)
        k8, sk = hadamard_rotate_quant(k, signs, stream=stream, fp8_format=fp8_format)
    else:
        q8, sq = rope_hadamard_rotate_quant(q, signs, stream=stream, fp8_format=fp8_format, **rope)
        k8, sk = rope_hadamard_rotate_quant(k, signs, stream=stream, fp8_format=fp8_format, **rope)
    v8t, sv = hadamard_rotate_quant(v, None, transpose_out=True, stream=stream, fp8_format=fp8_format)
    return attn_fwd_fp8(q8, sq, k8, sk, v8t, sv, causal=causal, softmax_scale=softmax_scale,
                        stream=stream, fp8_format=fp8_format)


__all__ = ["AttnError", "attn_bwd", "attn_bwd_noalloc", "clock_probe", "attn_fwd", "attn_fwd_fp8", "attn_fwd_fp8_e2e",
           "attn_fwd_fp8_qrot", "attn_fwd_splitkv", "attn_merge",
           "hadamard_rotate_quant", "load", "rope_hadamard_rotate_quant", "splitkv_chunk"]
