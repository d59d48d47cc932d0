"""ctypes binding of libattn.so: the same entry points as include/attn.h,
taking torch device tensors.  Argument marshalling only -- every step of the
computation runs in the HIP kernels; torch provides device memory and the
current stream.  There is no fallback: if the library is missing or a call
fails, an exception is raised."""
from __future__ import annotations

import ctypes
import math
import os

import torch

# ATTN_LIBRARY names another build of the same library (the host-sanitised
# build that the ABI tests run under); unset, the in-tree libattn.so.
LIB_PATH = os.environ.get("ATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "include", "attn.h")

ATTN_OK, ATTN_ERR_INVALID_ARGUMENT, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}
_DTYPE_CODE = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}

_c_i64_3 = ctypes.c_int64 * 3
_vp = ctypes.c_void_p
_i = ctypes.c_int

_SIGNATURES = {
    "attn_abi_version": ([], _i),
    "attn_status_string": ([_i], ctypes.c_char_p),
    "attn_last_error": ([], ctypes.c_char_p),
    "attn_fwd": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _i, _vp], _i),
    "hadamard_rotate_quant": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp], _i),
    "hadamard_rotate_quant_per_tensor": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp], _i),
    "attn_fwd_fp8": ([_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, ctypes.c_float,
                      _i, _vp], _i),
    "attn_fwd_fp8_qrot": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp,
                           ctypes.c_float, _i, _vp], _i),
    "attn_fwd_splitkv": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp,
                          ctypes.c_float, _i, _vp], _i),
    "attn_merge": ([_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp], _i),
    "rope_hadamard_rotate_quant": ([_i, _i, _i, _i, _i, _vp, _vp, _i, ctypes.c_double, _i, _vp, _i, _i, _vp,
                                    _vp, _vp], _i),
    "attn_bwd": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                  ctypes.c_float, _i, _vp], _i),
    "attn_clock_probe": ([_i, _vp, _vp], _i),
    "attn_bwd_noalloc": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          ctypes.c_float, _i, _vp], _i),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m exact_attention_forward_06_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int):
    if status != ATTN_OK:
        lib = load()
        raise AttnError(status, f"{lib.attn_status_string(status).decode()}: "
                                f"{lib.attn_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _buf(t, shape, dtype, device, name):
    """An output or workspace tensor: allocated when t is None, else checked
    to be contiguous with exactly the shape, dtype and device the kernels
    will write (the C ABI cannot see a tensor's size)."""
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous() or t.device != torch.device(device):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} on {device}; got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")
    return t


def _check_signs(signs, d):
    if signs is not None and (signs.dtype != torch.int8 or tuple(signs.shape) != (d,) or not signs.is_contiguous()):
        raise ValueError(f"signs must be a contiguous int8 vector of length d = {d}")


def _bhnd_strides(*ts):
    s = ts[0].stride()
    for t in ts:
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("expected [B, H, N, d] tensors with a contiguous last dim")
        if t.stride() != s or t.shape != ts[0].shape:
            raise ValueError("q, k and v must share shape and strides")
    return _c_i64_3(s[0], s[1], s[2])


def attn_fwd(q, k, v, causal=False, softmax_scale=None, out=None, lse=None, return_lse=True,
             stream=None):
    """O, LSE = attention forward of device tensors q, k, v [B, H, N, d]
    (fp32, fp16 or bf16).  Returns (o, lse) with lse fp32 [B, H, N]
    (None when return_lse is False and no lse buffer is given)."""
    lib = load()
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype among fp32, fp16, bf16")
    B, H, N, d = q.shape
    strides = _bhnd_strides(q, k, v)
    out = _buf(out, (B, H, N, d), q.dtype, q.device, "out")
    if lse is not None or return_lse:
        lse = _buf(lse, (B, H, N), torch.float32, q.device, "lse")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_fwd(_DTYPE_CODE[q.dtype], B, H, N, d, _ptr(q), _ptr(k), _ptr(v), strides,
                        _ptr(out), _ptr(lse), scale, int(bool(causal)), _stream(stream)))
    return out, lse


def splitkv_chunk(N: int, num_splits: int) -> int:
    """Keys per range of attn_fwd_splitkv (attn_splitkv_chunk in attn.h)."""
    per = -(-N // num_splits)
    return -(-per // 128) * 128


def attn_fwd_splitkv(q, k, v, num_splits, causal=False, softmax_scale=None, out=None, lse=None,
                     o_part=None, lse_part=None, stream=None):
    """attn_fwd as num_splits key-range partials plus their merge (fp16 /
    bf16, d = 64, 128 or 256).  Returns (o, lse, o_part, lse_part); the partial
    buffers (fp32 [S, B, H, N, d] and [S, B, H, N]) are allocated unless
    given."""
    lib = load()
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype among fp32, fp16, bf16")
    B, H, N, d = q.shape
    strides = _bhnd_strides(q, k, v)
    dev = q.device
    out = _buf(out, (B, H, N, d), q.dtype, dev, "out")
    lse = _buf(lse, (B, H, N), torch.float32, dev, "lse")
    o_part = _buf(o_part, (num_splits, B, H, N, d), torch.float32, dev, "o_part")
    lse_part = _buf(lse_part, (num_splits, B, H, N), torch.float32, dev, "lse_part")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_fwd_splitkv(_DTYPE_CODE[q.dtype], B, H, N, d, _ptr(q), _ptr(k), _ptr(v), strides,
                                int(num_splits), _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse),
                                scale, int(bool(causal)), _stream(stream)))
    return out, lse, o_part, lse_part


def attn_merge(o_part, lse_part, out_dtype=torch.bfloat16, out=None, lse=None, stream=None):
    """Merge S partials (o_part fp32 [S, B, H, N, d], lse_part fp32
    [S, B, H, N]) into (o [B, H, N, d] of out_dtype, lse fp32 [B, H, N])."""
    lib = load()
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise ValueError("partials must be fp32")
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("partials must be contiguous")
    S, B, H, N, d = o_part.shape
    if tuple(lse_part.shape) != (S, B, H, N):
        raise ValueError("lse_part must be [S, B, H, N]")
    out = _buf(out, (B, H, N, d), out_dtype if out is None else out.dtype, o_part.device, "out")
    lse = _buf(lse, (B, H, N), torch.float32, o_part.device, "lse")
    _check(lib.attn_merge(_DTYPE_CODE[out.dtype], S, B, H, N, d, _ptr(o_part), _ptr(lse_part), _ptr(out),
                          _ptr(lse), _stream(stream)))
    return out, lse


def hadamard_rotate_quant(x, signs=None, block_rows=128, transpose_out=False, out=None,
                          scales=None, stream=None, fp8_format="e4m3", per_tensor=False):
    """FP8 pre-pass of one [B, H, N, d] tensor: optional rotation by
    (1/sqrt(d)) H diag(signs), per-block amax scale and codes in fp8_format
    ("e4m3" or "e5m2"); per_tensor=True takes one scale per (b, h) instead
    (hadamard_rotate_quant_per_tensor: every slot of a head holds it).
    Returns (codes uint8 [B,H,N,d] or [B,H,d,N], scales fp32 [B,H,nblk])."""
    lib = load()
    if x.dtype not in _DTYPE_CODE:
        raise ValueError("x must be fp32, fp16 or bf16")
    B, H, N, d = x.shape
    strides = _bhnd_strides(x)
    nblk = -(-N // block_rows)
    out = _buf(out, (B, H, d, N) if transpose_out else (B, H, N, d), torch.uint8, x.device, "out")
    scales = _buf(scales, (B, H, nblk), torch.float32, x.device, "scales")
    _check_signs(signs, d)
    fn = lib.hadamard_rotate_quant_per_tensor if per_tensor else lib.hadamard_rotate_quant
    _check(fn(_DTYPE_CODE[x.dtype], B, H, N, d, _ptr(x), strides, _ptr(signs), block_rows,
              FP8_FORMATS[fp8_format], int(bool(transpose_out)), _ptr(out), _ptr(scales), _stream(stream)))
    return out, scales


ROPE_STYLES = {"interleaved": 1, "half": 2}


def rope_hadamard_rotate_quant(x, signs=None, style="interleaved", base=10000.0, pos_offset=0, block_rows=128,
                               out=None, scales=None, stream=None, fp8_format="e4m3"):
    """FP8 pre-pass of Q or K with RoPE in front: rows at positions
    pos_offset + n are rotary-embedded (pairs (2i, 2i+1) for "interleaved",
    (i, i + d/2) for "half", angle n * base^(-2i/d)), then optionally rotated
    by (1/sqrt(d)) H diag(signs), then block-quantised.
    Returns (codes uint8 [B,H,N,d], scales fp32 [B,H,nblk])."""
    lib = load()
    if x.dtype not in _DTYPE_CODE:
        raise ValueError("x must be fp32, fp16 or bf16")
    B, H, N, d = x.shape
    strides = _bhnd_strides(x)
    nblk = -(-N // block_rows)
    out = _buf(out, (B, H, N, d), torch.uint8, x.device, "out")
    scales = _buf(scales, (B, H, nblk), torch.float32, x.device, "scales")
    _check_signs(signs, d)
    _check(lib.rope_hadamard_rotate_quant(_DTYPE_CODE[x.dtype], B, H, N, d, _ptr(x), strides, ROPE_STYLES[style],
                                          float(base), int(pos_offset), _ptr(signs), block_rows,
                                          FP8_FORMATS[fp8_format], _ptr(out), _ptr(scales), _stream(stream)))
    return out, scales


def attn_fwd_fp8(q8, q_scale, k8, k_scale, v8t, v_scale, causal=False, softmax_scale=None,
                 block_rows=128, out=None, lse=None, return_lse=True, stream=None, fp8_format="e4m3"):
    """Attention forward on E4M3 codes (q8, k8 [B,H,N,d]; v8t [B,H,d,N]) with
    per-block fp32 scales.  Returns (o bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    lib = load()
    B, H, N, d = q8.shape
    for t in (q8, k8, v8t, q_scale, k_scale, v_scale):
        if not t.is_contiguous():
            raise ValueError("attn_fwd_fp8 takes contiguous tensors")
    nblk = -(-N // block_rows)
    for name, t, shape, dt in (("q8", q8, (B, H, N, d), torch.uint8), ("k8", k8, (B, H, N, d), torch.uint8),
                               ("v8t", v8t, (B, H, d, N), torch.uint8),
                               ("q_scale", q_scale, (B, H, nblk), torch.float32),
                               ("k_scale", k_scale, (B, H, nblk), torch.float32),
                               ("v_scale", v_scale, (B, H, nblk), torch.float32)):
        if tuple(t.shape) != shape or t.dtype != dt:
            raise ValueError(f"{name} must be {dt} of shape {shape}; got {t.dtype} {tuple(t.shape)}")
    out = _buf(out, (B, H, N, d), torch.bfloat16, q8.device, "out")
    if lse is not None or return_lse:
        lse = _buf(lse, (B, H, N), torch.float32, q8.device, "lse")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_fwd_fp8(B, H, N, d, _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale),
                            _ptr(v8t), _ptr(v_scale), block_rows, FP8_FORMATS[fp8_format], _ptr(out),
                            _ptr(lse), scale, int(bool(causal)), _stream(stream)))
    return out, lse


def attn_fwd_fp8_qrot(q, signs, k8, k_scale, v8t, v_scale, causal=False, softmax_scale=None,
                      block_rows=128, out=None, lse=None, return_lse=True, stream=None, fp8_format="e4m3"):
    """attn_fwd_fp8 with Q rotated (signs, the int8 [d] diagonal K was rotated
    with) and quantised by the attention kernel itself: q is fp16 / bf16
    [B,H,N,d] with a contiguous last dim; k8, k_scale, v8t, v_scale as in
    attn_fwd_fp8.  Returns (o bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    lib = load()
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q must be fp16 or bf16")
    B, H, N, d = q.shape
    strides = _bhnd_strides(q)
    for t in (k8, v8t, k_scale, v_scale, signs):
        if not t.is_contiguous():
            raise ValueError("attn_fwd_fp8_qrot takes contiguous codes, scales and signs")
    nblk = -(-N // block_rows)
    for name, t, shape, dt in (("k8", k8, (B, H, N, d), torch.uint8), ("v8t", v8t, (B, H, d, N), torch.uint8),
                               ("k_scale", k_scale, (B, H, nblk), torch.float32),
                               ("v_scale", v_scale, (B, H, nblk), torch.float32),
                               ("signs", signs, (d,), torch.int8)):
        if tuple(t.shape) != shape or t.dtype != dt:
            raise ValueError(f"{name} must be {dt} of shape {shape}; got {t.dtype} {tuple(t.shape)}")
    out = _buf(out, (B, H, N, d), torch.bfloat16, q.device, "out")
    if lse is not None or return_lse:
        lse = _buf(lse, (B, H, N), torch.float32, q.device, "lse")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_fwd_fp8_qrot(_DTYPE_CODE[q.dtype], B, H, N, d, _ptr(q), strides, _ptr(signs), _ptr(k8),
                                 _ptr(k_scale), _ptr(v8t), _ptr(v_scale), block_rows, FP8_FORMATS[fp8_format],
                                 _ptr(out), _ptr(lse), scale, int(bool(causal)), _stream(stream)))
    return out, lse


def attn_bwd(q, k, v, o, lse, dout, causal=False, softmax_scale=None, dq=None, dk=None, dv=None,
             delta=None, stream=None):
    """Gradients (dq, dk, dv) of attn_fwd for the upstream gradient dout,
    from the forward's inputs and outputs (o, lse) -- fp16 / bf16, d = 64 or
    128.  q, k, v are [B, H, N, d] with a contiguous last dim and shared
    strides (as in attn_fwd); o, dout and the gradients are contiguous.
    `delta` (fp32 [B, H, N]) is the library's workspace, allocated unless
    given; on return it holds dO_i . O_i.  Returns (dq, dk, dv, delta)."""
    lib = load()
    if q.dtype not in _DTYPE_CODE or any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must share a dtype among fp16, bf16")
    if lse.dtype != torch.float32:
        raise ValueError("lse must be fp32")
    for t in (o, dout, lse):
        if not t.is_contiguous():
            raise ValueError("attn_bwd takes contiguous o, dout and lse")
    strides = _bhnd_strides(q, k, v)
    B, H, N, d = q.shape
    for t in (k, v, o, dout):
        if t.shape != q.shape:
            raise ValueError("q, k, v, o, dout must share one [B, H, N, d] shape")
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    dev = q.device
    dq = _buf(dq, (B, H, N, d), q.dtype, dev, "dq")     # gradients are contiguous
    dk = _buf(dk, (B, H, N, d), q.dtype, dev, "dk")
    dv = _buf(dv, (B, H, N, d), q.dtype, dev, "dv")
    delta = _buf(delta, (B, H, N), torch.float32, dev, "delta")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_bwd(_DTYPE_CODE[q.dtype], B, H, N, d, _ptr(q), _ptr(k), _ptr(v), strides, _ptr(o), _ptr(lse),
                        _ptr(dout), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), scale, int(bool(causal)),
                        _stream(stream)))
    return dq, dk, dv, delta


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=False, softmax_scale=None, stream=None):
    """attn_bwd through the entry point that allocates nothing: the caller
    passes the outputs dq, dk, dv (contiguous, dtype of q); the D_i
    workspace is the library's scratch array (B*H*N <= 2^21).  Calls that
    overlap on one GPU race on that array."""
    lib = load()
    if q.dtype not in _DTYPE_CODE or any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must share a dtype among fp16, bf16")
    if lse.dtype != torch.float32:
        raise ValueError("lse must be fp32")
    for t in (o, dout, lse):
        if not t.is_contiguous():
            raise ValueError("attn_bwd_noalloc takes contiguous o, dout and lse")
    strides = _bhnd_strides(q, k, v)
    B, H, N, d = q.shape
    for t in (k, v, o, dout):
        if t.shape != q.shape:
            raise ValueError("q, k, v, o, dout must share one [B, H, N, d] shape")
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            raise ValueError(f"{name} is required: attn_bwd_noalloc allocates nothing")
        _buf(t, (B, H, N, d), q.dtype, q.device, name)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_bwd_noalloc(_DTYPE_CODE[q.dtype], B, H, N, d, _ptr(q), _ptr(k), _ptr(v), strides, _ptr(o),
                                _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), scale, int(bool(causal)),
                                _stream(stream)))
    return dq, dk, dv


def clock_probe(spin_us=300, out=None, stream=None):
    """Launch the shader-clock probe (a measurement aid): out (device int64
    [2], allocated if None) receives shader cycles and 100 MHz ticks over
    spin_us microseconds; MHz = out[0] / out[1] * 100 once the stream has
    run it."""
    dev = out.device if out is not None else torch.device("cuda", torch.cuda.current_device())
    out = _buf(out, (2,), torch.int64, dev, "out")
    _check(load().attn_clock_probe(int(spin_us), _ptr(out), _stream(stream)))
    return out


def declared_symbols(header: str = HEADER_PATH):
    """Function names declared in include/attn.h."""
    import re
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))
