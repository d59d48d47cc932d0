"""Host-side checks of the Python binding: caller-supplied outputs,
workspaces and FP8 inputs must have exactly the shape, dtype and layout the
kernels write or read (the C ABI receives bare pointers and cannot check a
tensor's size).  Every case is rejected before any library call, so these
run on CPU tensors."""
import pytest
import torch

import exact_attention_forward_06_amd as attn


def _qkv(B=1, H=2, N=64, d=64, dt=torch.bfloat16):
    return [torch.zeros(B, H, N, d, dtype=dt) for _ in range(3)]


def test_attn_fwd_rejects_wrong_out():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="out must be"):
        attn.attn_fwd(q, k, v, out=torch.zeros(1, 2, 63, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        attn.attn_fwd(q, k, v, out=torch.zeros(1, 2, 64, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="lse must be"):
        attn.attn_fwd(q, k, v, lse=torch.zeros(1, 2, 65))
    with pytest.raises(ValueError, match="not contiguous"):
        attn.attn_fwd(q, k, v, out=torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16).transpose(2, 3))


def test_attn_bwd_rejects_wrong_buffers():
    q, k, v = _qkv()
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError, match="dq must be"):
        attn.attn_bwd(q, k, v, o, lse, do, dq=torch.zeros(1, 2, 64, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dv must be"):
        attn.attn_bwd(q, k, v, o, lse, do, dv=torch.zeros(1, 2, 64, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="delta must be"):
        attn.attn_bwd(q, k, v, o, lse, do, delta=torch.zeros(2, 64))
    with pytest.raises(ValueError, match="lse must be"):
        attn.attn_bwd(q, k, v, o, torch.zeros(1, 2, 63), do)


def test_splitkv_and_merge_reject_wrong_partials():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="o_part must be"):
        attn.attn_fwd_splitkv(q, k, v, 2, o_part=torch.zeros(3, 1, 2, 64, 64))
    with pytest.raises(ValueError, match="out must be"):
        attn.attn_merge(torch.zeros(2, 1, 2, 64, 64), torch.zeros(2, 1, 2, 64),
                        out=torch.zeros(1, 2, 64, 65, dtype=torch.bfloat16))


def test_prepass_rejects_wrong_codes_scales_signs():
    x = torch.zeros(1, 2, 256, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must be"):
        attn.hadamard_rotate_quant(x, None, transpose_out=True, out=torch.zeros(1, 2, 256, 128, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales must be"):
        attn.hadamard_rotate_quant(x, None, scales=torch.zeros(1, 2, 3))
    with pytest.raises(ValueError, match="signs must be"):
        attn.hadamard_rotate_quant(x, torch.ones(64, dtype=torch.int8))
    with pytest.raises(ValueError, match="signs must be"):
        attn.rope_hadamard_rotate_quant(x, torch.ones(128, dtype=torch.int32))


def test_fp8_rejects_wrong_inputs():
    B, H, N, d = 1, 2, 256, 128
    q8 = torch.zeros(B, H, N, d, dtype=torch.uint8)
    sc = torch.ones(B, H, N // 128)
    with pytest.raises(ValueError, match="v8t must be"):
        attn.attn_fwd_fp8(q8, sc, q8, sc, q8, sc)          # V codes not transposed
    with pytest.raises(ValueError, match="k_scale must be"):
        attn.attn_fwd_fp8(q8, sc, q8, torch.ones(B, H, 1), q8.transpose(2, 3).contiguous(), sc)
