"""attn_bwd_noalloc (the entry point that allocates nothing) against attn_bwd
through the C ABI: two calls in a row, the second with a smaller input, each
bitwise equal to attn_bwd's result on the same inputs (the same kernels run;
only the D_i workspace differs: the library's scratch array instead of a
caller buffer), plus the capacity rejection."""
import pytest
import torch

from exact_attention_forward_06_amd import AttnError, attn_bwd, attn_bwd_noalloc, attn_fwd
from exact_attention_forward_06_amd.inputs import make_inputs, upstream_grad

pytestmark = pytest.mark.gpu


def _case(B, H, N, d, causal, seed):
    print(f"attn_bwd_noalloc B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    inp = make_inputs(B, H, N, d, "bf16", seed=seed)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    do = upstream_grad(B, H, N, d, "bf16", seed=seed).cuda()
    o, lse = attn_fwd(q, k, v, causal=causal)
    ref = attn_bwd(q, k, v, o, lse, do, causal=causal)[:3]
    outs = [torch.full_like(q, float("nan")) for _ in range(3)]
    got = attn_bwd_noalloc(q, k, v, o, lse, do, *outs, causal=causal)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(g, r), f"{name} differs from attn_bwd"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_noalloc_matches_attn_bwd_twice(gpu_lib, d):
    _case(2, 3, 1000, d, True, seed=61)        # first call on the device
    _case(1, 2, 333, d, False, seed=62)        # a smaller one after it


def test_noalloc_rejects_beyond_scratch(gpu_lib):
    q = torch.empty(1, 1, 2 ** 21 + 128, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(q) for _ in range(5)]
    with pytest.raises(AttnError, match="scratch"):
        attn_bwd_noalloc(q, outs[0], outs[1], outs[2], lse, outs[3], outs[4], torch.empty_like(q),
                         torch.empty_like(q))
