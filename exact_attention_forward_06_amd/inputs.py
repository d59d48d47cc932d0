"""Seeded synthetic inputs for the attention forward workloads.

This module is the only code shared by the HIP path's tests/bench and the
CPU oracle.  It draws random numbers and casts them to the storage dtype; it
holds none of the attention arithmetic.

Workloads (all Q, K, V entries i.i.d. N(0, 1) drawn in float32 from a
PCG64 stream, draw order Q, K, V, then the FP8 extras):

  small_fp32       fp32, B=1  H=2  N=256  d=64,  non-causal, seed 1
  bf16_n2048       bf16, B=4  H=16 N=2048 d=128, non-causal, seed 2
  bf16_causal_8k   bf16, B=2  H=16 N=8192 d=128, causal,     seed 3
  bf16_d64         bf16, B=8  H=16 N=4096 d=64,  non-causal, seed 4
  bf16_d256        bf16, B=4  H=8  N=4096 d=256, non-causal, seed 4
  fp8_hadamard_8k  bf16 inputs for the FP8 path, B=2 H=16 N=8192 d=128,
                   non-causal, seed 5; after V the generator draws the
                   outlier channel set (shared by Q and K, scaled x20
                   before the bf16 cast) and the +-1 sign vector D.
  bf16_few_heads_8k  bf16, B=1 H=2 N=8192 d=128, non-causal, seed 9: a
                   long sequence with few heads (64 Q blocks of 256 rows
                   for 256 compute units), the split-KV case.

The random sign diagonal is a random draw of the method (FlashAttention-3
page, section on incoherent processing), so it is produced here and passed
to both the kernel and the oracle as an input.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "fp32" | "fp16" | "bf16" | "fp8"
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    outlier_frac: float = 0.0   # fraction of head-dim channels scaled (FP8 workload)
    outlier_gain: float = 20.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def credited_flops(self) -> float:
        """4*B*H*N^2*d, halved for the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


WORKLOADS = {
    w.name: w
    for w in [
        Workload("small_fp32", "fp32", 1, 2, 256, 64, False, 1),
        Workload("bf16_n2048", "bf16", 4, 16, 2048, 128, False, 2),
        Workload("bf16_causal_8k", "bf16", 2, 16, 8192, 128, True, 3),
        Workload("bf16_d64", "bf16", 8, 16, 4096, 64, False, 4),
        Workload("bf16_d256", "bf16", 4, 8, 4096, 256, False, 4),
        Workload("fp8_hadamard_8k", "fp8", 2, 16, 8192, 128, False, 5, outlier_frac=0.005),
        # non-causal bf16 at the FP8 workload's shape and seed (its Q, K, V
        # before the outlier channels are scaled): the 16-bit context line
        Workload("bf16_8k", "bf16", 2, 16, 8192, 128, False, 5),
        Workload("bf16_few_heads_8k", "bf16", 1, 2, 8192, 128, False, 9),
    ]
}

_TORCH_DTYPE = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16,
                "fp8": torch.bfloat16}


def storage_dtype(dtype: str) -> torch.dtype:
    """Host/device dtype of Q, K, V (the FP8 path receives bf16 Q, K, V)."""
    return _TORCH_DTYPE[dtype]


def n_outlier_channels(d: int, frac: float) -> int:
    return max(1, int(round(frac * d))) if frac > 0 else 0


def make_inputs(B, H, N, d, dtype="bf16", seed=0, outlier_frac=0.0, outlier_gain=20.0):
    """Return a dict with CPU torch tensors q, k, v ([B,H,N,d], storage dtype)
    and, when outlier_frac > 0 or dtype == "fp8", the int8 sign vector
    `signs` [d] and the int64 outlier channel indices `outlier_channels`.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    out = {}
    if dtype == "fp8" or outlier_frac > 0:
        n_out = n_outlier_channels(d, outlier_frac)
        ch = rng.choice(d, n_out, replace=False) if n_out else np.zeros(0, np.int64)
        signs = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
        if n_out:
            q[..., ch] *= np.float32(outlier_gain)
            k[..., ch] *= np.float32(outlier_gain)
        out["signs"] = torch.from_numpy(signs)
        out["outlier_channels"] = torch.from_numpy(np.asarray(ch, dtype=np.int64))
    td = storage_dtype(dtype)
    out["q"] = torch.from_numpy(q).to(td)
    out["k"] = torch.from_numpy(k).to(td)
    out["v"] = torch.from_numpy(v).to(td)
    return out


def workload_inputs(w: Workload | str):
    if isinstance(w, str):
        w = WORKLOADS[w]
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.outlier_frac, w.outlier_gain)


def upstream_grad(B, H, N, d, dtype="bf16", seed=0):
    """The backward's upstream gradient dO [B,H,N,d]: i.i.d. N(0, 1) in
    float32 from its own PCG64 stream (seed sequence [seed, 1]), so the Q, K,
    V of make_inputs(..., seed) are unchanged, cast to the storage dtype."""
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    g = rng.standard_normal((B, H, N, d), dtype=np.float32)
    return torch.from_numpy(g).to(storage_dtype(dtype))


def random_signs(d: int, seed: int) -> torch.Tensor:
    rng = np.random.Generator(np.random.PCG64(seed))
    return torch.from_numpy((rng.integers(0, 2, d) * 2 - 1).astype(np.int8))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of the stored values for the oracle."""
    return t.detach().to("cpu").to(torch.float64).numpy()
