"""Full-size comparisons against the fp64 oracle, one head per task.

Test harness only.  The oracle functions are called unchanged; this module
only runs them for many heads at once in worker processes (one BLAS thread
each, at most 16 workers) and reduces each head's comparison with the GPU
result to a few sums, so a whole workload can be checked element by element
in seconds of wall time.  Workers are started with "spawn": they import
numpy and the oracle, never the GPU runtime.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

import oracle


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is installed here
        pass


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def map_heads(fn, tasks):
    """[fn(*t) for t in tasks], computed in worker processes."""
    tasks = list(tasks)
    if len(tasks) <= 1:
        return [fn(*t) for t in tasks]
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=min(workers(), len(tasks)), mp_context=ctx,
                                initializer=_init_worker) as ex:
        return list(ex.map(fn, *zip(*tasks)))


def head_errors(q, k, v, o_gpu, lse_gpu, scale, causal):
    """One head: the exact oracle against the GPU's O and LSE.  Arrays may
    come as float32 (bf16 values are exact in it); they are upcast to fp64.
    Returns the sums a whole-workload check needs."""
    q, k, v, o_gpu, lse_gpu = (np.asarray(x, np.float64) for x in (q, k, v, o_gpu, lse_gpu))
    o_ref, lse_ref = oracle.attention_head(q, k, v, scale, causal)
    err = np.abs(o_gpu - o_ref)
    lerr = np.abs(lse_gpu - lse_ref)
    return {"max_abs": float(err.max()), "sum_abs": float(err.sum()), "count": int(err.size),
            "lse_max": float(lerr.max()), "finite": bool(np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all())}


def reduce_errors(parts):
    """Combine head_errors results: max |O err|, mean |O err|, max |LSE err|."""
    n = sum(p["count"] for p in parts)
    return {"max_abs": max(p["max_abs"] for p in parts), "mean_abs": sum(p["sum_abs"] for p in parts) / n,
            "lse_max": max(p["lse_max"] for p in parts), "finite": all(p["finite"] for p in parts),
            "heads": len(parts)}


def fp8_head_errors(q, k, v, signs, o_gpu, lse_gpu, scale, causal, block_rows=128, fmt="e4m3"):
    """One head of the FP8 path.  q, k, v: the bf16 inputs upcast to fp64
    [N, d]; signs: the rotation's +-1 vector or None (unrotated codes);
    o_gpu, lse_gpu: the GPU result.  Returns squared-error sums of the GPU
    against (a) the oracle's simulation with the rounded P of the second
    product (the kernel's reading), (b) the simulation with P exact (the
    quantisation floor of Q, K and V alone), (c) exact attention, plus the
    same sums for the two simulations against exact attention and the LSE
    distance to (a)."""
    q, k, v, o_gpu, lse_gpu = (np.asarray(x, np.float64) for x in (q, k, v, o_gpu, lse_gpu))
    o_ex, _ = oracle.attention_head(q, k, v, scale, causal)
    o_p, lse_p = oracle.attention_fp8_simulated(q, k, v, signs, scale, causal, block_rows,
                                                quantize_p=True, fmt=fmt)
    o_f, _ = oracle.attention_fp8_simulated(q, k, v, signs, scale, causal, block_rows, fmt=fmt)

    def sq(a, b):
        return float(np.sum((a - b) ** 2))

    return {"gpu_simp": sq(o_gpu, o_p), "simp": float(np.sum(o_p ** 2)),
            "gpu_floor": sq(o_gpu, o_f), "floor": float(np.sum(o_f ** 2)),
            "gpu_exact": sq(o_gpu, o_ex), "exact": float(np.sum(o_ex ** 2)),
            "simp_exact": sq(o_p, o_ex), "floor_exact": sq(o_f, o_ex),
            "lse_simp_max": float(np.max(np.abs(lse_gpu - lse_p))),
            "lse_simp_sum": float(np.sum(np.abs(lse_gpu - lse_p))), "rows": int(lse_gpu.size),
            "lse_simp_abs": np.abs(lse_gpu - lse_p).astype(np.float32),
            "finite": bool(np.isfinite(o_gpu).all())}


def reduce_fp8(parts):
    """Relative RMS errors over all heads from fp8_head_errors sums."""
    s = {key: sum(p[key] for p in parts) for key in parts[0]
         if key not in ("lse_simp_max", "finite", "lse_simp_abs")}
    lse_mean = s["lse_simp_sum"] / s["rows"]
    lse_p99 = float(np.quantile(np.concatenate([p["lse_simp_abs"] for p in parts]), 0.99))
    return {"gpu_vs_simp": (s["gpu_simp"] / s["simp"]) ** 0.5,
            "gpu_vs_floor": (s["gpu_floor"] / s["floor"]) ** 0.5,
            "gpu_vs_exact": (s["gpu_exact"] / s["exact"]) ** 0.5,
            "simp_vs_exact": (s["simp_exact"] / s["exact"]) ** 0.5,
            "floor_vs_exact": (s["floor_exact"] / s["exact"]) ** 0.5,
            "lse_simp_max": max(p["lse_simp_max"] for p in parts), "lse_simp_mean": lse_mean,
            "lse_simp_p99": lse_p99,
            "finite": all(p["finite"] for p in parts), "heads": len(parts)}
