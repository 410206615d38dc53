"""Comparison rule between GPU outputs and the fp64 oracle.

Per output row (one (token, head) vector of head_dim values):
  rel = max |gpu - oracle| / max |oracle|.
fp32 passes when rel <= 1e-5 on every row.  bf16 passes when the largest
|gpu - oracle| over the whole output is <= 2e-2 AND rel <= 1e-2 on every row.
Rows where the oracle is exactly zero must be exactly zero on the GPU.
"""
import numpy as np
import torch

TOL = {"fp32": dict(rel=1e-5, abs=None), "bf16": dict(rel=1e-2, abs=2e-2)}


def gpu_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(gpu: np.ndarray, ref: np.ndarray, dtype: str):
    """Returns (ok, report) for gpu vs ref, both [..., head_dim]."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    err = np.abs(g - r)
    scale = np.abs(r).max(axis=1)
    zero_rows = scale == 0
    rel = np.where(zero_rows, 0.0, err.max(axis=1) / np.where(zero_rows, 1.0, scale))
    ok_zero = bool(np.all(err[zero_rows] == 0)) if zero_rows.any() else True
    tol = TOL[dtype]
    ok = ok_zero and bool(np.all(np.isfinite(g))) and bool(rel.max(initial=0.0) <= tol["rel"])
    max_abs = float(err.max(initial=0.0))
    if tol["abs"] is not None:
        ok = ok and max_abs <= tol["abs"]
    report = dict(rows=int(g.shape[0]), max_rel=float(rel.max(initial=0.0)), max_abs=max_abs,
                  zero_rows=int(zero_rows.sum()), zero_rows_exact=ok_zero,
                  allclose=int(np.isclose(g, r, atol=2e-2, rtol=1e-2).all(axis=1).sum()))
    return ok, report


def assert_close(gpu, ref, dtype, what=""):
    ok, rep = compare(gpu, ref, dtype)
    assert ok, f"{what} parity failed: {rep}"
    return rep


def tile_rows(cu_q, tile=32, every=8):
    """Rows for the oracle: every `every`-th row of each request, plus both
    edges of each of its `tile`-row q tiles (the rows one wave owns), plus
    its last row."""
    rows = []
    for b in range(len(cu_q) - 1):
        lo, hi = int(cu_q[b]), int(cu_q[b + 1])
        r = np.arange(hi - lo)
        keep = (r % every == 0) | (r % tile == 0) | (r % tile == tile - 1) | (r == hi - lo - 1)
        rows += (lo + r[keep]).tolist()
    return np.array(rows, dtype=np.int32)
