"""Helpers for the GPU parity tests: device transfer and the comparison rules.

Comparison rules (the parity bar):
* planes and codebook indices: bit-exact against the oracle;
* scales: exact, except a scale the oracle flags as tie-ambiguous (its exact quotient
  lies within a float64 summation error of a rounding midpoint), which may be either
  neighbour; that row's later planes are then checked against the oracle replayed with
  the scale the GPU chose;
* products: |y - y_ref| <= 1e-3 * sum|terms| element by element (fp32 accumulation,
  the output rounding included in the budget); for fp16 outputs the bound also admits
  the absolute floor of fp16's gradual underflow, half the subnormal spacing 2^-25,
  which an exact result rounded to fp16 can already reach when |y| < 2^-14.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import rb_oracle as O

TOL = 1e-3


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def planes_np(planes: torch.Tensor, K: int) -> np.ndarray:
    Kw = (K + 31) // 32
    return planes.cpu().numpy().view(np.uint32)[..., :Kw]


def scales_np(g: torch.Tensor, k: int, N: int) -> np.ndarray:
    a = g.float().cpu().numpy().astype(np.float64)
    return a.reshape(k, N, -1)


def assert_pack_matches(W: np.ndarray, k: int, h, fmt: str, group: int, planes_gpu: np.ndarray,
                        g_gpu: np.ndarray, rows=None):
    """Compare the GPU derivation of W's rows (all, or the given subset) with the oracle."""
    rows = np.arange(W.shape[0]) if rows is None else np.asarray(rows)
    Wr = W[rows]
    res = O.binarize(Wr, k, h=h, scale_fmt=fmt, group=group)
    g_or, amb = res["g"], res["ambiguous"]
    g_gp = g_gpu[:, rows, :]
    p_gp = planes_gpu[:, rows, :]
    bad = (g_gp != g_or) & ~amb
    assert not bad.any(), f"scale mismatch at (plane,row,group) {np.argwhere(bad)[:5].tolist()}: " \
                          f"gpu {g_gp[bad][:5]} oracle {g_or[bad][:5]}"
    replay_rows = sorted(set(np.argwhere((g_gp != g_or) & amb)[:, 1].tolist()))
    for r in replay_rows:
        forced = {(i, 0, q): g_gp[i, r, q] for i in range(k) for q in range(g_gp.shape[2])}
        rr = O.binarize(Wr[r:r + 1], k, h=h, scale_fmt=fmt, group=group, forced_g=forced)
        # the GPU's choice must be one of the two neighbours the exact quotient lies between
        assert np.array_equal(rr["planes"][:, 0], p_gp[:, r]), f"replayed row {rows[r]} planes differ"
    keep = np.setdiff1d(np.arange(len(rows)), replay_rows)
    diff = p_gp[:, keep] != res["planes"][:, keep]
    assert not diff.any(), f"plane bits differ at (plane,row,word) {np.argwhere(diff)[:5].tolist()}"
    return res


FP16_FLOOR = 2.0 ** -25


def assert_product_close(y_gpu: np.ndarray, y_ref: np.ndarray, sabs: np.ndarray, tol: float = TOL,
                         fp16_out: bool = True):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    lim = tol * sabs + (FP16_FLOOR if fp16_out else 0.0)
    bad = err > lim
    assert not bad.any(), (f"{bad.sum()} outputs out of tolerance; worst ratio "
                           f"{np.max(err / np.maximum(lim, 1e-300)):.3g} at {np.argwhere(bad)[:3].tolist()}")
    return float(np.max(err / np.maximum(lim, 1e-300)))
