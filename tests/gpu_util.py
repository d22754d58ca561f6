"""Helpers for the GPU parity tests: device transfer and the comparison rules.

Comparison rules (the parity bar):
* planes and codebook indices: bit-exact against the oracle;
* scales: exact, except a scale the oracle flags as tie-ambiguous (its exact quotient
  lies within a float64 summation error of a rounding midpoint), which may instead be
  the quotient's other rounding neighbour; that row's later planes and scales are then
  checked against the oracle replayed with the scales the GPU chose;
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
    # rows that agree with the oracle in every scale and bit pass as they are; a row that
    # differs is walked plane by plane with the oracle replayed on the GPU's earlier scales
    diff_rows = np.flatnonzero((g_gp != g_or).any(axis=(0, 2)) | (p_gp != res["planes"]).any(axis=(0, 2)))
    for r in diff_rows:
        forced = {}
        for i in range(k):
            rr = O.binarize(Wr[r:r + 1], k, h=h, scale_fmt=fmt, group=group, forced_g=forced or None)
            assert np.array_equal(rr["planes"][i, 0], p_gp[i, r]), \
                f"plane {i} bits of row {rows[r]} differ (earlier planes' scales as the GPU chose them)"
            for q in range(g_gp.shape[2]):
                gg, go = g_gp[i, r, q], rr["g"][i, 0, q]
                if gg != go:
                    # a scale rounded the other way is allowed only where the exact quotient
                    # is tie-ambiguous, and must then be its other rounding neighbour: one
                    # step of the storage format from the oracle's, on the quotient's side
                    assert rr["ambiguous"][i, 0, q], \
                        f"scale mismatch at (plane,row,group) ({i},{rows[r]},{q}): gpu {gg} oracle {go}"
                    ft = np.float16 if fmt == "f16" else np.float32
                    toward = ft(np.inf) if rr["quot"][i, 0, q] > go else ft(-np.inf)
                    nb = float(np.nextafter(ft(go), toward))
                    assert gg == nb, (f"ambiguous scale at (plane,row,group) ({i},{rows[r]},{q}) is {gg}, "
                                      f"not a rounding neighbour of the quotient (oracle {go}, other {nb})")
                forced[(i, 0, q)] = gg
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
