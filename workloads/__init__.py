"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module draws random numbers and nothing else: it holds none of the method's
arithmetic (no signs, scales, packing or products), so that the oracle under
``oracle/`` and the HIP path can both be fed from it without sharing code.

Every draw uses ``numpy.random.default_rng([cfg_id, role, variant])`` with
role 0 = weights, 1 = outlier columns, 2 = activations, 3 = codebook, 4 = learnable
scales, 5 = output gradients, so each
tensor of each workload is reproducible on its own.

Workloads (stand-ins for the layers the pages measure: the 4096x4096 q_proj of the
RaBiT summary's kernel-latency table, the LLaMA MLP 4096<->11008 projections, and
the "8192x28672 MLP layer" of the BTC-LLM page's LUT-GEMM section; the real
trained weights are not available, so the weight statistics are synthetic):

* ``tiny``     256x512, W ~ N(0, 0.02) fp32, k=1, x 1x512 fp32 ~ N(0,1), fp32 scales.
* ``square``   4096x4096, W ~ Student-t(nu=4)*0.02 with round(0.5% of K) input
               columns scaled x10, k=2, x fp16 ~ N(0,1), fp16 scales.
* ``down``     4096x11008 (the MLP down projection), same weight law, k=2, M in {1,4,16}.
* ``gateup``   11008x4096 (gate/up projections), same weight law, k=2, M in {1,4,16}.
* ``wide``     28672x8192, same weight law, k in {1,2}, M in {64,256} fp16 activations.
* ``codebook`` 4096x11008 sign source of the same weight law, v=20, c=65536 distinct
               seeded 20-bit codewords, fp16 scale per 16 weights, M=1.
* coupled training of the ``down`` layer: the same weights as the shared fp32 weight,
  learnable scales g_i ~ 0.8 * 0.02 * 2^-i * U(0.5, 1.5) per row and h_i ~ U(0.5, 1.5) per
  column (fp32), activations X ~ N(0,1) and output gradients dY ~ N(0, 0.01^2) for M tokens
  (drawn in fp32; the caller rounds them to bf16 or fp16).
"""
from __future__ import annotations

import numpy as np

ROLE_W, ROLE_OUTLIER, ROLE_X, ROLE_CODEBOOK, ROLE_SCALES, ROLE_GRAD = 0, 1, 2, 3, 4, 5

# cfg ids used in the seeds: one per workload family.
CFG_TINY, CFG_SQUARE, CFG_MLP, CFG_WIDE, CFG_CODEBOOK = 1, 2, 3, 4, 5
VARIANT = {"down": 0, "gateup": 1}

SHAPES = {
    "tiny": (256, 512),
    "square": (4096, 4096),
    "down": (4096, 11008),
    "gateup": (11008, 4096),
    "wide": (28672, 8192),
    "codebook": (4096, 11008),
}


def rng(cfg_id: int, role: int, variant: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg_id, role, variant])


def gaussian_weights(cfg_id: int, N: int, K: int, std: float = 0.02, variant: int = 0) -> np.ndarray:
    """W ~ N(0, std^2), fp32, shape (N, K)."""
    g = rng(cfg_id, ROLE_W, variant)
    return (g.standard_normal((N, K), dtype=np.float64) * std).astype(np.float32)


def outlier_columns(cfg_id: int, K: int, frac: float = 0.005, variant: int = 0) -> np.ndarray:
    """round(frac*K) distinct input-column indices, drawn uniformly without replacement."""
    n_out = int(round(frac * K))
    g = rng(cfg_id, ROLE_OUTLIER, variant)
    return np.sort(g.choice(K, size=n_out, replace=False))


def heavy_tailed_weights(cfg_id: int, N: int, K: int, variant: int = 0, nu: float = 4.0,
                         scale: float = 0.02, outlier_frac: float = 0.005,
                         outlier_gain: float = 10.0) -> np.ndarray:
    """W ~ Student-t(nu) * scale with a few whole input columns multiplied by ``outlier_gain``.

    Returned as fp32 (N, K), row-major. Rows are generated in blocks to bound memory.
    """
    g = rng(cfg_id, ROLE_W, variant)
    W = np.empty((N, K), dtype=np.float32)
    step = max(1, (1 << 24) // max(K, 1))
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        W[r0:r1] = (g.standard_t(nu, size=(r1 - r0, K)) * scale).astype(np.float32)
    cols = outlier_columns(cfg_id, K, outlier_frac, variant)
    if cols.size:
        W[:, cols] *= np.float32(outlier_gain)
    return W


def activations(cfg_id: int, M: int, K: int, dtype=np.float16, variant: int = 0) -> np.ndarray:
    """x ~ N(0,1) of shape (M, K) in ``dtype`` (rounded from an fp64 draw)."""
    g = rng(cfg_id, ROLE_X, variant * 1000 + M)
    return g.standard_normal((M, K)).astype(dtype)


def codebook(cfg_id: int = CFG_CODEBOOK, c: int = 65536, v: int = 20) -> np.ndarray:
    """c distinct v-bit integers drawn without replacement, stored as uint32 (upper bits 0)."""
    g = rng(cfg_id, ROLE_CODEBOOK)
    return g.choice(1 << v, size=c, replace=False).astype(np.uint32)


def weights_for(name: str, N: int | None = None, K: int | None = None) -> np.ndarray:
    """Weights of a named workload (optionally at a reduced shape, same law and seed)."""
    N0, K0 = SHAPES[name]
    N = N0 if N is None else N
    K = K0 if K is None else K
    if name == "tiny":
        return gaussian_weights(CFG_TINY, N, K)
    if name == "square":
        return heavy_tailed_weights(CFG_SQUARE, N, K)
    if name in ("down", "gateup"):
        return heavy_tailed_weights(CFG_MLP, N, K, variant=VARIANT[name])
    if name == "wide":
        return heavy_tailed_weights(CFG_WIDE, N, K)
    if name == "codebook":
        return heavy_tailed_weights(CFG_CODEBOOK, N, K)
    raise KeyError(name)


def activations_for(name: str, M: int, K: int | None = None) -> np.ndarray:
    K = SHAPES[name][1] if K is None else K
    if name == "tiny":
        return activations(CFG_TINY, M, K, dtype=np.float32)
    cfg = {"square": CFG_SQUARE, "down": CFG_MLP, "gateup": CFG_MLP, "wide": CFG_WIDE,
           "codebook": CFG_CODEBOOK}[name]
    return activations(cfg, M, K, dtype=np.float16, variant=VARIANT.get(name, 0))


def random_scales(seed: int, k: int, L: int, lo: float = 0.25, hi: float = 2.0,
                  negative_frac: float = 0.0, dtype=np.float16) -> np.ndarray:
    """Per-column scale vectors h (k, L) for the general-h test cases (seeded, optional negatives)."""
    g = np.random.default_rng([100, seed])
    h = g.uniform(lo, hi, size=(k, L))
    if negative_frac > 0:
        h *= np.where(g.random((k, L)) < negative_frac, -1.0, 1.0)
    return h.astype(dtype)


def training_scales(cfg_id: int, k: int, N: int, K: int, variant: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Learnable scales of a coupled-training layer: g (k, N) ~ 0.016 * 2^-i * U(0.5, 1.5) and
    h (k, K) ~ U(0.5, 1.5), fp32 (path i's magnitude halves with i, as residual paths do)."""
    g_ = rng(cfg_id, ROLE_SCALES, variant)
    g = g_.uniform(0.5, 1.5, size=(k, N)) * (0.016 * 0.5 ** np.arange(k))[:, None]
    h = g_.uniform(0.5, 1.5, size=(k, K))
    return g.astype(np.float32), h.astype(np.float32)


def output_grads(cfg_id: int, M: int, N: int, std: float = 0.01, variant: int = 0) -> np.ndarray:
    """dY ~ N(0, std^2) of shape (M, N), fp32."""
    g = rng(cfg_id, ROLE_GRAD, variant * 1000 + M)
    return (g.standard_normal((M, N)) * std).astype(np.float32)

