"""Plain, slow CPU oracle for residual binarized weights.

TEST INFRASTRUCTURE ONLY. The parity tests (``tests/``), ``__graft_entry__.smoke()``
and the CPU baseline timings of ``bench.py`` are the only callers. Nothing under
``residual_binarized_weight_amd/`` imports, links or runs this file, and this file
imports nothing from there: the two implementations share no code. Only the seeded
input generators (``workloads/``, random draws only) feed both.

Arithmetic is float64 on exactly widened fp32/fp16 inputs. Where a value is rounded
to a storage format (the fp16/fp32 scales) the rounding is done exactly, with
``fractions.Fraction``, to nearest with ties to even.

Sources (web pages on the method; cited by title and section):

* [RaBiT] "RaBiT: Residual-Aware Binarization Training for Accurate and Efficient
  LLMs" (paper summary page). Background section "Residual binarization" (k stacked
  +-1 layers, W ~ sum W_i; dual-scale form W_i = g (.) B (.) h with full-precision
  per-channel vectors g, h; matmul-free inference by additions and element-wise
  scaling). Sections "Core method" and "Method step details", Algorithm 2 (forward:
  R_0 = W_FP, B_i = sign(R_{i-1}), W_i = g_i (.) B_i (.) h_i, R_i = R_{i-1} - W_i;
  deployment: derive B_i once, freeze, drop W_FP). Section "Technical novelty"
  (32 columns packed into one uint32). Section "Limitations" (2.02 effective bits).
  Section "Method step details", Algorithm 1 (function-aware initialization: I/O
  channel importance scaling W' = s_out^a_out (.) W (.) s_in^a_in, iterative residual
  SVID over T_max = 20 Gauss-Seidel sweeps with rank-1 SVD scales, mapping back).
  Algorithm 2 also gives the coupled-training step: the forward derives the paths from
  the shared weight with the learnable scales, the backward passes the effective-weight
  gradient to the shared weight and differentiates the scales with B held constant.
* [BTC] "亚1比特大模型量化技术突破与实践" (BTC-LLM sub-1-bit binary codebook page).
  Section 2.1.1 (binary codebook; sign with 0 -> +1; Hamming distance by XOR +
  popcount; binary K-means whose M-step sets each centroid to the sign of its members'
  sum with 0 -> +1; the codebook shrinks to the distinct vectors when there are fewer of
  them than its preset size), 2.1.2 (LUT-GEMM: precompute input-block x codeword sums, accumulate by
  index), 3.2.1 (index | scale | offset layout, one scale group per 16 weights),
  5.1 (v=20, c=65536 for 13B+ models), 5.2 (index width ceil(log2 c) <= 16). Also
  the zero-mean preprocessing of 2.1.1 (each row shifted by its mean before binarization).
* [SigmoidBitLinear] the SigmoidBitLinear blog page: weights binarize to {0, scale_row}
  (a bit keeps the row's scale or gives 0).

Readings taken where the pages are silent:

1. sign(0) = +1, including -0.0 (BTC 2.1.1 maps zero centroid entries to +1).
2. bit value 1 <-> +1, bit 0 <-> -1; LSB-first: bit j of word w is column 32w+j.
3. Scale rule: for B = sign(R) and a given h, the L2-optimal row scale
   g = sum_k |R_k| h_k / sum_k h_k^2 (= row mean |R| when h = 1, the closed-form
   binarization scale), rounded to the scale format.
4. The residual subtracts the *stored* (rounded) scale: deployment runs on the
   stored values (RaBiT Algorithm 2 / deployment stage).
5. Group mode (codebook scales): the same rule over 16-column groups, h = 1.
6. Codebook blocks of v columns, the last one padded with +1 (signs of zero
   weights); ties in Hamming distance go to the lowest codeword index.
7. Initialization (RaBiT Algorithm 1): the residual of path i subtracts the other
   paths at their latest values (Gauss-Seidel, as the page names it; its formula's
   subscript is garbled), the paths start at zero (the first sweep is the greedy
   residual SVID), and the rank-1 fit of |R| is split evenly, ||g|| = ||h|| =
   sqrt(sigma_1). I/O scaling multiplies rows by s_out^a_out and columns by
   s_in^a_in before the sweeps and divides the scales by them afterwards.
8. Binary K-means (BTC 2.1.1): a codeword that no pattern chose keeps its value; the
   distinct patterns replace the codebook in ascending order when they number fewer
   than its size (the entries past them repeat the last distinct pattern, which never
   wins a tie, so an index still points at a distinct pattern); the caller supplies the
   initial codebook; an iteration is an E-step (nearest codeword) then an M-step, and
   a final E-step gives the indices of the returned codebook.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

WORD_BITS = 32

# (precision bits incl. the implicit one, minimum normal exponent, maximum exponent)
_FORMATS = {"f16": (11, -14, 15), "f32": (24, -126, 127)}



def tie_tolerance(L: int) -> float:
    """Relative distance to a rounding midpoint below which a scale over L columns is
    "tie-ambiguous": a float64 evaluation of the same quotient in another summation
    order (relative error <= (L + 2) * 2**-53 for L positive terms, one product
    rounding each and one division) may then round to either neighbour. A factor 4
    of headroom is added."""
    return 4.0 * (L + 2) * 2.0 ** -53


# ---------------------------------------------------------------------------
# rounding to a storage format
# ---------------------------------------------------------------------------
def _floor_log2(a: Fraction) -> int:
    """Largest e with 2**e <= a (a > 0)."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_format(q, fmt: str) -> float:
    """Round the exact rational ``q`` to the nearest value of ``fmt`` ('f16' or 'f32'),
    ties to even (IEEE 754 roundTiesToEven), with gradual underflow and overflow to inf.
    ``fmt == 'f64'`` returns float(q) (already a float64 when q is one)."""
    if fmt == "f64":
        return float(q)
    p, emin, emax = _FORMATS[fmt]
    q = Fraction(q)
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * quantum
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if val > max_finite:
        return sign * math.inf
    return sign * float(val)


def midpoint_distance(q, fmt: str) -> float:
    """Relative distance from the rational ``q`` to the nearest rounding midpoint of ``fmt``."""
    if fmt == "f64":
        return math.inf
    p, emin, _ = _FORMATS[fmt]
    q = abs(Fraction(q))
    if q == 0:
        return math.inf
    e = max(_floor_log2(q), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    m = q / quantum
    fl = m.numerator // m.denominator
    mid = (fl + Fraction(1, 2)) * quantum
    lower_mid = (fl - Fraction(1, 2)) * quantum
    d = min(abs(q - mid), abs(q - lower_mid))
    return float(d / q)


# ---------------------------------------------------------------------------
# signs and bit-planes
# ---------------------------------------------------------------------------
def sign_pm1(R: np.ndarray) -> np.ndarray:
    """sign with sign(0) = +1 (also for -0.0): +1 where R >= 0, else -1. [RaBiT Alg. 2; BTC 2.1.1]"""
    return np.where(R >= 0, 1, -1).astype(np.int8)


def pack_bits(B: np.ndarray) -> np.ndarray:
    """Pack a +-1 matrix (N, K) into uint32 words (N, ceil(K/32)).

    Bit j of word w holds column 32*w + j (LSB first); a set bit means +1. Bits for
    columns >= K are 0. [RaBiT "Technical novelty": 32 columns per uint32]
    """
    N, K = B.shape
    Kw = (K + WORD_BITS - 1) // WORD_BITS
    bits = np.zeros((N, Kw * WORD_BITS), dtype=np.uint8)
    bits[:, :K] = (B > 0)
    by = np.packbits(bits, axis=1, bitorder="little")          # byte b holds columns 8b..8b+7
    return np.ascontiguousarray(by).view("<u4").reshape(N, Kw)


def unpack_bits(words: np.ndarray, K: int) -> np.ndarray:
    """Inverse of :func:`pack_bits`: uint32 words (..., Kw) -> +-1 float64 (..., K)."""
    w = np.ascontiguousarray(words, dtype="<u4")
    by = w.view(np.uint8)
    bits = np.unpackbits(by, axis=-1, bitorder="little")[..., :K]
    return bits.astype(np.float64) * 2.0 - 1.0


# ---------------------------------------------------------------------------
# O1: residual binarization with dual scales
# ---------------------------------------------------------------------------
def _group_bounds(K: int, group: int):
    if group <= 0:
        return [(0, K)]
    return [(c0, min(K, c0 + group)) for c0 in range(0, K, group)]


def binarize(W: np.ndarray, k: int, h: np.ndarray | None = None, scale_fmt: str = "f16",
             group: int = 0, forced_g: dict | None = None):
    """Derive k residual sign planes and their row (or row-group) scales.

    [RaBiT, "Method step details", Algorithm 2, forward pass; "Residual binarization"]
      R_0 = W
      for i = 1..k:
          B_i = sign(R_{i-1})                      (sign(0) = +1)
          g_i = sum_k |R_{i-1}| h_i / sum_k h_i^2  (L2-optimal scale for this B_i and h_i,
                                                    rounded to ``scale_fmt``)
          W_i = g_i (.) B_i (.) h_i
          R_i = R_{i-1} - W_i                      (with the stored g_i)

    ``h`` is (k, K) (values of the stored scale format) or None for all ones.
    ``group > 0`` gives one scale per ``group`` consecutive columns of a row
    (g has shape (k, N, ceil(K/group))); otherwise one per row (k, N, 1).
    ``forced_g`` maps (i, n, q) -> scale, to replay a row with another admissible
    rounding of a tie-ambiguous scale.

    Returns a dict with planes (k, N, ceil(K/32)) uint32, g (k, N, G) float64 holding
    values of ``scale_fmt``, ambiguous (k, N, G) bool, the unrounded quotients as
    float64 (k, N, G) ``quot`` (which side of the stored scale the exact value lies on),
    and the residual row norms ||R_i||_2 for i = 0..k as ``res_norm`` (k+1, N).
    """
    if not np.all(np.isfinite(W)):
        raise ValueError("W holds NaN or Inf")
    W = np.asarray(W)
    N, K = W.shape
    R = W.astype(np.float64)                     # exact widening of fp32 / fp16 / bf16 values
    bounds = _group_bounds(K, group)
    G = len(bounds)
    Kw = (K + WORD_BITS - 1) // WORD_BITS
    planes = np.zeros((k, N, Kw), dtype=np.uint32)
    g = np.zeros((k, N, G), dtype=np.float64)
    amb = np.zeros((k, N, G), dtype=bool)
    quot64 = np.zeros((k, N, G), dtype=np.float64)
    res_norm = np.zeros((k + 1, N), dtype=np.float64)
    res_norm[0] = np.sqrt(np.sum(R * R, axis=1))
    for i in range(k):
        hi = np.ones(K, dtype=np.float64) if h is None else np.asarray(h[i], dtype=np.float64)
        B = sign_pm1(R)
        planes[i] = pack_bits(B)
        g_col = np.empty((N, K), dtype=np.float64)
        absRh = np.abs(R) * hi                   # products rounded once in float64
        for q, (c0, c1) in enumerate(bounds):
            den = math.fsum((hi[c0:c1] * hi[c0:c1]).tolist())
            for n in range(N):
                num = math.fsum(absRh[n, c0:c1].tolist())
                if den == 0.0:
                    gv = 0.0
                    quot = Fraction(0)
                else:
                    quot = Fraction(num) / Fraction(den)
                    gv = round_to_format(quot, scale_fmt)
                if forced_g is not None and (i, n, q) in forced_g:
                    gv = float(forced_g[(i, n, q)])
                else:
                    amb[i, n, q] = quot != 0 and midpoint_distance(quot, scale_fmt) <= tie_tolerance(c1 - c0)
                g[i, n, q] = gv
                quot64[i, n, q] = float(quot)
                g_col[n, c0:c1] = gv
        # W_i = g (.) B (.) h ; g*h is exact in float64 (<= 48 significant bits), *B exact.
        R = R - (g_col * hi[None, :]) * B
        res_norm[i + 1] = np.sqrt(np.sum(R * R, axis=1))
    return {"planes": planes, "g": g, "ambiguous": amb, "quot": quot64, "res_norm": res_norm}


def dequantize(planes: np.ndarray, g: np.ndarray, h: np.ndarray | None, K: int,
               group: int = 0) -> np.ndarray:
    """W_hat = sum_i g_i (.) B_i (.) h_i  [RaBiT "Residual binarization"]."""
    k, N, _ = planes.shape
    out = np.zeros((N, K), dtype=np.float64)
    for i in range(k):
        B = unpack_bits(planes[i], K)
        hi = np.ones(K) if h is None else np.asarray(h[i], dtype=np.float64)
        if group > 0:
            gcol = np.repeat(np.asarray(g[i], dtype=np.float64), group, axis=1)[:, :K]
        else:
            gcol = np.asarray(g[i], dtype=np.float64).reshape(N, -1)[:, :1]
        out += gcol * B * hi[None, :]
    return out


# ---------------------------------------------------------------------------
# O2: the matmul-free product on the packed planes
# ---------------------------------------------------------------------------
def gemv(planes: np.ndarray, g: np.ndarray, h: np.ndarray | None, x: np.ndarray, K: int,
         row_block: int = 512):
    """y[m, n] = sum_i g_i[n] * sum_k B_i[n, k] * h_i[k] * x[m, k]

    [RaBiT "Residual binarization": k parallel paths, each W_i = g_i (.) B_i (.) h_i, so
    y = sum_i g_i (.) (B_i (h_i (.) x)).] Computed in float64 from the unpacked +-1
    planes. Also returns the error scale sum|terms|[m, n] =
    sum_i |g_i[n]| * sum_k |h_i[k] x[m, k]| used by the tolerance
    |y - y_ref| <= 1e-3 * sum|terms|.
    """
    k, N, _ = planes.shape
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    M = x.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    sabs = np.zeros((M, N), dtype=np.float64)
    gg = np.asarray(g, dtype=np.float64).reshape(k, N, -1)[:, :, 0]
    for i in range(k):
        hi = np.ones(K) if h is None else np.asarray(h[i], dtype=np.float64)
        xh = x * hi[None, :]                                  # (M, K), exact products
        habs = np.abs(xh).sum(axis=1)                         # (M,)
        for r0 in range(0, N, row_block):
            r1 = min(N, r0 + row_block)
            B = unpack_bits(planes[i, r0:r1], K)              # (rows, K) +-1
            y[:, r0:r1] += gg[i, r0:r1][None, :] * (xh @ B.T)
            sabs[:, r0:r1] += np.abs(gg[i, r0:r1])[None, :] * habs[:, None]
    return y, sabs


def gemv_variant(planes: np.ndarray, g: np.ndarray, h: np.ndarray | None, mu: np.ndarray | None,
                 x: np.ndarray, K: int, zero_one: bool):
    """The product of the cheap weight variants, y = x W_hat^T, with
    W_hat[n, k] = sum_i g_i[n] * b_i[n, k] * h_i[k] + mu[n], where b is the plane bit read as
    {-1, +1} (zero_one False) or as {0, 1} (zero_one True), and mu an optional per-row offset.

    [SigmoidBitLinear blog: weights binarize to {0, scale_row}: bit 1 keeps the row's scale,
    bit 0 gives 0. BTC 2.1.1, zero-mean preprocessing: each row is shifted by its mean mu before
    binarization, so the row is mu + (binarized W - mu).] Dense float64 product on the
    dequantized matrix. Returns (y, sum|terms|) with sum|terms|[m, n] =
    sum_i |g_i[n]| sum_k |h_i[k] x[m, k]| + |mu[n]| sum_k |x[m, k]|.
    """
    k, N, _ = planes.shape
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    gg = np.asarray(g, dtype=np.float64).reshape(k, N, -1)[:, :, 0]
    What = np.zeros((N, K))
    sabs = np.zeros((x.shape[0], N))
    for i in range(k):
        B = unpack_bits(planes[i], K)                         # +-1
        b = (B > 0).astype(np.float64) if zero_one else B
        hi = np.ones(K) if h is None else np.asarray(h[i], dtype=np.float64)
        What += gg[i][:, None] * b * hi[None, :]
        sabs += np.abs(gg[i])[None, :] * (np.abs(x) @ np.abs(hi))[:, None]
    if mu is not None:
        mu = np.asarray(mu, dtype=np.float64)
        What += mu[:, None]
        sabs += np.abs(mu)[None, :] * np.abs(x).sum(axis=1)[:, None]
    return x @ What.T, sabs


# ---------------------------------------------------------------------------
# O3 / O4: sub-1-bit binary codebook
# ---------------------------------------------------------------------------
def sign_blocks(sign_words: np.ndarray, K: int, v: int) -> np.ndarray:
    """Cut each sign row into v-column blocks (last block padded with +1 signs) and
    return the v-bit patterns (N, ceil(K/v)) as int64; bit t <-> column v*j + t,
    1 <-> +1. [BTC 2.1.1: binary sub-vectors of the sign matrix]"""
    B = unpack_bits(sign_words, K)                          # (N, K) +-1
    N = B.shape[0]
    nb = (K + v - 1) // v
    padded = np.ones((N, nb * v), dtype=np.float64)
    padded[:, :K] = B
    bits = (padded.reshape(N, nb, v) > 0).astype(np.int64)
    weights = (np.int64(1) << np.arange(v, dtype=np.int64))
    return (bits * weights).sum(axis=2)


def hamming_encode(patterns: np.ndarray, codebook: np.ndarray, chunk: int = 64) -> np.ndarray:
    """idx = argmin_c popcount(pattern XOR C[c]), ties to the lowest c.

    Brute force over every codeword. [BTC 2.1.1: Hamming distance on packed +-1
    vectors by XOR + popcount]
    """
    flat = np.asarray(patterns, dtype=np.uint32).reshape(-1)
    C = np.asarray(codebook, dtype=np.uint32)
    out = np.empty(flat.shape[0], dtype=np.int64)
    for s in range(0, flat.shape[0], chunk):
        p = flat[s:s + chunk]
        d = np.bitwise_count(p[:, None] ^ C[None, :])          # (chunk, c)
        out[s:s + chunk] = np.argmin(d, axis=1)                  # first minimum = lowest index
    return out.reshape(np.shape(patterns)).astype(np.uint16 if C.shape[0] <= 65536 else np.int64)


def codebook_mstep(patterns: np.ndarray, idx: np.ndarray, codebook: np.ndarray, v: int):
    """M-step of binary K-means: each codeword becomes the elementwise sign of the sum of
    its members' +-1 vectors, a zero sum giving +1; a codeword without members keeps its
    value. Returns (new codebook as uint32, member count per codeword).

    [BTC 2.1.1: centroid update = sign(sum of the cluster's binary vectors), zeros -> +1]
    """
    P = np.asarray(patterns, dtype=np.int64).reshape(-1)
    I = np.asarray(idx, dtype=np.int64).reshape(-1)
    C = np.asarray(codebook, dtype=np.uint32)
    c = C.shape[0]
    count = np.bincount(I, minlength=c)
    out = C.copy()
    word = np.zeros(c, dtype=np.int64)
    for t in range(v):
        pm = 2.0 * ((P >> t) & 1) - 1.0                      # bit t of every pattern as +-1
        total = np.bincount(I, weights=pm, minlength=c)      # sum over each cluster
        word |= (total >= 0).astype(np.int64) << t
    has = count > 0
    out[has] = word[has].astype(np.uint32)
    return out, count


def codebook_distinct(patterns: np.ndarray) -> np.ndarray:
    """The distinct patterns in ascending order. [BTC 2.1.1: when the number M of distinct
    vectors is below the preset codebook size, the codebook size becomes M]"""
    return np.unique(np.asarray(patterns, dtype=np.int64).reshape(-1)).astype(np.uint32)


def total_hamming(patterns: np.ndarray, idx: np.ndarray, codebook: np.ndarray) -> int:
    """Sum over patterns of the Hamming distance to their assigned codeword."""
    P = np.asarray(patterns, dtype=np.uint32).reshape(-1)
    I = np.asarray(idx, dtype=np.int64).reshape(-1)
    return int(np.bitwise_count(P ^ np.asarray(codebook, dtype=np.uint32)[I]).sum())


def codebook_learn(patterns: np.ndarray, codebook: np.ndarray, v: int, iters: int):
    """Binary K-means on v-bit sign patterns from an initial codebook.

    [BTC 2.1.1] If the M distinct patterns are fewer than the c codewords, they become
    the codebook (ascending, then the last one repeated up to c: the effective size is
    M). Then `iters` iterations of E-step (nearest codeword by Hamming distance, ties to
    the lowest index) and M-step (codebook_mstep), and a final E-step. Returns
    (codebook, idx, M, history of the total Hamming distance after each E-step).
    """
    C = np.asarray(codebook, dtype=np.uint32).copy()
    c = C.shape[0]
    distinct = codebook_distinct(patterns)
    M = distinct.shape[0]
    if M < c:
        C[:M] = distinct
        C[M:] = distinct[-1]
    history = []
    for _ in range(iters):
        idx = hamming_encode(patterns, C)
        history.append(total_hamming(patterns, idx, C))
        C, _ = codebook_mstep(patterns, idx, C, v)
    idx = hamming_encode(patterns, C)
    history.append(total_hamming(patterns, idx, C))
    return C, idx, M, history


def codebook_gemv(idx: np.ndarray, codebook: np.ndarray, v: int, s: np.ndarray, group: int,
                  x: np.ndarray, K: int):
    """y[m, n] = sum_k s[n, k // group] * C[idx[n, k // v]]_(k mod v) * x[m, k], with
    codeword bits read as +-1 (bit 1 <-> +1).

    [BTC 2.1.2 (the LUT-GEMM computes exactly this dot product, with the x-block x
    codeword sums precomputed) and 3.2.1 (one scale per 16 weights)] Computed here as
    the dense dot product on the dequantized matrix, float64. Returns (y, sum|terms|)
    with sum|terms|[m, n] = sum_k |s[n, k // group] * x[m, k]|.
    """
    idx = np.asarray(idx, dtype=np.int64)
    N, nb = idx.shape
    C = np.asarray(codebook, dtype=np.int64)
    words = C[idx]                                            # (N, nb) v-bit patterns
    bits = (words[:, :, None] >> np.arange(v)[None, None, :]) & 1
    Bm = (bits.reshape(N, nb * v)[:, :K].astype(np.float64) * 2.0 - 1.0)
    scol = np.repeat(np.asarray(s, dtype=np.float64), group, axis=1)[:, :K]
    Wd = scol * Bm
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    y = x @ Wd.T
    sabs = np.abs(x) @ np.abs(scol).T
    return y, sabs


# ---------------------------------------------------------------------------
# storage accounting
# ---------------------------------------------------------------------------
def storage_bits_per_weight(N: int, K: int, k: int, scale_bits: int = 16, has_h: bool = True) -> float:
    """Bits per weight of k sign planes plus per-row g_i and (optionally) per-column h_i.

    [RaBiT "Limitations": a 2-bit model stores about 2.02 effective bits once the
    auxiliary scale vectors are counted]
    """
    per_plane_scales = N + (K if has_h else 0)
    return k + scale_bits * k * per_plane_scales / (N * K)


# ---------------------------------------------------------------------------
# initialization: I/O-importance scaling + iterative residual SVID
# ---------------------------------------------------------------------------
def svid_step(R: np.ndarray):
    """One sign-value-independent decomposition of a residual R (N x K):
    B = sign(R) (0 -> +1) and the top singular pair (sigma, u, v) of |R|, returned as
    g = sqrt(sigma) u and h = sqrt(sigma) v, both >= 0, so that B (.) g h^T approximates R.

    [RaBiT, "Method step details", Algorithm 1: each path's scales are extracted from its
    target residual by a rank-1 SVD approximation] |R| is nonnegative, so its top singular
    vectors can be taken nonnegative (Perron-Frobenius); the sign is fixed by making their
    sums positive. The top pair is a library SVD (full SVD when min(N, K) <= 512, else
    scipy's ARPACK svds from a deterministic start vector to machine precision).
    """
    R = np.asarray(R, dtype=np.float64)
    A = np.abs(R)
    N, K = A.shape
    if min(N, K) <= 512:
        U, S, Vt = np.linalg.svd(A, full_matrices=False)
        u, s, v = U[:, 0], S[0], Vt[0]
    else:
        from scipy.sparse.linalg import svds
        U, S, Vt = svds(A, k=1, tol=0, v0=np.ones(min(N, K)), random_state=0)
        u, s, v = U[:, 0], S[0], Vt[0]
    if u.sum() < 0:
        u, v = -u, -v
    B = np.where(R >= 0.0, 1.0, -1.0)          # -0.0 >= 0 holds: sign(0) = +1
    return B, math.sqrt(s) * u, math.sqrt(s) * v


def svid_init(W: np.ndarray, k: int, T: int = 20, s_in: np.ndarray | None = None,
              s_out: np.ndarray | None = None, a_in: float = 0.0, a_out: float = 0.0):
    """Function-aware initialization of k residual paths.

    [RaBiT, "Method step details", Algorithm 1]
      W' = s_out^a_out (.) W (.) s_in^a_in        (I/O channel importance scaling: s_in
                                                    per input column, s_out per output row)
      for t = 1..T, for path i = 1..k (Gauss-Seidel: the other paths at their latest values)
        R_i = W' - sum_{j != i} What_j;  B_i, g'_i, h'_i = SVID(R_i);  What_i = g'_i (.) B_i (.) h'_i
      g_i = s_out^-a_out (.) g'_i,  h_i = s_in^-a_in (.) h'_i  (back to the original domain)
    The paths start at What_j = 0, so the first sweep is the greedy residual SVID. Returns the
    sign planes (packed as in `pack_bits`), g [k][N], h [k][K] (original domain), the scaled-domain
    g', h', and the objective ||W' - sum_i What_i||_F after every path update.
    """
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    fo = np.ones(N) if s_out is None else np.asarray(s_out, dtype=np.float64) ** a_out
    fi = np.ones(K) if s_in is None else np.asarray(s_in, dtype=np.float64) ** a_in
    Wp = fo[:, None] * W * fi[None, :]
    What = np.zeros((k, N, K))
    B = np.ones((k, N, K))
    gp = np.zeros((k, N))
    hp = np.zeros((k, K))
    history = []
    for _ in range(T):
        What_prev = What.copy()  # the previous sweep's paths (a Jacobi sweep would use these)
        for i in range(k):
            R = Wp - (What.sum(axis=0) - What[i])
            B[i], gp[i], hp[i] = svid_step(R)
            What[i] = gp[i][:, None] * B[i] * hp[i][None, :]
            history.append(float(np.linalg.norm(Wp - What.sum(axis=0))))
    planes = np.stack([pack_bits(B[i]) for i in range(k)])
    return {"planes": planes, "B": B, "g": gp / fo[None, :], "h": hp / fi[None, :], "gp": gp, "hp": hp,
            "history": np.array(history)}


# ---------------------------------------------------------------------------
# coupled training step (forward with dynamically derived paths, straight-through backward)
# ---------------------------------------------------------------------------
def qat_forward(W: np.ndarray, g: np.ndarray, h: np.ndarray, X: np.ndarray):
    """Forward pass of a coupled-training layer.

    [RaBiT, "Method step details", Algorithm 2, forward] R_0 = W_FP; for each path i:
    B_i = sign(R_{i-1}) (0 -> +1), What_i = g_i (.) B_i (.) h_i, R_i = R_{i-1} - What_i; the
    layer multiplies by the effective weight What = sum_i What_i: Y = X What^T for X [M][K].
    g [k][N] and h [k][K] are the learnable scales (not recomputed from R). Returns Y, What,
    B [k][N][K] and the packed planes.
    """
    W = np.asarray(W, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    k = g.shape[0]
    R = W.copy()
    What = np.zeros_like(W)
    B = np.empty((k,) + W.shape)
    for i in range(k):
        B[i] = np.where(R >= 0.0, 1.0, -1.0)
        Wi = (g[i][:, None] * B[i]) * h[i][None, :]
        R = R - Wi
        What = What + Wi
    Y = np.atleast_2d(np.asarray(X, dtype=np.float64)) @ What.T
    planes = np.stack([pack_bits(B[i]) for i in range(k)])
    return Y, What, B, planes


def qat_backward(dY: np.ndarray, X: np.ndarray, What: np.ndarray, B: np.ndarray, g: np.ndarray,
                 h: np.ndarray):
    """Backward pass of the same layer.

    [RaBiT, "Method step details", Algorithm 2, backward] the shared weight takes the
    effective-weight gradient, grad W_FP = grad_What L = dY^T X (straight-through: the
    derivation of the paths is not differentiated); the scales follow the chain rule with the
    binary cores B_i held constant: dg_i[n] = sum_c dWhat[n, c] B_i[n, c] h_i[c] and
    dh_i[c] = sum_n dWhat[n, c] B_i[n, c] g_i[n]. Also dX = dY What for the layer below.
    """
    dY = np.atleast_2d(np.asarray(dY, dtype=np.float64))
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    dW = dY.T @ X
    dX = dY @ np.asarray(What, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    dg = np.stack([(dW * B[i]) @ h[i] for i in range(g.shape[0])])
    dh = np.stack([g[i] @ (dW * B[i]) for i in range(g.shape[0])])
    return dW, dX, dg, dh
