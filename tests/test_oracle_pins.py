"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU needed).

Each test checks the oracle against something other than itself: values worked by
hand from the pages' equations (tests/golden/), closed forms, brute force over all
candidates on tiny inputs, exact rational arithmetic, invariants, and library
routines applied to a *different* representation (the original matrix instead of
the unpacked planes).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import rb_oracle as O
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# rounding to the scale formats
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt,npdt", [("f16", np.float16), ("f32", np.float32)])
def test_round_to_format_matches_ieee_conversion(fmt, npdt):
    rng = np.random.default_rng(7)
    # magnitudes spanning subnormals, normals and overflow of both formats
    exps = rng.uniform(-30 if fmt == "f16" else -155, 17 if fmt == "f16" else 129, 4000)
    vals = np.ldexp(rng.uniform(1.0, 2.0, exps.size), np.floor(exps).astype(int))
    vals *= np.where(rng.random(vals.size) < 0.5, -1.0, 1.0)
    for v in vals:
        got = O.round_to_format(Fraction(float(v)), fmt)
        with np.errstate(over="ignore"):
            want = float(np.float64(v).astype(npdt))
        assert got == want or (math.isinf(got) and math.isinf(want) and np.sign(got) == np.sign(want)), v


def test_round_to_format_ties_to_even_fp16():
    # every rounding midpoint between adjacent positive finite fp16 values goes to the even neighbour
    bits = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = bits.view(np.float16).astype(np.float64)
    hi = (bits + 1).view(np.float16).astype(np.float64)
    for b, a, c in zip(bits[::37], lo[::37], hi[::37]):
        mid = (Fraction(float(a)) + Fraction(float(c))) / 2
        want = float(a) if b % 2 == 0 else float(c)
        assert O.round_to_format(mid, "f16") == want
        eps = (Fraction(float(c)) - Fraction(float(a))) / 1024
        assert O.round_to_format(mid - eps, "f16") == float(a)
        assert O.round_to_format(mid + eps, "f16") == float(c)
    # the largest finite value and the overflow threshold (65504 + 16 rounds to inf by ties-to-even)
    assert O.round_to_format(Fraction(65519), "f16") == 65504.0
    assert math.isinf(O.round_to_format(Fraction(65520), "f16"))


# ---------------------------------------------------------------------------
# O1: the scale rule and the sign rule
# ---------------------------------------------------------------------------
def test_alpha_scan_minimum_at_mean_abs():
    """For B = sign(w), ||w - a*B||^2 over a fine grid of a is minimal at the grid point
    nearest mean|w| (closed form: error(a) = ||w||^2 - 2a*sum|w| + a^2*K)."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        K = int(rng.integers(8, 300))
        w = rng.standard_t(4, size=(1, K)) * 0.02
        res = O.binarize(w, 1, scale_fmt="f64")
        a_or = res["g"][0, 0, 0]
        B = O.unpack_bits(res["planes"][0], K)[0]
        grid = np.linspace(0.5 * a_or, 1.5 * a_or, 10001)
        err = ((w[0][None, :] - grid[:, None] * B[None, :]) ** 2).sum(axis=1)
        best = grid[np.argmin(err)]
        nearest = grid[np.argmin(np.abs(grid - np.abs(w).mean()))]
        assert best == nearest
        assert abs(a_or - np.abs(w).mean()) <= 1e-15 * abs(a_or)


def test_sign_is_optimal_over_all_patterns():
    """Brute force over all 2^8 sign patterns of 1x8 rows: for a > 0, argmin_B ||w - aB||
    is sign(w); with exact zeros both choices tie (0 -> +1 is a tie-break)."""
    rng = np.random.default_rng(12)
    patterns = np.array(list(itertools.product([-1.0, 1.0], repeat=8)))
    for t in range(200):
        w = rng.standard_normal(8)
        if t % 4 == 0:
            w[rng.integers(0, 8, 2)] = 0.0
        res = O.binarize(w[None, :], 1, scale_fmt="f64")
        a = res["g"][0, 0, 0]
        B = O.unpack_bits(res["planes"][0], 8)[0]
        errs = ((w[None, :] - a * patterns) ** 2).sum(axis=1)
        e_or = ((w - a * B) ** 2).sum()
        assert e_or <= errs.min() * (1 + 1e-12)
        n_best = np.sum(np.isclose(errs, errs.min(), rtol=1e-12, atol=0))
        assert n_best == 2 ** int(np.sum(w == 0))
        # joint optimum over (a, B): for each B the best a is max(0, w.B/8)
        ab = np.maximum(0.0, patterns @ w / 8)
        joint = ((w[None, :] - ab[:, None] * patterns) ** 2).sum(axis=1)
        assert e_or <= joint.min() * (1 + 1e-12)


def test_negative_zero_and_zero_pack_to_plus_one():
    d = _golden("pack_layout.json")
    K = d["K"]
    w = np.full((1, K), -0.5, dtype=np.float32)
    w[0, d["nonnegative_columns"]] = 0.75
    w[0, d["zero_columns"]] = 0.0
    w[0, d["negative_zero_columns"]] = -0.0
    res = O.binarize(w, 1)
    want = [int(v, 16) for v in d["expected_words_hex"]]
    assert res["planes"][0, 0].tolist() == want


def test_hand_worked_example_k1_k2():
    d = _golden("worked_k2.json")
    W = np.array([d["W"]], dtype=np.float32)
    x = np.array([d["x"]], dtype=np.float16)
    r1 = O.binarize(W, 1)
    assert r1["planes"][0, 0, 0] == d["k1"]["word1"]
    assert r1["g"][0, 0, 0] == d["k1"]["g1"]
    y1, _ = O.gemv(r1["planes"], r1["g"], None, x, 4)
    assert y1[0, 0] == d["k1"]["y"]
    r2 = O.binarize(W, 2)
    assert r2["planes"][:, 0, 0].tolist() == [d["k1"]["word1"], d["k2"]["word2"]]
    assert r2["g"][:, 0, 0].tolist() == [d["k1"]["g1"], d["k2"]["g2"]]
    assert np.allclose(r2["res_norm"][:, 0] ** 2, d["k2"]["sq_norms"], rtol=0, atol=1e-15)
    y2, _ = O.gemv(r2["planes"], r2["g"], None, x, 4)
    assert y2[0, 0] == d["k2"]["y"]
    # dequantized residual equals the hand-derived R2
    What = O.dequantize(r2["planes"], r2["g"], None, 4)
    assert np.array_equal(W.astype(np.float64) - What, np.array([d["k2"]["R2"]]))


# ---------------------------------------------------------------------------
# O1: invariants and exact arithmetic
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("with_h", [False, True])
def test_residual_norm_non_increasing_in_k(with_h):
    """||R_i|| is non-increasing per row for k = 1..4 (also with fp16-rounded scales and a
    general h with negative entries: the L2-optimal g keeps each step a projection up to
    the rounding, and ||R - a s||^2 = ||R||^2 - K a'(2a - a') <= ||R||^2 for 0 <= a' <= 2a)."""
    W = wl.heavy_tailed_weights(9, 48, 301)
    h = wl.random_scales(3, 4, 301, negative_frac=0.3) if with_h else None
    res = O.binarize(W, 4, h=h)
    rn = res["res_norm"]
    assert np.all(rn[1:] <= rn[:-1] * (1 + 1e-15))
    assert np.all(rn[1] < rn[0])


def _exact_binarize(W, k, h, fmt, group):
    """Independent exact-rational derivation (loops, Fractions) of the same planes and scales."""
    N, K = W.shape
    R = [[Fraction(float(v)) for v in row] for row in W]
    bounds = [(0, K)] if group <= 0 else [(c, min(K, c + group)) for c in range(0, K, group)]
    planes, scales = [], []
    for i in range(k):
        hi = [Fraction(1)] * K if h is None else [Fraction(float(v)) for v in h[i]]
        words = np.zeros((N, (K + 31) // 32), dtype=np.uint32)
        gi = np.zeros((N, len(bounds)))
        for n in range(N):
            B = [1 if R[n][c] >= 0 else -1 for c in range(K)]
            for c in range(K):
                if B[c] > 0:
                    words[n, c // 32] |= np.uint32(1 << (c % 32))
            for q, (c0, c1) in enumerate(bounds):
                num = sum(abs(R[n][c]) * hi[c] for c in range(c0, c1))
                den = sum(hi[c] * hi[c] for c in range(c0, c1))
                g = Fraction(0) if den == 0 else Fraction(O.round_to_format(num / den, fmt))
                gi[n, q] = float(g)
                for c in range(c0, c1):
                    R[n][c] = R[n][c] - g * B[c] * hi[c]
        planes.append(words)
        scales.append(gi)
    return np.stack(planes), np.stack(scales), R


@pytest.mark.parametrize("k,fmt,with_h,group", [(1, "f32", False, 0), (2, "f16", False, 0),
                                                (3, "f16", True, 0), (4, "f16", True, 0),
                                                (2, "f16", False, 16), (1, "f16", False, 16)])
def test_float64_oracle_equals_exact_rationals(k, fmt, with_h, group):
    """On tiny inputs the float64 oracle reproduces an exact-rational derivation bit for bit
    (planes and scales): the float64 residual is exact where claimed and the scale
    rounding is decided correctly."""
    W = wl.heavy_tailed_weights(21 + k, 12, 61)
    W[0, :5] = 0.0
    W[1, 3] = -0.0
    h = wl.random_scales(5, k, 61, negative_frac=0.25) if with_h else None
    res = O.binarize(W, k, h=h, scale_fmt=fmt, group=group)
    assert not res["ambiguous"].any()
    pl, sc, _ = _exact_binarize(W, k, h, fmt, group)
    assert np.array_equal(res["planes"], pl)
    assert np.array_equal(res["g"], sc)


def test_pack_unpack_round_trip_ragged():
    rng = np.random.default_rng(4)
    for K in (1, 31, 32, 33, 100, 1000):
        B = np.where(rng.random((5, K)) < 0.5, -1.0, 1.0)
        words = O.pack_bits(B)
        assert words.shape == (5, (K + 31) // 32)
        assert np.array_equal(O.unpack_bits(words, K), B)
        # padding bits beyond K are zero
        if K % 32:
            assert np.all(words[:, -1] >> np.uint32(K % 32) == 0)


def test_storage_bits_per_weight_is_2_02():
    d = _golden("storage_bpw.json")
    bpw = O.storage_bits_per_weight(d["N"], d["K"], d["k"], d["scale_bits"])
    assert bpw == d["expected_bpw"]
    assert round(bpw, 2) == d["page_value_rounded"]


def test_all_zero_row_and_nan_rejection():
    W = np.zeros((2, 40), dtype=np.float32)
    W[1] = np.linspace(-1, 1, 40)
    res = O.binarize(W, 3)
    assert np.all(res["g"][:, 0, 0] == 0.0)
    assert res["planes"][0, 0, 0] == 0xFFFFFFFF and res["planes"][0, 0, 1] == 0xFF
    W[1, 7] = np.nan
    with pytest.raises(ValueError):
        O.binarize(W, 1)


# ---------------------------------------------------------------------------
# O2: the product, pinned on matrices with a closed-form binarization
# ---------------------------------------------------------------------------
def _walsh_patterns(N, K, rng, count):
    """count sign matrices (N, K) such that every pairwise product of rows is balanced
    (exactly K/2 agreements): B_j = B_1 * H_j with H_j distinct non-constant Walsh rows."""
    assert K % 4 == 0
    B1 = np.where(rng.random((N, K)) < 0.5, -1.0, 1.0)
    out = [B1]
    # Walsh functions of period 4 over the column index, permuted per matrix
    walsh = [np.array([1, -1, 1, -1]), np.array([1, 1, -1, -1]), np.array([1, -1, -1, 1])]
    perm = rng.permutation(K)
    for j in range(count - 1):
        Hj = np.tile(walsh[j], K // 4)[perm]
        out.append(B1 * Hj[None, :])
    return out


@pytest.mark.parametrize("k,N,K", [(1, 7, 64), (2, 5, 96), (3, 9, 40)])
def test_closed_form_recovery_and_product(k, N, K):
    """W = sum_i c_i (.) B_i with c_1 > c_2 + ... > 0 (fp16-exact) and balanced pattern
    products: the derivation recovers every c_i and B_i exactly, the dequantized matrix
    equals W, and the oracle product equals numpy's float64 W @ x on the original W."""
    rng = np.random.default_rng(100 + k)
    Bs = _walsh_patterns(N, K, rng, k)
    cs = []
    for i in range(k):
        c = rng.integers(1, 256, N).astype(np.float64) * 2.0 ** (-8 - 3 * i)
        cs.append(c)
    cs[0] = cs[0] + 1.0                        # c_1 dominates the rest
    if k == 3:
        cs[1] = cs[1] + 2.0 ** -6              # c_2 > c_3
    W = sum(cs[i][:, None] * Bs[i] for i in range(k)).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), sum(cs[i][:, None] * Bs[i] for i in range(k)))
    res = O.binarize(W, k)
    for i in range(k):
        assert np.array_equal(res["g"][i, :, 0], cs[i]), i
        assert np.array_equal(O.unpack_bits(res["planes"][i], K), Bs[i]), i
    assert np.array_equal(O.dequantize(res["planes"], res["g"], None, K), W.astype(np.float64))
    x = wl.activations(77, 3, K).astype(np.float64)
    y, sabs = O.gemv(res["planes"], res["g"], None, x, K)
    assert np.allclose(y, x @ W.astype(np.float64).T, rtol=1e-13, atol=1e-13)
    assert np.all(np.abs(y) <= sabs * (1 + 1e-13))


def test_product_with_general_h_against_dense_matrix():
    """With h != 1 the product equals x @ W_hat^T with W_hat[n,k] = sum_i g_i[n] B_i[n,k] h_i[k]
    assembled element by element (loops), not through the oracle's unpacking."""
    rng = np.random.default_rng(31)
    N, K, k = 6, 37, 2
    Bs = [np.where(rng.random((N, K)) < 0.5, -1.0, 1.0) for _ in range(k)]
    planes = np.stack([O.pack_bits(B) for B in Bs])
    g = rng.uniform(0.01, 0.03, (k, N, 1)).astype(np.float16).astype(np.float64)
    h = wl.random_scales(8, k, K, negative_frac=0.3).astype(np.float64)
    x = wl.activations(78, 2, K).astype(np.float64)
    Wd = np.zeros((N, K))
    for n in range(N):
        for c in range(K):
            Wd[n, c] = sum(g[i, n, 0] * Bs[i][n, c] * h[i, c] for i in range(k))
    y, _ = O.gemv(planes, g, h, x, K)
    assert np.allclose(y, x @ Wd.T, rtol=1e-13, atol=1e-15)


def test_masked_add_identity_exact():
    """sum_k (+-1)_k x_k = 2 * sum_{bit=1} x_k - sum_k x_k, in exact rationals."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        K = int(rng.integers(1, 70))
        x = [Fraction(float(v)) for v in rng.standard_normal(K).astype(np.float16)]
        bits = rng.random(K) < 0.5
        lhs = sum(xv if b else -xv for xv, b in zip(x, bits))
        rhs = 2 * sum(xv for xv, b in zip(x, bits) if b) - sum(x)
        assert lhs == rhs


# ---------------------------------------------------------------------------
# O3 / O4: binary codebook
# ---------------------------------------------------------------------------
def test_sign_blocks_padding_golden():
    d = _golden("sign_blocks.json")
    K, v = d["K"], d["v"]
    w = np.full((1, K), 0.3, dtype=np.float32)
    w[0, d["negative_columns"]] = -0.3
    res = O.binarize(w, 1)
    blocks = O.sign_blocks(res["planes"][0], K, v)
    assert blocks[0].tolist() == [int(s, 16) for s in d["expected_blocks_hex"]]


def test_hamming_encode_matches_bruteforce_loops():
    rng = np.random.default_rng(17)
    for v, c in ((6, 20), (8, 256), (8, 37)):
        C = rng.choice(1 << v, size=c, replace=False).astype(np.uint32)
        pats = rng.integers(0, 1 << v, size=(9, 7))
        got = O.hamming_encode(pats, C)
        for p, gi in zip(pats.reshape(-1), got.reshape(-1)):
            dists = [bin(int(p) ^ int(cw)).count("1") for cw in C]
            best = min(dists)
            assert gi == dists.index(best)      # first (lowest) index among the minima


def test_hamming_ties_go_to_lowest_index():
    C = np.array([0b1100, 0b0011, 0b0101, 0b1010], dtype=np.uint32)
    # 0b0000 is at distance 2 from all four codewords
    assert O.hamming_encode(np.array([[0]]), C)[0, 0] == 0
    # 0b0111 is at distance 1 from 0b0011 (index 1) and 0b0101 (index 2)
    assert O.hamming_encode(np.array([[0b0111]]), C)[0, 0] == 1


def test_nearest_in_hamming_is_max_plus_minus_one_dot():
    """dot(+-a, +-b) = v - 2*Hamming(a, b): the chosen codeword maximizes the +-1 dot
    product (computed with a float matmul), lowest index among equal maxima."""
    rng = np.random.default_rng(19)
    v, c = 10, 200
    C = rng.choice(1 << v, size=c, replace=False).astype(np.uint32)
    pats = rng.integers(0, 1 << v, size=300)
    pm = lambda a: ((a[:, None] >> np.arange(v)) & 1) * 2.0 - 1.0
    dots = pm(pats) @ pm(C.astype(np.int64)).T
    idx = O.hamming_encode(pats, C)
    for r in range(pats.size):
        assert idx[r] == int(np.flatnonzero(dots[r] == dots[r].max())[0])


def test_codebook_gemv_bruteforce_loops():
    rng = np.random.default_rng(23)
    N, K, v, group = 3, 45, 20, 16
    C = rng.choice(1 << v, size=64, replace=False).astype(np.uint32)
    nb = (K + v - 1) // v
    idx = rng.integers(0, 64, size=(N, nb))
    s = rng.uniform(0.01, 0.05, (N, (K + group - 1) // group)).astype(np.float16).astype(np.float64)
    x = wl.activations(90, 2, K).astype(np.float64)
    y, sabs = O.codebook_gemv(idx, C, v, s, group, x, K)
    for m in range(2):
        for n in range(N):
            acc = 0.0
            acc_abs = 0.0
            for kk in range(K):
                bit = (int(C[idx[n, kk // v]]) >> (kk % v)) & 1
                acc += s[n, kk // group] * (1.0 if bit else -1.0) * x[m, kk]
                acc_abs += abs(s[n, kk // group] * x[m, kk])
            assert math.isclose(y[m, n], acc, rel_tol=1e-12, abs_tol=1e-14)
            assert math.isclose(sabs[m, n], acc_abs, rel_tol=1e-12)


def test_codebook_exact_when_blocks_are_codewords():
    """If every sign block of W is itself a codeword, encoding is exact (distance 0) and the
    codebook product equals the group-scaled sign product computed directly on sign(W)."""
    rng = np.random.default_rng(29)
    N, K, v, group = 4, 80, 20, 16
    W = wl.heavy_tailed_weights(31, N, K)
    res = O.binarize(W, 1, group=group)
    pats = O.sign_blocks(res["planes"][0], K, v)
    others = rng.choice(1 << v, size=50, replace=False)
    C = np.unique(np.concatenate([pats.reshape(-1), others])).astype(np.uint32)
    rng.shuffle(C)
    idx = O.hamming_encode(pats, C)
    assert np.array_equal(C[idx.astype(np.int64)], pats.astype(np.uint32))
    x = wl.activations(91, 1, K).astype(np.float64)
    y, _ = O.codebook_gemv(idx, C, v, res["g"][0], group, x, K)
    S = np.where(W >= 0, 1.0, -1.0)
    scol = np.repeat(res["g"][0], group, axis=1)[:, :K]
    assert np.allclose(y, x @ (scol * S).T, rtol=1e-13, atol=1e-15)


def test_group_scales_recover_blockwise_constants():
    """Group mode: a row whose 16-column groups are c_q * (+-1) yields exactly c_q per group."""
    rng = np.random.default_rng(37)
    N, K, group = 3, 75, 16
    G = (K + group - 1) // group
    c = rng.integers(1, 512, (N, G)).astype(np.float64) * 2.0 ** -12
    S = np.where(rng.random((N, K)) < 0.5, -1.0, 1.0)
    W = (np.repeat(c, group, axis=1)[:, :K] * S).astype(np.float32)
    res = O.binarize(W, 1, group=group)
    assert np.array_equal(res["g"][0], c)
    assert np.array_equal(O.unpack_bits(res["planes"][0], K), S)


# ---------------------------------------------------------------------------
# initialization: iterative residual SVID with I/O-importance scaling
# ---------------------------------------------------------------------------
def _obj(R, B, g, h):
    return float(np.linalg.norm(R - B * np.outer(g, h)))


def test_svid_recovers_sign_times_rank1_magnitude_exactly():
    # W = S (.) a b^T with a, b > 0: one path, one sweep reproduces W, B = S (closed form)
    rng = np.random.default_rng(300)
    a, b = rng.uniform(0.5, 2.0, 23), rng.uniform(0.1, 3.0, 41)
    S = np.where(rng.random((23, 41)) < 0.5, -1.0, 1.0)
    W = S * np.outer(a, b)
    r = O.svid_init(W, 1, T=1)
    assert np.array_equal(r["B"][0], S)
    assert np.allclose(np.outer(r["g"][0], r["h"][0]), np.outer(a, b), rtol=1e-12, atol=0)
    assert r["history"][-1] <= 1e-12 * np.linalg.norm(W)
    assert np.all(r["g"][0] > 0) and np.all(r["h"][0] > 0)
    # the planes are the packed signs
    assert np.array_equal(O.unpack_bits(r["planes"][0], 41), S)


def test_svid_step_is_the_alternating_least_squares_optimum():
    # for B = sign(R), g h^T is the best rank-1 fit of |R|: an independent alternating least
    # squares solution (no SVD) reaches the same product, and neither a single sign flip nor
    # a small change of g or h lowers ||R - B (.) g h^T||
    rng = np.random.default_rng(301)
    R = rng.standard_t(4, (17, 29))
    B, g, h = O.svid_step(R)
    A = np.abs(R)
    ga, ha = np.ones(17), np.ones(29)
    for _ in range(2000):
        ga = A @ ha / (ha @ ha)
        ha = A.T @ ga / (ga @ ga)
    assert np.allclose(np.outer(g, h), np.outer(ga, ha), rtol=1e-9, atol=1e-12)
    best = _obj(R, B, g, h)
    for (n, c) in itertools.product(range(17), range(29)):
        Bf = B.copy()
        Bf[n, c] = -Bf[n, c]
        assert _obj(R, Bf, g, h) >= best
    for _ in range(50):
        assert _obj(R, B, g * (1 + 1e-3 * rng.standard_normal(17)), h) >= best
        assert _obj(R, B, g, h * (1 + 1e-3 * rng.standard_normal(29))) >= best


def test_svid_balanced_split():
    # only g h^T is determined by the fit; the split taken is the balanced one,
    # ||g|| = ||h|| = sqrt(sigma_1(|R|)) (a reading: the pages give the rank-1 fit only)
    R = np.random.default_rng(308).standard_normal((9, 14))
    B, g, h = O.svid_step(R)
    s1 = np.linalg.svd(np.abs(R), compute_uv=False)[0]
    assert math.isclose(np.linalg.norm(g), math.sqrt(s1), rel_tol=1e-12)
    assert math.isclose(np.linalg.norm(h), math.sqrt(s1), rel_tol=1e-12)


def test_svid_sign_of_zero_and_nonnegative_scales():
    W = wl.heavy_tailed_weights(302, 12, 40)
    W[3] = 0.0
    W[5, ::4] = -0.0
    r = O.svid_init(W, 2, T=2)
    assert np.all(r["B"][:, 3, :] == 1.0)
    assert np.all(r["g"] >= 0) and np.all(r["h"] >= 0)


@pytest.mark.parametrize("k", [1, 2, 3])
@pytest.mark.parametrize("scaled", [False, True])
def test_svid_gauss_seidel_objective_never_increases(k, scaled):
    # each path update minimises ||W' - sum What|| over that path's (B, g >= 0, h >= 0), so
    # the objective after every update is non-increasing (block coordinate descent)
    rng = np.random.default_rng(303 + k)
    W = wl.heavy_tailed_weights(304 + k, 48, 90)
    kw = {}
    if scaled:
        kw = dict(s_in=rng.lognormal(0, 0.7, 90), s_out=rng.lognormal(0, 0.5, 48), a_in=0.5, a_out=0.3)
    r = O.svid_init(W, k, T=6, **kw)
    hst = r["history"]
    assert np.all(np.diff(hst) <= 1e-12 * hst[0])
    if k > 1:
        assert hst[-1] < hst[k - 1]        # the later sweeps improve on the greedy first one
    else:
        assert np.allclose(hst, hst[0], rtol=1e-12)   # one path: every sweep repeats the same step


def test_svid_first_sweep_is_greedy_residual_svid():
    # with one sweep, path i is the SVID of W minus the paths before it
    W = wl.heavy_tailed_weights(305, 30, 70)
    r = O.svid_init(W, 3, T=1)
    R = W.copy()
    for i in range(3):
        B, g, h = O.svid_step(R)
        assert np.array_equal(B, r["B"][i])
        assert np.allclose(np.outer(g, h), np.outer(r["g"][i], r["h"][i]), rtol=1e-10, atol=1e-14)
        R = R - B * np.outer(g, h)


def test_svid_io_scaling_maps_back_consistently():
    # the scales returned in the original domain rebuild s_out^-a (.) What' (.) s_in^-a, and
    # zero exponents make the result independent of s_in and s_out
    rng = np.random.default_rng(306)
    W = wl.heavy_tailed_weights(307, 20, 50)
    s_in, s_out = rng.lognormal(0, 1, 50), rng.lognormal(0, 1, 20)
    r = O.svid_init(W, 2, T=3, s_in=s_in, s_out=s_out, a_in=0.7, a_out=0.4)
    for i in range(2):
        orig = r["B"][i] * np.outer(r["g"][i], r["h"][i])
        scaled = r["B"][i] * np.outer(r["gp"][i], r["hp"][i])
        assert np.allclose(orig, scaled / np.outer(s_out ** 0.4, s_in ** 0.7), rtol=1e-12, atol=0)
    r0 = O.svid_init(W, 2, T=3, s_in=s_in, s_out=s_out, a_in=0.0, a_out=0.0)
    r1 = O.svid_init(W, 2, T=3)
    assert np.array_equal(r0["B"], r1["B"]) and np.allclose(r0["g"], r1["g"], rtol=1e-12)


# ---------------------------------------------------------------------------
# coupled training step: forward derivation and straight-through backward
# ---------------------------------------------------------------------------
def _qat_case(seed, N=6, K=9, M=4, k=2):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K))
    g = rng.uniform(0.2, 0.6, (k, N))
    h = rng.uniform(0.5, 1.5, (k, K))
    X = rng.standard_normal((M, K))
    dY = rng.standard_normal((M, N))
    return W, g, h, X, dY


def _loss(W, g, h, X, dY):
    return float(np.sum(dY * O.qat_forward(W, g, h, X)[0]))


def test_qat_forward_matches_the_pack_derivation():
    # with the pack's own (L2-optimal, rounded) scales the forward derives the same planes,
    # and its effective weight is the pack's dequantized matrix
    W = wl.heavy_tailed_weights(500, 20, 70)
    for k in (1, 2, 3):
        res = O.binarize(W, k)
        g = res["g"].reshape(k, 20)
        Y, What, B, planes = O.qat_forward(W, g, np.ones((k, 70)), np.eye(70))
        assert np.array_equal(planes, res["planes"])
        assert np.allclose(What, O.dequantize(res["planes"], res["g"], None, 70), rtol=0, atol=1e-15)
        assert np.allclose(Y, What.T, rtol=0, atol=1e-15)


def test_qat_scale_gradients_match_finite_differences():
    # a small change of one scale flips no sign of any residual here, so B is locally constant
    # and the chain rule with B fixed is the exact derivative of the loss sum(dY * Y)
    W, g, h, X, dY = _qat_case(501)
    _, What, B, _ = O.qat_forward(W, g, h, X)
    dW, dX, dg, dh = O.qat_backward(dY, X, What, B, g, h)
    eps = 1e-6
    for (i, n) in itertools.product(range(2), range(6)):
        gp, gm = g.copy(), g.copy()
        gp[i, n] += eps
        gm[i, n] -= eps
        assert np.array_equal(O.qat_forward(W, gp, h, X)[2], B)
        num = (_loss(W, gp, h, X, dY) - _loss(W, gm, h, X, dY)) / (2 * eps)
        assert math.isclose(num, dg[i, n], rel_tol=1e-6, abs_tol=1e-8)
    for (i, c) in itertools.product(range(2), range(9)):
        hp, hm = h.copy(), h.copy()
        hp[i, c] += eps
        hm[i, c] -= eps
        num = (_loss(W, g, hp, X, dY) - _loss(W, g, hm, X, dY)) / (2 * eps)
        assert math.isclose(num, dh[i, c], rel_tol=1e-6, abs_tol=1e-8)


def test_qat_weight_and_input_gradients_match_finite_differences():
    # dW is the gradient with respect to the effective weight (straight-through), dX the
    # gradient with respect to the input
    W, g, h, X, dY = _qat_case(502)
    _, What, B, _ = O.qat_forward(W, g, h, X)
    dW, dX, _, _ = O.qat_backward(dY, X, What, B, g, h)
    eps = 1e-6
    f = lambda Wh, Xv: float(np.sum(dY * (Xv @ Wh.T)))
    for (n, c) in itertools.product(range(6), range(9)):
        E = np.zeros_like(What)
        E[n, c] = eps
        assert math.isclose((f(What + E, X) - f(What - E, X)) / (2 * eps), dW[n, c], rel_tol=1e-6, abs_tol=1e-8)
    for (m, c) in itertools.product(range(4), range(9)):
        E = np.zeros_like(X)
        E[m, c] = eps
        assert math.isclose((f(What, X + E) - f(What, X - E)) / (2 * eps), dX[m, c], rel_tol=1e-6, abs_tol=1e-8)


def test_qat_later_paths_fit_the_residual():
    # path i's signs are those of the residual left by the paths before it (sign(0) = +1)
    W, g, h, X, _ = _qat_case(503, k=3)
    W[2, 3] = 0.0
    _, What, B, _ = O.qat_forward(W, g, h, X)
    R = W.copy()
    for i in range(3):
        assert np.array_equal(B[i], np.where(R >= 0, 1.0, -1.0))
        R = R - g[i][:, None] * B[i] * h[i][None, :]
    assert np.allclose(What, W - R, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# binary codebook learning (binary K-means)
# ---------------------------------------------------------------------------
def test_codebook_mstep_hand_example():
    # v = 4; cluster 0: 1010, 1000, 0010 (bit sums -3, +1, -3, +1 -> 1010); cluster 1: 0001 and
    # 0110 tie on bits 0..2 (-> +1) and agree on bit 3 = 0 (-> 0111); cluster 2 has no member and
    # keeps its codeword
    P = np.array([0b1010, 0b1000, 0b0010, 0b0001, 0b0110])
    idx = np.array([0, 0, 0, 1, 1])
    C = np.array([0b0000, 0b0000, 0b1001], dtype=np.uint32)
    newC, count = O.codebook_mstep(P, idx, C, 4)
    assert newC.tolist() == [0b1010, 0b0111, 0b1001]
    assert count.tolist() == [3, 2, 0]


def test_codebook_mstep_majority_minimizes_hamming():
    # brute force over all 2^v codewords: the M-step word has the least total Hamming distance to
    # its cluster, and among the minimizers (which differ only in tied bits) it is the one with
    # every tied bit +1, i.e. the bitwise OR of all minimizers
    rng = np.random.default_rng(600)
    v, c = 6, 5
    P = rng.integers(0, 1 << v, size=60)
    idx = rng.integers(0, c, size=60)
    idx[:4] = [0, 0, 1, 1]
    P[:4] = [0b000111, 0b111000, 0b101010, 0b010101]       # cluster members forcing ties
    newC, _ = O.codebook_mstep(P, idx, np.zeros(c, np.uint32), v)
    allw = np.arange(1 << v, dtype=np.uint32)
    for j in range(c):
        mem = P[idx == j].astype(np.uint32)
        d = np.bitwise_count(mem[None, :] ^ allw[:, None]).sum(axis=1)
        mins = allw[d == d.min()]
        assert d[newC[j]] == d.min()
        assert newC[j] == np.bitwise_or.reduce(mins)


def test_codebook_learn_never_increases_distortion():
    rng = np.random.default_rng(601)
    v = 8
    P = rng.integers(0, 1 << v, size=(30, 17)) & rng.integers(0, 1 << v, size=(30, 17))   # skewed
    C0 = rng.choice(1 << v, size=24, replace=False).astype(np.uint32)
    C, idx, M, hist = O.codebook_learn(P, C0, v, 6)
    assert M > 24                                          # no shrinking here
    assert all(a >= b for a, b in zip(hist, hist[1:]))
    assert hist[-1] < hist[0]
    # the returned indices are the nearest codewords of the returned codebook
    d = np.bitwise_count(P.reshape(-1, 1).astype(np.uint32) ^ C[None, :])
    assert np.array_equal(d[np.arange(d.shape[0]), idx.reshape(-1).astype(np.int64)], d.min(axis=1))


def test_codebook_learn_shrinks_to_the_distinct_patterns():
    # 5 distinct patterns, 8 codewords: the codebook becomes them (ascending, the last repeated),
    # every pattern is encoded exactly and by its first occurrence
    rng = np.random.default_rng(602)
    vals = np.array([37, 3, 900, 511, 64])
    P = rng.choice(vals, size=(12, 9))
    C, idx, M, hist = O.codebook_learn(P, np.arange(8, dtype=np.uint32) * 101, 10, 3)
    assert M == 5
    assert C.tolist() == [3, 37, 64, 511, 900, 900, 900, 900]
    assert np.array_equal(C[idx.astype(np.int64)], P.astype(np.uint32))
    assert idx.max() <= 4 and hist[-1] == 0


def test_codebook_learn_keeps_the_codebook_when_not_fewer_patterns():
    # exactly c distinct patterns: no replacement; with no iteration the initial codebook comes back
    P = np.array([[5, 9, 12, 9], [12, 5, 7, 7]])
    C0 = np.array([12, 9, 7, 5], dtype=np.uint32)
    C, idx, M, _ = O.codebook_learn(P, C0, 4, 0)
    assert M == 4 and C.tolist() == [12, 9, 7, 5]
    assert np.array_equal(C[idx.astype(np.int64)], P.astype(np.uint32))


def test_codebook_learn_on_layer_signs():
    # signs of a heavy-tailed layer cut into v = 10 blocks: distortion falls over the iterations
    W = wl.heavy_tailed_weights(603, 40, 200)
    words = O.pack_bits(O.sign_pm1(W))
    P = O.sign_blocks(words, 200, 10)
    C0 = np.random.default_rng(603).choice(1 << 10, 64, replace=False).astype(np.uint32)
    _, _, M, hist = O.codebook_learn(P, C0, 10, 4)
    assert M > 64 and hist[-1] < hist[0]


# ---------------------------------------------------------------------------
# cheap product variants: {0, s} planes and a per-row offset
# ---------------------------------------------------------------------------
def test_gemv_variant_hand_example():
    # bits [[1,0,1],[0,1,1]], g = [2, 3], x = [1, 10, 100]
    planes = O.pack_bits(np.array([[1.0, -1.0, 1.0], [-1.0, 1.0, 1.0]]))[None]
    g = np.array([[2.0, 3.0]])
    x = np.array([[1.0, 10.0, 100.0]])
    y01, _ = O.gemv_variant(planes, g, None, None, x, 3, True)
    ypm, _ = O.gemv_variant(planes, g, None, None, x, 3, False)
    ymu, sabs = O.gemv_variant(planes, g, None, np.array([0.5, -1.0]), x, 3, True)
    assert y01.tolist() == [[202.0, 330.0]]
    assert ypm.tolist() == [[182.0, 327.0]]
    assert ymu.tolist() == [[257.5, 219.0]]
    assert sabs.tolist() == [[2 * 111 + 0.5 * 111, 3 * 111 + 1 * 111]]


def test_gemv_variant_matches_loops_and_the_masked_add_identity():
    rng = np.random.default_rng(610)
    k, N, K, M = 2, 5, 37, 3
    Bpm = np.where(rng.random((k, N, K)) < 0.5, -1.0, 1.0)
    planes = np.stack([O.pack_bits(Bpm[i]) for i in range(k)])
    g = rng.uniform(0.1, 1.0, (k, N))
    h = rng.uniform(-1.0, 2.0, (k, K))
    mu = rng.standard_normal(N)
    x = rng.standard_normal((M, K))
    y01, _ = O.gemv_variant(planes, g, h, mu, x, K, True)
    ypm, _ = O.gemv_variant(planes, g, h, None, x, K, False)
    for m in range(M):
        for n in range(N):
            acc = mu[n] * sum(x[m, c] for c in range(K))
            for i in range(k):
                acc += g[i, n] * sum(h[i, c] * x[m, c] for c in range(K) if Bpm[i, n, c] > 0)
            assert math.isclose(y01[m, n], acc, rel_tol=1e-12, abs_tol=1e-12)
    # {0,1} bits = (+-1 bits + 1) / 2: y01 = (ypm + sum_i g_i (h_i . x)) / 2 + mu sum x
    extra = sum(g[i][None, :] * (x @ h[i])[:, None] for i in range(k))
    assert np.allclose(y01, (ypm + extra) / 2 + mu[None, :] * x.sum(axis=1)[:, None], rtol=0, atol=1e-12)
    # with no offset and +-1 bits the variant is the plain product
    assert np.allclose(ypm, O.gemv(planes, g.reshape(k, N, 1), h, x, K)[0], rtol=0, atol=1e-12)
