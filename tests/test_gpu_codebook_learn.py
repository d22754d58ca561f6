"""GPU parity of binary codebook learning (rb_codebook_mstep, rb_codebook_distinct,
rb_codebook_learn) against the CPU oracle: all integer work, compared bit for bit. The sign
plane and the initial codebooks are inputs drawn on the host; at the full layer size the
indices are checked on sampled blocks (each must be a nearest codeword of the learned
codebook) and the distinct count against the oracle's."""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from oracle import rb_oracle as O
from tests.gpu_util import dev, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


def sign_plane(seed: int, N: int, K: int) -> np.ndarray:
    W = wl.heavy_tailed_weights(seed, N, K)
    return O.pack_bits(O.sign_pm1(W))


def init_codebook(seed: int, c: int, v: int) -> np.ndarray:
    return np.random.default_rng([700, seed]).choice(1 << v, size=c, replace=False).astype(np.uint32)


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("N,K,v,c", [(16, 1000, 20, 256), (33, 301, 7, 100), (8, 64, 32, 40), (50, 517, 10, 1024),
                                     (3, 45, 20, 1)])
@pytest.mark.parametrize("assign", ["nearest", "random"])
def test_mstep_matches_oracle(N, K, v, c, assign):
    words = sign_plane(710 + v, N, K)
    P = O.sign_blocks(words, K, v)
    C0 = init_codebook(v, c, min(v, 24))
    if assign == "nearest":
        idx = O.hamming_encode(P, C0).astype(np.uint16)
    else:  # arbitrary assignments, many codewords without members
        idx = np.random.default_rng(711).integers(0, c, size=P.shape).astype(np.uint16)
    C_ref, cnt_ref = O.codebook_mstep(P, idx, C0, v)
    C = to_dev(C0)
    cnt = rb.codebook_mstep(to_dev(words), K, to_dev(idx), C, v)
    torch.cuda.synchronize()
    assert np.array_equal(u32(C), C_ref)
    assert np.array_equal(u32(cnt), cnt_ref.astype(np.uint32))


def test_mstep_skewed_assignments():
    """Skewed memberships against the 4096-block slices the M-step counts in: one codeword with
    12000 members (three slices of one bucket), a bucket of exactly 4096 members (one full
    slice), one of 4097 (a full slice and a single member), the rest in the last, partial bucket
    (c = 65436 is not a multiple of 256), every other bucket empty; positions shuffled, K ragged."""
    N, K, v, c = 300, 1990, 20, 65436
    words = sign_plane(720, N, K)
    P = O.sign_blocks(words, K, v)
    total = P.size
    rng = np.random.default_rng(721)
    parts = [np.full(12000, 777), rng.integers(4864, 5120, 4096), rng.integers(51200, 51456, 4097)]
    parts.append(rng.integers(65280, c, total - sum(len(q) for q in parts)))
    idx = rng.permutation(np.concatenate(parts)).astype(np.uint16).reshape(P.shape)
    C0 = init_codebook(21, c, v)
    C_ref, cnt_ref = O.codebook_mstep(P, idx, C0, v)
    C = to_dev(C0)
    cnt = rb.codebook_mstep(to_dev(words), K, to_dev(idx), C, v)
    torch.cuda.synchronize()
    assert cnt_ref[777] == 12000 and cnt_ref[4864:5120].sum() == 4096 and cnt_ref[51200:51456].sum() == 4097
    assert np.array_equal(u32(C), C_ref)
    assert np.array_equal(u32(cnt), cnt_ref.astype(np.uint32))


@pytest.mark.parametrize("distinct_vals,c", [(5, 8), (8, 8), (1, 3), (300, 1000)])
def test_distinct_matches_oracle(distinct_vals, c):
    # rows built from a few repeated 10-column blocks, so the layer has few distinct blocks
    rng = np.random.default_rng(720 + distinct_vals)
    v, N, nb = 10, 24, 30
    vals = rng.choice(1 << v, size=distinct_vals, replace=False)
    P = rng.choice(vals, size=(N, nb))
    P.reshape(-1)[:distinct_vals] = vals                            # every value occurs
    bits = ((P[:, :, None] >> np.arange(v)) & 1).reshape(N, nb * v)
    words = O.pack_bits(np.where(bits > 0, 1.0, -1.0))
    K = nb * v
    C0 = init_codebook(distinct_vals, c, v)
    C = to_dev(C0)
    nd = rb.codebook_distinct(to_dev(words), K, C, v)
    torch.cuda.synchronize()
    distinct = O.codebook_distinct(O.sign_blocks(words, K, v))
    assert int(nd.item()) == len(distinct)
    if len(distinct) < c:
        expect = np.concatenate([distinct, np.full(c - len(distinct), distinct[-1], np.uint32)])
        assert np.array_equal(u32(C), expect)
    else:
        assert np.array_equal(u32(C), C0)                          # not touched


@pytest.mark.parametrize("N,K,v,c,iters", [(16, 1000, 20, 256, 0), (16, 1000, 20, 256, 3), (40, 777, 12, 512, 2),
                                           (24, 300, 10, 1000, 2), (7, 129, 6, 16, 5)])
def test_learn_matches_oracle(N, K, v, c, iters):
    words = sign_plane(730 + v, N, K)
    P = O.sign_blocks(words, K, v)
    C0 = init_codebook(v, c, v)
    C_ref, idx_ref, M_ref, _ = O.codebook_learn(P, C0, v, iters)
    C, idx, nd = rb.codebook_learn(to_dev(words), K, to_dev(C0), v, iters)
    torch.cuda.synchronize()
    assert int(nd.item()) == M_ref
    assert np.array_equal(u32(C), C_ref)
    assert np.array_equal(idx.cpu().numpy().view(np.uint16), idx_ref.astype(np.uint16))


def test_learn_is_deterministic_and_repeatable():
    words = to_dev(sign_plane(740, 64, 2000))
    C0 = init_codebook(740, 1024, 20)
    a = rb.codebook_learn(words, 2000, to_dev(C0), 20, 3)
    b = rb.codebook_learn(words, 2000, to_dev(C0), 20, 3)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_learn_mlp_down_layer_sampled():
    # the 4096 x 11008 sign matrix, v = 20, c = 65536, one iteration from the seeded codebook:
    # the distinct count equals the oracle's, sampled blocks are encoded to a nearest codeword of
    # the learned codebook, and every codeword is a v-bit word
    W = wl.weights_for("codebook")
    N, K = W.shape
    words = O.pack_bits(O.sign_pm1(W))
    C0 = wl.codebook()
    C, idx, nd = rb.codebook_learn(to_dev(words), K, to_dev(C0), 20, 1)
    torch.cuda.synchronize()
    P = O.sign_blocks(words, K, 20)
    assert int(nd.item()) == len(O.codebook_distinct(P))
    Cn = u32(C)
    assert np.all(Cn < (1 << 20))
    rs = np.random.default_rng(750)
    rows = rs.choice(N, 24, replace=False)
    sub = P[rows]
    got = idx.cpu().numpy().view(np.uint16)[rows]
    assert np.array_equal(got, O.hamming_encode(sub, Cn))


@pytest.mark.parametrize("N,K,v,c,iters", [(1, 1, 20, 1, 2), (1, 7, 3, 8, 2), (2, 45, 20, 3, 3), (1, 64, 24, 5, 1)])
def test_learn_degenerate_shapes(N, K, v, c, iters):
    # a single block, a codebook larger than the distinct blocks, one codeword, the widest v
    words = sign_plane(760 + K, N, K)
    P = O.sign_blocks(words, K, v)
    C0 = init_codebook(K, c, v)
    C_ref, idx_ref, M_ref, _ = O.codebook_learn(P, C0, v, iters)
    C, idx, nd = rb.codebook_learn(to_dev(words), K, to_dev(C0), v, iters)
    torch.cuda.synchronize()
    assert int(nd.item()) == M_ref
    assert np.array_equal(u32(C), C_ref)
    assert np.array_equal(idx.cpu().numpy().view(np.uint16), idx_ref.astype(np.uint16))


def test_mstep_mlp_down_layer_full():
    # the M-step on the whole 4096 x 11008 sign matrix (2.26 M blocks, v = 20, c = 65536), with
    # the indices of the nearest-codeword encode: codebook and member counts bit-exact
    W = wl.weights_for("codebook")
    N, K = W.shape
    words = O.pack_bits(O.sign_pm1(W))
    C0 = wl.codebook()
    wd = to_dev(words)
    idx = rb.codebook_encode(wd, K, to_dev(C0), 20, table=True)
    P = O.sign_blocks(words, K, 20)
    idx_np = idx.cpu().numpy().view(np.uint16)
    C_ref, cnt_ref = O.codebook_mstep(P, idx_np, C0, 20)
    C = to_dev(C0)
    cnt = rb.codebook_mstep(wd, K, idx, C, 20)
    torch.cuda.synchronize()
    assert np.array_equal(u32(C), C_ref)
    assert np.array_equal(u32(cnt), cnt_ref.astype(np.uint32))
