"""GPU parity of the binary-codebook path: rb_codebook_encode (bit-exact indices) and
rb_codebook_gemv (within 1e-3 * sum|terms|)."""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from oracle import rb_oracle as O
from tests.gpu_util import assert_pack_matches, assert_product_close, dev, planes_np, scales_np, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


def test_codebook_encode_full_codebook_sampled_rows():
    W = wl.weights_for("codebook")
    N, K = W.shape
    rows = np.random.default_rng(3).choice(N, 48, replace=False)
    C = wl.codebook()
    Ws = np.ascontiguousarray(W[rows])
    planes, s = rb.pack(torch.from_numpy(Ws).to(dev()), 1, group=16)
    idx = rb.codebook_encode(planes[0], K, to_dev(C), 20)
    idx = idx.cpu().numpy().view(np.uint16)
    res = assert_pack_matches(Ws, 1, None, "f16", 16, planes_np(planes, K), scales_np(s, 1, len(rows)))
    pats = O.sign_blocks(res["planes"][0], K, 20)
    idx_ref = O.hamming_encode(pats, C)
    assert np.array_equal(idx, idx_ref)


@pytest.mark.parametrize("K,v,c", [(45, 20, 64), (100, 7, 1000), (257, 32, 300), (64, 1, 2), (33, 12, 4096)])
def test_codebook_encode_shapes(K, v, c):
    W = wl.heavy_tailed_weights(80, 13, K)
    rng = np.random.default_rng(K + v)
    C = rng.choice(min(1 << v, 1 << 24), size=min(c, 1 << v), replace=False).astype(np.uint32)
    res = O.binarize(W, 1)
    idx = rb.codebook_encode(to_dev(res["planes"][0]), K, to_dev(C), v).cpu().numpy().view(np.uint16)
    assert np.array_equal(idx, O.hamming_encode(O.sign_blocks(res["planes"][0], K, v), C))


def test_codebook_gemv_config():
    N, K, v, group = 4096, 11008, 20, 16
    rng = np.random.default_rng(8)
    C = wl.codebook()
    idx = rng.integers(0, C.size, size=(N, (K + v - 1) // v)).astype(np.uint16)
    W = wl.weights_for("codebook")
    s = np.abs(W).reshape(N, K // group, group).mean(axis=2).astype(np.float16)  # any fp16 group scales
    x = wl.activations_for("codebook", 1)
    y = rb.codebook_gemv(to_dev(idx), to_dev(C), v, to_dev(s), group, to_dev(x), K)
    y = y.float().cpu().numpy()
    y_ref, sabs = O.codebook_gemv(idx, C, v, s.astype(np.float64), group, x, K)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("K,v,group,M", [(45, 20, 16, 1), (1000, 20, 16, 2), (333, 12, 8, 4), (64, 32, 64, 1)])
def test_codebook_gemv_shapes(K, v, group, M):
    N = 21
    rng = np.random.default_rng(K)
    c = 500
    C = rng.choice(1 << v, size=c, replace=False).astype(np.uint32)
    idx = rng.integers(0, c, size=(N, (K + v - 1) // v)).astype(np.uint16)
    s = rng.uniform(0.01, 0.05, (N, (K + group - 1) // group)).astype(np.float16)
    x = wl.activations(81, M, K)
    y = rb.codebook_gemv(to_dev(idx), to_dev(C), v, to_dev(s), group, to_dev(x), K).float().cpu().numpy()
    y_ref, sabs = O.codebook_gemv(idx, C, v, s.astype(np.float64), group, x, K)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("K", [16, 80, 81, 1000, 5519, 7760, 7761, 11008, 15520, 15521])
@pytest.mark.parametrize("N", [1, 37])
def test_codebook_lut_path_shapes(K, N):
    # M = 1, v = 20, group = 16 takes the nibble-table kernel for K <= 15520 (one phase up to
    # 7760 columns, two above); 15521 goes to the per-column kernel. Odd K exercises the
    # activation tail inside a dword; N = 37 leaves rows past N in the last block.
    v, group = 20, 16
    rng = np.random.default_rng(K * 7 + N)
    C = wl.codebook()
    idx = rng.integers(0, C.size, size=(N, (K + v - 1) // v)).astype(np.uint16)
    s = rng.uniform(0.001, 0.05, (N, (K + group - 1) // group)).astype(np.float16)
    x = wl.activations(82, 1, K)
    y = rb.codebook_gemv(to_dev(idx), to_dev(C), v, to_dev(s), group, to_dev(x), K).float().cpu().numpy()
    y_ref, sabs = O.codebook_gemv(idx, C, v, s.astype(np.float64), group, x, K)
    assert_product_close(y, y_ref, sabs)


def test_codebook_pipeline_pack_encode_product():
    # sign plane and group scales from rb_pack, indices from rb_codebook_encode, then the
    # LUT product, all on the GPU; the oracle recomputes every stage from W
    W = wl.weights_for("codebook", N=40)
    N, K = W.shape
    C = wl.codebook()
    planes, s = rb.pack(torch.from_numpy(W).to(dev()), 1, group=16)
    idx = rb.codebook_encode(planes[0], K, to_dev(C), 20)
    x = wl.activations_for("codebook", 1)
    y = rb.codebook_gemv(idx, to_dev(C), 20, s.reshape(N, -1), 16, to_dev(x), K).float().cpu().numpy()
    res = O.binarize(W, 1, group=16)
    assert not res["ambiguous"].any()
    idx_ref = O.hamming_encode(O.sign_blocks(res["planes"][0], K, 20), C)
    assert np.array_equal(idx.cpu().numpy().view(np.uint16), idx_ref)
    y_ref, sabs = O.codebook_gemv(idx_ref, C, 20, res["g"][0], 16, x, K)
    assert_product_close(y, y_ref, sabs)


# ---- encoding through the nearest-codeword table (breadth-first search over all 2^v patterns)

def _sign_words(seed, N, K):
    return O.binarize(wl.heavy_tailed_weights(seed, N, K), 1)["planes"][0]


@pytest.mark.parametrize("N,K,v,c,dups", [(37, 333, 8, 40, 0), (37, 333, 8, 40, 12), (13, 1000, 20, 3000, 50),
                                          (5, 97, 1, 2, 0), (9, 450, 12, 4096, 0), (4, 100, 24, 300, 20),
                                          (21, 700, 16, 1, 0)])
def test_codebook_encode_table_matches_oracle(N, K, v, c, dups):
    # distinct codewords plus repeats of some of them at later indices (a repeat must never win:
    # ties go to the lowest index), ragged K (the last block padded with +1)
    words = _sign_words(90 + v, N, K)
    rng = np.random.default_rng([91, v, c])
    C = rng.choice(1 << v, size=min(c, 1 << v), replace=False).astype(np.uint32)
    if dups:
        C = np.concatenate([C, C[rng.integers(0, len(C), dups)]])
    rng.shuffle(C[len(C) // 2:])
    P = O.sign_blocks(words, K, v)
    ref = O.hamming_encode(P, C)
    wd, Cd = to_dev(words), to_dev(C)
    got = rb.codebook_encode(wd, K, Cd, v, table=True).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    brute = rb.codebook_encode(wd, K, Cd, v).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, brute)


def test_codebook_encode_table_equidistant_ties():
    # two codewords 0000 and 1111 (v = 4): every block with two set bits is equidistant and
    # goes to index 0; the same codewords in the other order send it to index 0 again (1111)
    v, K = 4, 64
    blocks = np.array([[0b0011, 0b0101, 0b1001, 0b0110, 0b1010, 0b1100, 0b0001, 0b0111,
                        0b0000, 0b1111, 0b1011, 0b0010, 0b1101, 0b0100, 0b1000, 0b1110]])
    bits = ((blocks[:, :, None] >> np.arange(v)) & 1).reshape(1, K)
    words = O.pack_bits(np.where(bits > 0, 1.0, -1.0))
    for C in (np.array([0b0000, 0b1111], np.uint32), np.array([0b1111, 0b0000], np.uint32),
              np.array([0b0001, 0b0010, 0b0100, 0b1000], np.uint32)):
        ref = O.hamming_encode(O.sign_blocks(words, K, v), C)
        got = rb.codebook_encode(to_dev(words), K, to_dev(C), v, table=True).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref)


def test_codebook_encode_table_full_layer():
    # the 4096 x 11008 sign matrix against the full seeded codebook (v = 20, c = 65536): every
    # index equals the brute-force kernel's, and 24 sampled rows equal the oracle's
    W = wl.weights_for("codebook")
    N, K = W.shape
    words = O.pack_bits(O.sign_pm1(W))
    C = wl.codebook()
    wd, Cd = to_dev(words), to_dev(C)
    got = rb.codebook_encode(wd, K, Cd, 20, table=True)
    brute = rb.codebook_encode(wd, K, Cd, 20)
    torch.cuda.synchronize()
    assert torch.equal(got, brute)
    rows = np.random.default_rng(92).choice(N, 24, replace=False)
    P = O.sign_blocks(words[rows], K, 20)
    assert np.array_equal(got.cpu().numpy().view(np.uint16)[rows], O.hamming_encode(P, C))


@pytest.mark.parametrize("v", [1, 3, 7, 8])
def test_codebook_encode_table_stays_inside_its_workspace(v):
    # for v < 8 the 2^v patterns fill less than one 256-thread block: nothing past the table
    # and its flags may be read or written (a canary after rb_codebook_table_bytes(v))
    N, K, c = 3, 90, min(3, 1 << v)
    words = _sign_words(93, N, K)
    C = np.arange(c, dtype=np.uint32)
    need = rb.lib.rb_codebook_table_bytes(v)
    ws = torch.full(((need + 4096) // 4,), -1, dtype=torch.int32, device=dev())
    got = rb.codebook_encode(to_dev(words), K, to_dev(C), v, table=True, ws=ws.view(torch.uint8))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint16), O.hamming_encode(O.sign_blocks(words, K, v), C))
    tail = ws.view(torch.uint8)[need:].cpu().numpy()
    assert np.all(tail == 0xff)
