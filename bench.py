#!/usr/bin/env python3
"""Benchmark of the residual-binarized decode product on one MI355X.

Workload: the LLaMA-7B MLP down projection, W 4096 x 11008, k = 2 residual sign planes
(fp16 row scales, h = 1), x 1 x 11008 fp16, y fp16. One step = one rb_gemv call on one
activation vector. The planes are derived once by rb_pack (deploy-time; its time is
reported as pack_ms) and 40 copies of them (~460 MB, more than the 256 MB Infinity
Cache) are rotated so that every step reads its weights from HBM.

The timed steps are captured once in a HIP graph and replayed, so host launch overhead is
out of the measurement; HIP events on the replay stream around the whole timed region give
the average launch duration (total / steps), from which both the throughput `value` and the
roofline figure are computed. The replayed result is checked against an eager call.

`python bench.py --summarize-counters DIR` turns the CSV output of two rocprofv3 --pmc runs
of this script (FETCH_SIZE, WRITE_SIZE) into the HBM-traffic record that the roofline
block reads; the streaming-read kernel (bytes known) and the weight-copy kernel (bytes known)
of the same runs calibrate the counters.

Besides the metric, `rows` reports every other step of the path on its own seeded workload
with the roofline that bounds it: the deploy-time derivation (HBM), the batched product on
the matrix cores for the 28672 x 8192 layer at M = 64 / 256 (MFMA fp16 peak) with the M = 1
product on the same weights, the codebook encode (VALU) and the codebook LUT product (HBM).
`--no-rows` skips them.

Prints one JSON line (see the keys below). `python bench.py --gpus N` with N > 1 exits:
this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "k=2 4096×11008 M=1 binary GEMV µs; achieved HBM GB/s as % of MI355X peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, vendor figure
N_ROWS, K_COLS, K_PLANES = 4096, 11008, 2
SHAPE_GATEUP = (11008, 4096)          # the gate/up projection of the same MLP
COPIES = 40
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemv_nib_down_4096x11008_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "residual_binarized_weight_amd", "csrc", f)
                  for f in ("rb_gemv_nib.hip", "rb_device.hpp")]
PRODUCT_KERNEL = "gemv_nib1_kernel<2, 5, true, 1, 1, false>"  # the dominant kernel of a step


SETTLE_S = 0.25   # untimed replays before each timed graph (see graph_us)

# the batched product at k = 2 with fp16 scales and more than one 32-row batch tile
MERGE_NOTE = ("flops = 2 M N K k (one product per plane); the kernel forms +-g0 +-g1 as one fp16 operand "
              "(rounded once), so the matrix cores run mfma_flops = 2 M N K")


def algorithmic_bytes(N: int, K: int, k: int, M: int = 1) -> int:
    """Bytes the product must move: k*N*K/8 of sign bits, fp16 g (k*N), fp16 x (M*K) and
    fp16 y (M*N). h = 1 is implicit (not stored, not read)."""
    return k * N * K // 8 + 2 * k * N + 2 * M * K + 2 * M * N


def kernel_source_hash() -> str:
    """Hash of the product kernel's code: comments and whitespace are dropped, so a comment
    edit keeps the traffic record, while any change to the code voids it."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken
    on the current kernel source (else None)."""
    try:
        with open(COUNTERS_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(planes_np, g_np, x_np, budget_s: float = 12.0):
    """The CPU oracle (float64 NumPy, unpack + matmul) on the same layer, timed on the host."""
    from oracle import rb_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        O.gemv(planes_np, g_np, None, x_np, K_COLS)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= 20:
            break
    t = statistics.median(times)
    # the same on one thread (the matmul's BLAS pool limited to 1)
    t1 = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1, n1 = time_oracle(lambda: O.gemv(planes_np, g_np, None, x_np, K_COLS), budget_s=6.0, max_runs=4)
    except Exception:  # pragma: no cover
        t1 = None
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(algorithmic_bytes(N_ROWS, K_COLS, K_PLANES) / t / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "single_thread_value": None if t1 is None else round(algorithmic_bytes(N_ROWS, K_COLS, K_PLANES) / t1 / 1e9, 4),
        "sample": (f"full 4096x11008 k=2 layer, M=1: oracle unpack of the sign planes to float64 "
                   f"+ float64 matmul, median of {len(times)} runs ({t * 1e3:.0f} ms each); "
                   f"host {cpu_model or platform.processor()}, {len(os.sched_getaffinity(0))} cores visible"),
    }


PEAK_FP16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak, vendor figure
# VALU issue rate for plain 32-bit integer operations: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# = 39.3 T lane-operations/s. (The 157.3 TFLOP/s fp32 figure is this x 2 for an FMA's two flops
# x 2 for packed fp32, which the integer operations of the search do not have.) One (pattern,
# codeword) pair takes 3.5 of them: xor, popcount, the (distance, index) key, and half of a
# three-way minimum.
PEAK_VALU_OPS = 256 * 4 * 16 * 2.4e9
ENCODE_OPS_PER_PAIR = 3.5


FLUSH_BYTES = 512 << 20   # twice the 256 MB Infinity Cache


def flush_cache(torch, _lib, dev, stream=None):
    """Stream 512 MB through a plain read kernel, so that nothing a timed region reads next is
    still held in the 256 MB Infinity Cache or the L2s (run outside every timed region)."""
    import ctypes
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    st = stream if stream is not None else torch.cuda.current_stream()
    rc = _lib.lib.rb_bench_stream_read(ctypes.c_void_p(buf.data_ptr()), FLUSH_BYTES, ctypes.c_void_p(sink.data_ptr()),
                                       2048, ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise RuntimeError("cache flush launch failed")
    torch.cuda.synchronize()
    del buf


def graph_us(torch, calls, rounds: int = 5, settle_s: float = SETTLE_S) -> float:
    """Capture the calls once in a HIP graph on a side stream, replay it `rounds` times and
    return the average duration of one call (events on the replay stream). Before the timed
    replays the graph is replayed untimed for `settle_s` seconds: the GPU raises its clock over
    the first ~0.1 s of a load (a 5 ms burst of matrix-core work right after an idle second
    measured 25 % slower than the same work after 0.4 s of it), and a steady rate is wanted."""
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for c in calls[:2]:
            c()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(gr, stream=st):
            for c in calls:
                c()
    gr.replay()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        gr.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (rounds * len(calls))


def roof(bound: str, achieved: float, peak: float, unit: str, us: float, **extra) -> dict:
    d = {"us": round(us, 3), "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4)}
    d.update(extra)
    return d


def time_oracle(fn, budget_s: float = 2.0, max_runs: int = 5) -> tuple[float, int]:
    """Median wall time of repeated calls of an oracle function (at least one run)."""
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= max_runs:
            break
    return statistics.median(times), len(times)


def oracle_rate(fn, amount: float, scale: float, unit: str, sample: str) -> dict:
    """The CPU oracle on a bounded sample of a row's workload: `amount` units of the row's
    metric per call (bytes, flops or operations), reported in the row's unit (`scale` units
    each)."""
    t, n = time_oracle(fn)
    return {"value": round(amount / t / scale, 5), "unit": unit, "kind": "oracle",
            "sample": f"{sample}; median of {n} runs, {t * 1e3:.0f} ms each"}


PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure


def measure_qat_step(torch, np, rb, wl, dev, with_oracle: bool, M: int = 2048) -> dict:
    N, K, k = N_ROWS, K_COLS, K_PLANES
    W = torch.from_numpy(wl.weights_for("down")).to(dev)
    g, h = (torch.from_numpy(a).to(dev) for a in wl.training_scales(wl.CFG_MLP, k, N, K))
    X = torch.from_numpy(wl.activations(wl.CFG_MLP, M, K, dtype=np.float32)).to(dev).to(torch.bfloat16)
    dY = torch.from_numpy(wl.output_grads(wl.CFG_MLP, M, N)).to(dev).to(torch.bfloat16)
    C = 2
    Ws = [W] + [W.clone() for _ in range(C - 1)]
    pls = [torch.zeros((k, N, K // 32), dtype=torch.int32, device=dev) for _ in range(C)]
    Whs = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(C)]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.float32, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dg = torch.empty((k, N), dtype=torch.float32, device=dev)
    dh = torch.empty((k, K), dtype=torch.float32, device=dev)
    ws = torch.empty(rb.workspace_bytes(rb.RB_OP_QAT_BACKWARD, k, N, K, M), dtype=torch.uint8, device=dev)
    rb.qat_forward(Ws[0], g, h, X, planes=pls[0], What=Whs[0], Y=Y)
    t0 = time.perf_counter()
    rb.qat_autotune(X, dY, Whs[0], Y, dW, dX)
    tune_s = time.perf_counter() - t0

    def fwd(i):
        rb.qat_forward(Ws[i % C], g, h, X, planes=pls[i % C], What=Whs[i % C], Y=Y)

    def bwd(i):
        rb.qat_backward(dY, X, Whs[i % C], pls[i % C], g, h, ws=ws, dW=dW, dX=dX, dg=dg, dh=dh)

    def step(i):
        fwd(i)
        bwd(i)

    def timed(fn, reps=10):
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    der_us = timed(lambda i: rb.qat_derive(Ws[i % C], g, h, planes=pls[i % C], What=Whs[i % C]))
    fwd_us, bwd_us, step_us = timed(fwd), timed(bwd), timed(step)
    # the forward's product alone on each engine, and the product taken from the planes instead
    # of What (rb_gemm_small: one matrix-core pass per plane with h_i in the fp16 operand)
    mm_flops = 2.0 * M * N * K
    mm = {}
    for name, eng in (("mfma", rb.RB_QAT_ENGINE_MFMA), ("rocblas", rb.RB_QAT_ENGINE_ROCBLAS)):
        us = timed(lambda i, eng=eng: rb.qat_matmul(X, Whs[i % C], Y=Y, engine=eng))
        mm[name] = {"us": round(us, 2), "TFLOP/s": round(mm_flops / (us * 1e-6) / 1e12, 1),
                    "frac": round(mm_flops / (us * 1e-6) / 1e12 / PEAK_BF16_MFMA_TFLOPS, 4)}
    g16, h16, X16 = g.half(), h.half(), X.half()
    Yp = torch.empty((M, N), dtype=torch.float16, device=dev)
    wsp = torch.empty(max(16, rb.workspace_bytes(rb.RB_OP_GEMM_SMALL, k, N, K, M)), dtype=torch.uint8, device=dev)
    us = timed(lambda i: rb.gemm_small(pls[i % C], g16, h16, X16, K, ws=wsp, y=Yp))
    mm["planes_route"] = {"us": round(us, 2), "TFLOP/s": round(mm_flops / (us * 1e-6) / 1e12, 1),
                          "note": "Y from the k planes on the matrix cores (fp16 x, g and h): one product per "
                                  "plane, 2 k M N K flops of MFMA work against 2 M N K through What"}
    flops = 3 * 2.0 * M * N * K
    der_bytes = N * K * (4 + 2) + k * N * K // 8 + 4 * k * (N + K)   # W read, What + planes written
    row = roof("mfma", flops / (step_us * 1e-6) / 1e12, PEAK_BF16_MFMA_TFLOPS, "TFLOP/s", step_us, flops=flops,
               tokens=M, dtype="bf16 operands, fp32 accumulation, fp32 dW",
               forward_us=round(fwd_us, 2), backward_us=round(bwd_us, 2), autotune_s=round(tune_s, 2),
               forward_product=mm,
               derive={"us": round(der_us, 2), "algorithmic_bytes": der_bytes, "bound": "hbm",
                       "achieved": round(der_bytes / (der_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": round(der_bytes / (der_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
               derive_share_of_rest=round(der_us / (step_us - der_us), 4))
    out = {f"next_f2_qat_step_down_4096x11008_k2_m{M}": row}
    if with_oracle:
        from oracle import rb_oracle as O
        RQ, MQ = 64, 256
        Wq = wl.weights_for("down")[:RQ]
        gq, hq = (a.astype(np.float64) for a in wl.training_scales(wl.CFG_MLP, k, N, K))
        gq = gq[:, :RQ]
        Xq = X[:MQ].float().cpu().numpy().astype(np.float64)
        dYq = dY[:MQ, :RQ].float().cpu().numpy().astype(np.float64)

        def oracle_step():
            _, Wh_q, B_q, _ = O.qat_forward(Wq, gq, hq, Xq)
            O.qat_backward(dYq, Xq, Wh_q, B_q, gq, hq)
        row["cpu_oracle"] = oracle_rate(oracle_step, 3 * 2.0 * MQ * RQ * K, 1e12, "TFLOP/s",
                                        f"first {RQ} of the 4096 rows, {MQ} of the {M} tokens (fp64), flops "
                                        f"scaled to the sample")
    del Ws, pls, Whs, W, X, dY, dW, dX, ws
    torch.cuda.synchronize()
    return out


def measure_variants(torch, np, rb, wl, dev, with_oracle: bool) -> dict:
    N, K = N_ROWS, K_COLS
    Kw = (K + 31) // 32
    ldp = (Kw + 31) // 32 * 32
    W = torch.from_numpy(wl.weights_for("down")).to(dev)
    planes, g = rb.pack(W, 2, ldp=ldp)
    del W
    x = torch.from_numpy(wl.activations_for("down", 1)).to(dev)
    mu = torch.from_numpy(np.random.default_rng([900, 1]).normal(0, 0.002, N).astype(np.float16)).to(dev)
    ws = rb.workspace(rb.RB_OP_GEMV, 2, N, K, 1, device=dev)
    y = torch.empty((1, N), dtype=torch.float16, device=dev)
    out = {}
    # each variant beside the plain product of the same planes in the same harness (short graphs
    # of 40 rotated copies, so the figures sit a little above the metric's 2000-step graph)
    for name, kk, use_mu, zo in (("plain_k1", 1, False, False), ("zero_one_k1", 1, False, True),
                                 ("plain_k2", 2, False, False), ("offset_mu_k2", 2, True, False)):
        copies = [planes[:kk].clone() for _ in range(COPIES)]
        gk = g[:kk].contiguous()
        m = mu if use_mu else None
        us = graph_us(torch, [lambda c=c: rb.gemv_variant(c, gk, None, x, K, mu=m, zero_one=zo, ws=ws, y=y)
                              for c in copies], 5)
        byt = algorithmic_bytes(N, K, kk) + (2 * N if use_mu else 0)
        row = out[name] = roof("hbm", byt / (us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", us, algorithmic_bytes=byt)
        if with_oracle and name.startswith(("zero_one", "offset")):
            from oracle import rb_oracle as O
            RS = 512
            pl_s = np.ascontiguousarray(planes[:kk, :RS].cpu().numpy().view(np.uint32)[:, :, :Kw])
            g_s = g[:kk, :RS].float().cpu().numpy().astype(np.float64)
            mu_s = mu[:RS].float().cpu().numpy().astype(np.float64) if use_mu else None
            xh = x.float().cpu().numpy().astype(np.float64)
            row["cpu_oracle"] = oracle_rate(lambda: O.gemv_variant(pl_s, g_s, None, mu_s, xh, K, zo),
                                            algorithmic_bytes(RS, K, kk) + (2 * RS if use_mu else 0), 1e9, "GB/s",
                                            f"first {RS} of the 4096 rows, bytes scaled per row")
        del copies
    torch.cuda.synchronize()
    return {"next_f4_gemv_variants_down_4096x11008_m1": out}


def measure_codebook_learn(torch, np, rb, dev, pl, Kc: int, idx, C, enc_us, with_oracle: bool) -> dict:
    """Binary codebook learning on the sign plane pl[0] (Kc columns, v = 20, c = C.numel(), idx the
    indices of C): one standalone M-step (radix pass of the blocks, sliced counting, majority
    vote), the distinct-block count, and whole learning calls with 0 and 1 iterations (distinct +
    E-step + M-step + final E-step). enc_us is the brute-force E-step's time, None if unmeasured."""
    Nc, nb = idx.shape
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ws_l = torch.empty(rb.lib.rb_codebook_learn_workspace_bytes(Nc, Kc, C.numel(), 20), dtype=torch.uint8, device=dev)
    Cl = C.clone()

    def ev_us(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps
    ms_us = ev_us(lambda: rb.codebook_mstep(pl[0], Kc, idx, Cl, 20, counts=False, ws=ws_l), 10)
    ds_us = ev_us(lambda: rb.codebook_distinct(pl[0], Kc, Cl, 20, ws=ws_l), 10)
    l0_us = ev_us(lambda: rb.codebook_learn(pl[0], Kc, C.clone(), 20, 0, ws=ws_l), 2)
    lr_us = ev_us(lambda: rb.codebook_learn(pl[0], Kc, C.clone(), 20, 1, ws=ws_l), 2)
    words_np = pl[0].cpu().numpy().view(np.uint32)[:, :(Kc + 31) // 32]
    idx_np = idx.cpu().numpy().view(np.uint16)
    set_bits = int(np.bitwise_count(np.ascontiguousarray(words_np)).sum())
    # one per block (member) + one per +1 bit, the last block's padding columns counting as +1
    loop_atomics = Nc * nb + set_bits + Nc * (nb * 20 - Kc)
    # standalone M-step: idx read twice (histogram, scatter), the plane once, the records (one
    # word per block at v = 20: pattern and index byte) written and read, the slice tables
    # written and read, the codebook read and written
    nblk = Nc * nb
    n_slices = nblk // 4096 + min(-(-C.numel() // 256), nblk)
    ms_bytes = (pl[0].numel() * 4 + 2 * idx.numel() * 2 + 2 * nblk * 4 + 2 * n_slices * 256 * 21 * 4
                + 2 * 4 * C.numel())
    row = {
        "mstep": roof("hbm", ms_bytes / (ms_us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", ms_us, algorithmic_bytes=ms_bytes,
                      note="radix pass of the blocks on idx >> 8 writing one-word (pattern, index byte) records, "
                           "sliced counting with LDS atomics, per-codeword sums of the slices; no global "
                           "atomics"),
        "distinct_us": round(ds_us, 2),
        "learn_0_iterations_us": round(l0_us, 1),
        "learn_1_iteration_us": round(lr_us, 1),
        "iteration_us": round(lr_us - l0_us, 1),
        "e_step_alone_us": None if enc_us is None else round(enc_us, 1),
        "loop_counting_atomics": loop_atomics,
        "note": "learn with 0 iterations = distinct + the final E-step; each iteration adds an E-step and an "
                "M-step; at this size the E-steps go through the nearest-codeword table and the M-step is the "
                "radix pass + sliced vote (e_step_alone_us is the brute-force search, for comparison)",
    }
    if with_oracle:
        from oracle import rb_oracle as O
        pats = O.sign_blocks(words_np, Kc, 20)
        Cn = C.cpu().numpy().view(np.uint32)
        row["mstep"]["cpu_oracle"] = oracle_rate(
            lambda: O.codebook_mstep(pats, idx_np, Cn, 20), ms_bytes, 1e9, "GB/s",
            "the whole M-step (all 2.26 M blocks), bytes as for the GPU")
    del ws_l, Cl
    torch.cuda.synchronize()
    return row


def measure_rows(torch, np, rb, wl, dev, pack_ms: float, with_oracle: bool = True) -> dict:
    """Every step of the path besides the metric product, each on its own workload, timed
    on the GPU against the roofline that bounds it (inputs are seeded synthetic data). With
    `with_oracle`, each row also carries the CPU oracle's rate on a bounded sample of the same
    workload (`cpu_oracle`)."""
    rows = {}
    N, K, k = N_ROWS, K_COLS, K_PLANES
    pack_bytes = N * K * 4 + k * N * K // 8 + 2 * k * N      # W fp32 read once, planes + g written
    rows["a1_a2_pack_down_4096x11008_k2"] = roof("hbm", pack_bytes / (pack_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s",
                                                 pack_ms * 1e3, algorithmic_bytes=pack_bytes)
    if with_oracle:
        from oracle import rb_oracle as O
        R = 512
        Ws = wl.weights_for("down")[:R]
        rows["a1_a2_pack_down_4096x11008_k2"]["cpu_oracle"] = oracle_rate(
            lambda: O.binarize(Ws, k), R * pack_bytes / N, 1e9, "GB/s",
            f"first {R} of the 4096 rows (k=2, fp16 g), bytes scaled per row")
        del Ws

    # next row: function-aware initialization of the 4096x11008 layer, k = 2, T = 20 sweeps,
    # P = 4 power iterations per path update (each update: 2P + 1 passes over W and the planes)
    T_sw, P_it = 20, 4
    Wsv = torch.from_numpy(wl.weights_for("down")).to(dev)
    ws_sv = torch.empty(rb.workspace_bytes(rb.RB_OP_SVID_INIT, k, N, K, 1), dtype=torch.uint8, device=dev)
    rb.svid_init(Wsv, k, T=1, P=P_it, ws=ws_sv)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    rb.svid_init(Wsv, k, T=T_sw, P=P_it, ws=ws_sv)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    del Wsv, ws_sv

    def svid_bytes(rows, T):
        per_pass = rows * K * 4 + (k - 1) * rows * K // 8        # W and the other paths' planes
        return T * k * ((2 * P_it + 1) * per_pass + rows * K // 8)  # + the new plane
    byt = svid_bytes(N, T_sw)
    rows["next_f1_svid_init_down_4096x11008_k2_T20"] = roof(
        "hbm", byt / (us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", us, algorithmic_bytes=byt, sweeps=T_sw,
        power_iterations=P_it)
    if with_oracle:
        Rs = 256
        Wso = wl.weights_for("down")[:Rs]
        rows["next_f1_svid_init_down_4096x11008_k2_T20"]["cpu_oracle"] = oracle_rate(
            lambda: O.svid_init(Wso, k, T=2), svid_bytes(Rs, 2), 1e9, "GB/s",
            f"first {Rs} of the 4096 rows, 2 sweeps (exact fp64 SVD per path update), bytes counted as for "
            f"the GPU's {2 * P_it + 1} passes per update")
        del Wso

    # a3-a5 at M = 2, 4 and 16 on the same layer (fp16, 40 rotated copies): two rows in one
    # launch of the nibble kernel; four or more on the matrix cores (one pass over the planes)
    Wb = torch.from_numpy(wl.weights_for("down")).to(dev)
    planes_b, g_b = rb.pack(Wb, k, ldp=((K + 31) // 32 + 31) // 32 * 32)   # rows padded to 128 bytes
    del Wb
    copies_b = [planes_b.clone() for _ in range(COPIES)]
    for Mb in (2, 4, 16):
        xb = torch.from_numpy(wl.activations_for("down", Mb)).to(dev)
        yb = torch.empty((Mb, N), dtype=torch.float16, device=dev)
        wsb = rb.workspace(rb.RB_OP_GEMV, k, N, K, Mb, device=dev)
        us = graph_us(torch, [lambda c=c: rb.gemv(c, g_b, None, xb, K, ws=wsb, y=yb) for c in copies_b], 5)
        byt = algorithmic_bytes(N, K, k, Mb)
        row = rows[f"a3_a5_gemv_down_4096x11008_k2_m{Mb}"] = roof(
            "hbm", byt / (us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", us, algorithmic_bytes=byt,
            weight_bytes_streamed=k * N * K // 8,
            note="two rows: one launch of the nibble kernel (tables built and looked up per row, planes read "
                 "once); 4 or more rows on the matrix cores: one pass over the planes, K split into chunks whose "
                 "fp32 sums meet in the workspace")
        if with_oracle:
            from oracle import rb_oracle as O
            RS = 512
            pl_s = np.ascontiguousarray(planes_b[:, :RS].cpu().numpy().view(np.uint32)[:, :, :(K + 31) // 32])
            g_s = g_b[:, :RS].float().cpu().numpy().astype(np.float64).reshape(k, RS, 1)
            xh = xb.cpu().numpy()
            row["cpu_oracle"] = oracle_rate(lambda: O.gemv(pl_s, g_s, None, xh, K), algorithmic_bytes(RS, K, k, Mb),
                                            1e9, "GB/s", f"first {RS} of the 4096 rows, M={Mb}, bytes scaled per row")
    # the gate/up projection of the same MLP (11008x4096, k = 2) at M = 1, 4 and 16
    Ng, Kg = SHAPE_GATEUP
    Wg = torch.from_numpy(wl.weights_for("gateup")).to(dev)
    planes_g, g_g = rb.pack(Wg, k, ldp=((Kg + 31) // 32 + 31) // 32 * 32)
    del Wg
    copies_g = [planes_g.clone() for _ in range(COPIES)]
    for Mb in (1, 4, 16):
        xb = torch.from_numpy(wl.activations_for("gateup", Mb)).to(dev)
        yb = torch.empty((Mb, Ng), dtype=torch.float16, device=dev)
        wsb = rb.workspace(rb.RB_OP_GEMV, k, Ng, Kg, Mb, device=dev)
        us = graph_us(torch, [lambda c=c: rb.gemv(c, g_g, None, xb, Kg, ws=wsb, y=yb) for c in copies_g], 5)
        byt = algorithmic_bytes(Ng, Kg, k, Mb)
        row = rows[f"a3_a5_gemv_gateup_11008x4096_k2_m{Mb}"] = roof(
            "hbm", byt / (us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", us, algorithmic_bytes=byt,
            weight_bytes_streamed=k * Ng * Kg // 8)
        if with_oracle and Mb == 1:
            from oracle import rb_oracle as O
            RS = 1024
            pl_s = np.ascontiguousarray(planes_g[:, :RS].cpu().numpy().view(np.uint32)[:, :, :(Kg + 31) // 32])
            g_s = g_g[:, :RS].float().cpu().numpy().astype(np.float64).reshape(k, RS, 1)
            xh = xb.cpu().numpy()
            row["cpu_oracle"] = oracle_rate(lambda: O.gemv(pl_s, g_s, None, xh, Kg), algorithmic_bytes(RS, Kg, k, Mb),
                                            1e9, "GB/s", f"first {RS} of the 11008 rows, M=1, bytes scaled per row")
    del copies_g, planes_g
    # ... and with per-column scales h (fp16, the RaBiT dual-scale form) at M = 1: one nibble pass
    # per plane with x (.) h_i in its tables, chained through the workspace
    hb = torch.from_numpy(wl.random_scales(5, k, K, dtype=np.float16)).to(dev)
    Wb = torch.from_numpy(wl.weights_for("down")).to(dev)
    planes_h, g_h = rb.pack(Wb, k, h=hb, ldp=((K + 31) // 32 + 31) // 32 * 32)
    del Wb
    copies_h = [planes_h.clone() for _ in range(COPIES)]
    x1 = torch.from_numpy(wl.activations_for("down", 1)).to(dev)
    y1 = torch.empty((1, N), dtype=torch.float16, device=dev)
    ws1 = rb.workspace(rb.RB_OP_GEMV, k, N, K, 1, device=dev)
    us = graph_us(torch, [lambda c=c: rb.gemv(c, g_h, hb, x1, K, ws=ws1, y=y1) for c in copies_h], 5)
    byt = algorithmic_bytes(N, K, k) + 2 * k * K
    row = rows["a3_a5_gemv_down_4096x11008_k2_general_h_m1"] = roof(
        "hbm", byt / (us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", us, algorithmic_bytes=byt,
        note="one single-plane nibble pass per plane (x times that plane's h in the tables)")
    x16 = torch.from_numpy(wl.activations_for("down", 16)).to(dev)
    y16 = torch.empty((16, N), dtype=torch.float16, device=dev)
    us16 = graph_us(torch, [lambda c=c: rb.gemv(c, g_h, hb, x16, K, ws=ws1, y=y16) for c in copies_h], 5)
    byt16 = algorithmic_bytes(N, K, k, 16) + 2 * k * K
    rows["a3_a5_gemv_down_4096x11008_k2_general_h_m16"] = roof(
        "hbm", byt16 / (us16 * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", us16, algorithmic_bytes=byt16,
        note="on the matrix cores, h_i entering the fp16 operand")
    if with_oracle:
        from oracle import rb_oracle as O
        RS = 512
        pl_s = np.ascontiguousarray(planes_h[:, :RS].cpu().numpy().view(np.uint32)[:, :, :(K + 31) // 32])
        g_s = g_h[:, :RS].float().cpu().numpy().astype(np.float64).reshape(k, RS, 1)
        h_s = hb.float().cpu().numpy().astype(np.float64)
        xh = x1.cpu().numpy()
        row["cpu_oracle"] = oracle_rate(lambda: O.gemv(pl_s, g_s, h_s, xh, K), algorithmic_bytes(RS, K, k) + 2 * k * K,
                                        1e9, "GB/s", f"first {RS} of the 4096 rows, bytes scaled per row")
    # a6 on the 4096x11008 layer at M = 64 and 256 (prefill): 32 row tiles, so K is split
    # across blocks and the chunks meet in the workspace
    for Mb in (64, 256):
        xb = torch.from_numpy(wl.activations_for("down", Mb)).to(dev)
        yb = torch.empty((Mb, N), dtype=torch.float16, device=dev)
        wsg = rb.workspace(rb.RB_OP_GEMM_SMALL, k, N, K, Mb, device=dev)
        us = graph_us(torch, [lambda c=c: rb.gemm_small(c, g_b, None, xb, K, ws=wsg, y=yb) for c in copies_b], 3)
        flops = 2.0 * Mb * N * K * k
        rows[f"a6_gemm_small_down_4096x11008_k2_m{Mb}"] = roof(
            "mfma", flops / (us * 1e-6) / 1e12, PEAK_FP16_MFMA_TFLOPS, "TFLOP/s", us, flops=flops,
            k_chunks=(wsg.numel() // (4 * Mb * N)) if wsg is not None else 1, mfma_flops=flops / k,
            note=MERGE_NOTE)
    del copies_b, planes_b, copies_h, planes_h
    torch.cuda.synchronize()

    # next row: one coupled-training step of the 4096x11008 layer, k = 2, 2048 tokens in bf16:
    # forward (derive planes + What from the fp32 weight, Y = X What^T) and backward (dW, dX,
    # dg, dh); the GEMM kernels are chosen for the shape first (untimed setup); two weight
    # copies rotate so W is read from HBM
    rows.update(measure_qat_step(torch, np, rb, wl, dev, with_oracle))

    # next row: the cheap product variants on the metric's layer and launch shape (M = 1, fp16,
    # the nibble-table kernel, rotated weight copies): {0, s} bits on one plane, and k = 2 planes
    # with a per-row offset mu
    rows.update(measure_variants(torch, np, rb, wl, dev, with_oracle))

    # a6: the 28672x8192 layer on the matrix cores at M = 64 and 256, k = 1 and 2, and the
    # M = 1 product on the same weights; 8 weight copies rotate (470 MB > the 256 MB cache)
    Wd = torch.from_numpy(wl.weights_for("wide")).to(dev)
    NW, KW = Wd.shape
    planes2, g2 = rb.pack(Wd, 2)
    del Wd
    torch.cuda.synchronize()
    copies = [planes2.clone() for _ in range(8)]
    RS = 1024                                                 # oracle sample: rows of the layer
    if with_oracle:
        pl_s = np.ascontiguousarray(planes2[:, :RS].cpu().numpy().view(np.uint32)[:, :, :KW // 32])
        g_s = g2[:, :RS].float().cpu().numpy().astype(np.float64).reshape(2, RS, 1)
    for kk in (1, 2):
        cps = [c[:kk] for c in copies]
        gk = g2[:kk].contiguous()
        for M in (64, 256):
            xh = wl.activations_for("wide", M)
            x = torch.from_numpy(xh).to(dev)
            y = torch.empty((M, NW), dtype=torch.float16, device=dev)
            us = graph_us(torch, [lambda c=c: rb.gemm_small(c, gk, None, x, KW, y=y) for c in cps], 3)
            flops = 2.0 * M * NW * KW * kk
            row = rows[f"a6_gemm_small_28672x8192_k{kk}_m{M}"] = roof(
                "mfma", flops / (us * 1e-6) / 1e12, PEAK_FP16_MFMA_TFLOPS, "TFLOP/s", us, flops=flops,
                mfma_flops=2.0 * M * NW * KW)
            if kk == 2:
                row["note"] = MERGE_NOTE
            if with_oracle:
                row["cpu_oracle"] = oracle_rate(
                    lambda: O.gemv(pl_s[:kk], g_s[:kk], None, xh, KW), 2.0 * M * RS * KW * kk, 1e12, "TFLOP/s",
                    f"first {RS} of the 28672 rows, same M and k, flops scaled per row")
        x1h = wl.activations_for("wide", 1)
        x1 = torch.from_numpy(x1h).to(dev)
        ws = rb.workspace(rb.RB_OP_GEMV, kk, NW, KW, 1, device=dev)
        y1 = torch.empty((1, NW), dtype=torch.float16, device=dev)
        us = graph_us(torch, [lambda c=c: rb.gemv(c, gk, None, x1, KW, ws=ws, y=y1) for c in cps], 5)
        byt = algorithmic_bytes(NW, KW, kk)
        row = rows[f"gemv_m1_28672x8192_k{kk}"] = roof("hbm", byt / (us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", us,
                                                       algorithmic_bytes=byt)
        if with_oracle:
            row["cpu_oracle"] = oracle_rate(
                lambda: O.gemv(pl_s[:kk], g_s[:kk], None, x1h, KW), algorithmic_bytes(RS, KW, kk), 1e9, "GB/s",
                f"first {RS} of the 28672 rows, M=1, bytes scaled per row")
    del copies, planes2
    torch.cuda.synchronize()

    # a7, a8: the 4096x11008 sign matrix, v = 20, c = 65536, fp16 scales per 16 weights
    Wc = torch.from_numpy(wl.weights_for("codebook")).to(dev)
    Nc, Kc = Wc.shape
    pl, sc = rb.pack(Wc, 1, group=16)
    del Wc
    C = torch.from_numpy(wl.codebook().view(np.int32)).to(dev)
    idx = rb.codebook_encode(pl[0], Kc, C, 20)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        rb.codebook_encode(pl[0], Kc, C, 20)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 3
    nb = (Kc + 19) // 20
    pairs = Nc * nb * C.numel()
    rows["a7_codebook_encode_4096x11008_v20_c65536"] = roof(
        "alu", pairs * ENCODE_OPS_PER_PAIR / (us * 1e-6) / 1e12, PEAK_VALU_OPS / 1e12, "Tops/s", us,
        pairs=pairs, ops_per_pair=ENCODE_OPS_PER_PAIR)
    if with_oracle:
        RC = 16                                               # oracle sample: rows of the sign matrix
        pat = O.sign_blocks(pl[0, :RC].cpu().numpy().view(np.uint32)[:, :(Kc + 31) // 32], Kc, 20)
        Ch = C.cpu().numpy().view(np.uint32)
        rows["a7_codebook_encode_4096x11008_v20_c65536"]["cpu_oracle"] = oracle_rate(
            lambda: O.hamming_encode(pat, Ch), RC * nb * C.numel() * ENCODE_OPS_PER_PAIR, 1e12, "Tops/s",
            f"first {RC} of the 4096 rows ({RC * nb} patterns x 65536 codewords), operations scaled per pair")
    # the same encode through the nearest-codeword table (breadth-first search over the 2^20
    # patterns, then one lookup per block; identical indices)
    ws_t = torch.empty(rb.lib.rb_codebook_table_bytes(20), dtype=torch.uint8, device=dev)
    idx_t = rb.codebook_encode(pl[0], Kc, C, 20, table=True, ws=ws_t)
    torch.cuda.synchronize()
    if not torch.equal(idx_t, idx):
        raise RuntimeError("table encode differs from the brute-force encode")
    e0.record()
    for _ in range(10):
        rb.codebook_encode(pl[0], Kc, C, 20, table=True, ws=ws_t)
    e1.record()
    torch.cuda.synchronize()
    us_t = e0.elapsed_time(e1) * 1e3 / 10
    rows["a7_codebook_encode_4096x11008_v20_c65536"]["table"] = {
        "us": round(us_t, 2), "speedup_vs_search": round(us / us_t, 1),
        "note": "rb_codebook_encode_table: table of the nearest codeword of all 2^20 patterns by a multi-source "
                "breadth-first search over the hypercube (ties to the lowest index), then one lookup per block"}
    del ws_t, idx_t
    s2 = sc[0].reshape(Nc, -1).contiguous()
    xc = torch.from_numpy(wl.activations_for("codebook", 1)).to(dev)
    yc = torch.empty((1, Nc), dtype=torch.float16, device=dev)
    icp = [idx.clone() for _ in range(40)]
    scp = [s2.clone() for _ in range(40)]
    us = graph_us(torch, [lambda i=i, q=q: rb.codebook_gemv(i, C, 20, q, 16, xc, Kc, y=yc) for i, q in zip(icp, scp)], 5)
    byt = idx.numel() * 2 + s2.numel() * 2 + C.numel() * 4 + 2 * Kc + 2 * Nc
    rows["a8_codebook_gemv_4096x11008_m1"] = roof("hbm", byt / (us * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s", us,
                                                  algorithmic_bytes=byt,
                                                  note="bound in practice by 2.26 M random codeword reads from L2")
    # the codeword reads against the rate of random 4-byte reads from the same 256 KB table
    # (a plain gather kernel, timed here)
    import ctypes
    from residual_binarized_weight_amd import _lib
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    per_thread, blocks = 64, 1024
    gcall = lambda: _lib.lib.rb_bench_gather(ctypes.c_void_p(C.data_ptr()), C.numel(), per_thread,
                                              ctypes.c_void_p(sink.data_ptr()), blocks, None)
    for _ in range(2):
        assert gcall() == 0
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        gcall()
    e1.record()
    torch.cuda.synchronize()
    gps = blocks * 256 * per_thread / (e0.elapsed_time(e1) * 1e-3 / 5) / 1e9
    gathers = Nc * nb
    rows["a8_codebook_gemv_4096x11008_m1"]["gather_roofline"] = {
        "gathers": gathers, "achieved": round(gathers / (us * 1e-6) / 1e9, 2), "peak": round(gps, 2),
        "unit": "G gathers/s", "frac": round(gathers / (us * 1e-6) / 1e9 / gps, 4)}
    if with_oracle:
        RG = 1024
        idx_s = idx[:RG].cpu().numpy().view(np.uint16)
        s_s = s2[:RG].float().cpu().numpy()
        xch = xc.cpu().numpy()
        per_row = idx.shape[1] * 2 + s2.shape[1] * 2 + 2
        rows["a8_codebook_gemv_4096x11008_m1"]["cpu_oracle"] = oracle_rate(
            lambda: O.codebook_gemv(idx_s, Ch, 20, s_s, 16, xch, Kc), RG * per_row + C.numel() * 4 + 2 * Kc,
            1e9, "GB/s", f"first {RG} of the 4096 rows, M=1, index and scale bytes scaled per row")
    rows["next_f3_codebook_learn_4096x11008_v20_c65536"] = measure_codebook_learn(
        torch, np, rb, dev, pl, Kc, idx, C, rows["a7_codebook_encode_4096x11008_v20_c65536"]["us"], with_oracle)
    del icp, scp
    torch.cuda.synchronize()
    return rows


def summarize_counters(root: str, out_path: str = COUNTERS_FILE) -> int:
    """Read rocprofv3 --pmc CSVs (FETCH_SIZE and WRITE_SIZE runs of this script) under
    `root`, calibrate each counter against a kernel whose traffic is known, and write the
    per-launch HBM traffic of the product kernel to the counters record `out_path`."""
    import csv
    import glob
    per = {}  # (counter, kernel) -> list of per-dispatch totals
    for path in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        tot = {}
        for r in csv.DictReader(open(path)):
            key = (r["Counter_Name"], r["Kernel_Name"], r["Dispatch_Id"])
            tot[key] = tot.get(key, 0.0) + float(r["Counter_Value"])
        for (c, kname, _), v in tot.items():
            per.setdefault((c, kname), []).append(v)

    def med(c, pat):
        vals = [v for (cc, kn), vs in per.items() if cc == c and pat in kn for v in vs]
        return statistics.median(vals) if vals else None

    nbytes = algorithmic_bytes(N_ROWS, K_COLS, K_PLANES)
    stream_bytes = nbytes // 256 * 256                     # the stream-read kernel's footprint
    Kw = (K_COLS + 31) // 32
    copy_bytes = K_PLANES * N_ROWS * ((Kw + 31) // 32 * 32) * 4   # one weight-copy dispatch
    f_gemv, f_stream = med("FETCH_SIZE", PRODUCT_KERNEL), med("FETCH_SIZE", "stream_read")
    w_gemv, w_copy = med("WRITE_SIZE", PRODUCT_KERNEL), med("WRITE_SIZE", "copyBuffer")
    rec = {"kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_dispatch": f_gemv, "write_kib_per_dispatch": w_gemv,
           "stream_read_fetch_kib": f_stream, "stream_read_bytes": stream_bytes,
           "copy_write_kib": w_copy, "copy_bytes": copy_bytes}
    if None not in (f_gemv, f_stream, w_gemv, w_copy) and f_stream > 0 and w_copy > 0:
        fetch_scale = stream_bytes / (f_stream * 1024.0)
        write_scale = copy_bytes / (w_copy * 1024.0)
        rec.update({"fetch_scale": fetch_scale, "write_scale": write_scale,
                    "hbm_bytes_per_launch": round(f_gemv * 1024.0 * fetch_scale + w_gemv * 1024.0 * write_scale)})
    os.makedirs(os.path.dirname(os.path.abspath(out_path)), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


def summarize_trace(root: str, kernel: str = PRODUCT_KERNEL) -> int:
    """Per-dispatch duration distribution of `kernel` in the rocprofv3 --kernel-trace CSVs under
    `root` (all dispatches whose name contains it), printed as one JSON line."""
    import csv
    import glob
    durs = []
    for path in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not durs:
        print(json.dumps({"kernel": kernel, "dispatches": 0}))
        return 1
    durs.sort()
    q = lambda f: durs[min(len(durs) - 1, int(f * len(durs)))]
    print(json.dumps({"kernel": kernel, "dispatches": len(durs), "mean_us": round(statistics.fmean(durs), 3),
                      "p10_us": round(q(0.10), 3), "median_us": round(q(0.50), 3), "p90_us": round(q(0.90), 3),
                      "min_us": round(durs[0], 3), "max_us": round(durs[-1], 3)}))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row measurements of the other steps")
    ap.add_argument("--summarize-counters", metavar="DIR", help="write the traffic record from rocprofv3 CSVs")
    ap.add_argument("--summarize-trace", metavar="DIR", help="per-dispatch durations of the product kernel "
                                                              "from rocprofv3 kernel-trace CSVs")
    ap.add_argument("--kernel", default=PRODUCT_KERNEL, help="kernel name for --summarize-trace")
    ap.add_argument("--only-row", choices=["qat", "codebook_learn"], help="run one row's measurement alone (for profiling) "
                                                        "and print it as the JSON line")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.kernel)
    if args.gpus != 1:
        print(json.dumps({"error": "the product runs on one GPU here; --gpus must be 1 "
                                   "(a row-sharded multi-GPU layout is not implemented)"}))
        return 2

    import numpy as np
    import torch

    import residual_binarized_weight_amd as rb
    from residual_binarized_weight_amd import _lib
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only_row == "qat":
        print(json.dumps(measure_qat_step(torch, np, rb, wl, dev, with_oracle=False)))
        return 0
    if args.only_row == "codebook_learn":
        Wc = torch.from_numpy(wl.weights_for("codebook")).to(dev)
        Kc = Wc.shape[1]
        pl, _ = rb.pack(Wc, 1, group=16)
        del Wc
        C = torch.from_numpy(wl.codebook().view(np.int32)).to(dev)
        idx = rb.codebook_encode(pl[0], Kc, C, 20, table=True)
        print(json.dumps(measure_codebook_learn(torch, np, rb, dev, pl, Kc, idx, C, None, with_oracle=False)))
        return 0
    N, K, k = N_ROWS, K_COLS, K_PLANES
    Kw = (K + 31) // 32
    ldp = (Kw + 31) // 32 * 32          # rows padded to 128-byte multiples

    # ---- inputs (synthetic, seeded; see workloads/) and the deploy-time derivation -------
    W = torch.from_numpy(wl.weights_for("down")).to(dev)
    x = torch.from_numpy(wl.activations_for("down", 1)).to(dev)
    planes, g = rb.pack(W, k, ldp=ldp)
    torch.cuda.synchronize()
    # the pack timed like the other rows: a graph of calls, here alternating two copies of W
    # (360 MB, more than the 256 MB Infinity Cache, so every call reads W from HBM)
    W2, planes2 = W.clone(), planes.clone()
    pk = [lambda: rb.pack(W, k, ldp=ldp, planes=planes2), lambda: rb.pack(W2, k, ldp=ldp, planes=planes2)]
    pack_ms = graph_us(torch, [pk[i % 2] for i in range(20)]) / 1e3
    del W, W2, planes2
    copies = [planes.clone() for _ in range(COPIES)]
    ws = rb.workspace(rb.RB_OP_GEMV, k, N, K, 1, device=dev)
    y = torch.empty((1, N), dtype=torch.float16, device=dev)
    y_ref = rb.gemv(planes, g, None, x, K, ws=ws)
    torch.cuda.synchronize()

    import ctypes
    steps, warmup = args.steps, args.warmup
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        for i in range(warmup):
            rb.gemv(copies[i % COPIES], g, None, x, K, ws=ws, y=y)
    torch.cuda.synchronize()
    if not torch.equal(y, y_ref):
        raise RuntimeError("eager result changed across calls")

    # ---- throughput: the same steps captured once in a HIP graph and replayed ------------
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                rb.gemv(copies[i % COPIES], g, None, x, K, ws=ws, y=y)
    torch.cuda.synchronize()
    graph.replay()                      # warm replay, checked against the eager result
    torch.cuda.synchronize()
    if not torch.equal(y, y_ref):
        raise RuntimeError("graph replay result differs from the eager result")
    # cold reads at any step count: the warm replay's weights are pushed out of every cache
    # before the timed replay (within it, a copy comes back only after 39 others, 450 MB)
    flush_cache(torch, _lib, dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    graph.replay()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    if not torch.equal(y, y_ref):
        raise RuntimeError("timed replay result differs from the eager result")

    # ---- the same layer with per-column scales h (fp16, random: the dual-scale form), same
    # steps and rotation, cold: the general path, whose bytes include h ------------------
    hh = torch.from_numpy(wl.random_scales(5, k, K, dtype=np.float16)).to(dev)
    Wh = torch.from_numpy(wl.weights_for("down")).to(dev)
    planes_h, g_h = rb.pack(Wh, k, h=hh, ldp=ldp)
    del Wh
    copies_h = [planes_h.clone() for _ in range(COPIES)]
    yh = torch.empty((1, N), dtype=torch.float16, device=dev)
    yh_ref = rb.gemv(planes_h, g_h, hh, x, K, ws=ws)
    hgraph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for i in range(min(warmup, 2 * COPIES)):
            rb.gemv(copies_h[i % COPIES], g_h, hh, x, K, ws=ws, y=yh)
        torch.cuda.synchronize()
        with torch.cuda.graph(hgraph, stream=stream):
            for i in range(steps):
                rb.gemv(copies_h[i % COPIES], g_h, hh, x, K, ws=ws, y=yh)
    torch.cuda.synchronize()
    hgraph.replay()
    torch.cuda.synchronize()
    flush_cache(torch, _lib, dev)
    t0.record()
    hgraph.replay()
    t1.record()
    torch.cuda.synchronize()
    if not torch.equal(yh, yh_ref):
        raise RuntimeError("general-h replay result differs from the eager result")
    h_us = t0.elapsed_time(t1) * 1e3 / steps
    h_bytes = algorithmic_bytes(N, K, k) + 2 * k * K
    del copies_h, planes_h, hgraph

    nbytes = algorithmic_bytes(N, K, k)
    ms_per_step = total_ms / steps
    kern_us = ms_per_step * 1e3
    value = nbytes / (kern_us * 1e-6) / 1e9
    achieved = value

    # ---- streaming-read ceiling at the same footprint (plain kernel, same rotation) -------
    sz = nbytes // 256 * 256
    buf = torch.empty(sz * COPIES, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    sgraph = torch.cuda.CUDAGraph()
    reps = 400
    with torch.cuda.stream(stream):
        _lib.lib.rb_bench_stream_read(ctypes.c_void_p(buf.data_ptr()), sz, ctypes.c_void_p(sink.data_ptr()), 1024,
                                      ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        with torch.cuda.graph(sgraph, stream=stream):
            for i in range(reps):
                _lib.lib.rb_bench_stream_read(ctypes.c_void_p(buf.data_ptr() + (i % COPIES) * sz), sz,
                                              ctypes.c_void_p(sink.data_ptr()), 1024,
                                              ctypes.c_void_p(stream.cuda_stream))
    sgraph.replay()
    torch.cuda.synchronize()
    t0.record()
    sgraph.replay()
    t1.record()
    torch.cuda.synchronize()
    stream_gbs = sz * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del buf

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded Student-t(4)*0.02 weights with 0.5% x10 outlier columns; N(0,1) fp16 activations)",
        "config": {
            "workload": "MLP down projection W 4096x11008, k=2 sign planes, fp16 g, h=1, M=1 fp16 x -> fp16 y; "
                        f"weights rotated over {COPIES} copies (cold HBM)",
            "N": N, "K": K, "k": k, "M": 1, "ldp_words": ldp,
        },
        "gemv_us": round(kern_us, 3),
        "pct_of_hbm_peak": round(100.0 * achieved / PEAK_HBM_GBS, 2),
        "algorithmic_bytes_per_step": nbytes,
        "stream_read_ceiling_GBps": round(stream_gbs, 1),
        "general_h": {
            "note": "the same layer and launch shape with fp16 per-column scales h_i (read by the product): "
                    "the headline times the h = 1 form of the workload, which stores and reads no h",
            "us": round(h_us, 3), "algorithmic_bytes": h_bytes,
            "achieved_GBps": round(h_bytes / (h_us * 1e-6) / 1e9, 2),
            "frac": round(h_bytes / (h_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "pack_ms": round(pack_ms, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(),
        },
    }
    if not args.no_rows:
        out["rows"] = measure_rows(torch, np, rb, wl, dev, pack_ms, with_oracle=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np.ascontiguousarray(planes.cpu().numpy().view(np.uint32)[:, :, :Kw]),
                                           g.float().cpu().numpy().astype(np.float64).reshape(k, N, 1),
                                           x.cpu().numpy())
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
