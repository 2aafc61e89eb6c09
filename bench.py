"""Prefill throughput of log-linear Mamba-2 attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one ll_attn_fwd over the 16K-token workload (B=2, H=16, T=16384,
dk=dv=64, bf16 q/k/v/o, fp32 gates and lambda, 15 levels, chunk 64): the whole
hot path (ll_chunk_state, ll_fenwick_scan, ll_chunk_attn) on inputs already
resident in HBM.  Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The GPU raises its clocks over the first milliseconds of sustained work:
# after 5 warm-up steps the 16K prefill step measured 0.12 ms, after 300 of
# them 0.103 ms on the same box.  Before each timed section, settle() runs the
# section's step untimed, in bursts of 10 with a wait after each, for
# SETTLE_MS of wall time, so that the timed steps see the clocks a sustained
# job runs at.
SETTLE_MS = 100.0


def settle(fn) -> int:
    import torch

    n = 0
    t_end = time.perf_counter() + SETTLE_MS * 1e-3
    while SETTLE_MS > 0 and time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    return n


def algorithmic_bytes_per_token_head(w) -> int:
    """Compulsory HBM traffic of one token-head: read q, k, v, lambda, the
    log-gate, write o."""
    esz = 2 if w.io == "bf16" else 4
    return (2 * w.dk + 2 * w.dv) * esz + 4 * w.L + 4


def useful_flops_per_token_head(w) -> float:
    """Matrix-core work the chunked form must do per token-head: the chunk's
    own key-value state (2 dk dv), the causal half of the in-chunk scores and
    their product with V (~ (C+1)(dk+dv)), and one q^T S read per non-empty
    chunk-or-coarser level (2 dk dv each; on average half of the log2(T/C)
    chunk levels are non-empty)."""
    import math

    chunk_levels = math.log2(w.T // w.C)
    return 2 * w.dk * w.dv + (w.C + 1) * (w.dk + w.dv) + 2 * w.dk * w.dv * chunk_levels / 2


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "prefill-16k_kernels.md")
ATTN_SOURCES = ["chunk_attn.hip", "ll_device.hpp", "ll_launch.hpp"]


def measured_traffic():
    """HBM bytes per ll_chunk_attn launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, if it was taken on the kernel sources as they are now (else None)."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "fenwick_tree_linear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"traffic ll_chunk_attn: sources-sha256=([0-9a-f]+) read-bytes=(\d+) write-bytes=(\d+)", text)
    if not m or m.group(1) != h.hexdigest():
        return None
    return int(m.group(2)) + int(m.group(3))


def cpu_baseline(w, min_seconds: float = 10.0) -> dict:
    """The oracle's recurrent form on the whole workload (both batch entries, all heads, all
    tokens), repeated until at least ``min_seconds`` of host time, timed on the host cores."""
    import oracle
    from fenwick_tree_linear_amd import workloads as W

    import platform
    import tempfile

    x = W.prefill_inputs(w)
    np_in = {k: (None if v is None else v.float().numpy()) for k, v in x.items()}
    # a copy of the oracle built for this host's own instruction set
    tmpdir = tempfile.mkdtemp(prefix="llref_native_")
    lib = oracle.load(oracle.build(os.path.join(tmpdir, "libllref_native.so"), opt_flags=("-O3", "-march=native")))
    cpu_model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    runs, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        oracle.fwd_recurrent(np_in["q"], np_in["k"], np_in["v"], np_in["log_gate"], np_in["lam"], lib=lib)
        dt += time.perf_counter() - t0
        runs += 1
    cores = min(oracle.threads(lib), w.B * w.H)
    return {"value": runs * w.B * w.T / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"recurrent O(T log T) form over the whole workload ({w.B} x {w.H} heads x {w.T} tokens), "
                      f"fp64, {runs} runs in {dt:.1f} s",
            "build": "gcc -O3 -march=native -std=c11 -fopenmp", "cpu_model": cpu_model, "nproc": os.cpu_count(),
            "omp_threads": oracle.threads(lib)}


def decode_bench(steps: int, cold_reps: int = 10) -> dict:
    """ll_decode_step on the decode workload (B64 H16 d64 bf16, 17 levels): ``steps`` tokens at
    positions 32768.. from a resident per-level state (random values; the step's cost does not
    depend on them), one launch per token, timed with HIP events on the launch stream."""
    import torch

    import fenwick_tree_linear_amd as F
    from fenwick_tree_linear_amd import workloads as W

    w = W.WORKLOADS["decode-32k"]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    state = F.decode_state_tensor(w.B, w.H, w.dk, w.dv, w.L, device=dev)
    nmat = w.B * w.H * w.L * w.dk * w.dv
    state[:nmat].normal_(0.0, 0.05, generator=gen)
    x = W.decode_inputs(W.with_shape(w, steps=1), device=dev)
    q, k, v = (x[n][0].contiguous() for n in ("q", "k", "v"))
    g, lam = x["log_gate"][0].contiguous(), x["lam"][0].contiguous()
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    def step(pos):
        F.ll_decode_step(w.B, w.H, w.dk, w.dv, w.L, F.LL_BF16, F.LL_MAMBA2, pos, q, k, v, g, lam, None, o, state, stream)

    settle(lambda: step(w.T))
    for i in range(8):
        step(w.T + i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(w.T + i)
    stop.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) * 1e3 / steps
    mask = (1 << (w.L - 1)) - 1
    level_bytes = w.dk * w.dv * 4
    io_bytes = (4 * w.dk * 2 + 4 + 2 * w.L * 4)  # q, k, v, o; gate; lambda; sigma read + written

    def step_bytes(pos):  # the non-empty levels read, the merged level written, the token's I/O
        return w.B * w.H * ((bin(pos & mask).count("1") + 1) * level_bytes + io_bytes)

    bytes_per_step = sum(step_bytes(w.T + i) for i in range(steps)) / steps
    achieved = bytes_per_step / (us * 1e-6) / 1e9
    # cold: single steps, each after a 512 MiB write that leaves none of the state in the
    # 256 MB last-level cache (median of ``cold_reps``; positions continue where the run above ended)
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    cold = []
    for r in range(cold_reps):
        flush.fill_(float(r))
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        step(w.T + steps + r)
        b_ev.record(stream)
        torch.cuda.synchronize()
        cold.append((a_ev.elapsed_time(b_ev) * 1e3, step_bytes(w.T + steps + r)))
    del flush
    out = {"workload": "ll_decode_step B64 H16 d64 bf16, 17 levels, positions 32768.." + str(w.T + steps - 1),
           "us_per_step": round(us, 2), "tokens_per_s": round(w.B / (us * 1e-6), 1),
           "bytes_per_step": int(bytes_per_step), "achieved_GBs": round(achieved, 1), "peak_GBs": HBM_PEAK_GBS,
           "frac": round(achieved / HBM_PEAK_GBS, 4)}
    if cold:
        cold.sort()
        c_us, c_bytes = cold[len(cold) // 2]
        out["cold"] = {"us_per_step_median": round(c_us, 2), "bytes": int(c_bytes),
                       "achieved_GBs": round(c_bytes / (c_us * 1e-6) / 1e9, 1),
                       "frac": round(c_bytes / (c_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "reps": len(cold),
                       "note": "one step after a 512 MiB write; includes the launch of a lone kernel"}
    return out


def ragged_decode_bench(steps: int) -> dict:
    """ll_decode_step_ragged on the decode workload's shape (B64 H16 d64 bf16, 17 levels) with the
    64 sequences at different positions (32768 + 37 b, so their non-empty levels differ), all
    advanced by one token per step on the device; HIP events on the launch stream."""
    import torch

    import fenwick_tree_linear_amd as F
    from fenwick_tree_linear_amd import workloads as W

    w = W.WORKLOADS["decode-32k"]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    state = F.decode_state_tensor(w.B, w.H, w.dk, w.dv, w.L, device=dev)
    nmat = w.B * w.H * w.L * w.dk * w.dv
    state[:nmat].normal_(0.0, 0.05, generator=gen)
    x = W.decode_inputs(W.with_shape(w, steps=1), device=dev)
    q, k, v = (x[n][0].contiguous() for n in ("q", "k", "v"))
    g, lam = x["log_gate"][0].contiguous(), x["lam"][0].contiguous()
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    start_pos = [w.T + 37 * b for b in range(w.B)]
    pos = torch.tensor(start_pos, dtype=torch.int64, device=dev)

    def step():
        F.ll_decode_step_ragged(w.B, w.H, w.dk, w.dv, w.L, F.LL_BF16, F.LL_MAMBA2, pos, q, k, v, g, lam, None, o,
                                state, stream)
        pos.add_(1)

    settle(lambda: F.ll_decode_step_ragged(w.B, w.H, w.dk, w.dv, w.L, F.LL_BF16, F.LL_MAMBA2, pos, q, k, v, g, lam,
                                           None, o, state, stream))
    for _ in range(8):
        step()
    torch.cuda.synchronize()
    first = [p + 8 for p in start_pos]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) * 1e3 / steps  # includes the position increment (a tiny torch kernel)
    mask = (1 << (w.L - 1)) - 1
    level_bytes = w.dk * w.dv * 4
    io_bytes = (4 * w.dk * 2 + 4 + 2 * w.L * 4 + 8)
    total = sum(w.H * ((bin((p + i) & mask).count("1") + 1) * level_bytes + io_bytes)
                for p in first for i in range(steps)) / steps
    achieved = total / (us * 1e-6) / 1e9
    return {"workload": "ll_decode_step_ragged B64 H16 d64 bf16, 17 levels, sequence b at position 32768 + 37 b",
            "us_per_step": round(us, 2), "tokens_per_s": round(w.B / (us * 1e-6), 1),
            "bytes_per_step": int(total), "achieved_GBs": round(achieved, 1), "peak_GBs": HBM_PEAK_GBS,
            "frac": round(achieved / HBM_PEAK_GBS, 4)}


def from_state_bench(reps: int) -> dict:
    """ll_attn_fwd_from_state on the second half of the 16K prefill (tokens 8192..16383 of
    B2 H16 d64 bf16, 15 levels, chunk 64) after the per-level state of the first half (its one
    bucket, level 14): whole-call time and per-kernel averages (HIP events on the launch stream);
    where a separate ll_prior_read adds the earlier levels, its algorithmic bytes: q read, o read
    and written, the one level's weight and the gates per token-head, and the prior level once per
    head."""
    import torch

    import fenwick_tree_linear_amd as F
    from fenwick_tree_linear_amd import workloads as W

    w = W.WORKLOADS["prefill-16k"]
    T0 = w.T // 2
    dev = torch.device("cuda:0")
    x = W.prefill_inputs(w, device=dev)
    half = {k: (None if v is None else v[:, T0:].contiguous()) for k, v in x.items()}
    first = {k: (None if v is None else v[:, :T0].contiguous()) for k, v in x.items()}
    state = F.decode_state_tensor(w.B, w.H, w.dk, w.dv, w.L, device=dev)
    prob0 = F.LLProblem(w.B, T0, w.H, w.dk, w.dv, w.L, w.C, F.LL_BF16, F.LL_MAMBA2)
    ws_bytes = F.ll_attn_fwd_workspace_bytes(prob0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty(w.B, T0, w.H, w.dv, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    F.ll_attn_fwd(prob0, first["q"], first["k"], first["v"], first["log_gate"], first["lam"], None, o, state, ws,
                  ws_bytes, stream)

    def step():
        F.ll_attn_fwd_from_state(prob0, T0, state, half["q"], half["k"], half["v"], half["log_gate"], half["lam"],
                                 None, o, None, ws, ws_bytes, stream)

    settle(step)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    F.ll_kernel_timing_read()
    F.ll_kernel_timing_enable(True)
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    kt = F.ll_kernel_timing_read()
    F.ll_kernel_timing_enable(False)
    kernels = {name: round(t / n * 1e3, 2) for name, (t, n) in kt.items()}
    out = {"workload": "ll_attn_fwd_from_state B2 H16 d64 bf16, 15 levels, chunk 64: tokens 8192..16383 after "
                       "the state of 0..8191",
           "ms_per_step": round(ms, 5), "tokens_per_s": round(w.B * T0 / (ms * 1e-3), 1), "kernels_us": kernels}
    if "ll_prior_read" in kt:
        # a separate ll_prior_read: its algorithmic bytes
        th = w.B * T0 * w.H
        prior_bytes = th * (w.dk * 2 + 2 * w.dv * 2 + 4 + 4) + w.B * w.H * w.dk * w.dv * 4
        t_prior = kt["ll_prior_read"][0] / kt["ll_prior_read"][1] * 1e-3
        gbs = prior_bytes / t_prior / 1e9
        out["prior_read"] = {"bytes": int(prior_bytes), "achieved_GBs": round(gbs, 1), "peak_GBs": HBM_PEAK_GBS,
                             "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        out["prior_read"] = "inside ll_chunk_attn (the read takes the levels of [0, pos0) itself)"
    return out


def measured_peaks() -> dict:
    """What this machine reaches on plain library work, as context for the spec-sheet peaks: a 1 GiB
    device-to-device copy (HBM read + write, beyond the 256 MB last-level cache) and an
    8192 x 8192 x 8192 bf16 matrix product through torch (hipBLASLt), each the median of 5."""
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def median_ms(fn, reps=5):
        settle(fn)
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return sorted(out)[len(out) // 2]

    n = 1 << 28  # fp32 elements: 1 GiB
    src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    ms = median_ms(lambda: dst.copy_(src))
    copy_gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    del src, dst
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    y = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    ms = median_ms(lambda: torch.mm(x, y))
    gemm_tflops = 2 * m ** 3 / (ms * 1e-3) / 1e12
    del x, y
    return {"copy_1GiB_GBs": round(copy_gbs, 1), "bf16_gemm_8192_TFLOPs": round(gemm_tflops, 1),
            "hbm_spec_GBs": HBM_PEAK_GBS, "bf16_mfma_spec_TFLOPs": MFMA_BF16_PEAK_TFLOPS}


def ccq_bench(reps: int) -> dict:
    """ll_ccq_query (the curvature-conditioned query) on the 16K prefill's q and k (B2 H16 T16384
    d64 bf16): per-call time and per-kernel averages (HIP events on the launch stream), then the
    prefill step that reads with the contracted queries."""
    import torch

    import fenwick_tree_linear_amd as F
    from fenwick_tree_linear_amd import workloads as W

    w = W.WORKLOADS["prefill-16k"]
    dev = torch.device("cuda:0")
    x = W.prefill_inputs(w, device=dev)
    g = W.ccq_inputs(w.H, w.dk, seed=w.seed, device=dev)
    stream = torch.cuda.current_stream(dev)
    nbytes = F.ll_ccq_query_workspace_bytes(w.B, w.T, w.H, w.dk, F.LL_BF16)
    cws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    qc = torch.empty_like(x["q"])
    prob = F.LLProblem(w.B, w.T, w.H, w.dk, w.dv, w.L, w.C, F.LL_BF16, F.LL_MAMBA2)
    ws_bytes = F.ll_attn_fwd_workspace_bytes(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty(w.B, w.T, w.H, w.dv, dtype=torch.bfloat16, device=dev)

    def ccq():
        F.ll_ccq_query(w.B, w.T, w.H, w.dk, F.LL_BF16, x["q"], x["k"], g["w"], g["b"], qc, cws, nbytes, stream)

    def step():
        ccq()
        F.ll_attn_fwd(prob, qc, x["k"], x["v"], x["log_gate"], x["lam"], None, o, None, ws, ws_bytes, stream)

    def timed(fn, n):
        settle(fn)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    ms = timed(ccq, reps)
    F.ll_kernel_timing_read()
    F.ll_kernel_timing_enable(True)
    for _ in range(reps):
        ccq()
    torch.cuda.synchronize()
    kt = F.ll_kernel_timing_read()
    F.ll_kernel_timing_enable(False)
    step_ms = timed(step, reps)
    return {"workload": "ll_ccq_query B2 H16 T16384 d64 bf16 (running second moment from an all-ones, "
                        "no-decay prefill; running key sum from a chunked fp32 prefix sum)",
            "ms_per_call": round(ms, 5), "kernels_us": {k: round(t / n * 1e3, 2) for k, (t, n) in kt.items()},
            "prefill_with_ccq": {"ms_per_step": round(step_ms, 5),
                                 "tokens_per_s": round(w.B * w.T / (step_ms * 1e-3), 1)}}


def bwd_bench(reps: int) -> dict:
    """ll_attn_bwd on the 2K prefill's shape (B4 H16 T2048 d64 bf16, 12 levels, chunk 64): time per
    backward call (HIP events on the launch stream) and per-kernel averages, beside the forward's."""
    import torch

    import fenwick_tree_linear_amd as F
    from fenwick_tree_linear_amd import workloads as W

    w = W.WORKLOADS["prefill-2k"]
    dev = torch.device("cuda:0")
    x = W.prefill_inputs(w, device=dev)
    dO = torch.randn(w.B, w.T, w.H, w.dv, device=dev, generator=torch.Generator(device=dev).manual_seed(7)).to(
        torch.bfloat16)
    stream = torch.cuda.current_stream(dev)
    prob = F.LLProblem(w.B, w.T, w.H, w.dk, w.dv, w.L, w.C, F.LL_BF16, F.LL_MAMBA2)
    fws_bytes = F.ll_attn_fwd_workspace_bytes(prob)
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty(w.B, w.T, w.H, w.dv, dtype=torch.bfloat16, device=dev)
    bws_bytes = F.ll_attn_bwd_workspace_bytes(prob)
    bws = torch.empty(bws_bytes, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    dg, dl = torch.empty_like(x["log_gate"]), torch.empty_like(x["lam"])

    def fwd():
        F.ll_attn_fwd(prob, x["q"], x["k"], x["v"], x["log_gate"], x["lam"], None, o, None, fws, fws_bytes, stream)

    def bwd():
        F.ll_attn_bwd(prob, x["q"], x["k"], x["v"], x["log_gate"], x["lam"], o, dO, dq, dk, dv, dg, dl, bws,
                      bws_bytes, stream)

    def timed(fn, n):
        settle(fn)
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    f_ms = timed(fwd, reps)
    b_ms = timed(bwd, reps)
    F.ll_kernel_timing_read()
    F.ll_kernel_timing_enable(True)
    bwd()
    torch.cuda.synchronize()
    kt = F.ll_kernel_timing_read()
    F.ll_kernel_timing_enable(False)
    return {"workload": "ll_attn_bwd B4 H16 T2048 d64 bf16, 12 levels, chunk 64 (Mamba-2)",
            "fwd_ms": round(f_ms, 5), "bwd_ms": round(b_ms, 5), "bwd_over_fwd": round(b_ms / f_ms, 1),
            "tokens_per_s": round(w.B * w.T / (b_ms * 1e-3), 1),
            "kernels_in_one_call": {k: {"ms": round(t, 4), "launches": n} for k, (t, n) in kt.items()}}


MFMA_FP32_PEAK_TFLOPS = 157.3  # dense fp32 matrix cores


def lambda_mlp_bench(reps: int) -> dict:
    """ll_lambda_mlp (the adaptive-decay level-weight MLP, hidden 2L) over every row of the 16K
    prefill (2 x 16384 x 16 rows of 15 levels), back to back, HIP events on the launch stream;
    then the prefill step with the MLP in front of ll_attn_fwd."""
    import torch

    import fenwick_tree_linear_amd as F
    from fenwick_tree_linear_amd import workloads as W

    w = W.WORKLOADS["prefill-16k"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    m = W.lambda_mlp_inputs((w.B, w.T, w.H), w.L, seed=w.seed, device=dev)
    rows, L, hidden = w.B * w.T * w.H, w.L, m["w1"].shape[1]
    lam = torch.empty_like(m["d"])

    def mlp():
        F.ll_lambda_mlp(rows, L, hidden, m["d"], m["w1"], m["w2"], m["bias"], lam, stream)

    def timed(fn, n):
        settle(fn)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    ms = timed(mlp, reps)
    nbytes = rows * L * 4 * 2 + (2 * L * hidden + L) * 4
    flops = 4 * rows * L * hidden
    x = W.prefill_inputs(w, device=dev, parts=("q", "k", "v", "log_gate"))
    prob = F.LLProblem(w.B, w.T, w.H, w.dk, w.dv, w.L, w.C, F.LL_BF16, F.LL_MAMBA2)
    ws_bytes = F.ll_attn_fwd_workspace_bytes(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty(w.B, w.T, w.H, w.dv, dtype=torch.bfloat16, device=dev)

    def step_two_launches():
        mlp()
        F.ll_attn_fwd(prob, x["q"], x["k"], x["v"], x["log_gate"], lam, None, o, None, ws, ws_bytes, stream)

    mlp_ws_bytes = F.ll_attn_fwd_lambda_mlp_workspace_bytes(prob, hidden)
    mlp_ws = ws if mlp_ws_bytes <= ws_bytes else torch.empty(mlp_ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        F.ll_attn_fwd_lambda_mlp(prob, x["q"], x["k"], x["v"], x["log_gate"], m["d"], hidden, m["w1"], m["w2"],
                                 m["bias"], None, o, None, mlp_ws, max(mlp_ws_bytes, ws_bytes), stream)

    step_ms = timed(step, reps)
    two_ms = timed(step_two_launches, reps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"ll_lambda_mlp {rows} rows (B2 T16384 H16), L={L}, hidden={hidden}, fp32",
            "us_per_launch": round(ms * 1e3, 2), "bytes": nbytes, "achieved_GBs": round(gbs, 1),
            "peak_GBs": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
            "fp32_mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 2), "fp32_mfma_peak_tflops": MFMA_FP32_PEAK_TFLOPS,
            "prefill_with_mlp": {"ms_per_step": round(step_ms, 5),
                                 "tokens_per_s": round(w.B * w.T / (step_ms * 1e-3), 1),
                                 "entry": "ll_attn_fwd_lambda_mlp (the read makes the level weights)",
                                 "two_launches_ms_per_step": round(two_ms, 5)}}


def gdn_bench(steps: int) -> dict:
    """ll_attn_fwd with the Gated DeltaNet write on its 8K-token workload (B2 H16 T8192 d128 bf16,
    14 levels, chunk 64): whole-step time and per-kernel averages, both from HIP events on the
    launch stream, inputs resident in HBM."""
    import torch

    import fenwick_tree_linear_amd as F
    from fenwick_tree_linear_amd import workloads as W

    w = W.WORKLOADS["gdn-8k"]
    dev = torch.device("cuda:0")
    x = W.prefill_inputs(w, device=dev)
    prob = F.LLProblem(w.B, w.T, w.H, w.dk, w.dv, w.L, w.C, F.LL_BF16, F.LL_GATED_DELTANET)
    ws_bytes = F.ll_attn_fwd_workspace_bytes(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty(w.B, w.T, w.H, w.dv, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        F.ll_attn_fwd(prob, x["q"], x["k"], x["v"], x["log_gate"], x["lam"], x["beta"], o, None, ws, ws_bytes,
                      stream)

    settle(step)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    F.ll_kernel_timing_read()  # drop anything counted before
    F.ll_kernel_timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kt = F.ll_kernel_timing_read()
    F.ll_kernel_timing_enable(False)
    return {"workload": "gated-deltanet prefill B2 H16 T8192 dk=dv=128 bf16, 14 levels, chunk 64",
            "ms_per_step": round(ms, 5), "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
            "kernels_us": {name: round(t / n * 1e3, 2) for name, (t, n) in kt.items()},
            "algorithmic_bytes": gdn_algorithmic_bytes(w),
            "algorithmic_frac": round(gdn_algorithmic_bytes(w) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_io": gdn_hbm_fractions(w, kt)}


def gdn_algorithmic_bytes(w) -> int:
    """Compulsory HBM traffic of the Gated DeltaNet prefill: q, k, v read and o written (bf16), the
    gate, beta and the level weights read (fp32)."""
    rows = w.B * w.T * w.H
    return rows * (2 * w.dk + 2 * w.dv) * 2 + rows * (w.L + 2) * 4


def gdn_hbm_fractions(w, kt) -> dict:
    """Kernel I/O bytes of each Gated DeltaNet prefill kernel on this workload (what each kernel of
    this design must read and write, including the design's own intermediates W, U', U, the block
    states and the Fenwick nodes, but not the bf16 node copies or re-reads of earlier blocks' nodes)
    and the rate they give at the kernel's measured average time, as a fraction of the 8 TB/s peak.
    These are not the step's algorithmic bytes: those are the compulsory inputs and outputs (q, k, v,
    gates, beta, lambda read, o written), reported beside them.  The read runs at chunk 32 (the bf16
    d = 128 tile) in blocks of 8 chunks."""
    rows = w.B * w.T * w.H
    rb = w.dk * 2  # one bf16 row
    nb = w.T // (32 * 8)  # blocks per head
    heads = w.B * w.H
    node = w.dk * w.dv * 4
    alg = {
        "ll_gdn_wy": 4 * rows * rb + 2 * rows * 4,            # k, v, gates, beta in; W, U' out
        "ll_gdn_state": 4 * rows * rb + rows * 4,             # W, k, U', gates in; U out
        "ll_chunk_state": 2 * rows * rb + rows * 4 + heads * nb * node,  # k, U, gates in; block states out
        "ll_fenwick_scan": heads * nb * node + heads * (nb // 2) * node,  # block states read, nodes written
        "ll_chunk_attn": 4 * rows * rb + rows * (w.L + 1) * 4,  # q, k, U, lambda, gates in; o out
    }
    out = {}
    for name, nbytes in alg.items():
        if name in kt and kt[name][1]:
            us = kt[name][0] / kt[name][1] * 1e3
            out[name] = {"bytes": nbytes, "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "frac": round(nbytes / (us * 1e-6) / 8e12, 4)}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=512,
                    help="also time this many ll_decode_step tokens on the decode workload (0: skip)")
    ap.add_argument("--gdn-steps", type=int, default=20,
                    help="also time this many Gated DeltaNet prefill steps on its 8K-token workload (0: skip)")
    ap.add_argument("--ragged-steps", type=int, default=512,
                    help="also time this many ll_decode_step_ragged steps with per-sequence positions (0: skip)")
    ap.add_argument("--from-state-reps", type=int, default=20,
                    help="also time this many prefills of the 16K workload's second half from a state (0: skip)")
    ap.add_argument("--bwd-reps", type=int, default=5,
                    help="also time this many backward passes on the 2K prefill's shape (0: skip)")
    ap.add_argument("--ccq-reps", type=int, default=10,
                    help="also time this many curvature-conditioned query calls on the 16K workload (0: skip)")
    ap.add_argument("--mlp-reps", type=int, default=50,
                    help="also time this many ll_lambda_mlp launches over the 16K workload's rows (0: skip)")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="also time this many single steps with the last-level cache flushed before each (0: skip)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="run the step untimed for this long before the warm-up steps, so that the timed steps "
                         "see the GPU's clocks after they have ramped up under load (0: skip)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy and GEMM rates")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (each (batch, head) pair is "
              "independent, so more GPUs would shard the heads with no communication)", file=sys.stderr)
        return 2

    import torch

    import fenwick_tree_linear_amd as F
    from fenwick_tree_linear_amd import workloads as W

    w = W.WORKLOADS["prefill-16k"]
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: generating inputs on the GPU")
    x = W.prefill_inputs(w, device=dev)
    prob = F.LLProblem(w.B, w.T, w.H, w.dk, w.dv, w.L, w.C, F.LL_BF16, F.LL_MAMBA2)
    ws_bytes = F.ll_attn_fwd_workspace_bytes(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty(w.B, w.T, w.H, w.dv, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        F.ll_attn_fwd(prob, x["q"], x["k"], x["v"], x["log_gate"], x["lam"], None, o, None, ws, ws_bytes, stream)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * 1024 * 1024 // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del src, dst

    global SETTLE_MS
    SETTLE_MS = args.settle_ms
    settle_steps = settle(step)
    if settle_steps:
        log(f"[bench] settle: {settle_steps} untimed steps in {args.settle_ms:g} ms")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    start_ev = torch.cuda.Event(enable_timing=True)
    stop_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start_ev.record(stream)
    for _ in range(args.steps):
        step()
    stop_ev.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start_ev.elapsed_time(stop_ev) / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (events), wall {wall * 1e6 / args.steps:.1f} us/step")

    # per-kernel durations: HIP events around every launch, on the launch stream,
    # right after the timed steps (the same clocks)
    F.ll_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = F.ll_kernel_timing_read()
    F.ll_kernel_timing_enable(False)
    kernels = {name: round(ms / n * 1e3, 2) for name, (ms, n) in kt.items()}
    log(f"[bench] per-kernel average us: {kernels}")

    # cold: the 256 MB last-level cache flushed by writing a 512 MiB buffer
    # before each of a few individually timed steps (median reported)
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    cold_ms = []
    for r in range(args.cold_reps):
        flush.fill_(float(r))
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        step()
        b_ev.record(stream)
        torch.cuda.synchronize()
        cold_ms.append(a_ev.elapsed_time(b_ev))
    del flush
    cold = None
    if cold_ms:
        med = sorted(cold_ms)[len(cold_ms) // 2]
        cold = {"ms_per_step_median": round(med, 5), "tokens_per_s": round(w.B * w.T / (med * 1e-3), 1),
                "reps": len(cold_ms), "flush_bytes": 512 * 1024 * 1024}
        log(f"[bench] cold (last-level cache flushed): median {med * 1e3:.1f} us/step over {len(cold_ms)} steps")

    token_heads = w.B * w.T * w.H
    alg_bytes = algorithmic_bytes_per_token_head(w) * token_heads
    # ll_fenwick_scan: the block states it must read and the level >= 1 nodes it writes
    # (64 x 64 fp32 each): the workspace holds exactly those and their gate sums
    scan_bytes = F.ll_attn_fwd_workspace_bytes(prob)
    t_scan = kt["ll_fenwick_scan"][0] / kt["ll_fenwick_scan"][1] * 1e-3
    scan = {"bytes": scan_bytes, "us": round(t_scan * 1e6, 2), "achieved_GBs": round(scan_bytes / t_scan / 1e9, 1),
            "frac": round(scan_bytes / t_scan / 1e9 / HBM_PEAK_GBS, 4)}
    t_attn = kt["ll_chunk_attn"][0] / kt["ll_chunk_attn"][1] * 1e-3
    achieved = alg_bytes / t_attn / 1e9
    flops = useful_flops_per_token_head(w) * token_heads
    tokens_per_s = w.B * w.T / (ms_per_step * 1e-3)

    result = {
        "metric": "prefill tokens/s (log-linear Mamba-2, T=16K) + % of MFMA/HBM peak",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "log-linear Mamba-2 prefill B2 H16 T16384 dk=dv=64 bf16, 15 levels, chunk 64",
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "head_dim": w.dk, "levels": w.L,
                   "chunk": w.C},
        "roofline": {"bound": "hbm", "kernel": "ll_chunk_attn", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "algorithmic_bytes": alg_bytes},
        "mfma": {"useful_gflop": round(flops / 1e9, 2),
                 "achieved_tflops_step": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac_step": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "kernels_us": kernels,
        "scan": scan,
        "cold": cold,
        "cpu_baseline": None,
    }
    if args.decode_steps:
        result["decode"] = decode_bench(args.decode_steps, args.cold_reps)
        log(f"[bench] decode: {result['decode']}")
    if args.gdn_steps:
        result["gdn"] = gdn_bench(args.gdn_steps)
        log(f"[bench] gdn: {result['gdn']}")
    if args.ragged_steps:
        result["ragged_decode"] = ragged_decode_bench(args.ragged_steps)
        log(f"[bench] ragged decode: {result['ragged_decode']}")
    if args.from_state_reps:
        result["from_state"] = from_state_bench(args.from_state_reps)
        log(f"[bench] prefill from a state: {result['from_state']}")
    if args.bwd_reps:
        result["backward"] = bwd_bench(args.bwd_reps)
        log(f"[bench] backward: {result['backward']}")
    if args.ccq_reps:
        result["ccq"] = ccq_bench(args.ccq_reps)
        log(f"[bench] curvature-conditioned query: {result['ccq']}")
    if args.mlp_reps:
        result["lambda_mlp"] = lambda_mlp_bench(args.mlp_reps)
        log(f"[bench] lambda mlp: {result['lambda_mlp']}")
    if not args.no_peaks:
        result["measured_peaks"] = measured_peaks()
        log(f"[bench] measured peaks: {result['measured_peaks']}")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
