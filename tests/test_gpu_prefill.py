"""GPU parity of the chunk-parallel prefill (ll_attn_fwd) against the oracle.

Element-by-element at sizes the oracle finishes in seconds, sampled outputs at
the 16K-token workload in the launch configuration the benchmark times, plus
chunk-size invariance, ragged and degenerate shapes, state export, causality
and run-to-run determinism.  Tolerance: max|o - ref| / max|ref| <= 1e-4 for
fp32 io, <= 2e-2 for bf16 io.
"""

import numpy as np
import pytest
import torch

import oracle
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, gpu_prefill, np32, oracle_prefill, rel_err, say, to_dev, true_state

pytestmark = pytest.mark.gpu


def check(case, gpu, ref, io):
    err = rel_err(gpu, ref)
    say(f"[prefill] {case}: rel err {err:.3e} (tol {TOL[io]:g})")
    assert err <= TOL[io], case


@pytest.fixture(scope="module")
def prefill_2k():
    w = W.WORKLOADS["prefill-2k"]
    x = W.prefill_inputs(w)
    say("[prefill] oracle for prefill-2k (64 heads x 2048 tokens)")
    return w, x, oracle_prefill(x)


def test_tiny_fp32_every_chunk_size():
    w = W.WORKLOADS["tiny"]
    x = W.prefill_inputs(w)
    ref = oracle_prefill(x)
    for C in (16, 32, 64):
        check(f"tiny C={C}", gpu_prefill(x, C, w.L), ref, "f32")


def test_prefill_2k_full(prefill_2k):
    w, x, ref = prefill_2k
    check("prefill-2k C=64", gpu_prefill(x, 64, w.L), ref, "bf16")


def test_prefill_2k_chunk_invariance(prefill_2k):
    w, x, ref = prefill_2k
    o64 = gpu_prefill(x, 64, w.L)
    o32 = gpu_prefill(x, 32, w.L)
    check("prefill-2k C=32", o32, ref, "bf16")
    check("prefill-2k C=32 vs C=64", o32, o64, "bf16")


def test_prefill_16k_sampled():
    """The benchmarked workload (B2 H16 T16384 d64 bf16, C=64), checked on
    windows of tokens at the start, middle and end of every head."""
    w = W.WORKLOADS["prefill-16k"]
    x = W.prefill_inputs(w)
    o = gpu_prefill(x, w.C, w.L)
    assert np.isfinite(o).all()
    for lo, hi in ((0, 96), (8160, 8224), (12288 - 32, 12288 + 32), (16384 - 96, 16384)):
        ref = oracle_prefill(x, t_range=(lo, hi))
        check(f"prefill-16k tokens [{lo},{hi})", o[:, lo:hi], ref[:, lo:hi], "bf16")


@pytest.mark.parametrize("io,T,d,C,L", [("bf16", 32768, 64, 64, 16), ("bf16", 16384, 32, 32, 15)])
def test_many_blocks_no_decay(io, T, d, C, L):
    """64 blocks of 8 chunks per head: block 63 has six earlier-block Fenwick
    nodes, one more than the read holds in registers, so its last node comes
    through the per-chunk path.  No decay, so every node carries weight."""
    w = W.Workload("many blocks", W.MAMBA2, 1, 2, T, d, d, L, C, io, 31 + d)
    x = W.prefill_inputs(w, variant="nodecay")
    o = gpu_prefill(x, C, L)
    assert np.isfinite(o).all()
    for lo, hi in ((T - 64, T), (T * 47 // 64, T * 47 // 64 + 32)):
        ref = oracle_prefill(x, t_range=(lo, hi))
        check(f"{io} T{T} d{d} C{C} no decay, tokens [{lo},{hi})", o[:, lo:hi], ref[:, lo:hi], io)


@pytest.mark.parametrize("variant", ["nodecay", "slowdecay", "deep"])
def test_every_level_bf16(variant):
    """Inputs under which high levels carry weight (no or slow decay), and
    lambda one-hot at a random level per token."""
    w = W.with_shape(W.WORKLOADS["prefill-2k"], B=1, H=4)
    x = W.prefill_inputs(w, variant=variant)
    check(f"bf16 {variant}", gpu_prefill(x, 64, w.L), oracle_prefill(x), "bf16")


@pytest.mark.parametrize("variant", ["default", "nodecay", "deep"])
def test_every_level_fp32(variant):
    w = W.Workload("fp32 d32 T2048", W.MAMBA2, 1, 2, 2048, 32, 32, 12, 64, "f32", 11)
    x = W.prefill_inputs(w, variant=variant)
    ref = oracle_prefill(x)
    for C in (16, 64):
        check(f"fp32 d32 {variant} C={C}", gpu_prefill(x, C, w.L), ref, "f32")


RAGGED = [
    # io, B, H, T, d, C, L    (T/C chunks: odd counts give one-chunk blocks)
    ("bf16", 3, 5, 320, 64, 64, 10),    # 5 chunks
    ("bf16", 1, 2, 1536, 64, 64, 12),   # 24 chunks: 3 blocks of 8
    ("bf16", 2, 3, 224, 32, 32, 9),     # 7 chunks of 32, d=32
    ("bf16", 2, 2, 64, 64, 64, 7),      # a single chunk
    ("bf16", 1, 3, 320, 64, 64, 20),    # more levels than needed
    ("bf16", 1, 2, 1024, 128, 32, 11),  # d=128 (chunks of 32)
    ("bf16", 1, 1, 4096, 128, 32, 13),  # d=128: 16 blocks of 8 chunks, 4 block-level node levels
    ("bf16", 1, 1, 1568, 128, 32, 12),  # d=128: 49 chunks, one-chunk blocks
    ("f32", 2, 3, 48, 16, 16, 7),       # 3 chunks of 16
    ("f32", 1, 1, 16, 16, 16, 5),       # a single fp32 chunk
    ("f32", 1, 2, 96, 64, 32, 8),       # d=64 fp32
]


@pytest.mark.parametrize("io,B,H,T,d,C,L", RAGGED)
def test_ragged_and_degenerate_shapes(io, B, H, T, d, C, L):
    w = W.Workload("ragged", W.MAMBA2, B, H, T, d, d, L, C, io, 100 + T + d)
    x = W.prefill_inputs(w)
    check(f"{io} B{B} H{H} T{T} d{d} C{C} L{L}", gpu_prefill(x, C, L), oracle_prefill(x), io)


@pytest.mark.parametrize("io,T,d,C,L", [("bf16", 1536, 64, 64, 12), ("bf16", 2048, 64, 64, 13),
                                        ("f32", 208, 16, 16, 9), ("bf16", 320, 32, 32, 10),
                                        ("bf16", 1280, 128, 32, 12)])
def test_state_export_matches_bucket_states(io, T, d, C, L):
    """The exported per-level states of [0,T) (decayed through token T-1) equal
    the oracle's bucket sums; empty levels are zero and log-scales 0."""
    w = W.Workload("export", W.MAMBA2, 2, 3, T, d, d, L, C, io, 7 + T)
    x = W.prefill_inputs(w)
    o, (s_hat, sigma) = gpu_prefill(x, C, L, want_state=True)
    ref = oracle.state_direct(np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), L)
    assert (sigma == 0).all()
    err = rel_err(true_state(s_hat, sigma), ref)
    say(f"[prefill] export {io} T{T} d{d} C{C} L{L}: state rel err {err:.3e}")
    assert err <= TOL[io]
    empty = [l for l in range(L) if not (l >= 1 and (T >> (l - 1)) & 1)]
    assert (s_hat[:, :, empty] == 0).all()
    check(f"export-run output T{T}", o, oracle_prefill(x), io)


def test_state_only_prefill_needs_no_q_or_lambda():
    w = W.Workload("export", W.MAMBA2, 1, 2, 512, 64, 64, 11, 64, "bf16", 5)
    x = W.prefill_inputs(w, parts=("k", "v", "log_gate"))
    _, (s_hat, sigma) = gpu_prefill(x, 64, w.L, want_output=False, want_state=True)
    ref = oracle.state_direct(np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), w.L)
    assert rel_err(true_state(s_hat, sigma), ref) <= TOL["bf16"]


def test_causality(prefill_2k):
    """Changing tokens from t0 on leaves every earlier output bit-identical."""
    w, x, _ = prefill_2k
    t0 = 1000  # inside a chunk
    y = {k: (None if v is None else v.clone()) for k, v in x.items()}
    gen = torch.Generator().manual_seed(99)
    for name in ("q", "k", "v"):
        y[name][:, t0:] = torch.randn(y[name][:, t0:].shape, generator=gen).to(y[name].dtype)
    y["log_gate"][:, t0:] = -torch.rand(y["log_gate"][:, t0:].shape, generator=gen)
    y["lam"][:, t0:] = torch.rand(y["lam"][:, t0:].shape, generator=gen)
    a = gpu_prefill(x, 64, w.L)
    b = gpu_prefill(y, 64, w.L)
    assert np.array_equal(a[:, :t0], b[:, :t0])
    assert not np.array_equal(a[:, t0:], b[:, t0:])


def test_bitwise_deterministic(prefill_2k):
    w, x, _ = prefill_2k
    d = to_dev(x)
    a = gpu_prefill(x, 64, w.L, dev_inputs=d)
    b = gpu_prefill(x, 64, w.L, dev_inputs=d)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T", [15872, 16384])
def test_state_export_many_blocks(T):
    """At 31 and 32 blocks of 8 chunks per head the Fenwick scan splits each
    head's blocks into segments; the exported states then include nodes that
    combine several segments (slow decay, so every level carries weight)."""
    w = W.Workload("export many blocks", W.MAMBA2, 1, 2, T, 64, 64, 16, 64, "bf16", 17 + T)
    x = W.prefill_inputs(w, variant="slowdecay", parts=("k", "v", "log_gate"))
    _, (s_hat, sigma) = gpu_prefill(x, 64, 16, want_output=False, want_state=True)
    ref = oracle.state_direct(np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), 16)
    for lvl in range(16):
        if lvl >= 1 and (T >> (lvl - 1)) & 1:
            err = rel_err(true_state(s_hat[:, :, lvl], sigma[:, :, lvl]), ref[:, :, lvl])
            say(f"[prefill] export T{T} level {lvl}: state rel err {err:.3e}")
            assert err <= TOL["bf16"], lvl
