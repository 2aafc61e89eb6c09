"""GPU parity of the Gated DeltaNet write against the oracle (rule GDN): the
prefill (pseudo-value pass, then the log-linear read of q, k and the
pseudo-values), its exported state, the 8K-token d=128 workload on sampled
heads and windows, and the decode step from the empty state and from a
prefill's exported state.  Tolerance: max|o - ref| / max|ref| <= 1e-4 for fp32
io, <= 2e-2 for bf16 io.
"""

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, gpu_prefill, np32, oracle_prefill, rel_err, say, split_state, true_state

pytestmark = pytest.mark.gpu


def gdn(B, H, T, d, C, L, io, seed):
    return W.Workload("gdn", W.GATED_DELTANET, B, H, T, d, d, L, C, io, seed)


def check(case, gpu, ref, io):
    err = rel_err(gpu, ref)
    say(f"[gdn] {case}: rel err {err:.3e} (tol {TOL[io]:g})")
    assert err <= TOL[io], case


@pytest.mark.parametrize("C", [16, 32, 64])
def test_gdn_tiny_fp32_every_chunk_size(C):
    w = gdn(1, 2, 256, 16, C, 9, "f32", 40)
    x = W.prefill_inputs(w)
    check(f"tiny fp32 C={C}", gpu_prefill(x, C, w.L), oracle_prefill(x), "f32")


SHAPES = [
    # io, B, H, T, d, C, L
    ("bf16", 2, 3, 512, 64, 64, 10),
    ("bf16", 1, 2, 256, 32, 32, 9),
    ("bf16", 1, 2, 1024, 128, 64, 11),  # the read runs on chunks of 32
    ("bf16", 1, 2, 1024, 128, 32, 11),
    ("f32", 1, 2, 256, 64, 32, 9),
    ("f32", 2, 2, 96, 32, 16, 8),       # 6 chunks of 16
    ("f32", 1, 1, 64, 32, 64, 7),       # a single chunk
]


@pytest.mark.parametrize("io,B,H,T,d,C,L", SHAPES)
def test_gdn_shapes(io, B, H, T, d, C, L):
    w = gdn(B, H, T, d, C, L, io, 200 + T + d + C)
    x = W.prefill_inputs(w)
    check(f"{io} B{B} H{H} T{T} d{d} C{C} L{L}", gpu_prefill(x, C, L), oracle_prefill(x), io)


def test_gdn_chunk_size_invariance():
    """The pseudo-values and the read do not depend on C beyond rounding."""
    w = gdn(1, 2, 512, 64, 64, 10, "bf16", 77)
    x = W.prefill_inputs(w)
    check("C=32 vs C=64", gpu_prefill(x, 32, w.L), gpu_prefill(x, 64, w.L), "bf16")


def test_gdn_8k_sampled():
    """The 8K-token workload (B2 H16 T8192 d128 bf16, 14 levels, C=64) on two
    heads, at the start, middle and end of the sequence."""
    w = W.WORKLOADS["gdn-8k"]
    x = W.prefill_inputs(w)
    o = gpu_prefill(x, w.C, w.L)
    assert np.isfinite(o).all()
    heads = [(0, 0), (1, 15)]
    for lo, hi in ((0, 64), (4096 - 32, 4096 + 32), (8192 - 64, 8192)):
        ref = oracle_prefill(x, heads=heads, t_range=(lo, hi))
        for b, h in heads:
            check(f"gdn-8k head ({b},{h}) tokens [{lo},{hi})", o[b, lo:hi, h], ref[b, lo:hi, h], "bf16")


@pytest.mark.parametrize("io,T,d,C,L", [("bf16", 1536, 64, 64, 12), ("f32", 208, 16, 16, 9)])
def test_gdn_state_export(io, T, d, C, L):
    w = gdn(2, 2, T, d, C, L, io, 9 + T)
    x = W.prefill_inputs(w)
    _, (s_hat, sigma) = gpu_prefill(x, C, L, want_state=True)
    ref = oracle.state_direct(np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), L, beta=np32(x["beta"]),
                              rule=oracle.RULE_GDN)
    err = rel_err(true_state(s_hat, sigma), ref)
    say(f"[gdn] export {io} T{T} d{d}: state rel err {err:.3e}")
    assert err <= TOL[io]


def gpu_decode(x, state, t_lo, t_hi, L, io):
    B, _, H, dk = x["k"].shape
    dv = x["v"].shape[-1]
    dev = {k: (None if v is None else v.cuda()) for k, v in x.items()}
    code = F.LL_BF16 if io == "bf16" else F.LL_F32
    outs = []
    for t in range(t_lo, t_hi):
        o = torch.empty(B, H, dv, dtype=dev["v"].dtype, device="cuda")
        s = {k: (None if v is None else v[:, t].contiguous()) for k, v in dev.items()}
        F.ll_decode_step(B, H, dk, dv, L, code, F.LL_GATED_DELTANET, t, s["q"], s["k"], s["v"], s["log_gate"],
                         s["lam"], s["beta"], o, state)
        outs.append(o)
    torch.cuda.synchronize()
    return np.stack([np32(o) for o in outs], axis=1)


@pytest.mark.parametrize("io,d,T,L", [("bf16", 64, 200, 9), ("f32", 32, 200, 9), ("bf16", 128, 40, 7)])
def test_gdn_decode_from_empty_state(io, d, T, L):
    w = gdn(2, 3, T, d, 16, L, io, 51 + d)
    x = W.prefill_inputs(w)
    state = F.decode_state_tensor(w.B, w.H, d, d, L)
    o = gpu_decode(x, state, 0, T, L, io)
    check(f"decode from empty {io} d{d} T{T}", o, oracle_prefill(x), io)
    s_hat, sigma = split_state(state, w.B, w.H, L, d, d)
    ref = oracle.state_direct(np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), L, beta=np32(x["beta"]),
                              rule=oracle.RULE_GDN)
    live = [l for l in range(1, L) if (T >> (l - 1)) & 1]
    err = rel_err(true_state(s_hat, sigma)[:, :, live], ref[:, :, live])
    say(f"[gdn] decode final state {io} d{d}: rel err {err:.3e}")
    assert err <= TOL[io]


def test_gdn_decode_resumes_from_prefill_export():
    T0, T1, L = 1024, 1088, 12
    w = gdn(2, 2, T1, 64, 64, L, "bf16", 61)
    x = W.prefill_inputs(w)
    pre = {k: (None if v is None else v[:, :T0].contiguous()) for k, v in x.items()}
    _, flat = F.attn_fwd(*(pre[n].cuda() for n in ("q", "k", "v", "log_gate", "lam", "beta")), C=64, L=L,
                         rule=F.LL_GATED_DELTANET, want_state=True)
    o = gpu_decode(x, flat, T0, T1, L, "bf16")
    ref = oracle_prefill(x, t_range=(T0, T1))[:, T0:T1]
    check("decode after prefill export", o, ref, "bf16")
