"""GPU parity over the whole shape set of the boundary: head sizes 16, 32, 64
and 128 for dk and dv each (unequal too), chunk sizes 16, 32 and 64, both io
dtypes.  Shapes the kernels do not run natively run on zero-padded copies (a
square head; bf16 d = 16 at 32), in bf16 32-token chunks (bf16 C = 16, the
length padded to a multiple of 32 where needed), or in chunks halved until a
tile fits (fp32 d = 128); each is compared with the oracle, element by
element, at the io tolerance: the prefill of both write rules, the state
export and the prefill that continues from it, the decode step and the
backward pass.
"""

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, gpu_prefill, np32, oracle_prefill, rel_err, say, split_state, to_dev, true_state

pytestmark = pytest.mark.gpu

PREFILL = [
    # io, dk, dv, C, T
    ("bf16", 64, 32, 64, 512),
    ("bf16", 32, 128, 32, 256),
    ("bf16", 16, 16, 32, 256),
    ("bf16", 16, 64, 16, 256),
    ("bf16", 64, 64, 16, 208),  # 32-token chunks, T padded to 224
    ("bf16", 128, 128, 64, 256),  # 32-token chunks for the read
    ("f32", 16, 64, 16, 256),
    ("f32", 128, 32, 32, 128),
    ("f32", 128, 128, 16, 128),
    ("f32", 128, 128, 64, 192),  # 16-token chunks for the read
]


@pytest.mark.parametrize("rule", [W.MAMBA2, W.GATED_DELTANET])
@pytest.mark.parametrize("io,dk,dv,C,T", PREFILL)
def test_prefill_shape(io, dk, dv, C, T, rule):
    L = max(2, int(np.ceil(np.log2(T))) + 2)
    w = W.Workload("shape", rule, 1, 2, T, dk, dv, L, C, io, 500 + dk + 3 * dv + C)
    x = W.prefill_inputs(w)
    o = gpu_prefill(x, C, L)
    assert o.shape == (1, T, 2, dv)
    err = rel_err(o, oracle_prefill(x))
    say(f"[shape] rule {rule} {io} dk{dk} dv{dv} C{C} T{T}: rel err {err:.3e} (tol {TOL[io]:g})")
    assert err <= TOL[io]


@pytest.mark.parametrize("io,dk,dv,C", [("bf16", 64, 32, 64), ("bf16", 16, 128, 32), ("f32", 32, 16, 16),
                                        ("f32", 128, 64, 16)])
def test_state_export_and_continue(io, dk, dv, C):
    """Export the state of 512 tokens (dk != dv), continue with a 256-token
    segment from it, then decode 3 steps: outputs and states against the oracle."""
    T0, T1, L = 512, 256, 12
    w = W.Workload("shape chain", W.MAMBA2, 2, 2, T0 + T1 + 3, dk, dv, L, C, io, 700 + dk + dv)
    x = W.prefill_inputs(w, variant="slowdecay")
    d = to_dev(x)
    seg = lambda lo, hi: {k: (None if v is None else v[:, lo:hi].contiguous()) for k, v in d.items()}
    state = F.decode_state_tensor(w.B, w.H, dk, dv, L)
    s0 = seg(0, T0)
    o0, _ = F.attn_fwd(s0["q"], s0["k"], s0["v"], s0["log_gate"], s0["lam"], C=C, L=L, want_state=True,
                       state_out=state)
    torch.cuda.synchronize()
    s_hat, sigma = split_state(state, w.B, w.H, L, dk, dv)
    ref_state = oracle.state_direct(np32(x["k"])[:, :T0], np32(x["v"])[:, :T0], np32(x["log_gate"])[:, :T0], L)
    live = [lv for lv in range(1, L) if (T0 >> (lv - 1)) & 1]
    serr = rel_err(true_state(s_hat, sigma)[:, :, live], ref_state[:, :, live])
    s1 = seg(T0, T0 + T1)
    o1, _ = F.attn_fwd(s1["q"], s1["k"], s1["v"], s1["log_gate"], s1["lam"], C=C, L=L, want_state=True,
                       pos0=T0, state_in=state, state_out=state)
    code = F.LL_BF16 if io == "bf16" else F.LL_F32
    o_dec = []
    for t in range(T0 + T1, T0 + T1 + 3):
        od = torch.empty(w.B, w.H, dv, dtype=d["v"].dtype, device="cuda")
        F.ll_decode_step(w.B, w.H, dk, dv, L, code, F.LL_MAMBA2, t, d["q"][:, t].contiguous(),
                         d["k"][:, t].contiguous(), d["v"][:, t].contiguous(), d["log_gate"][:, t].contiguous(),
                         d["lam"][:, t].contiguous(), None, od, state)
        o_dec.append(od)
    torch.cuda.synchronize()
    ref = oracle_prefill(x)
    o_all = np.concatenate([np32(o0), np32(o1), np.stack([np32(v) for v in o_dec], axis=1)], axis=1)
    err = rel_err(o_all, ref)
    say(f"[shape] {io} dk{dk} dv{dv} C{C}: export rel err {serr:.3e}; prefill + continue + decode rel err {err:.3e}")
    assert serr <= TOL[io] and err <= TOL[io]


BWD = [
    # io, dk, dv, C, T
    ("bf16", 64, 32, 64, 512),
    ("bf16", 16, 16, 32, 256),
    ("bf16", 32, 64, 16, 208),  # 32-token chunks, T padded to 224
    ("bf16", 128, 128, 64, 256),
    ("f32", 16, 32, 64, 256),  # 32-token chunks
    ("f32", 128, 64, 16, 128),
]


@pytest.mark.parametrize("io,dk,dv,C,T", BWD)
def test_bwd_shape(io, dk, dv, C, T):
    L = max(2, int(np.ceil(np.log2(T))) + 2)
    w = W.Workload("shape bwd", W.MAMBA2, 1, 2, T, dk, dv, L, C, io, 800 + dk + 3 * dv + C)
    x = W.prefill_inputs(w)
    g = torch.Generator().manual_seed(900 + T)
    dO = torch.randn(1, T, 2, dv, generator=g).to(x["v"].dtype)
    dev = to_dev(x)
    o = F.attn_fwd(dev["q"], dev["k"], dev["v"], dev["log_gate"], dev["lam"], C=C, L=L)
    grads = F.attn_bwd(dev["q"], dev["k"], dev["v"], dev["log_gate"], dev["lam"], o, dO.cuda(), C=C, L=L)
    torch.cuda.synchronize()
    ref = oracle.bwd_direct(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), np32(x["lam"]), np32(dO))
    errs = {n: rel_err(np32(grads[n]), ref[n]) for n in ("dq", "dk", "dv", "dlambda", "dlog_gate")}
    say(f"[shape bwd] {io} dk{dk} dv{dv} C{C} T{T}: " + ", ".join(f"{n} {e:.3e}" for n, e in errs.items()))
    assert all(e <= TOL[io] for e in errs.values()), errs
