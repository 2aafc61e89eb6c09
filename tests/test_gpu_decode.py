"""GPU parity of the recurrent decode step (ll_decode_step) against the oracle.

Covers decoding from the empty state, resuming from an oracle-built state,
resuming from the prefill's exported state, the largest admissible position,
and the 32K-prefix workload (B64 H16 d64 bf16, 512 steps) on sampled heads.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, np32, oracle_prefill, rel_err, say, split_state, true_state

pytestmark = pytest.mark.gpu


def gpu_decode(x, state, t_lo, t_hi, L, io):
    """Steps positions t_lo..t_hi-1 with token t taken from x[:, t]; returns o
    [B, t_hi-t_lo, H, dv] as numpy."""
    B, _, H, dk = x["k"].shape
    dv = x["v"].shape[-1]
    dev = {k: (None if v is None else v.cuda()) for k, v in x.items()}
    outs = []
    code = F.LL_BF16 if io == "bf16" else F.LL_F32
    for t in range(t_lo, t_hi):
        o = torch.empty(B, H, dv, dtype=dev["v"].dtype, device="cuda")
        step = {k: (None if v is None else v[:, t].contiguous()) for k, v in dev.items()}
        F.ll_decode_step(B, H, dk, dv, L, code, F.LL_MAMBA2, t, step["q"], step["k"], step["v"], step["log_gate"],
                         step["lam"], None, o, state)
        outs.append(o)
    torch.cuda.synchronize()
    return np.stack([np32(o) for o in outs], axis=1)


@pytest.mark.parametrize("io,d,T,L", [("bf16", 64, 300, 10), ("f32", 32, 300, 10), ("f32", 16, 31, 6),
                                      ("bf16", 128, 70, 8)])
def test_decode_from_empty_state(io, d, T, L):
    """Decoding token by token from the zero state reproduces every output of
    the direct form (T=31, L=6 ends at the largest admissible position 30)."""
    w = W.Workload("decode", W.MAMBA2, 2, 3, T, d, d, L, 16, io, 21 + d)
    x = W.prefill_inputs(w)
    state = F.decode_state_tensor(w.B, w.H, d, d, L)
    o = gpu_decode(x, state, 0, T, L, io)
    err = rel_err(o, oracle_prefill(x))
    say(f"[decode] from empty {io} d{d} T{T}: rel err {err:.3e}")
    assert err <= TOL[io]
    s_hat, sigma = split_state(state, w.B, w.H, L, d, d)
    ref = oracle.state_direct(np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), L)
    live = [l for l in range(1, L) if (T >> (l - 1)) & 1]
    err = rel_err(true_state(s_hat, sigma)[:, :, live], ref[:, :, live])
    say(f"[decode] final state {io} d{d} T{T}: rel err {err:.3e}")
    assert err <= TOL[io]


@pytest.mark.parametrize("io,d", [("bf16", 64), ("f32", 32)])
def test_decode_resumes_from_oracle_state(io, d):
    T0, T1, L = 1000, 1200, 12
    w = W.Workload("resume", W.MAMBA2, 2, 2, T1, d, d, L, 16, io, 31)
    x = W.prefill_inputs(w)
    ref_state = oracle.state_direct(np32(x["k"])[:, :T0], np32(x["v"])[:, :T0], np32(x["log_gate"])[:, :T0], L)
    n = w.B * w.H * L * d * d
    flat = np.zeros(F.ll_decode_state_bytes(w.B, w.H, d, d, L) // 4, np.float32)
    flat[:n] = ref_state.astype(np.float32).reshape(-1)
    state = torch.from_numpy(flat).cuda()
    o = gpu_decode(x, state, T0, T1, L, io)
    ref = oracle_prefill(x, t_range=(T0, T1))[:, T0:T1]
    err = rel_err(o, ref)
    say(f"[decode] resume from oracle state {io} d{d}: rel err {err:.3e}")
    assert err <= TOL[io]


def test_decode_resumes_from_prefill_export():
    T0, T1, L = 2048, 2112, 13
    w = W.Workload("export+decode", W.MAMBA2, 2, 4, T1, 64, 64, L, 64, "bf16", 41)
    x = W.prefill_inputs(w)
    pre = {k: (None if v is None else v[:, :T0].contiguous()) for k, v in x.items()}
    dev = {k: (None if v is None else v.cuda()) for k, v in pre.items()}
    _, state = F.attn_fwd(dev["q"], dev["k"], dev["v"], dev["log_gate"], dev["lam"], C=64, L=L, want_state=True)
    o = gpu_decode(x, state, T0, T1, L, "bf16")
    err = rel_err(o, oracle_prefill(x, t_range=(T0, T1))[:, T0:T1])
    say(f"[decode] resume from prefill export: rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_decode_32k_workload_sampled_heads():
    """B64 H16 d64 bf16: the per-level states of a 32768-token prefix come from
    the prefill's export on the GPU; then 512 decode steps (positions 32768..
    33279).  Sampled heads are checked against the oracle, which builds its own
    prefix states from the same inputs."""
    w = W.WORKLOADS["decode-32k"]
    L, d = w.L, w.dk
    say("[decode] generating the 32768-token prefix on the GPU")
    pre = W.prefill_inputs(w, device="cuda", parts=("k", "v", "log_gate"))
    _, state = F.attn_fwd(None, pre["k"], pre["v"], pre["log_gate"], None, C=64, L=L, want_output=False,
                          want_state=True)
    torch.cuda.synchronize()
    steps = W.decode_inputs(w)
    dev = {k: (None if v is None else v.cuda()) for k, v in steps.items()}
    B, H = w.B, w.H
    o_all = torch.empty(w.steps, B, H, d, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    t0 = time.time()
    for i in range(w.steps):
        F.ll_decode_step(B, H, d, d, L, F.LL_BF16, F.LL_MAMBA2, w.T + i, dev["q"][i], dev["k"][i], dev["v"][i],
                         dev["log_gate"][i], dev["lam"][i], None, o_all[i], state)
    torch.cuda.synchronize()
    say(f"[decode] 512 steps in {time.time() - t0:.3f} s (with launch overhead)")
    o_all = np32(o_all)

    heads = [(0, 0), (17, 5), (40, 11), (63, 15)]
    for b, h in heads:
        k = np32(pre["k"][b:b + 1, :, h:h + 1])
        v = np32(pre["v"][b:b + 1, :, h:h + 1])
        g = np32(pre["log_gate"][b:b + 1, :, h:h + 1])
        st = oracle.state_direct(k, v, g, L)
        ref = []
        for i in range(w.steps):
            sl = lambda name: np32(steps[name][i, b:b + 1, h:h + 1])
            ref.append(oracle.decode_step(st, w.T + i, sl("q"), sl("k"), sl("v"), sl("log_gate"), sl("lam"))[0, 0])
        err = rel_err(o_all[:, b, h], np.stack(ref))
        say(f"[decode] 32k head (b={b}, h={h}): rel err {err:.3e}")
        assert err <= TOL["bf16"]
