"""GPU parity of the decode step with one position per sequence
(ll_decode_step_ragged) against the oracle, which steps each sequence on its
own from the same per-level states.

Also: equal positions give bit-for-bit the result of ll_decode_step, and a
sequence whose position does not fit the levels gets NaN outputs with its
state untouched while the others are computed.  Tolerance as for the other
decode tests: max|o - ref| / max|ref| <= 1e-4 (fp32 io), 2e-2 (bf16 io).
"""

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, np32, rel_err, say, split_state, true_state

pytestmark = pytest.mark.gpu


def setup(io, d, L, positions, steps, rule, seed):
    """Inputs for B = len(positions) sequences (row b's prefix is its first
    positions[b] tokens, then `steps` decode tokens) and the oracle's
    per-level states of each prefix."""
    B, H = len(positions), 3
    T = max(max(positions), 0) + steps
    w = W.Workload("ragged decode", rule, B, H, T, d, d, L, 16, io, seed)
    x = W.prefill_inputs(w)
    st = np.zeros((B, H, L, d, d))
    for b, p in enumerate(positions):
        if p > 0:
            sl = lambda name: None if x[name] is None else np32(x[name][b:b + 1, :p])
            st[b] = oracle.state_direct(sl("k"), sl("v"), sl("log_gate"), L, beta=sl("beta"),
                                        rule=oracle.RULE_GDN if rule == W.GATED_DELTANET else oracle.RULE_MAMBA2)[0]
    return w, x, st


def flat_state(st, w, d):
    flat = np.zeros(F.ll_decode_state_bytes(w.B, w.H, d, d, w.L) // 4, np.float32)
    flat[:st.size] = st.astype(np.float32).reshape(-1)
    return torch.from_numpy(flat).cuda()


def token(x, b, t):
    """Token t of sequence b as [H, ...] arrays (clamped into range for rows
    whose position is invalid: their values are never used)."""
    t = min(max(t, 0), x["k"].shape[1] - 1)
    return {k: (None if v is None else v[b, t]) for k, v in x.items()}


def run_gpu(w, x, positions, steps, state, d):
    code = F.LL_BF16 if w.io == "bf16" else F.LL_F32
    outs = []
    for i in range(steps):
        toks = [token(x, b, p + i) for b, p in enumerate(positions)]
        dev = {k: (None if toks[0][k] is None else torch.stack([tk[k] for tk in toks]).contiguous().cuda())
               for k in toks[0]}
        pos = torch.tensor([p + i for p in positions], dtype=torch.int64, device="cuda")
        o = torch.empty(w.B, w.H, d, dtype=dev["v"].dtype, device="cuda")
        F.ll_decode_step_ragged(w.B, w.H, d, d, w.L, code, w.rule, pos, dev["q"], dev["k"], dev["v"],
                                dev["log_gate"], dev["lam"], dev["beta"], o, state)
        outs.append(o)
    torch.cuda.synchronize()
    return np.stack([np32(o) for o in outs], axis=1)  # [B, steps, H, d]


def run_oracle(w, x, positions, steps, st, rows):
    rule = oracle.RULE_GDN if w.rule == W.GATED_DELTANET else oracle.RULE_MAMBA2
    ref = np.zeros((w.B, steps, w.H, w.dv))
    for b in rows:
        s = np.ascontiguousarray(st[b:b + 1])
        for i in range(steps):
            tk = token(x, b, positions[b] + i)
            a = {k: (None if v is None else np32(v)[None]) for k, v in tk.items()}
            ref[b, i] = oracle.decode_step(s, positions[b] + i, a["q"], a["k"], a["v"], a["log_gate"], a["lam"],
                                           a["beta"], rule=rule)[0]
        st[b] = s[0]
    return ref


@pytest.mark.parametrize("io,d,rule", [("bf16", 64, W.MAMBA2), ("f32", 32, W.MAMBA2), ("bf16", 128, W.MAMBA2),
                                       ("bf16", 64, W.GATED_DELTANET)])
def test_ragged_positions_match_oracle(io, d, rule):
    L, steps = 13, 3
    positions = [0, 1, 777, 2048, 4091]  # the last steps up to 4093: pos + 1 < 2^12
    w, x, st = setup(io, d, L, positions, steps, rule, seed=60 + d)
    state = flat_state(st, w, d)
    o = run_gpu(w, x, positions, steps, state, d)
    ref = run_oracle(w, x, positions, steps, st, range(w.B))
    err = rel_err(o, ref)
    say(f"[ragged decode] {io} d{d} rule {rule} positions {positions}: rel err {err:.3e} (tol {TOL[io]:g})")
    assert err <= TOL[io]
    s_hat, sigma = split_state(state, w.B, w.H, L, d, d)
    for b, p in enumerate(positions):
        live = [l for l in range(1, L) if ((p + steps) >> (l - 1)) & 1]
        err = rel_err(true_state(s_hat, sigma)[b][:, live], st[b][:, live])
        say(f"[ragged decode] state of sequence {b} after position {p + steps - 1}: rel err {err:.3e}")
        assert err <= TOL[io]


def test_equal_positions_match_uniform_step_bitwise():
    L, d, p = 12, 64, 1500
    w, x, st = setup("bf16", d, L, [p] * 4, 1, W.MAMBA2, seed=71)
    tk = {k: (None if v is None else v[:, p].contiguous().cuda()) for k, v in x.items()}
    s1, s2 = flat_state(st, w, d), flat_state(st, w, d)
    o1 = torch.empty(w.B, w.H, d, dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    F.ll_decode_step(w.B, w.H, d, d, L, F.LL_BF16, F.LL_MAMBA2, p, tk["q"], tk["k"], tk["v"], tk["log_gate"],
                     tk["lam"], None, o1, s1)
    pos = torch.full((w.B,), p, dtype=torch.int64, device="cuda")
    F.ll_decode_step_ragged(w.B, w.H, d, d, L, F.LL_BF16, F.LL_MAMBA2, pos, tk["q"], tk["k"], tk["v"],
                            tk["log_gate"], tk["lam"], None, o2, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)


def test_invalid_positions_give_nan_and_keep_state():
    """Rows at position -1 and 2^(L-1) - 1 (whose successor does not fit) are
    refused by the kernel: NaN outputs, state bytes unchanged; the other rows
    are stepped normally."""
    L, d = 10, 64
    positions = [5, -1, 511, 300]
    w, x, st = setup("bf16", d, L, [5, 0, 0, 300], 1, W.MAMBA2, seed=81)
    state = flat_state(st, w, d)
    before = state.clone()
    o = run_gpu(w, x, positions, 1, state, d)
    ref = run_oracle(w, x, positions, 1, st, [0, 3])
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all()
    err = rel_err(o[[0, 3]], ref[[0, 3]])
    say(f"[ragged decode] valid rows beside invalid ones: rel err {err:.3e}")
    assert err <= TOL["bf16"]
    s_now, _ = split_state(state, w.B, w.H, L, d, d)
    s_was, _ = split_state(before, w.B, w.H, L, d, d)
    assert np.array_equal(s_now[[1, 2]], s_was[[1, 2]])
    n = w.B * w.H * L * d * d
    sig_now = state[n:].view(w.B, w.H, L).cpu()
    sig_was = before[n:].view(w.B, w.H, L).cpu()
    assert torch.equal(sig_now[[1, 2]], sig_was[[1, 2]])
