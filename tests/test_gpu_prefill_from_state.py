"""GPU parity of the prefill that continues a sequence from its per-level
states (ll_attn_fwd_from_state), chained segment by segment with the state
updated in place, against the oracle's direct form over the whole sequence
and its bucket states.

Both write rules (for Gated DeltaNet the pseudo-value pass continues from the
prior plain state).  Segment boundaries cover both cases of the export: the segment's bucket
merging with a run of prior levels (pos0 = 512, 1536 with 512-token
segments) and prior levels kept beside the segment's own (pos0 = 1024; a
1536-token segment after 2048).  Tolerance: max|o - ref| / max|ref| <= 1e-4
(fp32 io), 2e-2 (bf16 io).
"""

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, np32, oracle_prefill, rel_err, say, split_state, to_dev, true_state

pytestmark = pytest.mark.gpu


def chained_prefill(x, cuts, C, L):
    """Prefill x [B, N, H, ...] as segments [cuts[i], cuts[i+1]) on the GPU,
    each from the state the previous one left (in place)."""
    d = to_dev(x)
    B, N, H, dk = d["k"].shape
    state = F.decode_state_tensor(B, H, dk, dk, L)
    outs = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        seg = {k: (None if v is None else v[:, lo:hi].contiguous()) for k, v in d.items()}
        rule = F.LL_MAMBA2 if seg.get("beta") is None else F.LL_GATED_DELTANET
        o, _ = F.attn_fwd(seg["q"], seg["k"], seg["v"], seg["log_gate"], seg["lam"], seg.get("beta"), C=C, L=L,
                          rule=rule, want_state=True, pos0=lo, state_in=state if lo > 0 else None, state_out=state)
        outs.append(o)
    torch.cuda.synchronize()
    return np.concatenate([np32(o) for o in outs], axis=1), state


@pytest.mark.parametrize("io,d,C,seg,variant,rule", [
    ("bf16", 64, 64, 512, "slowdecay", W.MAMBA2), ("bf16", 64, 64, 512, "default", W.MAMBA2),
    ("f32", 32, 32, 128, "slowdecay", W.MAMBA2), ("bf16", 128, 32, 256, "nodecay", W.MAMBA2),
    ("bf16", 64, 64, 512, "slowdecay", W.GATED_DELTANET), ("f32", 32, 16, 64, "slowdecay", W.GATED_DELTANET),
    ("bf16", 128, 64, 256, "slowdecay", W.GATED_DELTANET)])
def test_chained_segments_match_whole_sequence(io, d, C, seg, variant, rule):
    N, L = 4 * seg, 13
    w = W.Workload("chained", rule, 1, 3, N, d, d, L, C, io, 90 + d + seg)
    x = W.prefill_inputs(w, variant=variant)
    cuts = [0, seg, 2 * seg, 3 * seg, 4 * seg]
    o, state = chained_prefill(x, cuts, C, L)
    err = rel_err(o, oracle_prefill(x))
    say(f"[from state] rule {rule} {io} d{d} C{C} segments of {seg} ({variant}): output rel err {err:.3e} "
        f"(tol {TOL[io]:g})")
    assert err <= TOL[io]
    s_hat, sigma = split_state(state, w.B, w.H, L, d, d)
    ref = oracle.state_direct(np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), L, beta=np32(x["beta"]),
                              rule=oracle.RULE_GDN if rule == W.GATED_DELTANET else oracle.RULE_MAMBA2)
    live = [l for l in range(1, L) if (N >> (l - 1)) & 1]
    assert (sigma == 0).all()
    err = rel_err(true_state(s_hat, sigma)[:, :, live], ref[:, :, live])
    say(f"[from state] final state after {N} tokens: rel err {err:.3e}")
    assert err <= TOL[io]
    empty = [l for l in range(L) if l not in live]
    assert (s_hat[:, :, empty] == 0).all()


def test_uneven_segment_then_decode():
    """2048 tokens, then a 1536-token segment (prior level kept, two segment
    levels beside it), then decode steps from the exported state."""
    L, d, N, T1 = 14, 64, 3584, 2048
    w = W.Workload("segment+decode", W.MAMBA2, 2, 2, N + 8, d, d, L, 64, "bf16", 97)
    x = W.prefill_inputs(w, variant="slowdecay")
    pre = {k: (None if v is None else v[:, :N]) for k, v in x.items()}
    o, state = chained_prefill(pre, [0, T1, N], 64, L)
    ref_all = oracle_prefill(x)
    err = rel_err(o, ref_all[:, :N])
    say(f"[from state] 2048 + 1536 tokens: output rel err {err:.3e}")
    assert err <= TOL["bf16"]
    dev = to_dev(x)
    outs = []
    for t in range(N, N + 8):
        ot = torch.empty(w.B, w.H, d, dtype=torch.bfloat16, device="cuda")
        F.ll_decode_step(w.B, w.H, d, d, L, F.LL_BF16, F.LL_MAMBA2, t, dev["q"][:, t].contiguous(),
                         dev["k"][:, t].contiguous(), dev["v"][:, t].contiguous(),
                         dev["log_gate"][:, t].contiguous(), dev["lam"][:, t].contiguous(), None, ot, state)
        outs.append(ot)
    torch.cuda.synchronize()
    od = np.stack([np32(t) for t in outs], axis=1)
    err = rel_err(od, ref_all[:, N:])
    say(f"[from state] decode after the chained prefill: rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_state_only_continuation():
    """o = NULL: only the state of [0, pos0 + T) is produced (q and lambda
    not needed), and a fresh output buffer is not touched."""
    L, d, seg = 12, 64, 256
    w = W.Workload("state only", W.MAMBA2, 1, 2, 2 * seg, d, d, L, 64, "bf16", 99)
    x = W.prefill_inputs(w, variant="slowdecay")
    dev = to_dev(x)
    _, state = F.attn_fwd(dev["q"][:, :seg].contiguous(), dev["k"][:, :seg].contiguous(),
                          dev["v"][:, :seg].contiguous(), dev["log_gate"][:, :seg].contiguous(),
                          dev["lam"][:, :seg].contiguous(), C=64, L=L, want_state=True)
    F.attn_fwd(None, dev["k"][:, seg:].contiguous(), dev["v"][:, seg:].contiguous(),
               dev["log_gate"][:, seg:].contiguous(), None, C=64, L=L, want_output=False, want_state=True,
               pos0=seg, state_in=state, state_out=state)
    torch.cuda.synchronize()
    s_hat, sigma = split_state(state, w.B, w.H, L, d, d)
    ref = oracle.state_direct(np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), L)
    live = [l for l in range(1, L) if ((2 * seg) >> (l - 1)) & 1]
    err = rel_err(true_state(s_hat, sigma)[:, :, live], ref[:, :, live])
    say(f"[from state] state-only continuation: rel err {err:.3e}")
    assert err <= TOL["bf16"]
