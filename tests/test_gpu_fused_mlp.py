"""GPU parity of the prefill whose level weights come from the adaptive-decay
MLP inside the call (ll_attn_fwd_lambda_mlp; "Adaptive memory decay for
log-linear attention", section "Method", LambdaMLPSoftplus).

Two checks per case:
  - against the oracle: its own fp64 MLP, then its direct form, at the io
    tolerance;
  - against ll_lambda_mlp followed by ll_attn_fwd on the same inputs: equal bit
    for bit.  The read that makes the weights forms the composite W1 W2 and the
    fp32 row products with the same operations in the same order as
    ll_lambda_mlp and cuts the sequence into the plain read's blocks; where it
    cannot make the weights the call runs those same launches.
"""

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, np32, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

# io, dk, dv, C, T, L, hidden, rule
CASES = [
    ("bf16", 64, 64, 64, 512, 10, 20, W.MAMBA2),    # made by the read, one block of 8 chunks
    ("bf16", 64, 64, 64, 2048, 12, 24, W.MAMBA2),   # made by the read, 4 blocks (the plain read: 2)
    ("bf16", 64, 64, 64, 960, 12, 24, W.MAMBA2),    # a last block of fewer chunks
    ("bf16", 32, 32, 32, 512, 10, 20, W.MAMBA2),    # d = 32, chunks of 32
    ("bf16", 32, 64, 64, 1024, 11, 22, W.MAMBA2),   # dk != dv (square head 64)
    ("bf16", 64, 64, 16, 496, 10, 32, W.MAMBA2),    # chunks of 16 run as 32 (length padded)
    ("bf16", 64, 64, 64, 512, 16, 32, W.MAMBA2),    # L at its fused limit
    ("bf16", 64, 64, 64, 4096, 16, 32, W.MAMBA2),   # L 16, 8 blocks
    ("bf16", 64, 64, 64, 1024, 11, 22, W.GATED_DELTANET),
    ("bf16", 64, 64, 64, 1024, 11, 33, W.MAMBA2),   # hidden 33 (made by the read: any hidden size)
    ("bf16", 64, 64, 64, 512, 12, 64, W.MAMBA2),    # hidden 64, the largest ll_lambda_mlp takes
    ("bf16", 64, 64, 64, 512, 17, 34, W.MAMBA2),    # L 17: ll_lambda_mlp first
    ("bf16", 128, 128, 64, 512, 10, 20, W.MAMBA2),  # d = 128: ll_lambda_mlp first
    ("f32", 32, 32, 32, 512, 10, 20, W.MAMBA2),     # fp32: ll_lambda_mlp first
]


def fused_case(io, dk, dv, C, T, L, hidden, rule, B=1, H=3):
    w = W.Workload("fused mlp", rule, B, H, T, dk, dv, L, C, io, 300 + dk + dv + T % 97 + L)
    x = W.prefill_inputs(w)
    m = W.lambda_mlp_inputs((B, T, H), L, hidden, seed=w.seed)
    return w, x, m


def run_both(w, x, m, rule_code):
    d, md = to_dev(x), to_dev(m)
    o_fused = F.attn_fwd_lambda_mlp(d["q"], d["k"], d["v"], d["log_gate"], md["d"], md["w1"], md["w2"], md["bias"],
                                    d.get("beta"), C=w.C, rule=rule_code)
    lam = F.lambda_mlp(md["d"], md["w1"], md["w2"], md["bias"])
    o_two = F.attn_fwd(d["q"], d["k"], d["v"], d["log_gate"], lam, d.get("beta"), C=w.C, L=w.L, rule=rule_code)
    torch.cuda.synchronize()
    return o_fused, o_two


@pytest.mark.parametrize("io,dk,dv,C,T,L,hidden,rule", CASES)
def test_fused_mlp_prefill(io, dk, dv, C, T, L, hidden, rule):
    w, x, m = fused_case(io, dk, dv, C, T, L, hidden, rule)
    rule_code = F.LL_MAMBA2 if rule == W.MAMBA2 else F.LL_GATED_DELTANET
    o_fused, o_two = run_both(w, x, m, rule_code)
    same = torch.equal(o_fused, o_two)
    two_err = rel_err(np32(o_fused), np32(o_two))
    lam_ref = oracle.lambda_mlp(np32(m["d"]), np32(m["w1"]), np32(m["w2"]), np32(m["bias"]))
    x["lam"] = torch.from_numpy(lam_ref.astype(np.float32))
    err = rel_err(np32(o_fused), oracle_prefill(x))
    say(f"[fused mlp] {io} dk{dk} dv{dv} C{C} T{T} L{L} hidden {hidden} rule {rule}: rel err {err:.3e} "
        f"(tol {TOL[io]:g}); against ll_lambda_mlp + ll_attn_fwd: equal {same}, rel diff {two_err:.3e}")
    assert same
    assert two_err <= TOL[io]
    assert err <= TOL[io]


def test_fused_mlp_16k_workload():
    """The 16K prefill (B2 H16 T16384 d64 bf16, 15 levels, chunk 64) with its level weights
    from the MLP (hidden 2L = 30), which the read makes itself: every output against
    ll_lambda_mlp + ll_attn_fwd (both in blocks of 16 chunks: bit for bit), and the last 256
    tokens of every head against the oracle's direct form."""
    w = W.WORKLOADS["prefill-16k"]
    x = W.prefill_inputs(w, parts=("q", "k", "v", "log_gate"))
    m = W.lambda_mlp_inputs((w.B, w.T, w.H), w.L, seed=w.seed)
    o_fused, o_two = run_both(w, x, m, F.LL_MAMBA2)
    two_err = rel_err(np32(o_fused), np32(o_two))
    say(f"[fused mlp] 16K workload: rel diff against ll_lambda_mlp + ll_attn_fwd {two_err:.3e}")
    assert torch.equal(o_fused, o_two)
    lam_ref = oracle.lambda_mlp(np32(m["d"]), np32(m["w1"]), np32(m["w2"]), np32(m["bias"]))
    x["lam"] = torch.from_numpy(lam_ref.astype(np.float32))
    t_range = (w.T - 256, w.T)
    ref = oracle_prefill(x, t_range=t_range)[:, t_range[0]:t_range[1]]
    err = rel_err(np32(o_fused)[:, t_range[0]:t_range[1]], ref)
    say(f"[fused mlp] 16K workload: last 256 tokens rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_fused_mlp_32k_far_nodes():
    """B1 H8 T32768 d64 bf16, 16 levels (the MLP's limit), hidden 2L: the read that makes the
    weights in blocks of 16 chunks with block indices up to 31 (a Fenwick node past the four held
    ones), against ll_lambda_mlp + ll_attn_fwd bit for bit."""
    w = W.Workload("fused mlp 32k", W.MAMBA2, 1, 8, 32768, 64, 64, 16, 64, "bf16", 11)
    x = W.prefill_inputs(w, parts=("q", "k", "v", "log_gate"))
    m = W.lambda_mlp_inputs((w.B, w.T, w.H), w.L, seed=w.seed)
    o_fused, o_two = run_both(w, x, m, F.LL_MAMBA2)
    say(f"[fused mlp] 32K, 16 levels: equal {torch.equal(o_fused, o_two)}")
    assert torch.isfinite(o_fused.float()).all()
    assert torch.equal(o_fused, o_two)
