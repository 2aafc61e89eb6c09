"""GPU check of ll_attn_fwd_noalloc, the allocation-free prefill: through the
C ABI, its outputs must equal those of ll_attn_fwd (same kernels, workspace
from the library's scratch array instead of the caller) on consecutive calls,
the second one smaller than the first, so that it runs over what the first
left in the scratch.  Bit-equality is asked for: both run the same kernels in
the same launch configuration."""

import pytest
import torch

import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from fenwick_tree_linear_amd.binding import io_code
from _parity import say, to_dev

pytestmark = pytest.mark.gpu


def run_both(w, want_state):
    x = to_dev(W.prefill_inputs(w))
    B, T, H, dk = x["k"].shape
    dv = x["v"].shape[-1]
    rule = F.LL_MAMBA2 if x.get("beta") is None else F.LL_GATED_DELTANET
    prob = F.LLProblem(B, T, H, dk, dv, w.L, w.C, io_code(x["k"].dtype), rule)
    ws = torch.empty(max(F.ll_attn_fwd_workspace_bytes(prob), 1), dtype=torch.uint8, device="cuda")
    o_ref = torch.empty(B, T, H, dv, dtype=x["v"].dtype, device="cuda")
    o_na = torch.full_like(o_ref, float("nan"))
    n_state = F.ll_decode_state_bytes(B, H, dk, dv, w.L) // 4
    s_ref = torch.empty(n_state, dtype=torch.float32, device="cuda") if want_state else None
    s_na = torch.full((n_state,), float("nan"), dtype=torch.float32, device="cuda") if want_state else None
    args = (x["q"], x["k"], x["v"], x["log_gate"], x["lam"], x.get("beta"))
    F.ll_attn_fwd(prob, *args, o_ref, s_ref, ws, ws.numel())
    F.ll_attn_fwd_noalloc(prob, *args, o_na, s_na)
    torch.cuda.synchronize()
    return o_ref, o_na, s_ref, s_na


def check(name, ref, got):
    diff = (ref.float() - got.float()).abs().max().item()
    say(f"[noalloc] {name}: max |noalloc - ll_attn_fwd| = {diff:.3e}, bit-equal {torch.equal(ref, got)}")
    assert torch.equal(ref, got), name


def test_noalloc_matches_ll_attn_fwd_on_consecutive_calls():
    # 1) the 16K-token prefill (25 MB of scratch), 2) a smaller one with state
    # export, run over the first call's scratch contents, 3) a Gated DeltaNet
    # prefill, whose row buffers also live in the scratch
    cases = [
        (W.WORKLOADS["prefill-16k"], False),
        (W.Workload("noalloc small", W.MAMBA2, 1, 3, 1536, 64, 64, 12, 64, "bf16", 71), True),
        (W.Workload("noalloc gdn", W.GATED_DELTANET, 1, 2, 512, 32, 32, 11, 32, "f32", 72), True),
    ]
    for w, want_state in cases:
        say(f"[noalloc] case {w.name}: B{w.B} H{w.H} T{w.T} d{w.dk} {w.io} C{w.C} L{w.L}")
        o_ref, o_na, s_ref, s_na = run_both(w, want_state)
        check(f"{w.name} o", o_ref, o_na)
        if want_state:
            check(f"{w.name} state", s_ref, s_na)
