"""GPU parity of the backward pass (ll_attn_bwd) against the oracle's
gradients from the definition (themselves pinned by central differences of the
forward oracle).  Every gradient tensor is compared element by element:
max|g - ref| / max|ref| <= 1e-4 (fp32 io), 2e-2 (bf16 io).

The cases cover one block per head (T = C P), several blocks (block-level
reverse buckets, a block count that is not a power of two), blocks of one and
two chunks, and the 2048-token bf16 shape the benchmark times (d 64, C 64,
12 levels), where the gate gradient's suffix sums run longest.
"""

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, np32, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # io, B, H, T, d, C, L, variant
    ("f32", 1, 2, 256, 16, 16, 9, "default"),
    ("f32", 2, 2, 192, 32, 64, 9, "slowdecay"),   # reversed reads padded to 256
    ("f32", 1, 2, 128, 64, 32, 8, "nodecay"),
    ("bf16", 2, 4, 512, 64, 64, 10, "default"),
    ("bf16", 1, 2, 320, 64, 64, 10, "slowdecay"),  # padded to 512
    ("bf16", 1, 2, 256, 128, 32, 9, "default"),
    ("f32", 1, 2, 1024, 32, 16, 11, "default"),     # 8 blocks of 8 chunks
    ("f32", 1, 3, 384, 16, 32, 10, "slowdecay"),    # 3 blocks of 4 chunks
    ("bf16", 2, 2, 384, 32, 64, 10, "default"),     # 3 blocks of 2 chunks
    ("bf16", 1, 2, 1536, 128, 32, 12, "slowdecay"), # 6 blocks of 8 chunks
    ("bf16", 1, 4, 2048, 64, 64, 12, "default"),    # 4 blocks of 8 chunks
]


@pytest.mark.parametrize("io,B,H,T,d,C,L,variant", CASES)
def test_bwd_matches_oracle(io, B, H, T, d, C, L, variant):
    w = W.Workload("bwd", W.MAMBA2, B, H, T, d, d, L, C, io, 200 + T + d)
    x = W.prefill_inputs(w, variant=variant)
    g = torch.Generator().manual_seed(300 + T + d)
    dO = torch.randn(B, T, H, d, generator=g).to(x["v"].dtype)
    dev = to_dev(x)
    dOd = dO.cuda()
    o = F.attn_fwd(dev["q"], dev["k"], dev["v"], dev["log_gate"], dev["lam"], C=C, L=L)
    grads = F.attn_bwd(dev["q"], dev["k"], dev["v"], dev["log_gate"], dev["lam"], o, dOd, C=C, L=L)
    torch.cuda.synchronize()
    ref = oracle.bwd_direct(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), np32(x["lam"]), np32(dO))
    errs = {}
    for name in ("dq", "dk", "dv", "dlambda", "dlog_gate"):
        tol = TOL[io]
        err = rel_err(np32(grads[name]), ref[name])
        say(f"[bwd] {io} B{B} H{H} T{T} d{d} C{C} {variant}: {name} rel err {err:.3e} (tol {tol:g})")
        errs[name] = err
    assert all(errs[n] <= TOL[io] for n in errs), errs
