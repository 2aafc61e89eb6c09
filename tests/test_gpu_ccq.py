"""GPU parity of the curvature-conditioned query (ll_ccq_query) against the
oracle, and of a prefill that reads with it.

Keys get one crowded direction per head (with_dense_key_direction), so the
contraction moves the queries by much more than the tolerance; the tests check
that as well.  Tolerance: max|x - ref| / max|ref| <= 1e-4 (fp32 io), 2e-2
(bf16 io).
"""

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, gpu_prefill, np32, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [
    # io, B, H, T, d
    ("f32", 1, 2, 256, 16),
    ("f32", 2, 2, 48, 32),     # chunks of 16
    ("f32", 1, 3, 512, 64),    # chunks of 32 (tile limit)
    ("bf16", 2, 4, 2048, 64),
    ("bf16", 1, 2, 96, 32),    # chunks of 32
    ("bf16", 1, 2, 1024, 128),
    ("f32", 1, 2, 256, 128),   # four 16-byte loads a tensor, two rows each
    ("bf16", 2, 3, 128, 16),   # two lanes a row: a quarter of the lanes hold rows
]


def inputs(io, B, H, T, d, seed):
    w = W.Workload("ccq", W.MAMBA2, B, H, T, d, d, W.levels_for(T), 16, io, seed)
    x = W.prefill_inputs(w)
    x["k"] = W.with_dense_key_direction(x["k"], seed=seed)
    g = W.ccq_inputs(H, d, seed=seed)
    return w, x, g


@pytest.mark.parametrize("io,B,H,T,d", SHAPES)
def test_ccq_query_matches_oracle(io, B, H, T, d):
    w, x, g = inputs(io, B, H, T, d, 50 + T + d)
    dev, gd = to_dev(x), to_dev(g)
    qc = np32(F.ccq_query(dev["q"], dev["k"], gd["w"], gd["b"]))
    torch.cuda.synchronize()
    ref = oracle.ccq_query(np32(x["q"]), np32(x["k"]), np32(g["w"]), np32(g["b"]))
    err = rel_err(qc, ref)
    moved = rel_err(np32(x["q"]), ref)
    say(f"[ccq] {io} B{B} H{H} T{T} d{d}: rel err {err:.3e} (tol {TOL[io]:g}); contraction moves q by {moved:.2e}")
    assert err <= TOL[io]
    assert moved > 10 * TOL[io]


def test_ccq_in_place():
    """q_clean may be q itself."""
    w, x, g = inputs("bf16", 1, 2, 512, 64, 77)
    dev, gd = to_dev(x), to_dev(g)
    out = F.ccq_query(dev["q"], dev["k"], gd["w"], gd["b"])
    q2 = dev["q"].clone()
    F.ccq_query(q2, dev["k"], gd["w"], gd["b"], out=q2)
    torch.cuda.synchronize()
    assert torch.equal(out, q2)


@pytest.mark.parametrize("io,d,C", [("bf16", 64, 64), ("f32", 32, 32)])
def test_prefill_reads_with_the_contracted_query(io, d, C):
    """q_clean from the GPU feeds ll_attn_fwd; the oracle contracts its own
    queries and runs its direct form."""
    w, x, g = inputs(io, 1, 3, 1024, d, 88 + d)
    dev, gd = to_dev(x), to_dev(g)
    dev["q"] = F.ccq_query(dev["q"], dev["k"], gd["w"], gd["b"])
    o = gpu_prefill(None, C, w.L, dev_inputs=dev)
    xr = dict(x)
    xr["q"] = torch.from_numpy(oracle.ccq_query(np32(x["q"]), np32(x["k"]), np32(g["w"]), np32(g["b"]))
                               .astype(np.float32))
    err = rel_err(o, oracle_prefill(xr))
    say(f"[ccq] prefill {io} d{d} with contracted queries: rel err {err:.3e} (tol {TOL[io]:g})")
    assert err <= TOL[io]


def test_ccq_16k_every_output():
    """The 16K workload the benchmark times (B2 H16 T16384 d64 bf16, chunks of
    64; the all-ones prefill then has 15 levels): every output against the
    oracle, which runs the whole batch from its fp64 running sums."""
    w = W.WORKLOADS["prefill-16k"]
    x = W.prefill_inputs(w)
    g = W.ccq_inputs(w.H, w.dk, seed=w.seed)
    dev, gd = to_dev(x), to_dev(g)
    qc = np32(F.ccq_query(dev["q"], dev["k"], gd["w"], gd["b"]))
    torch.cuda.synchronize()
    ref = oracle.ccq_query(np32(x["q"]), np32(x["k"]), np32(g["w"]), np32(g["b"]))
    err = rel_err(qc, ref)
    moved = rel_err(np32(x["q"]), ref)
    say(f"[ccq] 16K workload, every output: rel err {err:.3e} (tol {TOL['bf16']:g}); contraction moves q by "
        f"{moved:.2e}")
    assert err <= TOL["bf16"]
