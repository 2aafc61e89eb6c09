"""GPU parity of the level-weight MLP (ll_lambda_mlp) against the oracle, and
of a prefill whose level weights come from it.

ll_lambda_mlp computes softplus(d (W1 W2) + b) per row in fp32, the composite
W1 W2 first (no activation lies between the layers), the row product on the
matrix cores; the oracle computes the two layers as written, softplus((d W1) W2
+ b), in fp64 ("Adaptive memory decay for log-linear attention", section
"Method").  Tolerance: max|lambda - ref| / max|ref| <= 1e-5 (fp32 sums of at
most 64 products for the composite and 32 for the row, of O(1) terms, plus the
fp32 exponential and logarithm of softplus, stay well below it).
"""

import numpy as np
import pytest
import torch

import oracle
import fenwick_tree_linear_amd as F
from fenwick_tree_linear_amd import workloads as W
from _parity import TOL, gpu_prefill, np32, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

MLP_TOL = 1e-5


def ref_lambda(x):
    return oracle.lambda_mlp(np32(x["d"]), np32(x["w1"]), np32(x["w2"]), np32(x["bias"]))


def gpu_lambda(x):
    d = to_dev(x)
    lam = F.lambda_mlp(d["d"], d["w1"], d["w2"], d["bias"])
    torch.cuda.synchronize()
    return np32(lam)


# rows, L, hidden: every pair of level tiles (L <= 16, <= 32) and hidden tiles
# (<= 16, 32, 48, 64), ragged row counts (not a multiple of 64 or of 256)
SHAPES = [
    (1, 9, 18), (63, 9, 18), (64, 12, 24), (1000, 15, 30), (4097, 17, 34), (300, 24, 48), (129, 32, 64),
    (77, 5, 7), (50, 1, 1), (200, 16, 16), (200, 16, 17), (513, 31, 40), (255, 14, 60),
]


@pytest.mark.parametrize("rows,L,hidden", SHAPES)
def test_lambda_mlp_matches_oracle(rows, L, hidden):
    x = W.lambda_mlp_inputs((rows,), L, hidden, seed=rows + L)
    lam, ref = gpu_lambda(x), ref_lambda(x)
    err = rel_err(lam, ref)
    say(f"[lambda-mlp] rows {rows} L {L} hidden {hidden}: rel err {err:.3e} (tol {MLP_TOL:g})")
    assert err <= MLP_TOL
    assert (lam >= 0).all()


def test_lambda_mlp_large_preactivations():
    """|z| in the hundreds: softplus stays finite (z for large z, e^z for very
    negative z), no overflow in the exponential."""
    x = W.lambda_mlp_inputs((4, 96), 15, seed=5)
    x["d"] = x["d"] * 200.0
    lam, ref = gpu_lambda(x), ref_lambda(x)
    assert np.isfinite(lam).all()
    err = rel_err(lam, ref)
    say(f"[lambda-mlp] large pre-activations (max {ref.max():.1f}): rel err {err:.3e}")
    assert err <= MLP_TOL


def test_lambda_mlp_16k_workload_rows():
    """All 2 x 16384 x 16 rows of the 16K prefill at its 15 levels (hidden 30)."""
    w = W.WORKLOADS["prefill-16k"]
    x = W.lambda_mlp_inputs((w.B, w.T, w.H), w.L, seed=w.seed)
    lam, ref = gpu_lambda(x), ref_lambda(x)
    err = rel_err(lam, ref)
    say(f"[lambda-mlp] 16K workload rows: rel err {err:.3e}")
    assert err <= MLP_TOL


@pytest.mark.parametrize("io,d,C", [("bf16", 64, 64), ("f32", 32, 16)])
def test_prefill_with_mlp_level_weights(io, d, C):
    """Level weights from the MLP feed ll_attn_fwd on the GPU; the oracle runs
    its own MLP and its direct form on the same inputs."""
    w = W.Workload("mlp prefill", W.MAMBA2, 1, 4, 2048, d, d, 12, C, io, 21)
    x = W.prefill_inputs(w, parts=("q", "k", "v", "log_gate"))
    m = W.lambda_mlp_inputs((w.B, w.T, w.H), w.L, seed=21)
    dev = to_dev(x)
    md = to_dev(m)
    dev["lam"] = F.lambda_mlp(md["d"], md["w1"], md["w2"], md["bias"])
    o = gpu_prefill(None, C, w.L, dev_inputs=dev)
    x["lam"] = torch.from_numpy(ref_lambda(m).astype(np.float32))
    err = rel_err(o, oracle_prefill(x))
    say(f"[lambda-mlp] prefill {io} d{d} C{C} with MLP weights: rel err {err:.3e} (tol {TOL[io]:g})")
    assert err <= TOL[io]


def test_lambda_mlp_unaligned_rows():
    """Rows and weights not on 16-byte boundaries (views one float into larger
    buffers) take the 4-byte path and give the same values."""
    rows, L, hidden = 640, 15, 30
    x = W.lambda_mlp_inputs((rows,), L, hidden, seed=13)
    ref = ref_lambda(x)
    d = to_dev(x)
    buf = torch.empty(rows * L + 1, dtype=torch.float32, device="cuda")
    buf[1:] = d["d"].reshape(-1)
    din = buf[1:].view(rows, L)
    out = torch.empty(rows * L + 1, dtype=torch.float32, device="cuda")
    lam = F.lambda_mlp(din, d["w1"], d["w2"], d["bias"], out=out[1:].view(rows, L))
    torch.cuda.synchronize()
    err = rel_err(np32(lam), ref)
    say(f"[lambda-mlp] unaligned rows: rel err {err:.3e}")
    assert err <= MLP_TOL
    aligned = np32(F.lambda_mlp(d["d"], d["w1"], d["w2"], d["bias"]))
    assert np.array_equal(np32(lam), aligned)
