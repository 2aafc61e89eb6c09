"""Every output of the three large workloads against the oracle, element by
element, in the launch configuration the benchmark times:

  - the 16K-token prefill (B2 H16 T16384 d64 bf16, 15 levels, C=64): all
    524,288 token-heads against the oracle's recurrent form;
  - the decode workload (B64 H16 d64 bf16, 17 levels): the prefill's export
    of the 32768-token prefix against the oracle's bucket sums for all 1024
    heads, then all 512 decode steps of all heads against the oracle's
    recurrent step started from its own prefix states;
  - the Gated DeltaNet 8K prefill (B2 H16 T8192 d128 bf16, 14 levels, C=64):
    all 262,144 token-heads against the oracle's recurrent form.

The oracle's recurrent form is pinned to its direct form on the CPU
(tests/test_oracle_pins.py); the sampled direct-form windows of
test_gpu_prefill.py and test_gpu_gdn.py stay as a second check.  The metric is
max |gpu - ref| / max |ref| over all outputs of a workload, one line per
workload in the log.  Also here: the Gated DeltaNet special cases on the GPU
(beta == 0 writes nothing; a == 1, beta == 1 with one-hot keys keeps the last
value written under each key).
"""

import time

import numpy as np
import pytest
import torch

import oracle
from fenwick_tree_linear_amd import workloads as W
import fenwick_tree_linear_amd as F
from _parity import TOL, gpu_prefill, np32, rel_err, say, split_state, to_dev, true_state

pytestmark = pytest.mark.gpu


def recurrent_ref(x):
    rule = oracle.RULE_MAMBA2 if x.get("beta") is None else oracle.RULE_GDN
    return oracle.fwd_recurrent(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), np32(x["lam"]),
                                np32(x.get("beta")), rule=rule)


def test_prefill_16k_every_output():
    w = W.WORKLOADS["prefill-16k"]
    x = W.prefill_inputs(w)
    say(f"[full] {w.name}: GPU prefill")
    o = gpu_prefill(x, w.C, w.L)
    t0 = time.time()
    ref = recurrent_ref(x)
    say(f"[full] oracle recurrent form over {w.B * w.H} heads x {w.T} tokens in {time.time() - t0:.1f} s")
    assert np.isfinite(ref).all()
    err = rel_err(o, ref)
    say(f"[full] PARITY {w.name}: all {o.size} outputs, rel err {err:.3e} (tol {TOL['bf16']:g})")
    assert err <= TOL["bf16"]


def test_prefill_32k_far_nodes_every_output():
    """B1 H8 T32768 d64 bf16, 16 levels, C=64: blocks of 16 chunks (8 heads x 32 blocks keep every
    CU a block to read), so the block index J runs to 31 and its bit 4, past the four Fenwick
    nodes the read holds in registers, is read from the workspace at every chunk.  Every output
    against the oracle's recurrent form."""
    w = W.Workload("prefill 32k, far nodes", W.MAMBA2, 1, 8, 32768, 64, 64, 16, 64, "bf16", 7)
    x = W.prefill_inputs(w)
    o = gpu_prefill(x, w.C, w.L)
    ref = recurrent_ref(x)
    err = rel_err(o, ref)
    say(f"[full] PARITY {w.name}: all {o.size} outputs, rel err {err:.3e} (tol {TOL['bf16']:g})")
    assert err <= TOL["bf16"]


def test_gdn_8k_every_output():
    w = W.WORKLOADS["gdn-8k"]
    x = W.prefill_inputs(w)
    say(f"[full] {w.name}: GPU prefill")
    o = gpu_prefill(x, w.C, w.L)
    t0 = time.time()
    ref = recurrent_ref(x)
    say(f"[full] oracle recurrent form over {w.B * w.H} heads x {w.T} tokens in {time.time() - t0:.1f} s")
    assert np.isfinite(ref).all()
    err = rel_err(o, ref)
    say(f"[full] PARITY {w.name}: all {o.size} outputs, rel err {err:.3e} (tol {TOL['bf16']:g})")
    assert err <= TOL["bf16"]


def test_decode_32k_every_output():
    w = W.WORKLOADS["decode-32k"]
    B, H, L, d = w.B, w.H, w.L, w.dk
    say(f"[full] {w.name}: the 32768-token prefix on the GPU, exported")
    pre = W.prefill_inputs(w, device="cuda", parts=("k", "v", "log_gate"))
    _, state = F.attn_fwd(None, pre["k"], pre["v"], pre["log_gate"], None, C=64, L=L, want_output=False,
                          want_state=True)
    torch.cuda.synchronize()
    s_hat, sigma = split_state(state, B, H, L, d, d)
    gpu_prefix = true_state(s_hat, sigma)
    del s_hat, sigma

    # the oracle's prefix states, one batch entry (16 heads) per call
    t0 = time.time()
    st = np.zeros((B, H, L, d, d), dtype=np.float64)
    for b in range(B):
        sl = lambda n: np32(pre[n][b:b + 1])
        st[b] = oracle.state_direct(sl("k"), sl("v"), sl("log_gate"), L)[0]
    say(f"[full] oracle prefix states of {B * H} heads in {time.time() - t0:.1f} s")
    del pre
    live = [lv for lv in range(1, L) if (w.T >> (lv - 1)) & 1]
    err = rel_err(gpu_prefix[:, :, live], st[:, :, live])
    say(f"[full] PARITY {w.name} prefix export: levels {live} of all {B * H} heads, rel err {err:.3e} "
        f"(tol {TOL['bf16']:g})")
    assert err <= TOL["bf16"]
    del gpu_prefix

    steps = W.decode_inputs(w)
    dev = to_dev(steps)
    o_all = torch.empty(w.steps, B, H, d, dtype=torch.bfloat16, device="cuda")
    for i in range(w.steps):
        F.ll_decode_step(B, H, d, d, L, F.LL_BF16, F.LL_MAMBA2, w.T + i, dev["q"][i], dev["k"][i], dev["v"][i],
                         dev["log_gate"][i], dev["lam"][i], None, o_all[i], state)
    torch.cuda.synchronize()
    o_all = np32(o_all)

    t0 = time.time()
    ref = np.empty((w.steps, B, H, d), dtype=np.float64)
    for i in range(w.steps):
        sl = lambda n: np32(steps[n][i])
        ref[i] = oracle.decode_step(st, w.T + i, sl("q"), sl("k"), sl("v"), sl("log_gate"), sl("lam"))
    say(f"[full] oracle decode of {w.steps} steps x {B * H} heads in {time.time() - t0:.1f} s")
    err = rel_err(o_all, ref)
    say(f"[full] PARITY {w.name}: all {o_all.size} outputs of {w.steps} steps, rel err {err:.3e} "
        f"(tol {TOL['bf16']:g})")
    assert err <= TOL["bf16"]


# ----------------------------------------------------- Gated DeltaNet cases

@pytest.mark.parametrize("io,d,C", [("bf16", 64, 64), ("f32", 32, 16), ("bf16", 128, 64)])
def test_gdn_zero_beta_writes_nothing(io, d, C):
    w = W.Workload("gdn beta 0", W.GATED_DELTANET, 2, 3, 512, d, d, 11, C, io, 81 + d)
    x = W.prefill_inputs(w)
    x["beta"] = torch.zeros_like(x["beta"])
    o, (s_hat, sigma) = gpu_prefill(x, C, w.L, want_state=True)
    say(f"[gdn] beta == 0 {io} d{d}: max |o| = {np.max(np.abs(o)):.3e}, max |state| = "
        f"{np.max(np.abs(true_state(s_hat, sigma))):.3e}")
    assert np.max(np.abs(o)) == 0.0
    assert np.max(np.abs(true_state(s_hat, sigma))) == 0.0


@pytest.mark.parametrize("io,d,C", [("f32", 32, 16), ("f32", 64, 64), ("bf16", 64, 64)])
def test_gdn_one_hot_keys_keep_last_value(io, d, C):
    """a == 1, beta == 1, lambda == 1 and keys drawn from the one-hot basis:
    the delta rule overwrites the slot of each key, so with q_t = e_j the read
    returns the last value written under key j up to t (zero before the first),
    and the exported state holds row j = that value."""
    T, L, H = 256, 10, 2
    rng = np.random.default_rng(5 + d)
    keys = rng.integers(0, d, (1, T, H))
    qsel = rng.integers(0, d, (1, T, H))
    eye = np.eye(d, dtype=np.float32)
    x = {
        "q": torch.from_numpy(eye[qsel]),
        "k": torch.from_numpy(eye[keys]),
        "v": torch.from_numpy(rng.standard_normal((1, T, H, d)).astype(np.float32)),
        "log_gate": torch.zeros(1, T, H),
        "lam": torch.ones(1, T, H, L),
        "beta": torch.ones(1, T, H),
    }
    if io == "bf16":
        for n in ("q", "k", "v"):
            x[n] = x[n].to(torch.bfloat16)
    v = np32(x["v"])
    ref = np.zeros((1, T, H, d))
    rows = np.zeros((H, d, d))
    for h in range(H):
        for t in range(T):
            rows[h, keys[0, t, h]] = v[0, t, h]
            ref[0, t, h] = rows[h, qsel[0, t, h]]
    o, (s_hat, sigma) = gpu_prefill(x, C, L, want_state=True)
    err = rel_err(o, ref)
    total = true_state(s_hat, sigma).sum(axis=2)[0]  # the plain state: the sum of the levels
    serr = rel_err(total, rows)
    say(f"[gdn] one-hot keys {io} d{d} C{C}: o rel err {err:.3e}, state rel err {serr:.3e} (tol {TOL[io]:g})")
    assert err <= TOL[io] and serr <= TOL[io]
