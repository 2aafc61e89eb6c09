"""Shared helpers of the GPU parity tests (not collected by pytest).

The HIP path is always called through the C ABI (fenwick_tree_linear_amd.binding);
the oracle only ever receives inputs from fenwick_tree_linear_amd.workloads.
"""

import sys

import numpy as np
import torch

import oracle
import fenwick_tree_linear_amd as F

# max-abs error / max-abs reference, per io dtype
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np32(t):
    return None if t is None else t.detach().float().cpu().numpy()


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(ref).all()
    if not np.isfinite(gpu).all():
        return float("inf")
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


def to_dev(x, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in x.items()}


def gpu_prefill(x, C, L, want_output=True, want_state=False, dev_inputs=None):
    """Runs ll_attn_fwd on cuda copies of the inputs ``x``; returns numpy o
    (and the decode-layout state split into S_hat, sigma)."""
    d = dev_inputs if dev_inputs is not None else to_dev(x)
    rule = F.LL_MAMBA2 if d.get("beta") is None else F.LL_GATED_DELTANET
    res = F.attn_fwd(d["q"], d["k"], d["v"], d["log_gate"], d["lam"], d.get("beta"), C=C, L=L, rule=rule,
                     want_output=want_output, want_state=want_state)
    torch.cuda.synchronize()
    if want_state:
        o, st = res
        B, _, H, dk = d["k"].shape
        dv = d["v"].shape[-1]
        return (np32(o) if o is not None else None), split_state(st, B, H, L, dk, dv)
    return np32(res)


def split_state(flat, B, H, L, dk, dv):
    flat = flat.detach().cpu().numpy()
    n = B * H * L * dk * dv
    s_hat = flat[:n].reshape(B, H, L, dk, dv).astype(np.float64)
    sigma = flat[n:n + B * H * L].reshape(B, H, L).astype(np.float64)
    return s_hat, sigma


def true_state(s_hat, sigma):
    return np.exp(sigma)[..., None, None] * s_hat


def oracle_rule(x):
    return oracle.RULE_MAMBA2 if x.get("beta") is None else oracle.RULE_GDN


def oracle_prefill(x, heads=None, t_range=None):
    return oracle.fwd_direct(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["log_gate"]), np32(x["lam"]),
                             np32(x.get("beta")), rule=oracle_rule(x), heads=heads, t_range=t_range)
