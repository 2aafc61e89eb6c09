"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of the oracle's C source (a
dropped term, a wrong sign, an index off by one, a transposed operand), builds
it on the CPU, and checks that at least one pin rejects it; the unmodified
source must pass every pin.  Nothing here touches the GPU path.
"""

import ctypes
import math
import os
import subprocess

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "llref.c")

# (name, original text, planted text)
MUTANTS = [
    ("level-0 dropped", "if (s == t) return 0;", "if (s == t) return 1;"),
    ("bucket level off by one", "if (s >= end - size) return floor_log2(size) + 1;",
     "if (s >= end - size) return floor_log2(size);"),
    ("largest bucket peeled first", "int64_t size = end & (-end);",
     "int64_t size = (int64_t)1 << floor_log2(end);"),
    ("own gate decays own write", "double logw = 0.0; /* sum_{r=s+1}^{t} log a_r */",
     "double logw = log_gate[ix_tok(&d, b, t, h)];"),
    ("decay sign flipped", "double a = exp(log_a);", "double a = exp(-log_a);"),
    ("read uses transposed state", "r += S[l * per_level + (size_t)i * dv + j] * (double)qt[i];",
     "r += S[l * per_level + (size_t)j * dk + i] * (double)qt[i];"),
    ("merge into wrong level", "double *dst = S + (size_t)(c + 1) * per_level;",
     "double *dst = S + (size_t)(c > 0 ? c : 1) * per_level;"),
    ("gdn beta dropped", "w[j] = bt * ((double)vt[j] - acc);", "w[j] = ((double)vt[j] - acc);"),
    ("gdn u ignores decay", "double w = exp(logw) * dot_f(kt, ks, d->dk);", "double w = dot_f(kt, ks, d->dk);"),
    ("state decayed one token too far", "double logw = 0.0; /* sum_{r=s+1}^{T-1} log a_r */",
     "double logw = log_gate[ix_tok(&d, b, T - 1, h)];"),
    ("mlp W1 read transposed", "acc += (double)dr[m] * (double)w1[(size_t)m * hidden + j];",
     "acc += (double)dr[m] * (double)w1[(size_t)j * L + m];"),
    ("mlp bias dropped", "double z = (double)bias[l];", "double z = 0.0;"),
    ("mlp hidden layer activated", "h[j] = acc;", "h[j] = acc > 0.0 ? acc : 0.0;"),
    ("mlp softplus replaced by exp", "lambda[r * L + l] = (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));",
     "lambda[r * L + l] = exp(z);"),
    ("ccq mean term dropped", "sig[(size_t)i * dk + j] = kk[(size_t)i * dk + j] / n - (ksum[i] / n) * (ksum[j] / n);",
     "sig[(size_t)i * dk + j] = kk[(size_t)i * dk + j] / n;"),
    ("ccq covariance over t, not t + 1", "const double n = (double)(t + 1);", "const double n = (double)(t > 0 ? t : 1);"),
    ("ccq gate sign flipped", "const double gamma = 1.0 / (1.0 + exp(-z));", "const double gamma = 1.0 / (1.0 + exp(z));"),
    ("ccq query expanded, not contracted", "q_clean[row * dk + i] = qt[i] - gamma * sq;",
     "q_clean[row * dk + i] = qt[i] + gamma * sq;"),
    ("bwd dk without the level weight", "dk_out[is * dk + i] += lam * w * A * qt[i];",
     "dk_out[is * dk + i] += w * A * qt[i];"),
    ("bwd gate gradient with the wrong sign at the source", "dG[s] -= lam * w * P * A;", "dG[s] += lam * w * P * A;"),
    ("bwd gate gradient summed forward", "for (int64_t r = T - 1; r >= 0; r--) {",
     "for (int64_t r = 0; r < T; r++) {"),
]


def _inputs(T, L, gdn, seed=1):
    rng = np.random.default_rng(seed)
    B, H, dk, dv = 1, 2, 3, 5
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    if gdn:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    g = (-rng.uniform(0.001, 0.3, (B, T, H))).astype(np.float32)
    lam = np.log1p(np.exp(rng.normal(0.54, 0.5, (B, T, H, L)))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    return q, k, v, g, lam, beta


def _xor_level(t, s):
    return (t ^ s).bit_length()


def pin_failures(lib):
    """Run a compact set of the pins against ``lib``; return the names that fail."""
    fails = []

    # hand-worked partition of [0,13) and the XOR characterisation
    if list(oracle.levels_row(13, lib=lib)) != [4] * 8 + [3] * 4 + [1, 0]:
        fails.append("partition")

    T, L = 29, 6
    for gdn in (False, True):
        rule = oracle.RULE_GDN if gdn else oracle.RULE_MAMBA2
        q, k, v, g, lam, beta = _inputs(T, L, gdn)
        beta_arg = beta if gdn else None
        # lambda == 1: textbook (gated) linear attention / gated delta rule
        ones = np.ones_like(lam)
        ref = np.zeros((1, T, 2, 5))
        for h in range(2):
            S = np.zeros((3, 5))
            for t in range(T):
                kt = k[0, t, h].astype(np.float64)
                vt = v[0, t, h].astype(np.float64)
                a = math.exp(float(g[0, t, h]))
                if gdn:
                    bt = float(beta[0, t, h])
                    S = a * (np.eye(3) - bt * np.outer(kt, kt)) @ S + bt * np.outer(kt, vt)
                else:
                    S = a * S + np.outer(kt, vt)
                ref[0, t, h] = S.T @ q[0, t, h].astype(np.float64)
        for form in (oracle.fwd_direct, oracle.fwd_recurrent):
            o = form(q, k, v, g, ones, beta_arg, rule=rule, lib=lib)
            if not np.allclose(o, ref, rtol=1e-10, atol=1e-10):
                fails.append(f"textbook-{form.__name__}-{rule}")
        # two independent forms agree with random lambda
        a = oracle.fwd_direct(q, k, v, g, lam, beta_arg, rule=rule, lib=lib)
        b = oracle.fwd_recurrent(q, k, v, g, lam, beta_arg, rule=rule, lib=lib)
        if not np.allclose(a, b, rtol=1e-10, atol=1e-10):
            fails.append(f"direct-vs-recurrent-{rule}")
        # decode from the empty state reproduces the prefill outputs
        st = np.zeros((1, 2, L, 3, 5))
        for t in range(T):
            o = oracle.decode_step(st, t, q[:, t], k[:, t], v[:, t], g[:, t], lam[:, t],
                                   beta[:, t] if gdn else None, rule=rule, lib=lib)
            if not np.allclose(o, a[:, t], rtol=1e-10, atol=1e-10):
                fails.append(f"decode-{rule}")
                break

    # one-hot lambda at each level against brute force over XOR buckets,
    # and the exported state against bucket sums
    q, k, v, g, lam, _ = _inputs(T, L, False)
    cum = np.cumsum(g.astype(np.float64), axis=1)
    for level in range(L):
        lam1 = np.zeros_like(lam)
        lam1[..., level] = 1.0
        o = oracle.fwd_direct(q, k, v, g, lam1, lib=lib)
        ref = np.zeros_like(o)
        for h in range(2):
            for t in range(T):
                for s in range(t + 1):
                    if _xor_level(t, s) == level:
                        w = math.exp(cum[0, t, h] - cum[0, s, h]) * float(
                            q[0, t, h].astype(np.float64) @ k[0, s, h].astype(np.float64))
                        ref[0, t, h] += w * v[0, s, h].astype(np.float64)
        if not np.allclose(o, ref, rtol=1e-10, atol=1e-10):
            fails.append(f"one-hot-{level}")
    st = oracle.state_direct(k, v, g, L, lib=lib)
    ref = np.zeros_like(st)
    for h in range(2):
        for s in range(T):
            ref[0, h, _xor_level(T, s)] += math.exp(cum[0, T - 1, h] - cum[0, s, h]) * np.outer(
                k[0, s, h].astype(np.float64), v[0, s, h].astype(np.float64))
    if not np.allclose(st, ref, rtol=1e-10, atol=1e-10):
        fails.append("state")

    # the level-weight MLP: a hand-worked case, the identity special case and
    # linearity of the pre-activation
    d = np.array([[1.0, 2.0]])
    w1 = np.array([[1, 0, 2, -1], [0, 1, -1, 1]], dtype=np.float64)
    w2 = np.array([[1, 0], [-1, 0], [5, 7], [1, 10]], dtype=np.float64)
    lam = oracle.lambda_mlp(d, w1, w2, np.array([0.0, 20.0]), lib=lib)
    if not (abs(lam[0, 0] - math.log(2.0)) < 1e-15 and abs(lam[0, 1] - 30.0) < 1e-12):
        fails.append("mlp-hand")
    x = np.array([[-3.0, -0.5, 0.0, 0.5, 3.0]])
    if not np.allclose(oracle.lambda_mlp(x, np.eye(5), np.eye(5), np.zeros(5), lib=lib), np.logaddexp(0.0, x),
                       rtol=1e-14, atol=0):
        fails.append("mlp-identity")
    rng = np.random.default_rng(2)
    w1 = rng.standard_normal((3, 6)).astype(np.float32)
    w2 = rng.standard_normal((6, 3)).astype(np.float32)
    b = rng.standard_normal(3).astype(np.float32)
    d1 = rng.standard_normal((4, 3)).astype(np.float32)
    pre1 = np.log(np.expm1(oracle.lambda_mlp(d1, w1, w2, b, lib=lib))) - b
    pre2 = np.log(np.expm1(oracle.lambda_mlp(-d1, w1, w2, b, lib=lib))) - b
    if not np.allclose(pre1, -pre2, atol=1e-8):
        fails.append("mlp-linear")

    # the curvature-conditioned query: numpy's population covariance, and a
    # hand-worked two-token case
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 6, 2, 3)).astype(np.float32)
    k = rng.standard_normal((1, 6, 2, 3)).astype(np.float32)
    w = rng.standard_normal((2, 3)).astype(np.float32)
    b = rng.standard_normal(2).astype(np.float32)
    qc = oracle.ccq_query(q, k, w, b, lib=lib)
    ref = _ccq_numpy(q, k, w, b)
    if not np.allclose(qc, ref, rtol=1e-10, atol=1e-12):
        fails.append("ccq-numpy")
    # the backward: central differences of the forward's loss on a few coordinates
    rng = np.random.default_rng(6)
    T, H, d, L = 10, 1, 2, 5
    xb = {n: rng.standard_normal((1, T, H, d)).astype(np.float32) for n in ("q", "k", "v")}
    xb["g"] = (-rng.uniform(0.01, 0.3, (1, T, H))).astype(np.float32)
    xb["lam"] = rng.uniform(0.5, 1.5, (1, T, H, L)).astype(np.float32)
    dO = rng.standard_normal((1, T, H, d)).astype(np.float32)
    gr = oracle.bwd_direct(xb["q"], xb["k"], xb["v"], xb["g"], xb["lam"], dO, lib=lib)

    def loss(x):
        return float(np.sum(oracle.fwd_direct(x["q"], x["k"], x["v"], x["g"], x["lam"], lib=lib) * dO))

    for name, key, idx in (("k", "dk", (0, 2, 0, 1)), ("g", "dlog_gate", (0, 3, 0)), ("g", "dlog_gate", (0, 7, 0)),
                           ("q", "dq", (0, 8, 0, 0)), ("v", "dv", (0, 1, 0, 1)), ("lam", "dlambda", (0, 9, 0, 2))):
        xp = {kk: vv.copy() for kk, vv in xb.items()}
        xm = {kk: vv.copy() for kk, vv in xb.items()}
        xp[name][idx] += np.float32(1e-3)
        xm[name][idx] -= np.float32(1e-3)
        fd = (loss(xp) - loss(xm)) / (float(xp[name][idx]) - float(xm[name][idx]))
        if abs(fd - gr[key][idx]) > 1e-6 * (1 + abs(fd)):
            fails.append("bwd-" + key)
            break
    qh, kh = _ccq_hand()
    if not np.allclose(oracle.ccq_query(qh, kh, np.zeros((1, 2)), np.zeros(1), lib=lib)[0, 1, 0], [1.0, 3.0],
                       atol=1e-14):
        fails.append("ccq-hand")
    return fails


def _ccq_numpy(q, k, w, b):
    """q - sigmoid(w.q + b) Cov(k_0..k_t) q with numpy's population covariance."""
    B, T, H, dk = q.shape
    out = np.zeros((B, T, H, dk))
    for bb in range(B):
        for h in range(H):
            for t in range(T):
                ks = k[bb, :t + 1, h].astype(np.float64)
                cov = np.cov(ks.T, bias=True).reshape(dk, dk) if t > 0 else np.zeros((dk, dk))
                qt = q[bb, t, h].astype(np.float64)
                g = 1.0 / (1.0 + math.exp(-(float(w[h].astype(np.float64) @ qt) + float(b[h]))))
                out[bb, t, h] = qt - g * (cov @ qt)
    return out


def _ccq_hand():
    """Keys (1, 0) then (-1, 0): at t = 1 the mean is 0 and the covariance
    diag(1, 0); with w = 0, b = 0 the gate is 1/2, so q = (2, 3) becomes (1, 3)."""
    q = np.array([[[[5.0, 5.0]], [[2.0, 3.0]]]], dtype=np.float32)
    k = np.array([[[[1.0, 0.0]], [[-1.0, 0.0]]]], dtype=np.float32)
    return q, k


def _build_variant(tmp_path, name, text):
    src = tmp_path / f"{name.replace(' ', '_')}.c"
    src.write_text(text)
    so = tmp_path / f"{name.replace(' ', '_')}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(src), "-lm"],
                   check=True)
    return oracle.load(str(so))


def test_unmodified_oracle_passes_every_pin(tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert pin_failures(_build_variant(tmp_path, "original", text)) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    lib = _build_variant(tmp_path, name, text.replace(old, new))
    try:
        fails = pin_failures(lib)
    except ValueError:
        fails = ["raised"]
    assert fails, f"no pin caught: {name}"
