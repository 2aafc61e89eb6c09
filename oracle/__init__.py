"""CPU oracle for the log-linear (Fenwick-tree) attention forward pass.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``fenwick_tree_linear_amd``) never imports this package and shares no code
with it.

The arithmetic lives in ``llref.c`` (plain C, fp64, OpenMP over heads); this
module builds it with gcc and wraps it for numpy arrays.  Every function states
the passage it evaluates: of the "Log-Linear Attention" page (technical
summary, section 2) for the attention itself, of the "Adaptive memory decay for
log-linear attention" page (section "Method") for the level-weight MLP, of the
curvature-conditioned query page (section 2, "Mechanism") for the query
contraction.  The
pins that tie it to the pages and to the mathematics are in
``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "llref.c")
_LIB = os.path.join(_HERE, "libllref.so")

RULE_MAMBA2 = 0
RULE_GDN = 1

_ERRORS = {-1: "inconsistent arguments", -2: "too few levels for the positions", -3: "out of memory"}


# x86-64-v3 (AVX2, FMA) runs on every host these tests meet and lets gcc
# vectorise the fp64 loops; -std=c11 keeps floating-point contraction off, so
# the results are the same bit for bit as an unvectorised build.
PORTABLE_FLAGS = ("-O3", "-march=x86-64-v3")


def build(out: str = _LIB, extra_flags: tuple[str, ...] = (), opt_flags: tuple[str, ...] = PORTABLE_FLAGS) -> str:
    """Compile ``llref.c`` into a shared library with gcc and return its path."""
    cmd = ["gcc", *opt_flags, "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", out + ".tmp", _SRC, "-lm",
           *extra_flags]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library, building it first when it is missing or stale."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int, ctypes.c_int64
    lib.llref_threads.argtypes = []
    lib.llref_threads.restype = i32
    lib.llref_level.argtypes = [i64, i64]
    lib.llref_level.restype = i32
    lib.llref_levels_row.argtypes = [i64, P]
    lib.llref_levels_row.restype = None
    lib.llref_fwd_direct.argtypes = [i32] * 7 + [P] * 6 + [i32, P, i64, i64, P]
    lib.llref_fwd_direct.restype = i32
    lib.llref_state_direct.argtypes = [i32] * 7 + [P] * 4 + [i32, P, P]
    lib.llref_state_direct.restype = i32
    lib.llref_fwd_recurrent.argtypes = [i32] * 7 + [P] * 6 + [i32, P, P, P]
    lib.llref_fwd_recurrent.restype = i32
    lib.llref_decode_step.argtypes = [i32] * 6 + [i64] + [P] * 8
    lib.llref_decode_step.restype = i32
    lib.llref_lambda_mlp.argtypes = [i64, i32, i32] + [P] * 5
    lib.llref_lambda_mlp.restype = i32
    lib.llref_ccq_query.argtypes = [i32] * 4 + [P] * 5
    lib.llref_ccq_query.restype = i32
    lib.llref_bwd_direct.argtypes = [i32] * 6 + [P] * 11
    lib.llref_bwd_direct.restype = i32
    return lib


def _f32(x):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _heads(heads):
    if heads is None:
        return 0, None
    h = np.ascontiguousarray(np.asarray(heads, dtype=np.int32).reshape(-1, 2))
    return h.shape[0], h


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"{what}: {_ERRORS.get(rc, rc)}")


def threads(lib=None) -> int:
    """OpenMP threads the oracle's parallel loops use (over heads)."""
    return (lib or load()).llref_threads()


def level(t: int, s: int, lib=None) -> int:
    """Fenwick level of source ``s`` seen from position ``t`` (section 2.2)."""
    return (lib or load()).llref_level(t, s)


def levels_row(t: int, lib=None) -> np.ndarray:
    """``[level(t, s) for s in 0..t]`` as an int32 array."""
    out = np.empty(t + 1, dtype=np.int32)
    (lib or load()).llref_levels_row(t, _ptr(out))
    return out


def fwd_direct(q, k, v, log_gate, lam, beta=None, rule=RULE_MAMBA2, heads=None, t_range=None,
               lib=None) -> np.ndarray:
    """Direct O(T^2) masked form (section 2.2/2.3), fp64 output [B,T,H,dv].

    ``heads`` (pairs b,h) and ``t_range`` (lo, hi) restrict what is computed;
    rows not computed are NaN.
    """
    q, k, v, g, lam, beta = map(_f32, (q, k, v, log_gate, lam, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    lo, hi = t_range if t_range is not None else (0, T)
    nh, hs = _heads(heads)
    o = np.full((B, T, H, dv), np.nan, dtype=np.float64)
    rc = (lib or load()).llref_fwd_direct(B, T, H, dk, dv, L, rule, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                          _ptr(lam), _ptr(beta), nh, _ptr(hs), lo, hi, _ptr(o))
    _check(rc, "llref_fwd_direct")
    return o


def state_direct(k, v, log_gate, L, beta=None, rule=RULE_MAMBA2, heads=None, lib=None) -> np.ndarray:
    """Per-level states of the prefix [0,T) from the bucket sums (section 2.2).

    Returns fp64 [B,H,L,dk,dv], decayed through the last token.
    """
    k, v, g, beta = map(_f32, (k, v, log_gate, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    nh, hs = _heads(heads)
    st = np.zeros((B, H, L, dk, dv), dtype=np.float64)
    rc = (lib or load()).llref_state_direct(B, T, H, dk, dv, L, rule, _ptr(k), _ptr(v), _ptr(g),
                                            _ptr(beta), nh, _ptr(hs), _ptr(st))
    _check(rc, "llref_state_direct")
    return st


def fwd_recurrent(q, k, v, log_gate, lam, beta=None, rule=RULE_MAMBA2, heads=None, want_state=False,
                  lib=None):
    """Recurrent O(T log T) form (section 2.3).

    Returns ``o`` (fp64 [B,T,H,dv], NaN for heads not computed), and the
    exported per-level states [B,H,L,dk,dv] when ``want_state``.
    """
    q, k, v, g, lam, beta = map(_f32, (q, k, v, log_gate, lam, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    nh, hs = _heads(heads)
    o = np.full((B, T, H, dv), np.nan, dtype=np.float64)
    st = np.zeros((B, H, L, dk, dv), dtype=np.float64) if want_state else None
    rc = (lib or load()).llref_fwd_recurrent(B, T, H, dk, dv, L, rule, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                             _ptr(lam), _ptr(beta), nh, _ptr(hs), _ptr(o), _ptr(st))
    _check(rc, "llref_fwd_recurrent")
    return (o, st) if want_state else o


def decode_step(state, pos, q, k, v, log_gate, lam, beta=None, rule=RULE_MAMBA2, lib=None) -> np.ndarray:
    """One recurrent step at ``pos`` (section 2.3), updating ``state`` in place.

    ``state`` is fp64 [B,H,L,dk,dv] holding the true per-level states of
    [0,pos); inputs drop the T axis.  Returns o fp64 [B,H,dv].
    """
    assert state.dtype == np.float64 and state.flags["C_CONTIGUOUS"]
    q, k, v, g, lam, beta = map(_f32, (q, k, v, log_gate, lam, beta))
    B, H, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    o = np.zeros((B, H, dv), dtype=np.float64)
    rc = (lib or load()).llref_decode_step(B, H, dk, dv, L, rule, pos, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _ptr(lam), _ptr(beta), _ptr(o), _ptr(state))
    _check(rc, "llref_decode_step")
    return o


def lambda_mlp(d, w1, w2, bias, lib=None) -> np.ndarray:
    """Level weights from the adaptive-decay MLP ("Adaptive memory decay for
    log-linear attention", section "Method", LambdaMLPSoftplus):
    ``lambda = softplus((d W1) W2 + b)`` per token and head, fp64.

    ``d`` [..., L] (any leading axes), ``w1`` [L, hidden], ``w2`` [hidden, L],
    ``bias`` [L]; returns lambda with the shape of ``d``.
    """
    d, w1, w2, bias = map(_f32, (d, w1, w2, bias))
    L = d.shape[-1]
    hidden = w1.shape[1]
    if w1.shape != (L, hidden) or w2.shape != (hidden, L) or bias.shape != (L,):
        raise ValueError("lambda_mlp: inconsistent arguments")
    rows = d.size // L
    lam = np.empty(d.shape, dtype=np.float64)
    rc = (lib or load()).llref_lambda_mlp(rows, L, hidden, _ptr(d), _ptr(w1), _ptr(w2), _ptr(bias), _ptr(lam))
    _check(rc, "llref_lambda_mlp")
    return lam


def ccq_query(q, k, w, b, lib=None) -> np.ndarray:
    """Curvature-conditioned query (the curvature-conditioned query page,
    section 2, "Mechanism"): q_clean = q_t - sigmoid(w_h . q_t + b_h) Sigma_t q_t
    with Sigma_t the plain covariance of keys 0..t, per token and head, fp64.

    ``q``, ``k`` [B,T,H,dk], ``w`` [H,dk], ``b`` [H]; returns q_clean [B,T,H,dk].
    """
    q, k, w, b = map(_f32, (q, k, w, b))
    B, T, H, dk = q.shape
    if k.shape != q.shape or w.shape != (H, dk) or b.shape != (H,):
        raise ValueError("ccq_query: inconsistent arguments")
    out = np.empty(q.shape, dtype=np.float64)
    _check((lib or load()).llref_ccq_query(B, T, H, dk, _ptr(q), _ptr(k), _ptr(w), _ptr(b), _ptr(out)),
           "llref_ccq_query")
    return out


def bwd_direct(q, k, v, log_gate, lam, dO, lib=None) -> dict:
    """Gradients of the Mamba-2 log-linear read ("Log-Linear Attention",
    sections 2.2-2.3, masked form) for a loss with gradient dO at o, from the
    definition term by term, fp64.  Returns dq, dk, dv, dlog_gate, dlambda."""
    q, k, v, g, lam, dO = map(_f32, (q, k, v, log_gate, lam, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    out = dict(dq=np.empty((B, T, H, dk)), dk=np.empty((B, T, H, dk)), dv=np.empty((B, T, H, dv)),
               dlog_gate=np.empty((B, T, H)), dlambda=np.empty((B, T, H, L)))
    rc = (lib or load()).llref_bwd_direct(B, T, H, dk, dv, L, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(lam),
                                          _ptr(dO), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                          _ptr(out["dlog_gate"]), _ptr(out["dlambda"]))
    _check(rc, "llref_bwd_direct")
    return out
