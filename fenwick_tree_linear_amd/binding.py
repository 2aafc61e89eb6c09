"""ctypes binding of libllattn.so: argument marshalling only.

Every function named ``ll_*`` mirrors the C entry point of the same name in
``include/ll_attn.h``; tensors are passed as device pointers and the current
torch stream is passed as the hipStream.  Non-OK statuses raise ``LLError``
carrying ``ll_last_error()``.  The library is loaded on first use and its
absence is an error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

LL_F32, LL_BF16 = 0, 1
LL_MAMBA2, LL_GATED_DELTANET = 0, 1

_STATUS = {0: "LL_OK", -1: "LL_ERR_NULL", -2: "LL_ERR_SHAPE", -3: "LL_ERR_DTYPE", -4: "LL_ERR_UNSUPPORTED",
           -5: "LL_ERR_WORKSPACE", -6: "LL_ERR_POSITION", -7: "LL_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.environ.get("LLATTN_LIB") or os.path.join(_HERE, "libllattn.so")


class LLError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


class LLProblem(ctypes.Structure):
    """``ll_problem``: B, T, H, dk, dv, L, C, io, rule."""

    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int),
                ("dv", ctypes.c_int), ("L", ctypes.c_int), ("C", ctypes.c_int), ("io", ctypes.c_int),
                ("rule", ctypes.c_int)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libllattn.so (built by ``python -m fenwick_tree_linear_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fenwick_tree_linear_amd.build` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
    lib.ll_attn_fwd_workspace_bytes.argtypes = [ctypes.POINTER(LLProblem), ctypes.POINTER(sz)]
    lib.ll_attn_fwd.argtypes = [ctypes.POINTER(LLProblem), P, P, P, P, P, P, P, P, P, sz, P]
    lib.ll_decode_state_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.ll_decode_step.argtypes = [i32, i32, i32, i32, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P]
    lib.ll_last_error.argtypes = []
    lib.ll_last_error.restype = ctypes.c_char_p
    lib.ll_kernel_timing_enable.argtypes = [i32]
    lib.ll_kernel_timing_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int), i32, ctypes.POINTER(ctypes.c_int)]
    lib.ll_lambda_mlp.argtypes = [i64, i32, i32, P, P, P, P, P, P]
    lib.ll_attn_fwd_noalloc.argtypes = [ctypes.POINTER(LLProblem), P, P, P, P, P, P, P, P, P]
    lib.ll_attn_fwd_from_state.argtypes = [ctypes.POINTER(LLProblem), i64, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.ll_ccq_query_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.ll_ccq_query.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, sz, P]
    lib.ll_attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(LLProblem), ctypes.POINTER(sz)]
    lib.ll_attn_bwd.argtypes = [ctypes.POINTER(LLProblem)] + [P] * 13 + [sz, P]
    lib.ll_decode_step_ragged.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
    lib.ll_attn_fwd_lambda_mlp_workspace_bytes.argtypes = [ctypes.POINTER(LLProblem), i32, ctypes.POINTER(sz)]
    lib.ll_attn_fwd_lambda_mlp.argtypes = [ctypes.POINTER(LLProblem), P, P, P, P, P, i32, P, P, P, P, P, P, P, sz, P]
    for fn in ("ll_attn_fwd_workspace_bytes", "ll_attn_fwd", "ll_decode_state_bytes", "ll_decode_step",
               "ll_kernel_timing_enable", "ll_kernel_timing_read", "ll_lambda_mlp", "ll_attn_fwd_noalloc", "ll_decode_step_ragged", "ll_attn_fwd_from_state",
               "ll_ccq_query_workspace_bytes", "ll_ccq_query", "ll_attn_bwd_workspace_bytes", "ll_attn_bwd",
               "ll_attn_fwd_lambda_mlp_workspace_bytes", "ll_attn_fwd_lambda_mlp"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def ll_last_error() -> str:
    return load_library().ll_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise LLError(status, ll_last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libllattn must be contiguous")
    return t.data_ptr()


_IO_DTYPES = {LL_F32: torch.float32, LL_BF16: torch.bfloat16}


def _io_dtype(io: int):
    return _IO_DTYPES.get(io)  # None for an unknown code: the library reports LL_ERR_DTYPE


def _validate(*specs) -> None:
    """Checks every tensor argument against the ABI's layout before the library
    is called: the C ABI sees only pointers, so a host tensor, a tensor on
    another device, a wrong dtype or a short buffer would otherwise reach a
    kernel.  Each spec is (name, tensor, element count, dtype); plain integers
    (raw device addresses) and None pass through unchecked (the library checks
    NULLs).  A count or dtype of None is not checked."""
    tensors = []
    for name, t, numel, dtype in specs:  # layout first, then where the memory is
        if t is None or isinstance(t, int):
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor or a device address, got {type(t).__name__}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if numel is not None and t.numel() != numel:
            raise ValueError(f"{name} must hold {numel} elements for this problem, got {t.numel()} "
                             f"(shape {tuple(t.shape)})")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        tensors.append((name, t))
    device = None
    for name, t in tensors:
        if not t.is_cuda:
            raise ValueError(f"{name} is on {t.device}: libllattn takes device memory only")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, other arguments on {device}")
    if device is not None and device.index is not None and device.index != torch.cuda.current_device():
        raise ValueError(f"arguments are on {device} but the current device is cuda:{torch.cuda.current_device()}")


def _workspace_spec(workspace, workspace_bytes: int):
    if isinstance(workspace, torch.Tensor) and workspace.numel() * workspace.element_size() < workspace_bytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"fewer than the {workspace_bytes} passed as its size")
    return ("workspace", workspace, None, None)


def _state_elems(B: int, H: int, dk: int, dv: int, L: int) -> int:
    # S_hat [B,H,L,dk,dv] then sigma [B,H,L], fp32 (ll_decode_state_bytes / 4)
    return B * H * L * (dk * dv + 1)


def _prefill_specs(p: LLProblem, q, k, v, log_gate, lam, beta, o):
    if p is None:
        return []
    io = _io_dtype(p.io)
    rows = p.B * p.T * p.H
    specs = [("q", q, rows * p.dk, io), ("k", k, rows * p.dk, io), ("v", v, rows * p.dv, io),
             ("log_gate", log_gate, rows, torch.float32), ("lambda", lam, rows * p.L, torch.float32),
             ("o", o, rows * p.dv, io)]
    if p.rule == LL_GATED_DELTANET:
        specs.append(("beta", beta, rows, torch.float32))
    return specs


def _decode_specs(B, H, dk, dv, L, io, rule, q, k, v, log_gate, lam, beta, o, state):
    dt = _io_dtype(io)
    specs = [("q", q, B * H * dk, dt), ("k", k, B * H * dk, dt), ("v", v, B * H * dv, dt),
             ("log_gate", log_gate, B * H, torch.float32), ("lambda", lam, B * H * L, torch.float32),
             ("o", o, B * H * dv, dt), ("state", state, _state_elems(B, H, dk, dv, L), torch.float32)]
    if rule == LL_GATED_DELTANET:
        specs.append(("beta", beta, B * H, torch.float32))
    return specs


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream if isinstance(stream, int) else stream.cuda_stream


def ll_attn_fwd_workspace_bytes(problem: LLProblem) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ll_attn_fwd_workspace_bytes(ctypes.byref(problem), ctypes.byref(out)))
    return out.value


def ll_attn_fwd(problem: LLProblem, q, k, v, log_gate, lam, beta, o, state_out, workspace, workspace_bytes: int,
                stream=None) -> None:
    p = problem
    _validate(*_prefill_specs(p, q, k, v, log_gate, lam, beta, o),
              *([("state_out", state_out, _state_elems(p.B, p.H, p.dk, p.dv, p.L), torch.float32)] if p else []),
              _workspace_spec(workspace, workspace_bytes))
    _check(load_library().ll_attn_fwd(None if problem is None else ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _ptr(lam),
                                      _ptr(beta), _ptr(o), _ptr(state_out), _ptr(workspace), workspace_bytes,
                                      _stream(stream)))


def ll_attn_fwd_noalloc(problem: LLProblem, q, k, v, log_gate, lam, beta, o, state_out, stream=None) -> None:
    p = problem
    _validate(*_prefill_specs(p, q, k, v, log_gate, lam, beta, o),
              *([("state_out", state_out, _state_elems(p.B, p.H, p.dk, p.dv, p.L), torch.float32)] if p else []))
    _check(load_library().ll_attn_fwd_noalloc(None if problem is None else ctypes.byref(problem), _ptr(q), _ptr(k),
                                              _ptr(v), _ptr(log_gate), _ptr(lam), _ptr(beta), _ptr(o),
                                              _ptr(state_out), _stream(stream)))


def ll_attn_fwd_from_state(problem: LLProblem, pos0: int, state_in, q, k, v, log_gate, lam, beta, o, state_out,
                           workspace, workspace_bytes: int, stream=None) -> None:
    p = problem
    n_state = _state_elems(p.B, p.H, p.dk, p.dv, p.L) if p else None
    _validate(*_prefill_specs(p, q, k, v, log_gate, lam, beta, o),
              *([("state_in", state_in, n_state, torch.float32), ("state_out", state_out, n_state, torch.float32)]
                if p else []),
              _workspace_spec(workspace, workspace_bytes))
    _check(load_library().ll_attn_fwd_from_state(None if problem is None else ctypes.byref(problem), pos0,
                                                 _ptr(state_in), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate),
                                                 _ptr(lam), _ptr(beta), _ptr(o), _ptr(state_out), _ptr(workspace),
                                                 workspace_bytes, _stream(stream)))


def ll_attn_fwd_lambda_mlp_workspace_bytes(problem: LLProblem, hidden: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ll_attn_fwd_lambda_mlp_workspace_bytes(None if problem is None else ctypes.byref(problem),
                                                                 hidden, ctypes.byref(out)))
    return out.value


def ll_attn_fwd_lambda_mlp(problem: LLProblem, q, k, v, log_gate, d, hidden: int, w1, w2, bias, beta, o, state_out,
                           workspace, workspace_bytes: int, stream=None) -> None:
    p = problem
    f32 = torch.float32
    specs = []
    if p:
        specs = [s for s in _prefill_specs(p, q, k, v, log_gate, d, beta, o) if s[0] != "lambda"]
        specs += [("d", d, p.B * p.T * p.H * p.L, f32), ("w1", w1, p.L * hidden, f32),
                  ("w2", w2, hidden * p.L, f32), ("bias", bias, p.L, f32)]
        if state_out is not None:
            specs.append(("state_out", state_out, _state_elems(p.B, p.H, p.dk, p.dv, p.L), f32))
    _validate(*specs, _workspace_spec(workspace, workspace_bytes))
    _check(load_library().ll_attn_fwd_lambda_mlp(None if problem is None else ctypes.byref(problem), _ptr(q), _ptr(k),
                                                 _ptr(v), _ptr(log_gate), _ptr(d), hidden, _ptr(w1), _ptr(w2),
                                                 _ptr(bias), _ptr(beta), _ptr(o), _ptr(state_out), _ptr(workspace),
                                                 workspace_bytes, _stream(stream)))


def ll_decode_state_bytes(B: int, H: int, dk: int, dv: int, L: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ll_decode_state_bytes(B, H, dk, dv, L, ctypes.byref(out)))
    return out.value


def ll_decode_step(B, H, dk, dv, L, io, rule, pos, q, k, v, log_gate, lam, beta, o, state, stream=None) -> None:
    _validate(*_decode_specs(B, H, dk, dv, L, io, rule, q, k, v, log_gate, lam, beta, o, state))
    _check(load_library().ll_decode_step(B, H, dk, dv, L, io, rule, pos, _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate),
                                         _ptr(lam), _ptr(beta), _ptr(o), _ptr(state), _stream(stream)))


def ll_lambda_mlp(rows: int, L: int, hidden: int, d, w1, w2, bias, lam, stream=None) -> None:
    f32 = torch.float32
    _validate(("d", d, rows * L, f32), ("w1", w1, L * hidden, f32), ("w2", w2, hidden * L, f32),
              ("bias", bias, L, f32), ("lambda", lam, rows * L, f32))
    _check(load_library().ll_lambda_mlp(rows, L, hidden, _ptr(d), _ptr(w1), _ptr(w2), _ptr(bias), _ptr(lam),
                                        _stream(stream)))


def ll_decode_step_ragged(B, H, dk, dv, L, io, rule, pos, q, k, v, log_gate, lam, beta, o, state,
                          stream=None) -> None:
    """``pos``: int64 device tensor [B], one position per sequence."""
    _validate(("pos", pos, B, torch.int64), *_decode_specs(B, H, dk, dv, L, io, rule, q, k, v, log_gate, lam, beta,
                                                           o, state))
    _check(load_library().ll_decode_step_ragged(B, H, dk, dv, L, io, rule, _ptr(pos), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(log_gate), _ptr(lam), _ptr(beta), _ptr(o), _ptr(state),
                                                _stream(stream)))


def ll_ccq_query_workspace_bytes(B: int, T: int, H: int, dk: int, io: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ll_ccq_query_workspace_bytes(B, T, H, dk, io, ctypes.byref(out)))
    return out.value


def ll_ccq_query(B, T, H, dk, io, q, k, w, b, q_clean, workspace, workspace_bytes: int, stream=None) -> None:
    dt, n = _io_dtype(io), B * T * H * dk
    _validate(("q", q, n, dt), ("k", k, n, dt), ("w", w, H * dk, torch.float32), ("b", b, H, torch.float32),
              ("q_clean", q_clean, n, dt), _workspace_spec(workspace, workspace_bytes))
    _check(load_library().ll_ccq_query(B, T, H, dk, io, _ptr(q), _ptr(k), _ptr(w), _ptr(b), _ptr(q_clean),
                                       _ptr(workspace), workspace_bytes, _stream(stream)))


def ll_attn_bwd_workspace_bytes(problem: LLProblem) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ll_attn_bwd_workspace_bytes(ctypes.byref(problem), ctypes.byref(out)))
    return out.value


def ll_attn_bwd(problem: LLProblem, q, k, v, log_gate, lam, o, dO, dq, dk, dv, dlog_gate, dlam, workspace,
                workspace_bytes: int, stream=None) -> None:
    p = problem
    if p is not None:
        io, rows, f32 = _io_dtype(p.io), p.B * p.T * p.H, torch.float32
        _validate(*_prefill_specs(p, q, k, v, log_gate, lam, None, o), ("dO", dO, rows * p.dv, io),
                  ("dq", dq, rows * p.dk, io), ("dk", dk, rows * p.dk, io), ("dv", dv, rows * p.dv, io),
                  ("dlog_gate", dlog_gate, rows, f32), ("dlambda", dlam, rows * p.L, f32),
                  _workspace_spec(workspace, workspace_bytes))
    _check(load_library().ll_attn_bwd(None if problem is None else ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(log_gate), _ptr(lam), _ptr(o), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(dlog_gate), _ptr(dlam), _ptr(workspace), workspace_bytes,
                                      _stream(stream)))


def ll_kernel_timing_enable(on: bool) -> None:
    _check(load_library().ll_kernel_timing_enable(1 if on else 0))


def ll_kernel_timing_read() -> dict:
    """{kernel name: (total ms, launches)} since the last read."""
    cap = 16
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    n_launch = (ctypes.c_int * cap)()
    count = ctypes.c_int(0)
    _check(load_library().ll_kernel_timing_read(names, ms, n_launch, cap, ctypes.byref(count)))
    return {names[i].decode(): (ms[i], n_launch[i]) for i in range(min(count.value, cap))}


# ---------------------------------------------------------------- helpers

def io_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return LL_F32
    if dtype == torch.bfloat16:
        return LL_BF16
    raise TypeError(f"io dtype must be float32 or bfloat16, got {dtype}")


def decode_state_tensor(B: int, H: int, dk: int, dv: int, L: int, device="cuda") -> torch.Tensor:
    """A zeroed decode state (the empty prefix) as a flat fp32 tensor."""
    n = ll_decode_state_bytes(B, H, dk, dv, L) // 4
    return torch.zeros(n, dtype=torch.float32, device=device)


def attn_fwd(q, k, v, log_gate, lam, beta=None, C: int = 64, rule: int = LL_MAMBA2, L: int | None = None,
             want_output: bool = True, want_state: bool = False, workspace=None, out=None, stream=None,
             pos0: int = 0, state_in=None, state_out=None):
    """Allocate outputs and workspace with torch, then call ``ll_attn_fwd``
    (or ``ll_attn_fwd_from_state`` for a segment starting at ``pos0`` after
    the per-level states ``state_in``).

    Returns ``o`` (or None), and the exported state (flat fp32) when
    ``want_state`` (written into ``state_out`` if given, which may be
    ``state_in``).
    """
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    L = L if L is not None else lam.shape[-1]
    prob = LLProblem(B, T, H, dk, dv, L, C, io_code(k.dtype), rule)
    nbytes = ll_attn_fwd_workspace_bytes(prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    o = None
    if want_output:
        o = out if out is not None else torch.empty(B, T, H, dv, dtype=v.dtype, device=v.device)
    st = None
    if want_state:
        st = state_out if state_out is not None else torch.empty(ll_decode_state_bytes(B, H, dk, dv, L) // 4,
                                                                  dtype=torch.float32, device=k.device)
    if pos0 or state_in is not None:
        ll_attn_fwd_from_state(prob, pos0, state_in, q, k, v, log_gate, lam, beta, o, st, workspace,
                               workspace.numel(), stream)
    else:
        ll_attn_fwd(prob, q, k, v, log_gate, lam, beta, o, st, workspace, workspace.numel(), stream)
    return (o, st) if want_state else o


def lambda_mlp(d, w1, w2, bias, out=None, stream=None):
    """Level weights softplus((d W1) W2 + b) for every row of ``d`` [..., L]
    (fp32 on the GPU); returns a tensor shaped like ``d``."""
    L = d.shape[-1]
    hidden = w1.shape[1]
    if tuple(w1.shape) != (L, hidden) or tuple(w2.shape) != (hidden, L) or tuple(bias.shape) != (L,):
        raise ValueError("lambda_mlp: w1 [L, hidden], w2 [hidden, L] and bias [L] must match d [..., L]")
    for t in (d, w1, w2, bias):
        if t.dtype != torch.float32:
            raise TypeError("lambda_mlp takes fp32 tensors")
    lam = out if out is not None else torch.empty_like(d)
    ll_lambda_mlp(d.numel() // L, L, hidden, d, w1, w2, bias, lam, stream)
    return lam


def attn_fwd_lambda_mlp(q, k, v, log_gate, d, w1, w2, bias, beta=None, C: int = 64, rule: int = LL_MAMBA2,
                        want_state: bool = False, workspace=None, out=None, stream=None):
    """The prefill with level weights softplus((d W1) W2 + b) made by the read
    (``ll_attn_fwd_lambda_mlp``); returns ``o`` (and the exported state when
    ``want_state``)."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    L, hidden = d.shape[-1], w1.shape[1]
    prob = LLProblem(B, T, H, dk, dv, L, C, io_code(k.dtype), rule)
    nbytes = ll_attn_fwd_lambda_mlp_workspace_bytes(prob, hidden)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    o = out if out is not None else torch.empty(B, T, H, dv, dtype=v.dtype, device=v.device)
    st = None
    if want_state:
        st = torch.empty(ll_decode_state_bytes(B, H, dk, dv, L) // 4, dtype=torch.float32, device=k.device)
    ll_attn_fwd_lambda_mlp(prob, q, k, v, log_gate, d, hidden, w1, w2, bias, beta, o, st, workspace,
                           workspace.numel(), stream)
    return (o, st) if want_state else o


def ccq_query(q, k, w, b, out=None, workspace=None, stream=None):
    """The curvature-conditioned query q - sigmoid(w_h . q + b_h) Cov(k_0..k_t) q
    for q, k [B,T,H,dk] (io dtype), w [H,dk], b [H] (fp32); returns q_clean."""
    B, T, H, dk = q.shape
    io = io_code(q.dtype)
    nbytes = ll_ccq_query_workspace_bytes(B, T, H, dk, io)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    qc = out if out is not None else torch.empty_like(q)
    ll_ccq_query(B, T, H, dk, io, q, k, w, b, qc, workspace, workspace.numel(), stream)
    return qc


def attn_bwd(q, k, v, log_gate, lam, o, dO, C: int = 64, L: int | None = None, workspace=None, stream=None):
    """Gradients (dq, dk, dv, dlog_gate, dlambda) of the Mamba-2 prefill for
    the output gradient dO; allocates outputs and workspace with torch."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    L = L if L is not None else lam.shape[-1]
    prob = LLProblem(B, T, H, dk, dv, L, C, io_code(k.dtype), LL_MAMBA2)
    nbytes = ll_attn_bwd_workspace_bytes(prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    dq, dkk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(log_gate)
    dl = torch.empty_like(lam)
    ll_attn_bwd(prob, q, k, v, log_gate, lam, o, dO, dq, dkk, dvv, dg, dl, workspace, workspace.numel(), stream)
    return dict(dq=dq, dk=dkk, dv=dvv, dlog_gate=dg, dlambda=dl)
