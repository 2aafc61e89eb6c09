"""CPU-only checks of the C ABI: the library loads, exports every declared
entry point, sizes its buffers as documented, and rejects bad arguments before
touching the GPU (a rejected call enqueues nothing, so these run without one)."""

import ctypes
import os
import re

import pytest

import fenwick_tree_linear_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ll_attn.h")

DUMMY = 0x1000  # a non-NULL pointer that validation must never dereference


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ll_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["ll_attn_bwd", "ll_attn_bwd_workspace_bytes", "ll_attn_fwd", "ll_attn_fwd_from_state",
         "ll_attn_fwd_lambda_mlp", "ll_attn_fwd_lambda_mlp_workspace_bytes", "ll_attn_fwd_noalloc",
         "ll_attn_fwd_workspace_bytes", "ll_ccq_query",
         "ll_ccq_query_workspace_bytes", "ll_decode_state_bytes", "ll_decode_step", "ll_decode_step_ragged",
         "ll_kernel_timing_enable", "ll_kernel_timing_read", "ll_lambda_mlp", "ll_last_error"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(F.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def prob(**kw):
    base = dict(B=2, T=16384, H=16, dk=64, dv=64, L=15, C=64, io=F.LL_BF16, rule=F.LL_MAMBA2)
    base.update(kw)
    return F.LLProblem(*(base[k] for k in ("B", "T", "H", "dk", "dv", "L", "C", "io", "rule")))


def status_of(fn, *args):
    try:
        fn(*args)
    except F.LLError as e:
        return e.name, str(e)
    return "LL_OK", ""


def test_workspace_bytes_for_the_16k_prefill():
    # 32 heads x 16 blocks of 16 chunks (the bf16 d <= 64 read keeps four
    # within-block levels): 512 block states + 256 Fenwick nodes of 64x64 fp32,
    # plus their gate sums
    n = F.ll_attn_fwd_workspace_bytes(prob())
    assert 768 * 64 * 64 * 4 <= n <= 768 * 64 * 64 * 4 + 4 * 4096 + 4 * 256
    assert n % 256 == 0
    # at d = 128 (bf16) the read takes the nodes from a bf16 copy of all of them:
    # 32 heads x 32 blocks of 8 chunks of 32 -> 1024 states, 512 nodes, 1024 copies
    m = F.ll_attn_fwd_workspace_bytes(prob(T=8192, L=14, dk=128, dv=128, C=32))
    base = 1536 * 128 * 128 * 4 + 1024 * 128 * 128 * 2
    assert base <= m <= base + 4 * 4096 + 5 * 256


def test_gdn_workspace_holds_three_row_buffers():
    """The Gated DeltaNet pass adds W, U' and the pseudo-values U, each [B,T,H,d] in the io dtype;
    d=128 bf16 with C=64 is accepted (the read then uses chunks of 32)."""
    m = F.ll_attn_fwd_workspace_bytes(prob(T=2048, L=12))
    g = F.ll_attn_fwd_workspace_bytes(prob(T=2048, L=12, rule=F.LL_GATED_DELTANET))
    rows = 2 * 2048 * 16 * 64 * 2
    assert 3 * rows <= g - m <= 3 * rows + 3 * 256
    assert F.ll_attn_fwd_workspace_bytes(prob(T=8192, L=14, dk=128, dv=128, rule=F.LL_GATED_DELTANET)) > 0


@pytest.mark.parametrize("io", [F.LL_F32, F.LL_BF16])
def test_full_shape_set_is_accepted(io):
    """Every head size (dk and dv each in 16, 32, 64, 128, also unequal) and
    chunk size (16, 32, 64) of the boundary is accepted by every prefill, the
    backward (Mamba-2) and the decode; shapes the kernels do not run natively
    run zero-padded to a square head, in bf16 32-token chunks, or in chunks
    halved until a tile fits."""
    for dk in (16, 32, 64, 128):
        for dv in (16, 32, 64, 128):
            for C in (16, 32, 64):
                for rule in (F.LL_MAMBA2, F.LL_GATED_DELTANET):
                    p = prob(B=1, T=256, H=2, dk=dk, dv=dv, L=9, C=C, io=io, rule=rule)
                    assert F.ll_attn_fwd_workspace_bytes(p) > 0, (dk, dv, C, rule)
                assert F.ll_attn_bwd_workspace_bytes(prob(B=1, T=256, H=2, dk=dk, dv=dv, L=9, C=C, io=io)) > 0
            assert F.ll_decode_state_bytes(2, 3, dk, dv, 9) == 2 * 3 * 9 * (dk * dv + 1) * 4
    # bf16 chunks of 16 with T not a multiple of 32 run padded to the next multiple
    assert F.ll_attn_fwd_workspace_bytes(prob(B=1, T=48, H=2, L=7, C=16, io=io)) > 0


def test_workspace_grows_with_problem():
    a = F.ll_attn_fwd_workspace_bytes(prob(T=2048, L=12))
    b = F.ll_attn_fwd_workspace_bytes(prob(T=4096, L=13))
    assert 0 < a < b


@pytest.mark.parametrize("kw,name,frag", [
    (dict(T=16384, L=14), "LL_ERR_SHAPE", "levels"),
    (dict(T=1000), "LL_ERR_SHAPE", "multiple"),
    (dict(C=48), "LL_ERR_SHAPE", "power of two"),
    (dict(C=128), "LL_ERR_UNSUPPORTED", "chunk"),
    (dict(dk=48, dv=48), "LL_ERR_UNSUPPORTED", "head size"),
    (dict(dk=64, dv=24), "LL_ERR_UNSUPPORTED", "head size"),
    (dict(C=16, T=16, L=5), "LL_ERR_UNSUPPORTED", "L >= 6"),  # bf16 runs T = 16 padded to 32 tokens
    (dict(io=7), "LL_ERR_DTYPE", "dtype"),
    (dict(rule=5), "LL_ERR_UNSUPPORTED", "rule"),
    (dict(B=0), "LL_ERR_SHAPE", "positive"),
    (dict(T=2 ** 24, L=25), "LL_ERR_UNSUPPORTED", "levels"),
])
def test_invalid_problems_are_rejected(kw, name, frag):
    st, msg = status_of(F.ll_attn_fwd_workspace_bytes, prob(**kw))
    assert st == name and frag in msg, msg


def test_fp32_supports_small_heads_and_chunks():
    assert F.ll_attn_fwd_workspace_bytes(prob(T=256, dk=16, dv=16, L=9, C=16, io=F.LL_F32)) > 0


def test_fwd_validation_before_any_launch():
    p = prob()
    ws = F.ll_attn_fwd_workspace_bytes(p)
    D = DUMMY
    cases = [
        ((p, D, None, D, D, D, None, D, None, D, ws), "LL_ERR_NULL"),           # k NULL
        ((p, D, D, D, D, D, None, None, None, D, ws), "LL_ERR_NULL"),           # nothing requested
        ((p, None, D, D, D, D, None, D, None, D, ws), "LL_ERR_NULL"),           # q NULL with output
        ((p, D, D, D, D, None, None, D, None, D, ws), "LL_ERR_NULL"),           # lambda NULL with output
        ((p, D, D, D, D, D, None, D, None, D, ws - 1), "LL_ERR_WORKSPACE"),     # workspace too small
        ((p, D, D, D, D, D, None, D, None, None, ws), "LL_ERR_WORKSPACE"),      # workspace NULL
        ((p, D, D, D, D, D, None, D, D, D, ws), "LL_ERR_SHAPE"),                # export of [0,2^14) needs L=16
        ((prob(rule=F.LL_GATED_DELTANET), D, D, D, D, D, None, D, None, D, ws), "LL_ERR_NULL"),  # GDN needs beta
        ((None, D, D, D, D, D, None, D, None, D, ws), "LL_ERR_NULL"),
    ]
    for args, name in cases:
        st, msg = status_of(F.ll_attn_fwd, *args, 0)
        assert st == name, (name, msg)


def test_decode_state_bytes():
    # S_hat [B,H,L,dk,dv] + sigma [B,H,L], fp32
    assert F.ll_decode_state_bytes(64, 16, 64, 64, 17) == 64 * 16 * 17 * (64 * 64 + 1) * 4
    assert status_of(F.ll_decode_state_bytes, 1, 1, 64, 64, 1)[0] == "LL_ERR_SHAPE"


def test_decode_validation_before_any_launch():
    D = DUMMY
    good = [64, 16, 64, 64, 17, F.LL_BF16, F.LL_MAMBA2, 32768, D, D, D, D, D, None, D, D, 0]
    # largest position whose successor state still fits: pos + 1 < 2^16
    cases = [
        (dict(pos=2 ** 16 - 1), "LL_ERR_POSITION"),
        (dict(pos=-1), "LL_ERR_POSITION"),
        (dict(L=33, pos=5), "LL_ERR_UNSUPPORTED"),
        (dict(io=3), "LL_ERR_DTYPE"),
        (dict(rule=F.LL_GATED_DELTANET), "LL_ERR_NULL"),  # Gated DeltaNet needs beta
        (dict(dk=64, dv=24), "LL_ERR_UNSUPPORTED"),
        (dict(state=None), "LL_ERR_NULL"),
        (dict(q=None), "LL_ERR_NULL"),
    ]
    idx = dict(B=0, H=1, dk=2, dv=3, L=4, io=5, rule=6, pos=7, q=8, k=9, v=10, g=11, lam=12, beta=13, o=14, state=15)
    for kw, name in cases:
        args = list(good)
        for key, val in kw.items():
            args[idx[key]] = val
        st, msg = status_of(F.ll_decode_step, *args)
        assert st == name, (kw, msg)


def test_last_error_is_cleared_by_a_good_call():
    status_of(F.ll_attn_fwd_workspace_bytes, prob(C=48))
    assert F.ll_last_error() != ""
    F.ll_attn_fwd_workspace_bytes(prob())
    assert F.ll_last_error() == ""


def test_lambda_mlp_validation_before_any_launch():
    D = DUMMY
    good = dict(rows=1024, L=15, hidden=30, d=D, w1=D, w2=D + 64, bias=D + 128, lam=D + 4096)
    cases = [
        (dict(rows=-1), "LL_ERR_SHAPE"),
        (dict(L=0), "LL_ERR_SHAPE"),
        (dict(hidden=0), "LL_ERR_SHAPE"),
        (dict(L=33), "LL_ERR_UNSUPPORTED"),
        (dict(hidden=65), "LL_ERR_UNSUPPORTED"),
        (dict(rows=2 ** 40), "LL_ERR_UNSUPPORTED"),
        (dict(d=None), "LL_ERR_NULL"),
        (dict(bias=None), "LL_ERR_NULL"),
        (dict(lam=None), "LL_ERR_NULL"),
        (dict(lam=D), "LL_ERR_SHAPE"),  # lambda over d
        (dict(rows=0, d=None, w1=None, w2=None, bias=None, lam=None), "LL_OK"),  # nothing to do
    ]
    order = ("rows", "L", "hidden", "d", "w1", "w2", "bias", "lam")
    for kw, name in cases:
        a = dict(good, **kw)
        st, msg = status_of(F.ll_lambda_mlp, *(a[k] for k in order), 0)
        assert st == name, (kw, msg)


def test_fused_mlp_prefill_workspace():
    """The read makes the level weights itself for bf16 with a run head <= 64, run chunks >= 32
    and L <= 16 (any hidden size), in the plain prefill's blocks: the workspace is then exactly a
    prefill's.  Otherwise the weights of every row go through the workspace after the plain
    prefill's (256-byte aligned)."""
    for kw, hidden in [(dict(), 30), (dict(), 33), (dict(), 64), (dict(T=32768, L=16), 30),
                       (dict(T=2048, L=12, dk=32, dv=16, C=16), 24)]:
        p = prob(**kw)
        assert F.ll_attn_fwd_lambda_mlp_workspace_bytes(p, hidden) == F.ll_attn_fwd_workspace_bytes(p), (kw, hidden)
    # the 16K prefill: blocks of 16 chunks, 32 heads x 16 blocks, 512 states + 256 nodes of 64 x 64 fp32
    n = F.ll_attn_fwd_lambda_mlp_workspace_bytes(prob(), 30)
    assert 768 * 64 * 64 * 4 <= n <= 768 * 64 * 64 * 4 + 4 * 4096 + 4 * 256
    for kw, hidden in [(dict(T=2048, L=17), 30), (dict(T=2048, L=12, io=F.LL_F32, C=32), 24),
                       (dict(T=2048, L=12, dk=128, dv=128, C=32), 24)]:
        p = prob(**kw)
        base = (F.ll_attn_fwd_workspace_bytes(p) + 255) // 256 * 256
        assert F.ll_attn_fwd_lambda_mlp_workspace_bytes(p, hidden) == base + p.B * p.T * p.H * p.L * 4, (kw, hidden)


def test_fused_mlp_prefill_validation_before_any_launch():
    D = DUMMY
    p = prob(T=2048, L=12)
    n = F.ll_attn_fwd_lambda_mlp_workspace_bytes(p, 24)
    good = dict(p=p, q=D, k=D, v=D, g=D, d=D, hidden=24, w1=D, w2=D, bias=D, beta=None, o=D, st=None, ws=D, n=n)
    cases = [
        (dict(hidden=0), "LL_ERR_SHAPE"),
        (dict(hidden=65), "LL_ERR_UNSUPPORTED"),
        (dict(p=prob(T=2048, L=33)), "LL_ERR_UNSUPPORTED"),
        (dict(o=None), "LL_ERR_NULL"),
        (dict(d=None), "LL_ERR_NULL"),
        (dict(w2=None), "LL_ERR_NULL"),
        (dict(n=n - 1), "LL_ERR_WORKSPACE"),
        (dict(p=prob(T=2048, L=12, C=48)), "LL_ERR_SHAPE"),
    ]
    order = ("p", "q", "k", "v", "g", "d", "hidden", "w1", "w2", "bias", "beta", "o", "st", "ws", "n")
    for kw, name in cases:
        a = dict(good, **kw)
        st, msg = status_of(F.ll_attn_fwd_lambda_mlp, *(a[x] for x in order), 0)
        assert st == name, (kw, msg)


def test_ragged_decode_validation_before_any_launch():
    D = DUMMY
    good = [64, 16, 64, 64, 17, F.LL_BF16, F.LL_MAMBA2, D, D, D, D, D, D, None, D, D, 0]
    cases = [
        (dict(pos=None), "LL_ERR_NULL"),
        (dict(L=33), "LL_ERR_UNSUPPORTED"),
        (dict(L=1), "LL_ERR_SHAPE"),
        (dict(io=3), "LL_ERR_DTYPE"),
        (dict(rule=F.LL_GATED_DELTANET), "LL_ERR_NULL"),
        (dict(dk=64, dv=24), "LL_ERR_UNSUPPORTED"),
        (dict(dk=48, dv=48), "LL_ERR_UNSUPPORTED"),
        (dict(state=None), "LL_ERR_NULL"),
        (dict(o=None), "LL_ERR_NULL"),
    ]
    idx = dict(B=0, H=1, dk=2, dv=3, L=4, io=5, rule=6, pos=7, q=8, k=9, v=10, g=11, lam=12, beta=13, o=14, state=15)
    for kw, name in cases:
        args = list(good)
        for key, val in kw.items():
            args[idx[key]] = val
        st, msg = status_of(F.ll_decode_step_ragged, *args)
        assert st == name, (kw, msg)


def test_prefill_from_state_validation_before_any_launch():
    D = DUMMY
    ws = F.ll_attn_fwd_workspace_bytes(prob(T=2048, L=16))

    def call(p, pos0, state_in=D, o=D, state_out=None, beta=None):
        return status_of(F.ll_attn_fwd_from_state, p, pos0, state_in, D, D, D, D, D, beta, o, state_out, D, ws, 0)

    assert call(prob(T=2048, L=16), -1)[0] == "LL_ERR_POSITION"
    assert call(prob(T=2048, L=16), 1024)[0] == "LL_ERR_POSITION"  # segment longer than lowbit(pos0)
    assert call(prob(T=2048, L=16), 3 * 1024)[0] == "LL_ERR_POSITION"
    assert call(prob(T=2048, L=16), 2048, state_in=None)[0] == "LL_ERR_NULL"
    assert call(prob(T=2048, L=16, rule=F.LL_GATED_DELTANET), 2048, beta=None)[0] == "LL_ERR_NULL"
    # outputs up to position 2^15 - 1 fit 16 levels; the state of [0, 2^15) needs 17
    assert call(prob(T=2048, L=16), 2 ** 15 - 2048, state_out=D)[0] == "LL_ERR_SHAPE"
    assert call(prob(T=2048, L=16), 2 ** 15, state_out=None)[0] == "LL_ERR_SHAPE"
    assert call(prob(T=2048, L=13), 2048 * 3)[0] == "LL_ERR_SHAPE"  # position 8191 needs 14 levels


def test_ccq_validation_before_any_launch():
    D = DUMMY
    n = F.ll_ccq_query_workspace_bytes(2, 16384, 16, 64, F.LL_BF16)
    # the prefill's inputs ones [rows, 15] and zeros (fp32), its output kkq (bf16 rows), the
    # per-chunk key sums [2, 16, 256, 64] fp32 and the prefill workspace
    rows = 2 * 16384 * 16
    need = rows * 15 * 4 + rows * 4 + rows * 64 * 2 + 2 * 16 * 256 * 64 * 4 + F.ll_attn_fwd_workspace_bytes(prob())
    assert need <= n <= need + 5 * 256

    def call(B=2, T=16384, H=16, dk=64, io=F.LL_BF16, q=D, k=D, w=D, b=D, qc=D, ws=D, wsb=n):
        return status_of(F.ll_ccq_query, B, T, H, dk, io, q, k, w, b, qc, ws, wsb, 0)[0]

    assert call(T=100) == "LL_ERR_UNSUPPORTED"  # no supported chunk divides 100
    assert call(dk=48) == "LL_ERR_UNSUPPORTED"
    assert call(io=7) == "LL_ERR_DTYPE"
    assert call(B=0) == "LL_ERR_SHAPE"
    assert call(w=None) == "LL_ERR_NULL"
    assert call(qc=None) == "LL_ERR_NULL"
    assert call(wsb=n - 1) == "LL_ERR_WORKSPACE"
    assert call(ws=None) == "LL_ERR_WORKSPACE"


def test_bwd_validation_before_any_launch():
    D = DUMMY
    n = F.ll_attn_bwd_workspace_bytes(prob(T=2048, L=12))
    # the forward's workspace, dO.o and v.dv per row (fp32), the block shares of the
    # reverse bucket states (4 blocks of 8 chunks per head: 2 block levels) and 3
    # chunk-level states per block, all fp32 64 x 64
    def need(T, L, nb, nbl):
        # the block states and Fenwick nodes of (v, k) in blocks of 8 chunks (the backward's
        # walks keep three chunk levels), two fp32 values per row, the reverse bucket states
        # (one fp32 64 x 64 state per block and block level) and one fp32 sum per block; at
        # d = 64 the chunk-level states live in LDS
        rows, heads, state = 2 * T * 16, 2 * 16, 64 * 64 * 4
        a256 = lambda x: (x + 255) // 256 * 256
        fwd = a256(heads * nb * state) + a256(heads * nb * 4) + a256(heads * (nb // 2) * state) + a256(heads * max(nb // 2, 1) * 4)
        return fwd + 2 * rows * 4 + heads * nb * nbl * state + heads * nb * 4

    assert need(2048, 12, 4, 2) <= n <= need(2048, 12, 4, 2) + 6 * 256  # 4 blocks of 8 chunks: 2 block levels
    m = F.ll_attn_bwd_workspace_bytes(prob(T=4096, L=13))  # 8 blocks: 3 block levels
    assert need(4096, 13, 8, 3) <= m <= need(4096, 13, 8, 3) + 6 * 256

    def call(p, q=D, o=D, dO=D, dq=D, dlam=D, ws=D, wsb=n):
        return status_of(F.ll_attn_bwd, p, q, D, D, D, D, o, dO, dq, D, D, D, dlam, ws, wsb, 0)[0]

    assert call(prob(T=2048, L=12, rule=F.LL_GATED_DELTANET)) == "LL_ERR_UNSUPPORTED"
    assert call(prob(T=2048, L=11)) == "LL_ERR_SHAPE"
    assert call(prob(T=2048, L=12, C=48)) == "LL_ERR_SHAPE"
    assert call(prob(T=2048, L=12), dO=None) == "LL_ERR_NULL"
    assert call(prob(T=2048, L=12), dq=None) == "LL_ERR_NULL"
    assert call(prob(T=2048, L=12), dlam=None) == "LL_ERR_NULL"
    assert call(prob(T=2048, L=12), wsb=n - 1) == "LL_ERR_WORKSPACE"
    assert call(prob(T=2048, L=12), ws=None) == "LL_ERR_WORKSPACE"


def test_noalloc_validation_before_any_launch():
    """The allocation-free prefill validates like ll_attn_fwd, and rejects a
    problem whose workspace exceeds its 64 MiB scratch before touching the GPU."""
    d = DUMMY
    args = (d, d, d, d, d, None, d, None)
    big = prob(B=16)  # 16 x 16 heads x 16384 tokens: 100 MB of block states and nodes
    assert F.ll_attn_fwd_workspace_bytes(prob()) <= 64 << 20
    assert F.ll_attn_fwd_workspace_bytes(big) > 64 << 20
    name, msg = status_of(F.ll_attn_fwd_noalloc, big, *args)
    assert name == "LL_ERR_WORKSPACE" and "allocation-free" in msg
    gdn = prob(T=8192, L=14, dk=128, dv=128, rule=F.LL_GATED_DELTANET)
    assert status_of(F.ll_attn_fwd_noalloc, gdn, d, d, d, d, d, d, d, None)[0] == "LL_ERR_WORKSPACE"
    assert status_of(F.ll_attn_fwd_noalloc, prob(C=48), *args)[0] == "LL_ERR_SHAPE"
    assert status_of(F.ll_attn_fwd_noalloc, prob(), d, None, d, d, d, None, d, None)[0] == "LL_ERR_NULL"
    assert status_of(F.ll_attn_fwd_noalloc, None, *args)[0] == "LL_ERR_NULL"
    assert status_of(F.ll_attn_fwd_noalloc, prob(rule=F.LL_GATED_DELTANET), *args)[0] == "LL_ERR_NULL"


# ------------------------------------------------ binding argument checks

@pytest.fixture
def no_library(monkeypatch):
    """Any call that reaches the library fails the test: the binding's checks
    must raise first."""
    from fenwick_tree_linear_amd import binding

    def refuse():
        raise AssertionError("the library was called")

    monkeypatch.setattr(binding, "load_library", refuse)


def _prefill_tensors(p, io=None):
    import torch

    dt = io or (torch.bfloat16 if p.io == F.LL_BF16 else torch.float32)
    rows = (p.B, p.T, p.H)
    return dict(q=torch.zeros(*rows, p.dk, dtype=dt), k=torch.zeros(*rows, p.dk, dtype=dt),
                v=torch.zeros(*rows, p.dv, dtype=dt), log_gate=torch.zeros(*rows), lam=torch.zeros(*rows, p.L),
                beta=torch.zeros(*rows), o=torch.zeros(*rows, p.dv, dtype=dt))


def test_binding_rejects_host_tensors(no_library):
    import torch

    p = prob(B=1, T=256, H=2, L=9)
    x = _prefill_tensors(p)
    with pytest.raises(ValueError, match="device memory only"):
        F.ll_attn_fwd(p, x["q"], x["k"], x["v"], x["log_gate"], x["lam"], None, x["o"], None, DUMMY, 0)
    with pytest.raises(ValueError, match="device memory only"):
        F.ll_attn_fwd_noalloc(p, x["q"], x["k"], x["v"], x["log_gate"], x["lam"], None, x["o"], None)
    # the int64 positions of the ragged decode step, on the host
    with pytest.raises(ValueError, match="device memory only"):
        F.ll_decode_step_ragged(2, 2, 64, 64, 9, F.LL_BF16, F.LL_MAMBA2, torch.zeros(2, dtype=torch.int64),
                                DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY, DUMMY)


def test_binding_rejects_wrong_dtypes_and_sizes(no_library):
    import torch

    p = prob(B=1, T=256, H=2, L=9)
    x = _prefill_tensors(p)
    args = lambda **kw: [kw.get(n, x[n]) for n in ("q", "k", "v", "log_gate", "lam")]
    # q in another dtype than the problem's io
    with pytest.raises(TypeError, match="q must be torch.bfloat16"):
        F.ll_attn_fwd(p, *args(q=x["q"].float()), None, x["o"], None, DUMMY, 0)
    # lambda with one level too few, a short gate, an fp32 o for bf16 io
    with pytest.raises(ValueError, match="lambda must hold"):
        F.ll_attn_fwd(p, *args(lam=x["lam"][..., :-1].contiguous()), None, x["o"], None, DUMMY, 0)
    with pytest.raises(ValueError, match="log_gate must hold"):
        F.ll_attn_fwd(p, *args(log_gate=x["log_gate"][:, :-1].contiguous()), None, x["o"], None, DUMMY, 0)
    with pytest.raises(TypeError, match="o must be"):
        F.ll_attn_fwd(p, *args(), None, x["o"].float(), None, DUMMY, 0)
    # the Gated DeltaNet write strength, short
    g = prob(B=1, T=256, H=2, L=9, rule=F.LL_GATED_DELTANET)
    with pytest.raises(ValueError, match="beta must hold"):
        F.ll_attn_fwd(g, *args(), x["beta"][:, :-1].contiguous(), x["o"], None, DUMMY, 0)
    # a state buffer of the wrong size, a workspace smaller than the size passed
    with pytest.raises(ValueError, match="state_out must hold"):
        F.ll_attn_fwd(p, *args(), None, x["o"], torch.zeros(10), DUMMY, 0)
    with pytest.raises(ValueError, match="workspace holds"):
        F.ll_attn_fwd(p, *args(), None, x["o"], None, torch.zeros(16, dtype=torch.uint8), 1 << 20)
    # decode: a short state, a pos of the wrong dtype
    with pytest.raises(ValueError, match="state must hold"):
        F.ll_decode_step(2, 2, 64, 64, 9, F.LL_BF16, F.LL_MAMBA2, 5, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None,
                         DUMMY, torch.zeros(100))
    with pytest.raises(TypeError, match="pos must be torch.int64"):
        F.ll_decode_step_ragged(2, 2, 64, 64, 9, F.LL_BF16, F.LL_MAMBA2, torch.zeros(2, dtype=torch.int32),
                                DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY, DUMMY)
    # the level-weight MLP with a transposed-size W2 buffer
    with pytest.raises(ValueError, match="w2 must hold"):
        F.ll_lambda_mlp(4, 15, 30, torch.zeros(4, 15), torch.zeros(15, 30), torch.zeros(29, 15), torch.zeros(15),
                        torch.zeros(4, 15))
