"""Log-linear (Fenwick-tree) attention forward pass for AMD MI355X (gfx950).

The compute lives in ``libllattn.so`` (hand-written HIP kernels behind the C
ABI of ``include/ll_attn.h``); this package only marshals torch tensors into
that ABI.  There is no fallback: if the library is missing, every call raises.

    from fenwick_tree_linear_amd import ll_attn_fwd, LLProblem
"""

from .binding import (  # noqa: F401
    LL_BF16,
    LL_F32,
    LL_GATED_DELTANET,
    LL_MAMBA2,
    LLError,
    LLProblem,
    attn_bwd,
    attn_fwd,
    attn_fwd_lambda_mlp,
    ccq_query,
    decode_state_tensor,
    lambda_mlp,
    lib_path,
    ll_attn_bwd,
    ll_attn_bwd_workspace_bytes,
    ll_attn_fwd,
    ll_attn_fwd_from_state,
    ll_attn_fwd_lambda_mlp,
    ll_attn_fwd_lambda_mlp_workspace_bytes,
    ll_attn_fwd_noalloc,
    ll_attn_fwd_workspace_bytes,
    ll_ccq_query,
    ll_ccq_query_workspace_bytes,
    ll_decode_state_bytes,
    ll_decode_step,
    ll_decode_step_ragged,
    ll_kernel_timing_enable,
    ll_kernel_timing_read,
    ll_lambda_mlp,
    ll_last_error,
    load_library,
)
