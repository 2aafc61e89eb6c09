/*
 * ll_attn.h -- C ABI of libllattn.so: log-linear (Fenwick-tree) attention
 * forward pass on AMD Instinct MI355X (gfx950).
 *
 * What is computed ("Log-Linear Attention", technical summary, section 2.2):
 *
 *   o_t = sum_{l=0}^{L-1} lambda_t^(l) q_t^T S_t^(l)
 *
 * where the prefix [0,t) is split by the Fenwick-tree decomposition into
 * disjoint power-of-two buckets (level l >= 1 holds 2^(l-1) tokens; level 0 is
 * token t itself) and S_t^(l) is the hidden state of bucket l.  Equivalently,
 * with 0-based tokens and lev(t,s) = bit_length(t XOR s) for s < t, lev(t,t) = 0:
 *
 *   o_t = sum_{s<=t} lambda_t^(lev(t,s)) * prod_{r=s+1}^{t} a_r * (q_t . k_s) * w_s
 *
 * The write w_s follows the host model the method is applied to (section 3):
 *   LL_MAMBA2          w_s = v_s                (scalar-gated state, S_t = a_t S_{t-1} + k_t v_t^T)
 *   LL_GATED_DELTANET  w_s = u_s = beta_s (v_s - a_s S_{s-1}^T k_s), the pseudo-value of the
 *                      gated delta rule S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T;
 *                      the level weights act on the read only.
 * The gate is passed as log a_t (a_t in (0,1], so log a_t <= 0; positive values
 * are accepted but can overflow exactly as the mathematics does).
 *
 * Conventions shared by every entry point:
 *  - All tensors are dense, row-major, in device memory owned by the caller.
 *    The library never allocates, frees or synchronises.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *  - Every argument is validated before any HIP call: a non-LL_OK return
 *    means nothing was enqueued; ll_last_error() then describes the problem.
 *  - LL_ERR_HIP reports a failed launch.  Faults inside kernels surface at the
 *    caller's next synchronisation of the stream.
 *  - No C++ exception crosses this interface.  The library is thread-safe for
 *    calls on different streams with disjoint output buffers.
 */
#ifndef LL_ATTN_H
#define LL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LL_OK = 0,
  LL_ERR_NULL = -1,        /* a required pointer is NULL */
  LL_ERR_SHAPE = -2,       /* sizes inconsistent (e.g. T % C != 0, too few levels) */
  LL_ERR_DTYPE = -3,       /* unknown io dtype */
  LL_ERR_UNSUPPORTED = -4, /* valid but not implemented (head size, chunk, rule) */
  LL_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
  LL_ERR_POSITION = -6,    /* decode position outside what the levels can hold */
  LL_ERR_HIP = -7          /* a HIP launch failed */
} ll_status;

typedef enum { LL_F32 = 0, LL_BF16 = 1 } ll_dtype;

typedef enum { LL_MAMBA2 = 0, LL_GATED_DELTANET = 1 } ll_rule;

/*
 * One prefill problem.
 *   B, T, H : batch, tokens, heads.       dk, dv : key and value head sizes.
 *   L       : number of Fenwick levels (level 0 = the token itself).  Outputs
 *             need T <= 2^(L-1); exporting the state of [0,T) needs
 *             T < 2^(L-1).  Levels beyond the largest used are ignored.
 *   C       : chunk size of the chunk-parallel form (section 2.3), a power of
 *             two with T % C == 0.  The result does not depend on C beyond
 *             rounding.
 *   io      : dtype of q, k, v and o.  Gates, lambda, beta and states are fp32.
 * Accepted (LL_ERR_UNSUPPORTED otherwise): dk and dv each in {16, 32, 64,
 *   128}, C in {16, 32, 64}, both io dtypes, T < 2^23.  The kernels run a
 *   square head D and their own chunk, since the read is the same sum
 *   whatever the head padding or the chunk size:
 *   - D = max(dk, dv), and 32 for bf16 at 16: q and k (dk < D) or v (dv < D)
 *     run on zero-padded copies in the workspace (zero key columns add nothing
 *     to q.k; the padded output columns are dropped);
 *   - bf16 runs chunks of at least 32 tokens (a bf16 matrix-core step
 *     contracts 32 values); where T is not a multiple of the run chunk, the
 *     inputs run zero-padded at the end (zero keys and values, no decay) and
 *     need L covering the padded length; the state export then needs T a
 *     multiple of the run chunk;
 *   - a C x D tile of the read stays within 8 KiB: larger chunks run halved
 *     (bf16 D = 128 at 32 tokens, fp32 D = 128 at 16).  For
 *     LL_GATED_DELTANET the pseudo-value pass runs at the requested chunk
 *     (fp32 D = 128: 16) and the read at the largest chunk that fits.
 */
typedef struct {
  int B, T, H, dk, dv, L, C;
  ll_dtype io;
  ll_rule rule;
} ll_problem;

/*
 * Bytes of device workspace ll_attn_fwd needs for `p` (0 is possible).  The
 * workspace holds, per head, the decayed key-value state of every aligned span
 * of chunks and its Fenwick combination (chunk-parallel form, section 2.3);
 * for LL_GATED_DELTANET also three [B,T,H,D] io-dtype row buffers: the
 * per-chunk WY factors (I + L)^-1 diag(beta e^G) K and (I + L)^-1 diag(beta) V
 * and the pseudo-values u the read runs on; and, for a problem not run in its
 * own shape, the padded copies of the inputs, the output and the states.
 * Errors: LL_ERR_NULL, and every validation error of ll_attn_fwd.
 */
ll_status ll_attn_fwd_workspace_bytes(const ll_problem* p, size_t* bytes);

/*
 * Chunk-parallel prefill (section 2.3, "training (parallel)": the hierarchical
 * mask evaluated chunk by chunk with matrix multiplications).
 *   q [B,T,H,dk], k [B,T,H,dk], v [B,T,H,dv]     io dtype
 *   log_gate [B,T,H]        fp32, log a_t
 *   lambda   [B,T,H,L]      fp32, per-token, per-head level weights
 *   beta     [B,T,H]        fp32, LL_GATED_DELTANET only (ignored otherwise);
 *                            the write strength, normally in (0, 1]; any finite
 *                            value is accepted
 *   o        [B,T,H,dv]     io dtype, written (may be NULL if state_out is not)
 *   state_out                nullable; if given, receives the per-level states
 *                            of [0,T) in the decode-state layout (see
 *                            ll_decode_state_bytes), decayed through token T-1
 *                            with all log-scales 0 and empty levels zeroed.
 *   workspace                device memory of >= ll_attn_fwd_workspace_bytes;
 *                            contents on entry do not matter.
 * q and lambda may be NULL when o is NULL.
 */
ll_status ll_attn_fwd(const ll_problem* p, const void* q, const void* k, const void* v,
                      const float* log_gate, const float* lambda, const float* beta, void* o,
                      void* state_out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * ll_attn_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and arguments without the workspace, which comes from a
 * scratch array inside the library instead.
 *   - The array holds LL_NOALLOC_SCRATCH_BYTES (64 MiB); a problem whose
 *     ll_attn_fwd_workspace_bytes exceeds it is rejected with
 *     LL_ERR_WORKSPACE before anything is enqueued.  64 MiB covers the
 *     LL_MAMBA2 prefill of 2 x 16 heads x 16384 tokens at dk = dv = 64
 *     (25 MB); the LL_GATED_DELTANET row buffers rarely fit.
 *   - Each GPU the library runs on holds its own copy of the array from the
 *     first call made with it current until the process ends; that first
 *     call also looks up the array's device address.
 *   - No part of the scratch needs to start at zero: every call writes all
 *     of it that it reads.  Nothing is allocated or freed by any call.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (on different streams, or from several threads without
 *     ordering) race on it and give undefined results.  Calls in one stream
 *     are ordered and safe.
 * The caller still owns and passes every input and output.
 */
#define LL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ll_status ll_attn_fwd_noalloc(const ll_problem* p, const void* q, const void* k, const void* v,
                              const float* log_gate, const float* lambda, const float* beta, void* o,
                              void* state_out, hipStream_t stream);

/*
 * Prefill of a segment that continues a sequence (section 2.2 and 2.3: the
 * buckets of positions before the segment are carried as per-level states),
 * for chunked prefill: tokens pos0 .. pos0 + T - 1, with the per-level
 * states of [0, pos0) in `state_in` (the decode-state layout below, e.g. the
 * export of the previous segment).  Everything else as ll_attn_fwd, whose
 * workspace size applies; o receives the outputs of the segment's tokens and
 * state_out (nullable) the states of [0, pos0 + T).  state_out may be
 * state_in (updated in place); no other overlap is allowed.
 * Requires (LL_ERR_POSITION otherwise) pos0 >= 0 and, for pos0 > 0,
 * T <= lowbit(pos0): the segment then never splits a prior bucket, and each
 * of its tokens sees the prior states at the set bits of pos0, above all of
 * the segment's own levels.  Outputs need pos0 + T <= 2^(L-1), exporting
 * pos0 + T < 2^(L-1) (LL_ERR_SHAPE).  pos0 > 0 needs state_in (LL_ERR_NULL);
 * pos0 == 0 is ll_attn_fwd (state_in ignored).  For LL_GATED_DELTANET the
 * pseudo-values of the segment continue the delta rule from the prior plain
 * state, the sum of the prior levels (they partition [0, pos0)).
 */
ll_status ll_attn_fwd_from_state(const ll_problem* p, int64_t pos0, const float* state_in, const void* q,
                                 const void* k, const void* v, const float* log_gate, const float* lambda,
                                 const float* beta, void* o, void* state_out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Size of the state the recurrent form carries between tokens ("Log-Linear
 * Attention", section 2.3, "inference": one hidden state per Fenwick level,
 * O(log T) of them, each dk x dv).
 * Bytes of one decode state: S_hat [B,H,L,dk,dv] fp32 followed by
 * sigma [B,H,L] fp32.  The true per-level state is exp(sigma_l) * S_hat_l
 * (the log-scale carries the decay lazily).  Level l >= 1 holds the bucket of
 * size 2^(l-1) of the prefix [0,pos) when bit l-1 of pos is set; the other
 * levels (and level 0) are ignored and may hold anything.
 * A zero-filled state is the state of the empty prefix (pos = 0).
 */
ll_status ll_decode_state_bytes(int B, int H, int dk, int dv, int L, size_t* bytes);

/*
 * One recurrent decode step at position `pos` (section 2.3, "inference":
 * O(log T) state and time per token), for all B*H heads at once.
 *   q, k [B,H,dk], v [B,H,dv]       io dtype, the new token
 *   log_gate [B,H], lambda [B,H,L]  fp32     beta [B,H] (LL_GATED_DELTANET only)
 *   o [B,H,dv]                      io dtype, written
 *   state                           in/out, the layout above, holding [0,pos) on
 *                                   entry and [0,pos+1) on return.
 * Requires pos + 1 < 2^(L-1) (LL_ERR_POSITION otherwise), so that the state
 * after the step still fits.  For LL_GATED_DELTANET beta must not be NULL
 * (LL_ERR_NULL); the step forms the pseudo-value u = beta (v - S^T k), with S
 * the sum of the live levels decayed through a_pos, reads with it, and
 * writes k u^T.
 * A state exported by ll_attn_fwd with the same rule resumes exactly.
 */
ll_status ll_decode_step(int B, int H, int dk, int dv, int L, ll_dtype io, ll_rule rule, int64_t pos,
                         const void* q, const void* k, const void* v, const float* log_gate,
                         const float* lambda, const float* beta, void* o, void* state,
                         hipStream_t stream);

/*
 * Level weights from the adaptive-decay MLP ("Adaptive memory decay for
 * log-linear attention", section "Method", LambdaMLPSoftplus), the producer of
 * the `lambda` argument above: for every row (a token and head),
 *   h = d W1,   lambda = softplus(h W2 + b),   softplus(z) = log(1 + e^z),
 * so every level of every token and head gets its own non-negative weight.
 *   d      [rows, L]        fp32, the per-level representation of each row
 *                           (rows = B*T*H for a prefill, B*H for a decode step;
 *                           row-major, so [B,T,H,L] is already this layout)
 *   w1     [L, hidden]      fp32, first layer (no bias)
 *   w2     [hidden, L]      fp32, second layer
 *   bias   [L]              fp32
 *   lambda [rows, L]        fp32, written; must not overlap d
 * The page uses hidden = 2L; implemented for 1 <= L <= 32, 1 <= hidden <= 64
 * (LL_ERR_UNSUPPORTED otherwise).  Computed in fp32: no activation lies between
 * the two layers, so the kernel forms the composite Wc = W1 W2 (L x L) and then
 * lambda = softplus(d Wc + b), one L x L product per row on the matrix cores
 * (the result agrees with the two layers to fp32 rounding).
 * rows == 0 enqueues nothing (pointers may then be NULL).
 */
ll_status ll_lambda_mlp(int64_t rows, int L, int hidden, const float* d, const float* w1, const float* w2,
                        const float* bias, float* lambda, hipStream_t stream);

/*
 * The chunk-parallel prefill with its level weights from the adaptive-decay
 * MLP ("Adaptive memory decay for log-linear attention", section "Method",
 * LambdaMLPSoftplus, and its "Complexity": the MLP acts on the O(log T) level
 * axis of each token): ll_attn_fwd with lambda = softplus((d W1) W2 + b)
 * taken from ll_lambda_mlp's arguments instead of a lambda tensor.
 *   d [B,T,H,L] fp32, the per-level representation of each token and head
 *   hidden, w1 [L, hidden], w2 [hidden, L], bias [L]: as ll_lambda_mlp
 *   every other argument as ll_attn_fwd (o must not be NULL)
 * For bf16 problems whose run shape has a head of at most 64 and chunks of at
 * least 32, with L <= 16, the read makes the weights of each chunk itself
 * (the composite Wc and the fp32 products of ll_lambda_mlp, in the same order)
 * and never writes them to memory; otherwise ll_lambda_mlp writes them into
 * the workspace first.  Either way the result is that of ll_lambda_mlp
 * followed by ll_attn_fwd, bit for bit (the same weights, the same blocks).
 * Workspace: ll_attn_fwd_lambda_mlp_workspace_bytes (the prefill's, plus
 * B*T*H*L floats when the weights go through memory).  Errors as ll_attn_fwd
 * and ll_lambda_mlp.
 */
ll_status ll_attn_fwd_lambda_mlp_workspace_bytes(const ll_problem* p, int hidden, size_t* bytes);
ll_status ll_attn_fwd_lambda_mlp(const ll_problem* p, const void* q, const void* k, const void* v,
                                 const float* log_gate, const float* d, int hidden, const float* w1, const float* w2,
                                 const float* bias, const float* beta, void* o, void* state_out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * The decode step for a batch whose sequences sit at different positions
 * (section 2.3, "inference", one token per sequence), for continuous batching:
 * as ll_decode_step, with
 *   pos [B]   int64 in device memory: the position of each sequence, read by
 *             the kernel (so a captured or replayed launch follows the values
 *             in memory); the caller advances them.
 * Positions are not visible to the host, so they are checked on the device:
 * a sequence with pos < 0 or pos + 1 >= 2^(L-1) gets NaN in every output of
 * its heads and its state is left unchanged.  Every other argument is
 * validated on the host as for ll_decode_step (LL_ERR_NULL for a NULL pos).
 */
ll_status ll_decode_step_ragged(int B, int H, int dk, int dv, int L, ll_dtype io, ll_rule rule, const int64_t* pos,
                                const void* q, const void* k, const void* v, const float* log_gate,
                                const float* lambda, const float* beta, void* o, void* state,
                                hipStream_t stream);

/*
 * The curvature-conditioned query ("Don't read everything: curvature-
 * conditioned query for linear attention", section 2, "Mechanism"), a
 * read-side correction applied before the read:
 *   q_clean_t = q_t - gamma_t Sigma_t q_t,   gamma_t = sigmoid(w_h . q_t + b_h),
 *   Sigma_t   = the covariance of keys 0..t of the head (population, no decay).
 * Pass q_clean as q to ll_attn_fwd: the contraction then applies to the read of
 * every level.
 *   q, k [B,T,H,dk]  io dtype        w [H,dk], b [H]  fp32, the gate of each head
 *   q_clean [B,T,H,dk]  io dtype, written (may be q itself)
 *   workspace  device memory of >= ll_ccq_query_workspace_bytes; contents on
 *              entry do not matter.
 * The running second moment comes from a chunk-parallel prefill with every
 * level weight 1 and no decay, the running key sum from a chunked fp32
 * prefix sum.  Implemented for the head sizes of ll_attn_fwd and T
 * a multiple of 16, T < 2^23 (LL_ERR_UNSUPPORTED otherwise).
 */
ll_status ll_ccq_query_workspace_bytes(int B, int T, int H, int dk, ll_dtype io, size_t* bytes);
ll_status ll_ccq_query(int B, int T, int H, int dk, ll_dtype io, const void* q, const void* k, const float* w,
                       const float* b, void* q_clean, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * Backward pass of the prefill for the LL_MAMBA2 write (training): given the
 * forward's inputs and the gradient dO of a loss at the output o, writes the
 * gradients of that loss with respect to every input ("Log-Linear Attention",
 * section 2.3: the masked form, whose pair weights are differentiated term by
 * term; section 3 trains through it):
 *   dq, dk [B,T,H,dk], dv [B,T,H,dv]   io dtype
 *   dlog_gate [B,T,H], dlambda [B,T,H,L]   fp32
 * With M[t,s] = lambda_t^{lev(t,s)} e^{G_t - G_s} for s <= t (G the running
 * sum of log_gate):
 *   dq_t = sum_s M[t,s] (dO_t . v_s) k_s      (the forward read of (dO, v, k))
 *   dv_s = sum_t M[t,s] (q_t . k_s) dO_t,     dk_s = sum_t M[t,s] (dO_t . v_s) q_t
 *   dlambda_t^l = sum over s at level l of e^{G_t - G_s} (q_t . k_s)(dO_t . v_s)
 *   dlog_gate_r = sum_{t >= r} (dO_t . o_t - k_t . dk_t)
 * dv and dk come from reads in which each source gathers the later tokens of
 * the one Fenwick bucket it reads at every level; dO . o and k . dk enter the
 * gate gradient in fp32, as sum_l lambda^l dlambda^l and v . dv.  `o` is not
 * read (it may be NULL).  Shapes as ll_attn_fwd (LL_ERR_UNSUPPORTED for
 * LL_GATED_DELTANET).  The workspace holds the forward's block states and
 * Fenwick nodes (of the dq read, then of (k, v)), two fp32 values per row, a
 * dk x dv fp32 state per block and block level (bit_length(blocks - 1) of them),
 * and max-depth chunk-level states per block; its contents on entry do not
 * matter.  Kernels run on `stream`, in order; the call returns after launching.
 */
ll_status ll_attn_bwd_workspace_bytes(const ll_problem* p, size_t* bytes);
ll_status ll_attn_bwd(const ll_problem* p, const void* q, const void* k, const void* v, const float* log_gate,
                      const float* lambda, const void* o, const void* dO, void* dq, void* dk, void* dv,
                      float* dlog_gate, float* dlambda, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Text of the last error on the calling thread; valid until its next call. */
const char* ll_last_error(void);

/*
 * Per-kernel timing, a measurement aid (off by default).  While enabled, each
 * kernel that the entry points launch is bracketed by two HIP
 * events recorded on the call's stream.  ll_kernel_timing_read() waits for the
 * recorded events, then reports for up to `capacity` kernels their name (a
 * static string: "ll_chunk_state", "ll_fenwick_scan", "ll_chunk_attn",
 * "ll_state_export", "ll_decode_step", "ll_gdn_wy", "ll_gdn_state",
 * "ll_lambda_mlp", "ll_prior_read", "ll_ccq", "ll_bwd"), the summed milliseconds and the launch
 * count, and clears the record.  Enabling creates HIP events lazily; timing
 * adds two event records per launch, so do not time throughput with it on.
 */
ll_status ll_kernel_timing_enable(int on);
ll_status ll_kernel_timing_read(const char** names, double* total_ms, int* launches, int capacity, int* count);

#ifdef __cplusplus
}
#endif

#endif /* LL_ATTN_H */
