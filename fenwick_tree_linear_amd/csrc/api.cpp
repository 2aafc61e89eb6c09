// api.cpp -- the C ABI of libllattn (declared in include/ll_attn.h):
// argument validation, workspace planning and the launch sequence.  Every
// check runs before the first HIP call, so a rejected call enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include <hip/hip_runtime.h>

#include "ll_attn.h"
#include "ll_launch.hpp"

using llattn::DecodeArgs;
using llattn::GdnArgs;
using llattn::PrefillArgs;

namespace {

thread_local char g_err[512] = "";

ll_status fail(ll_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

ll_status ok() {
  g_err[0] = '\0';
  return LL_OK;
}

int bit_length(int64_t x) {
  int n = 0;
  while (x > 0) {
    x >>= 1;
    ++n;
  }
  return n;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Enum arguments arrive from C callers as plain ints and may hold any value;
// they are read as ints, so that checking an out-of-range value is defined
// behaviour (loading it through the enum type would not be, in C++).
template <typename E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "the ABI's enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

// bf16 matrix-core steps contract 32 values: bf16 needs d >= 32 and C >= 32
bool supported_head(int d, ll_dtype io) {
  if (io == LL_BF16) return d == 32 || d == 64 || d == 128;
  return d == 16 || d == 32 || d == 64;
}

bool supported_chunk(int c, ll_dtype io) {
  if (io == LL_BF16) return c == 32 || c == 64;
  return c == 16 || c == 32 || c == 64;
}

constexpr int kMaxBlockChunks = 8;  // P <= 2^max_block_depth

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  int Cr;  // chunk size of the log-linear read (C, or smaller for Gated DeltaNet when a tile would not fit)
  int P, nb, nF, LS;
  size_t s_off, gs_off, f_off, gf_off, n16_off;
  size_t w_off, up_off, u_off;  // Gated DeltaNet: W, U' and the pseudo-values U
  size_t bytes;
};

// Validates a prefill problem and derives the block decomposition.
ll_status plan_prefill(const ll_problem* p, bool exporting, Plan* out) {
  if (!p) return fail(LL_ERR_NULL, "problem is NULL");
  const int io_v = enum_value(p->io), rule_v = enum_value(p->rule);
  if (io_v != LL_F32 && io_v != LL_BF16) return fail(LL_ERR_DTYPE, "unknown io dtype %d", io_v);
  if (rule_v != LL_MAMBA2 && rule_v != LL_GATED_DELTANET) return fail(LL_ERR_UNSUPPORTED, "unknown rule %d", rule_v);
  if (p->B < 1 || p->T < 1 || p->H < 1 || p->dk < 1 || p->dv < 1 || p->L < 1 || p->C < 1)
    return fail(LL_ERR_SHAPE, "sizes must be positive (B=%d T=%d H=%d dk=%d dv=%d L=%d C=%d)", p->B, p->T, p->H,
                p->dk, p->dv, p->L, p->C);
  if (!is_pow2(p->C)) return fail(LL_ERR_SHAPE, "chunk size C=%d is not a power of two", p->C);
  if (p->T % p->C != 0) return fail(LL_ERR_SHAPE, "T=%d is not a multiple of C=%d", p->T, p->C);
  if (p->L > 62) return fail(LL_ERR_SHAPE, "L=%d levels is more than positions can use", p->L);
  // outputs of positions t < T need levels up to bit_length(T-1)
  const int need = bit_length((int64_t)p->T - 1) + 1;
  if (p->L < need) return fail(LL_ERR_SHAPE, "T=%d needs at least %d levels, got L=%d", p->T, need, p->L);
  if (exporting && bit_length(p->T) > p->L - 1)
    return fail(LL_ERR_SHAPE, "exporting the state of [0,%d) needs at least %d levels, got L=%d", p->T,
                bit_length(p->T) + 1, p->L);
  if (p->dk != p->dv) return fail(LL_ERR_UNSUPPORTED, "dk=%d != dv=%d is not supported", p->dk, p->dv);
  if (!supported_head(p->dk, p->io))
    return fail(LL_ERR_UNSUPPORTED, "head size %d not supported for %s io", p->dk, p->io == LL_BF16 ? "bf16" : "fp32");
  if (!supported_chunk(p->C, p->io))
    return fail(LL_ERR_UNSUPPORTED, "chunk size C=%d not supported for %s io", p->C, p->io == LL_BF16 ? "bf16" : "fp32");
  const size_t esz = p->io == LL_BF16 ? 2 : 4;
  int Cr = p->C;
  if (p->rule == LL_GATED_DELTANET) {
    // the pseudo-value pass works on chunks of C; the read may use smaller ones
    while ((size_t)Cr * p->dk * esz > (size_t)llattn::kAttnTileBytesMax && supported_chunk(Cr / 2, p->io)) Cr /= 2;
  }
  if ((size_t)Cr * p->dk * esz > (size_t)llattn::kAttnTileBytesMax)
    return fail(LL_ERR_UNSUPPORTED, "a chunk tile of C=%d x d=%d %s values exceeds %d bytes", Cr, p->dk,
                p->io == LL_BF16 ? "bf16" : "fp32", llattn::kAttnTileBytesMax);
  if (need > llattn::kLevelsMax)
    return fail(LL_ERR_UNSUPPORTED, "T=%d needs %d levels; at most %d are supported", p->T, need, llattn::kLevelsMax);
  if ((int64_t)p->B * p->H * (p->T / p->C) > ((int64_t)1 << 31) - 1)
    return fail(LL_ERR_UNSUPPORTED, "problem too large for one launch");

  const int nc = p->T / Cr;
  const int depth_cap = 1 << llattn::max_block_depth(p->dk);
  int P = nc & -nc;  // lowest set bit: blocks tile the chunks exactly
  if (P > kMaxBlockChunks) P = kMaxBlockChunks;
  if (P > depth_cap) P = depth_cap;
  Plan pl;
  pl.Cr = Cr;
  pl.P = P;
  pl.nb = nc / P;
  pl.nF = pl.nb / 2;
  pl.LS = p->L < need ? p->L : need;
  const size_t bh = (size_t)p->B * p->H;
  const size_t dd = (size_t)p->dk * p->dv;
  size_t off = 0;
  pl.s_off = off;
  off = align256(off + bh * pl.nb * dd * sizeof(float));
  pl.gs_off = off;
  off = align256(off + bh * pl.nb * sizeof(float));
  pl.f_off = off;
  off = align256(off + bh * pl.nF * dd * sizeof(float));
  pl.gf_off = off;
  off = align256(off + bh * (pl.nF > 0 ? pl.nF : 1) * sizeof(float));
  pl.n16_off = 0;
  if (llattn::node_copies(p->io == LL_BF16 ? 1 : 0, p->dk) && pl.nb > 1) {  // bf16 copies of the nodes the read takes
    pl.n16_off = off;
    off = align256(off + bh * pl.nb * dd * 2);
  }
  pl.w_off = pl.up_off = pl.u_off = 0;
  if (p->rule == LL_GATED_DELTANET) {
    const size_t rows = (size_t)p->B * p->T * p->H * p->dk * esz;
    pl.w_off = off;
    off = align256(off + rows);
    pl.up_off = off;
    off = align256(off + rows);
    pl.u_off = off;
    off = align256(off + rows);
  }
  pl.bytes = off;
  *out = pl;
  return LL_OK;
}

// ---------------------------------------------------------- kernel timing
enum KernelId { K_CHUNK_STATE, K_FENWICK_SCAN, K_CHUNK_ATTN, K_STATE_EXPORT, K_DECODE_STEP, K_GDN_WY, K_GDN_STATE,
                K_LAMBDA_MLP, K_PRIOR_READ, K_CCQ, K_BWD, K_COUNT };
const char* const kKernelNames[K_COUNT] = {"ll_chunk_state", "ll_fenwick_scan", "ll_chunk_attn", "ll_state_export",
                                           "ll_decode_step", "ll_gdn_wy",       "ll_gdn_state",   "ll_lambda_mlp", "ll_prior_read", "ll_ccq", "ll_bwd"};

struct Timing {
  std::mutex mu;
  std::atomic<bool> on{false};  // read without the lock on every launch
  std::vector<hipEvent_t> pool;  // free events
  struct Pending {
    int kernel;
    hipEvent_t start, stop;
  };
  std::vector<Pending> pending;
  double total_ms[K_COUNT] = {};
  int launches[K_COUNT] = {};
};
Timing g_timing;

hipEvent_t take_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launches one kernel through `fn`, bracketed by events when timing is on.
template <typename Fn>
hipError_t timed(int kernel, hipStream_t stream, Fn fn) {
  if (!g_timing.on.load(std::memory_order_acquire)) return fn();
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (!g_timing.on.load(std::memory_order_relaxed)) return fn();  // switched off meanwhile
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) {  // no timing for this launch; keep whichever event was made
    if (a) g_timing.pool.push_back(a);
    if (b) g_timing.pool.push_back(b);
    return fn();
  }
  if (hipEventRecord(a, stream) != hipSuccess) {  // no timing for this launch
    g_timing.pool.push_back(a);
    g_timing.pool.push_back(b);
    return fn();
  }
  hipError_t e = fn();
  if (hipEventRecord(b, stream) != hipSuccess) {
    g_timing.pool.push_back(a);
    g_timing.pool.push_back(b);
    return e;
  }
  g_timing.pending.push_back({kernel, a, b});
  return e;
}

}  // namespace

extern "C" {

ll_status ll_kernel_timing_enable(int on) {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  g_timing.on.store(on != 0, std::memory_order_release);
  return ok();
}

ll_status ll_kernel_timing_read(const char** names, double* total_ms, int* launches, int capacity, int* count) {
  if (!count || (capacity > 0 && (!names || !total_ms || !launches)))
    return fail(LL_ERR_NULL, "output arrays must not be NULL");
  std::lock_guard<std::mutex> lock(g_timing.mu);
  for (auto& p : g_timing.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess)
      return fail(LL_ERR_HIP, "reading kernel timing events failed");
    g_timing.total_ms[p.kernel] += ms;
    g_timing.launches[p.kernel] += 1;
    g_timing.pool.push_back(p.start);
    g_timing.pool.push_back(p.stop);
  }
  g_timing.pending.clear();
  int n = 0;
  for (int kk = 0; kk < K_COUNT; ++kk) {
    if (g_timing.launches[kk] == 0) continue;
    if (n < capacity) {
      names[n] = kKernelNames[kk];
      total_ms[n] = g_timing.total_ms[kk];
      launches[n] = g_timing.launches[kk];
    }
    ++n;
    g_timing.total_ms[kk] = 0.0;
    g_timing.launches[kk] = 0;
  }
  *count = n;
  return ok();
}

const char* ll_last_error(void) { return g_err; }

ll_status ll_attn_fwd_workspace_bytes(const ll_problem* p, size_t* bytes) {
  if (!bytes) return fail(LL_ERR_NULL, "bytes is NULL");
  Plan pl;
  // plan as if exporting is not requested; the workspace does not depend on it
  ll_status st = plan_prefill(p, false, &pl);
  if (st != LL_OK) return st;
  *bytes = pl.bytes;
  return ok();
}

// ------------------------------------------------------ allocation-free prefill
// The workspace of ll_attn_fwd_noalloc: one copy of this array on every GPU the
// library runs on, alive until the process ends.  In host code its name is only
// a stand-in for the device symbol; host code uses the device address that
// hipGetSymbolAddress returns for the current device, never the name itself.
static __device__ __align__(256) char scratch[LL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept.
ll_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LL_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LL_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(LL_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    if (!ptr) return fail(LL_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LL_OK;
}

// Both prefill entry points: a segment at positions pos0 .. pos0 + T - 1 whose
// earlier positions (if any) are summarised by state_in.
// reuse_states: the workspace already holds the block states and Fenwick nodes
// of this (k, v, log_gate) from the previous call (a Mamba-2 read with other
// q or level weights); only the read runs.
ll_status run_prefill(const ll_problem* p, int64_t pos0, const float* state_in, const void* q, const void* k,
                      const void* v, const float* log_gate, const float* lambda, const float* beta, void* o,
                      void* state_out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                      bool reuse_states = false, bool noalloc = false) {
  if (reuse_states && (p->rule != LL_MAMBA2 || pos0 != 0 || state_out))
    return fail(LL_ERR_UNSUPPORTED, "reusing block states is only for a plain Mamba-2 read");
  Plan pl;
  ll_status st = plan_prefill(p, state_out != nullptr, &pl);
  if (st != LL_OK) return st;
  if (pos0 < 0) return fail(LL_ERR_POSITION, "pos0=%lld is negative", (long long)pos0);
  if (pos0 > 0) {
    if (!state_in) return fail(LL_ERR_NULL, "state_in must not be NULL when pos0 > 0");
    if ((pos0 & -pos0) < p->T)
      return fail(LL_ERR_POSITION, "pos0=%lld: the segment of T=%d tokens must fit below the lowest set bit of pos0",
                  (long long)pos0, p->T);
    if (pos0 > ((int64_t)1 << 61)) return fail(LL_ERR_POSITION, "pos0=%lld is too large", (long long)pos0);
    const int64_t end = pos0 + p->T;
    if (bit_length(end - 1) + 1 > p->L)
      return fail(LL_ERR_SHAPE, "positions up to %lld need at least %d levels, got L=%d", (long long)(end - 1),
                  bit_length(end - 1) + 1, p->L);
    if (state_out && bit_length(end) > p->L - 1)
      return fail(LL_ERR_SHAPE, "exporting the state of [0,%lld) needs at least %d levels, got L=%d", (long long)end,
                  bit_length(end) + 1, p->L);
  }
  if (!k || !v || !log_gate) return fail(LL_ERR_NULL, "k, v and log_gate must not be NULL");
  if (!o && !state_out) return fail(LL_ERR_NULL, "o and state_out are both NULL: nothing to compute");
  if (o && (!q || !lambda)) return fail(LL_ERR_NULL, "q and lambda must not be NULL when o is requested");
  if (p->rule == LL_GATED_DELTANET && !beta) return fail(LL_ERR_NULL, "beta must not be NULL for Gated DeltaNet");
  if (noalloc) {
    if (pl.bytes > LL_NOALLOC_SCRATCH_BYTES)
      return fail(LL_ERR_WORKSPACE, "this problem needs %zu bytes of workspace; the allocation-free prefill has %zu",
                  pl.bytes, (size_t)LL_NOALLOC_SCRATCH_BYTES);
    // validation is over: only now touch the device, for the scratch address
    st = scratch_of_current_device(&workspace);
    if (st != LL_OK) return st;
  } else {
    if (workspace_bytes < pl.bytes)
      return fail(LL_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes,
                  pl.bytes);
    if (pl.bytes > 0 && !workspace) return fail(LL_ERR_WORKSPACE, "workspace is NULL");
  }

  char* ws = static_cast<char*>(workspace);
  PrefillArgs a;
  a.B = p->B;
  a.T = p->T;
  a.H = p->H;
  a.L = p->L;
  a.LS = pl.LS;
  a.P = pl.P;
  a.nb = pl.nb;
  a.nF = pl.nF;
  a.q = q;
  a.k = k;
  a.v = p->rule == LL_GATED_DELTANET ? static_cast<const void*>(ws + pl.u_off) : v;
  a.g = log_gate;
  a.lam = lambda;
  a.o = o;
  a.S = reinterpret_cast<float*>(ws + pl.s_off);
  a.GS = reinterpret_cast<float*>(ws + pl.gs_off);
  a.F = reinterpret_cast<float*>(ws + pl.f_off);
  a.GF = reinterpret_cast<float*>(ws + pl.gf_off);
  a.N16 = (llattn::node_copies(p->io == LL_BF16 ? 1 : 0, p->dk) && pl.nb > 1) ? static_cast<void*>(ws + pl.n16_off)
                                                                                : nullptr;
  a.state = static_cast<float*>(state_out);
  a.state_in = pos0 > 0 ? state_in : nullptr;
  a.pos0 = pos0;
  const int io = p->io == LL_BF16 ? 1 : 0;
  const int D = p->dk;

  hipError_t e = hipSuccess;
  if (p->rule == LL_GATED_DELTANET) {
    // the pseudo-values U of the delta rule, then the read of (q, k, U)
    GdnArgs gd;
    gd.B = p->B;
    gd.T = p->T;
    gd.H = p->H;
    gd.k = k;
    gd.v = v;
    gd.g = log_gate;
    gd.beta = beta;
    gd.W = ws + pl.w_off;
    gd.Up = ws + pl.up_off;
    gd.U = ws + pl.u_off;
    gd.L = p->L;
    gd.state_in = a.state_in;
    gd.pos0 = a.pos0;
    e = timed(K_GDN_WY, stream, [&] { return llattn::launch_gdn_wy(io, D, p->C, gd, stream); });
    if (e == hipSuccess) e = timed(K_GDN_STATE, stream, [&] { return llattn::launch_gdn_state(io, D, p->C, gd, stream); });
  }
  const int C = pl.Cr;
  if (e == hipSuccess && !reuse_states)
    e = timed(K_CHUNK_STATE, stream, [&] { return llattn::launch_block_state(io, D, C, a, stream); });
  if (e == hipSuccess && a.nb > 1 && !reuse_states)
    e = timed(K_FENWICK_SCAN, stream, [&] { return llattn::launch_fenwick_scan(D, a, stream); });
  if (e == hipSuccess && o)
    e = timed(K_CHUNK_ATTN, stream, [&] { return llattn::launch_chunk_attn(io, D, C, a, stream); });
  if (e == hipSuccess && o && pos0 > 0)
    e = timed(K_PRIOR_READ, stream, [&] { return llattn::launch_prior_read(io, D, C, a, stream); });
  if (e == hipSuccess && state_out)
    e = timed(K_STATE_EXPORT, stream, [&] { return llattn::launch_state_export(D, C, a, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

ll_status ll_attn_fwd(const ll_problem* p, const void* q, const void* k, const void* v, const float* log_gate,
                      const float* lambda, const float* beta, void* o, void* state_out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return run_prefill(p, 0, nullptr, q, k, v, log_gate, lambda, beta, o, state_out, workspace, workspace_bytes, stream);
}

ll_status ll_attn_fwd_noalloc(const ll_problem* p, const void* q, const void* k, const void* v, const float* log_gate,
                              const float* lambda, const float* beta, void* o, void* state_out, hipStream_t stream) {
  return run_prefill(p, 0, nullptr, q, k, v, log_gate, lambda, beta, o, state_out, nullptr, 0, stream, false, true);
}

ll_status ll_attn_fwd_from_state(const ll_problem* p, int64_t pos0, const float* state_in, const void* q,
                                 const void* k, const void* v, const float* log_gate, const float* lambda,
                                 const float* beta, void* o, void* state_out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return run_prefill(p, pos0, state_in, q, k, v, log_gate, lambda, beta, o, state_out, workspace, workspace_bytes,
                     stream);
}

ll_status ll_decode_state_bytes(int B, int H, int dk, int dv, int L, size_t* bytes) {
  if (!bytes) return fail(LL_ERR_NULL, "bytes is NULL");
  if (B < 1 || H < 1 || dk < 1 || dv < 1 || L < 2)
    return fail(LL_ERR_SHAPE, "sizes must be positive and L >= 2 (B=%d H=%d dk=%d dv=%d L=%d)", B, H, dk, dv, L);
  *bytes = (size_t)B * H * L * ((size_t)dk * dv + 1) * sizeof(float);
  return ok();
}

namespace {

// Shared by both decode entry points: everything but the position.
ll_status check_decode(int B, int H, int dk, int dv, int L, ll_dtype io, ll_rule rule, const void* q, const void* k,
                       const void* v, const float* log_gate, const float* lambda, const float* beta, void* o,
                       void* state) {
  const int io_v = enum_value(io), rule_v = enum_value(rule);
  if (io_v != LL_F32 && io_v != LL_BF16) return fail(LL_ERR_DTYPE, "unknown io dtype %d", io_v);
  if (rule_v != LL_MAMBA2 && rule_v != LL_GATED_DELTANET) return fail(LL_ERR_UNSUPPORTED, "unknown rule %d", rule_v);
  if (B < 1 || H < 1 || dk < 1 || dv < 1 || L < 2)
    return fail(LL_ERR_SHAPE, "sizes must be positive and L >= 2 (B=%d H=%d dk=%d dv=%d L=%d)", B, H, dk, dv, L);
  if (L > 32) return fail(LL_ERR_UNSUPPORTED, "L=%d: at most 32 decode levels are supported", L);
  if (!q || !k || !v || !log_gate || !lambda || !o || !state)
    return fail(LL_ERR_NULL, "q, k, v, log_gate, lambda, o and state must not be NULL");
  if (rule == LL_GATED_DELTANET && !beta) return fail(LL_ERR_NULL, "beta must not be NULL for Gated DeltaNet");
  if (dk != dv) return fail(LL_ERR_UNSUPPORTED, "dk=%d != dv=%d is not supported", dk, dv);
  if (dk != 16 && dk != 32 && dk != 64 && dk != 128) return fail(LL_ERR_UNSUPPORTED, "head size %d not supported", dk);
  return LL_OK;
}

ll_status launch_decode(int B, int H, int dk, int L, ll_dtype io, ll_rule rule, int64_t pos, const int64_t* pos_dev,
                        const void* q, const void* k, const void* v, const float* log_gate, const float* lambda,
                        const float* beta, void* o, void* state, hipStream_t stream) {
  DecodeArgs a;
  a.B = B;
  a.H = H;
  a.L = L;
  a.pos = pos;
  a.pos_dev = pos_dev;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = log_gate;
  a.lam = lambda;
  a.beta = rule == LL_GATED_DELTANET ? beta : nullptr;
  a.o = o;
  a.state = static_cast<float*>(state);
  const int code = io == LL_BF16 ? 1 : 0;
  hipError_t e = timed(K_DECODE_STEP, stream, [&] { return llattn::launch_decode_step(code, dk, a, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

ll_status ll_decode_step(int B, int H, int dk, int dv, int L, ll_dtype io, ll_rule rule, int64_t pos, const void* q,
                         const void* k, const void* v, const float* log_gate, const float* lambda, const float* beta,
                         void* o, void* state, hipStream_t stream) {
  ll_status st = check_decode(B, H, dk, dv, L, io, rule, q, k, v, log_gate, lambda, beta, o, state);
  if (st != LL_OK) return st;
  if (pos < 0) return fail(LL_ERR_POSITION, "pos=%lld is negative", (long long)pos);
  if (pos + 1 >= ((int64_t)1 << (L - 1)))
    return fail(LL_ERR_POSITION, "pos=%lld: the state of [0,pos+1) does not fit in L=%d levels", (long long)pos, L);
  return launch_decode(B, H, dk, L, io, rule, pos, nullptr, q, k, v, log_gate, lambda, beta, o, state, stream);
}

ll_status ll_decode_step_ragged(int B, int H, int dk, int dv, int L, ll_dtype io, ll_rule rule, const int64_t* pos,
                                const void* q, const void* k, const void* v, const float* log_gate,
                                const float* lambda, const float* beta, void* o, void* state, hipStream_t stream) {
  ll_status st = check_decode(B, H, dk, dv, L, io, rule, q, k, v, log_gate, lambda, beta, o, state);
  if (st != LL_OK) return st;
  if (!pos) return fail(LL_ERR_NULL, "pos must not be NULL");
  return launch_decode(B, H, dk, L, io, rule, 0, pos, q, k, v, log_gate, lambda, beta, o, state, stream);
}

ll_status ll_lambda_mlp(int64_t rows, int L, int hidden, const float* d, const float* w1, const float* w2,
                        const float* bias, float* lambda, hipStream_t stream) {
  if (rows < 0 || L < 1 || hidden < 1)
    return fail(LL_ERR_SHAPE, "rows must be >= 0, L and hidden >= 1 (rows=%lld L=%d hidden=%d)", (long long)rows, L,
                hidden);
  if (L > 32 || hidden > 64)
    return fail(LL_ERR_UNSUPPORTED, "L=%d, hidden=%d: at most 32 levels and 64 hidden units are supported", L, hidden);
  if (rows > ((int64_t)1 << 36)) return fail(LL_ERR_UNSUPPORTED, "rows=%lld is too many for one launch", (long long)rows);
  if (rows == 0) return ok();  // nothing to compute
  if (!d || !w1 || !w2 || !bias || !lambda) return fail(LL_ERR_NULL, "d, w1, w2, bias and lambda must not be NULL");
  if ((const float*)lambda == d) return fail(LL_ERR_SHAPE, "lambda must not alias d");
  hipError_t e = timed(K_LAMBDA_MLP, stream,
                       [&] { return llattn::launch_lambda_mlp(rows, L, hidden, d, w1, w2, bias, lambda, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

namespace {

// The curvature-conditioned query: two prefills with all level weights 1 and
// no decay give the running sums it needs; their buffers, then the prefill
// workspace.
struct CcqPlan {
  ll_problem p;
  size_t ones_off, zeros_off, kkq_off, csum_off, fwd_off, fwd_bytes, bytes;
};

ll_status plan_ccq(int B, int T, int H, int dk, ll_dtype io, CcqPlan* out) {
  const int io_v = enum_value(io);
  if (io_v != LL_F32 && io_v != LL_BF16) return fail(LL_ERR_DTYPE, "unknown io dtype %d", io_v);
  if (B < 1 || T < 1 || H < 1 || dk < 1)
    return fail(LL_ERR_SHAPE, "sizes must be positive (B=%d T=%d H=%d dk=%d)", B, T, H, dk);
  if (!supported_head(dk, io))
    return fail(LL_ERR_UNSUPPORTED, "head size %d not supported for %s io", dk, io == LL_BF16 ? "bf16" : "fp32");
  const size_t esz = io == LL_BF16 ? 2 : 4;
  int C = 0;
  for (int c : {64, 32, 16})
    if (!C && supported_chunk(c, io) && T % c == 0 && (size_t)c * dk * esz <= (size_t)llattn::kAttnTileBytesMax) C = c;
  if (!C) return fail(LL_ERR_UNSUPPORTED, "T=%d is not a multiple of a supported chunk size for head size %d", T, dk);
  CcqPlan c;
  c.p.B = B;
  c.p.T = T;
  c.p.H = H;
  c.p.dk = c.p.dv = dk;
  c.p.L = bit_length((int64_t)T - 1) + 1;
  if (c.p.L < 2) c.p.L = 2;
  c.p.C = C;
  c.p.io = io;
  c.p.rule = LL_MAMBA2;
  Plan pl;
  ll_status st = plan_prefill(&c.p, false, &pl);
  if (st != LL_OK) return st;
  const size_t rows = (size_t)B * T * H;
  size_t off = 0;
  c.ones_off = off;
  off = align256(off + rows * c.p.L * 4);
  c.zeros_off = off;
  off = align256(off + rows * 4);
  c.kkq_off = off;
  off = align256(off + rows * dk * esz);
  c.csum_off = off;  // per-chunk key sums, [B,H,T/C,dk] fp32
  off = align256(off + (size_t)B * H * (T / C) * dk * 4);
  c.fwd_off = off;
  c.fwd_bytes = pl.bytes;
  c.bytes = off + pl.bytes;
  *out = c;
  return LL_OK;
}

}  // namespace

ll_status ll_ccq_query_workspace_bytes(int B, int T, int H, int dk, ll_dtype io, size_t* bytes) {
  if (!bytes) return fail(LL_ERR_NULL, "bytes is NULL");
  CcqPlan c;
  ll_status st = plan_ccq(B, T, H, dk, io, &c);
  if (st != LL_OK) return st;
  *bytes = c.bytes;
  return ok();
}

ll_status ll_ccq_query(int B, int T, int H, int dk, ll_dtype io, const void* q, const void* k, const float* w,
                       const float* b, void* q_clean, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  CcqPlan c;
  ll_status st = plan_ccq(B, T, H, dk, io, &c);
  if (st != LL_OK) return st;
  if (!q || !k || !w || !b || !q_clean) return fail(LL_ERR_NULL, "q, k, w, b and q_clean must not be NULL");
  if (workspace_bytes < c.bytes)
    return fail(LL_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, c.bytes);
  if (!workspace) return fail(LL_ERR_WORKSPACE, "workspace is NULL");
  char* ws = static_cast<char*>(workspace);
  float* ones = reinterpret_cast<float*>(ws + c.ones_off);
  float* zeros = reinterpret_cast<float*>(ws + c.zeros_off);
  void* kkq = ws + c.kkq_off;
  float* csum = reinterpret_cast<float*>(ws + c.csum_off);
  const int code = io == LL_BF16 ? 1 : 0;
  hipError_t e = timed(K_CCQ, stream, [&] { return llattn::launch_ccq_fill((int64_t)B * T * H, c.p.L, ones, zeros, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  // sum_{j<=t} (k_j . q_t) k_j
  st = run_prefill(&c.p, 0, nullptr, q, k, k, zeros, ones, nullptr, kkq, nullptr, ws + c.fwd_off, c.fwd_bytes, stream);
  if (st != LL_OK) return st;
  // sum_{j<=t} k_j: chunk sums and their prefix over the chunks, the rest in the combine
  e = timed(K_CCQ, stream, [&] { return llattn::launch_ccq_ksum(code, dk, B, T, H, c.p.C, k, csum, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  e = timed(K_CCQ, stream, [&] {
    return llattn::launch_ccq_combine(code, dk, B, T, H, c.p.C, q, k, kkq, csum, w, b, q_clean, stream);
  });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

namespace {

// The backward pass: the forward's block states and Fenwick nodes of (v, k),
// the per-row terms of the gate gradient, the reverse bucket states (block
// shares, then bucket sums, and their transposes), the per-block gate sums,
// and the chunk-level states of the walks where they do not fit in LDS.
struct BwdPlan {
  Plan pl;
  int nbl;  // block levels: bit_length(nb - 1)
  size_t fwd_off, doo_off, din_off, w_off, wt_off, bt_off, scratch_off, bytes;
};

ll_status plan_bwd(const ll_problem* p, BwdPlan* out) {
  Plan pl;
  ll_status st = plan_prefill(p, false, &pl);
  if (st != LL_OK) return st;
  if (p->rule != LL_MAMBA2) return fail(LL_ERR_UNSUPPORTED, "the backward pass is implemented for the Mamba-2 write");
  BwdPlan c;
  c.pl = pl;
  c.nbl = bit_length((int64_t)pl.nb - 1);
  const size_t bh = (size_t)p->B * p->H, rows = (size_t)p->B * p->T * p->H;
  const size_t dd = (size_t)p->dk * p->dv;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  c.fwd_off = take(pl.bytes);
  c.doo_off = take(rows * 4);
  c.din_off = take(rows * 4);
  c.w_off = take(bh * pl.nb * (size_t)c.nbl * dd * 4);
  c.wt_off = take(bh * pl.nb * (size_t)c.nbl * dd * 4);
  c.bt_off = take(bh * pl.nb * 4);
  c.scratch_off = take(llattn::bwd_states_in_lds(p->dk) ? 0
                                                        : bh * pl.nb * (size_t)llattn::max_block_depth(p->dk) * dd * 4);
  c.bytes = off;
  *out = c;
  return LL_OK;
}

}  // namespace

ll_status ll_attn_bwd_workspace_bytes(const ll_problem* p, size_t* bytes) {
  if (!bytes) return fail(LL_ERR_NULL, "bytes is NULL");
  BwdPlan c;
  ll_status st = plan_bwd(p, &c);
  if (st != LL_OK) return st;
  *bytes = c.bytes;
  return ok();
}

ll_status ll_attn_bwd(const ll_problem* p, const void* q, const void* k, const void* v, const float* log_gate,
                      const float* lambda, const void* o, const void* dO, void* dq, void* dk, void* dv,
                      float* dlog_gate, float* dlambda, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  (void)o;  // dO . o is formed from the level gradients: sum_l lambda^l dlambda^l
  BwdPlan c;
  ll_status st = plan_bwd(p, &c);
  if (st != LL_OK) return st;
  if (!q || !k || !v || !log_gate || !lambda || !dO)
    return fail(LL_ERR_NULL, "q, k, v, log_gate, lambda and dO must not be NULL");
  if (!dq || !dk || !dv || !dlog_gate || !dlambda)
    return fail(LL_ERR_NULL, "dq, dk, dv, dlog_gate and dlambda must not be NULL");
  if (workspace_bytes < c.bytes)
    return fail(LL_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, c.bytes);
  if (!workspace) return fail(LL_ERR_WORKSPACE, "workspace is NULL");
  char* ws = static_cast<char*>(workspace);
  const Plan& pl = c.pl;
  const int io = p->io == LL_BF16 ? 1 : 0;
  const int D = p->dk;

  // the forward's block states and Fenwick nodes of (v, k): the transposed
  // states of (k, v), which the forward walk reads as S dO
  PrefillArgs f;
  f.B = p->B;
  f.T = p->T;
  f.H = p->H;
  f.L = p->L;
  f.LS = pl.LS;
  f.P = pl.P;
  f.nb = pl.nb;
  f.nF = pl.nF;
  f.q = nullptr;
  f.k = v;
  f.v = k;
  f.g = log_gate;
  f.lam = lambda;
  f.o = nullptr;
  f.S = reinterpret_cast<float*>(ws + c.fwd_off + pl.s_off);
  f.GS = reinterpret_cast<float*>(ws + c.fwd_off + pl.gs_off);
  f.F = reinterpret_cast<float*>(ws + c.fwd_off + pl.f_off);
  f.GF = reinterpret_cast<float*>(ws + c.fwd_off + pl.gf_off);
  f.N16 = nullptr;
  f.state = nullptr;
  f.state_in = nullptr;
  f.pos0 = 0;
  hipError_t e = timed(K_BWD, stream, [&] { return llattn::launch_block_state(io, D, pl.Cr, f, stream); });
  if (e == hipSuccess && pl.nb > 1) e = timed(K_BWD, stream, [&] { return llattn::launch_fenwick_scan(D, f, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));

  llattn::BwdArgs a;
  a.B = p->B;
  a.T = p->T;
  a.H = p->H;
  a.D = D;
  a.L = p->L;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = log_gate;
  a.lam = lambda;
  a.dO = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_gate = dlog_gate;
  a.dlambda = dlambda;
  llattn::BwdFwdNodes n;
  n.nb = pl.nb;
  n.nF = pl.nF;
  n.P = pl.P;
  n.LS = pl.LS;
  n.S = f.S;
  n.GS = f.GS;
  n.F = f.F;
  n.GF = f.GF;
  llattn::BwdWork w;
  w.dOo = reinterpret_cast<float*>(ws + c.doo_off);
  w.din = reinterpret_cast<float*>(ws + c.din_off);
  w.W = reinterpret_cast<float*>(ws + c.w_off);
  w.WT = reinterpret_cast<float*>(ws + c.wt_off);
  w.BT = reinterpret_cast<float*>(ws + c.bt_off);
  w.nbl = c.nbl;
  w.scratch = llattn::bwd_states_in_lds(D) ? nullptr : reinterpret_cast<float*>(ws + c.scratch_off);
  // the forward walk; the reverse bucket states; the reverse walk; the gate's later blocks
  for (int pass = 0; pass < 4 && e == hipSuccess; ++pass)
    e = timed(K_BWD, stream, [&] { return llattn::launch_bwd_native(io, D, pl.Cr, a, n, w, pass, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
