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

// Head sizes (each of dk and dv) and chunk sizes a caller may pass.
bool accepted_head(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool accepted_chunk(int c) { return c == 16 || c == 32 || c == 64; }

// The square head size the kernels run a problem at: dk and dv zero-padded to
// the larger, and bf16 d = 16 to the 32 values one bf16 matrix-core step
// contracts (zero key columns add nothing to q.k; zero value columns give
// output columns that are dropped).
int run_head(int dk, int dv, ll_dtype io) {
  const int d = dk > dv ? dk : dv;
  return (io == LL_BF16 && d < 32) ? 32 : d;
}

// Chunks the kernels run natively for an io dtype.
bool native_chunk(int c, ll_dtype io) { return io == LL_BF16 ? (c == 32 || c == 64) : accepted_chunk(c); }

// The chunk the kernels run for a requested chunk C at run head size D.  The
// read is the same sum whatever the chunk size, so: a bf16 step contracts 32
// tokens (bf16 C = 16 runs 32-token chunks), and a C x D tile of the read must
// fit its LDS stage (larger chunks run halved).  Gated DeltaNet's pseudo-value
// pass runs the chunk it has for D (bf16: 32 or 64; fp32 at D = 128: 16).
int run_chunk(int c, int D, ll_dtype io, ll_rule rule) {
  const size_t esz = io == LL_BF16 ? 2 : 4;
  if (io == LL_BF16 && c < 32) c = 32;
  if (rule == LL_GATED_DELTANET) return (io == LL_F32 && D == 128) ? 16 : c;
  while ((size_t)c * D * esz > (size_t)llattn::kAttnTileBytesMax && native_chunk(c / 2, io)) c /= 2;
  return c;
}

constexpr int kMaxBlockChunks = 16;  // P <= 2^read_block_depth (or the depth a caller asks for)
// Blocks per prefill below which blocks of 16 chunks would leave CUs of the
// persistent read idle (the MI355X has 256): then blocks of 8.
constexpr int64_t kReadBlocksMin = 256;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  ll_problem r;  // the problem the kernels run: square head, run chunk and (padded) length
  int Cr;        // chunk size of the log-linear read (r.C, or smaller for Gated DeltaNet when a tile would not fit)
  int P, nb, nF, LS;
  size_t s_off, gs_off, f_off, gf_off, n16_off;
  size_t w_off, up_off, u_off;  // Gated DeltaNet: W, U' and the pseudo-values U
  // copies of the caller's tensors in the run shape, where it differs
  bool pad_qk, pad_v, pad_t, pad_state;
  size_t qp_off, kp_off, vp_off, op_off, gp_off, lp_off, bp_off, sin_off, sout_off;
  size_t bytes;
};

// Validates a prefill problem and derives the run problem, the block
// decomposition and the workspace.  The workspace does not depend on
// `exporting` (which only adds checks).
ll_status plan_prefill(const ll_problem* p, bool exporting, Plan* out, int depth = -1) {
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
  if (!accepted_head(p->dk) || !accepted_head(p->dv))
    return fail(LL_ERR_UNSUPPORTED, "head sizes dk=%d, dv=%d: each must be 16, 32, 64 or 128", p->dk, p->dv);
  if (!accepted_chunk(p->C)) return fail(LL_ERR_UNSUPPORTED, "chunk size C=%d not supported (16, 32 or 64)", p->C);
  const size_t esz = p->io == LL_BF16 ? 2 : 4;
  ll_problem r = *p;
  r.dk = r.dv = run_head(p->dk, p->dv, p->io);
  r.C = run_chunk(p->C, r.dk, p->io, p->rule);
  r.T = (p->T + r.C - 1) / r.C * r.C;
  const int D = r.dk;
  if (r.T != p->T) {
    if (exporting)
      return fail(LL_ERR_UNSUPPORTED, "exporting the state needs T a multiple of %d for %s io (T=%d)", r.C,
                  p->io == LL_BF16 ? "bf16" : "fp32", p->T);
    if (bit_length((int64_t)r.T - 1) + 1 > p->L)
      return fail(LL_ERR_UNSUPPORTED, "T=%d runs padded to %d tokens (%d-token chunks), which needs L >= %d", p->T,
                  r.T, r.C, bit_length((int64_t)r.T - 1) + 1);
  }
  int Cr = r.C;
  if (p->rule == LL_GATED_DELTANET) {
    // the pseudo-value pass works on chunks of r.C; the read may use smaller ones
    while ((size_t)Cr * D * esz > (size_t)llattn::kAttnTileBytesMax && native_chunk(Cr / 2, p->io)) Cr /= 2;
  }
  if ((size_t)Cr * D * esz > (size_t)llattn::kAttnTileBytesMax)
    return fail(LL_ERR_UNSUPPORTED, "a chunk tile of C=%d x d=%d %s values exceeds %d bytes", Cr, D,
                p->io == LL_BF16 ? "bf16" : "fp32", llattn::kAttnTileBytesMax);
  if (p->rule == LL_GATED_DELTANET && (size_t)r.C * D * esz > 2 * (size_t)llattn::kAttnTileBytesMax)
    return fail(LL_ERR_UNSUPPORTED, "the Gated DeltaNet pass has no %s chunk of C=%d x d=%d",
                p->io == LL_BF16 ? "bf16" : "fp32", r.C, D);
  const int need_r = bit_length((int64_t)r.T - 1) + 1;
  if (need_r > llattn::kLevelsMax)
    return fail(LL_ERR_UNSUPPORTED, "T=%d needs %d levels; at most %d are supported", r.T, need_r, llattn::kLevelsMax);
  if ((int64_t)p->B * p->H * (r.T / Cr) > ((int64_t)1 << 31) - 1)
    return fail(LL_ERR_UNSUPPORTED, "problem too large for one launch");

  const int nc = r.T / Cr;
  const int depth_cap = 1 << (depth >= 0 ? depth : llattn::read_block_depth(r.io == LL_BF16 ? 1 : 0, D, Cr));
  int P = nc & -nc;  // lowest set bit: blocks tile the chunks exactly
  if (P > kMaxBlockChunks) P = kMaxBlockChunks;
  if (P > depth_cap) P = depth_cap;
  // blocks of more than 8 chunks only while they leave every CU a block to read
  while (P > 8 && (int64_t)p->B * p->H * (nc / P) < kReadBlocksMin) P /= 2;
  Plan pl;
  pl.r = r;
  pl.Cr = Cr;
  pl.P = P;
  pl.nb = nc / P;
  pl.nF = pl.nb / 2;
  pl.LS = p->L < need_r ? p->L : need_r;
  const size_t bh = (size_t)p->B * p->H;
  const size_t dd = (size_t)D * D;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  pl.s_off = take(bh * pl.nb * dd * sizeof(float));
  pl.gs_off = take(bh * pl.nb * sizeof(float));
  pl.f_off = take(bh * pl.nF * dd * sizeof(float));
  pl.gf_off = take(bh * (pl.nF > 0 ? pl.nF : 1) * sizeof(float));
  pl.n16_off = 0;
  if (llattn::node_copies(p->io == LL_BF16 ? 1 : 0, D) && pl.nb > 1)  // bf16 copies of the nodes the read takes
    pl.n16_off = take(bh * pl.nb * dd * 2);
  const size_t rows_r = (size_t)p->B * r.T * p->H;
  pl.w_off = pl.up_off = pl.u_off = 0;
  if (p->rule == LL_GATED_DELTANET) {
    pl.w_off = take(rows_r * D * esz);
    pl.up_off = take(rows_r * D * esz);
    pl.u_off = take(rows_r * D * esz);
  }
  pl.pad_t = r.T != p->T;
  pl.pad_qk = p->dk != D || pl.pad_t;
  pl.pad_v = p->dv != D || pl.pad_t;
  pl.pad_state = p->dk != D || p->dv != D;
  pl.qp_off = pl.kp_off = pl.vp_off = pl.op_off = pl.gp_off = pl.lp_off = pl.bp_off = pl.sin_off = pl.sout_off = 0;
  if (pl.pad_qk) {
    pl.qp_off = take(rows_r * D * esz);
    pl.kp_off = take(rows_r * D * esz);
  }
  if (pl.pad_v) {
    pl.vp_off = take(rows_r * D * esz);
    pl.op_off = take(rows_r * D * esz);
  }
  if (pl.pad_t) {
    pl.gp_off = take(rows_r * 4);
    pl.lp_off = take(rows_r * p->L * 4);
    pl.bp_off = take(rows_r * 4);
  }
  if (pl.pad_state) {
    const size_t state_bytes = bh * p->L * (dd + 1) * 4;
    pl.sin_off = take(state_bytes);
    pl.sout_off = take(state_bytes);
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

// Copies between a caller's [B,T,H,d] (or [B,T,H]) tensor and its run shape.
hipError_t pad_rows(int esz, const void* src, int B, int Ts, int H, int ds, void* dst, int Td, int dd, hipStream_t s) {
  return llattn::launch_pad_copy(esz, src, dst, B, Ts, H, ds, Td, H, dd, s);
}

// A caller's decode-layout state [B,H,L,dk,dv] + sigma [B,H,L] and its run
// shape [B,H,L,D,D] + sigma.
hipError_t pad_state(const void* src, int dks, int dvs, void* dst, int dkd, int dvd, int64_t mats, hipStream_t s) {
  hipError_t e = llattn::launch_pad_copy(4, src, dst, mats, dks, 1, dvs, dkd, 1, dvd, s);
  if (e != hipSuccess) return e;
  return llattn::launch_pad_copy(4, static_cast<const float*>(src) + mats * dks * dvs,
                                 static_cast<float*>(dst) + mats * dkd * dvd, 1, 1, 1, (int)mats, 1, 1, (int)mats, s);
}

// The launch sequence of a validated prefill in its run shape.
// The level-weight MLP that the read runs itself (lambda then holds its input d).
struct ReadMlp {
  int hidden;
  const float *w1, *w2, *bias;
};

ll_status run_core(const Plan& pl, int64_t pos0, const float* state_in, const void* q, const void* k, const void* v,
                   const float* log_gate, const float* lambda, const float* beta, void* o, void* state_out,
                   void* workspace, hipStream_t stream, bool reuse_states, const ReadMlp* mlp = nullptr) {
  char* ws = static_cast<char*>(workspace);
  const ll_problem* p = &pl.r;
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
  const bool read_prior = llattn::read_takes_prior(p->io == LL_BF16 ? 1 : 0, p->dk, pl.Cr, pos0);
  if (read_prior) {
    // the read takes the levels of [0, pos0) too: stage up to level bit_length(pos0)
    int bl = 0;
    while ((pos0 >> bl) != 0) ++bl;
    a.prior = state_in;
    if (a.LS < bl + 1) a.LS = bl + 1 < p->L ? bl + 1 : p->L;
  }
  if (mlp) {
    a.w1 = mlp->w1;
    a.w2 = mlp->w2;
    a.mlp_bias = mlp->bias;
    a.hidden = mlp->hidden;
  }
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
  if (e == hipSuccess && o && pos0 > 0 && !read_prior)
    e = timed(K_PRIOR_READ, stream, [&] { return llattn::launch_prior_read(io, D, C, a, stream); });
  if (e == hipSuccess && state_out)
    e = timed(K_STATE_EXPORT, stream, [&] { return llattn::launch_state_export(D, C, a, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}


// Both prefill entry points: a segment at positions pos0 .. pos0 + T - 1 whose
// earlier positions (if any) are summarised by state_in.  A problem whose
// shape the kernels do not run natively runs on copies in its run shape.
// reuse_states: the workspace already holds the block states and Fenwick nodes
// of this (k, v, log_gate) from the previous call (a Mamba-2 read with other
// q or level weights); only the read runs.
ll_status run_prefill(const ll_problem* p, int64_t pos0, const float* state_in, const void* q, const void* k,
                      const void* v, const float* log_gate, const float* lambda, const float* beta, void* o,
                      void* state_out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                      bool reuse_states = false, bool noalloc = false, const ReadMlp* mlp = nullptr) {
  Plan pl;
  ll_status st = plan_prefill(p, state_out != nullptr, &pl);
  if (st != LL_OK) return st;
  if (reuse_states && (p->rule != LL_MAMBA2 || pos0 != 0 || state_out || pl.pad_qk || pl.pad_v))
    return fail(LL_ERR_UNSUPPORTED, "reusing block states is only for a plain Mamba-2 read in the run shape");
  const ll_problem& r = pl.r;
  if (pos0 < 0) return fail(LL_ERR_POSITION, "pos0=%lld is negative", (long long)pos0);
  if (pos0 > 0) {
    if (!state_in) return fail(LL_ERR_NULL, "state_in must not be NULL when pos0 > 0");
    if ((pos0 & -pos0) < r.T)
      return fail(LL_ERR_POSITION, "pos0=%lld: the segment of T=%d tokens must fit below the lowest set bit of pos0",
                  (long long)pos0, r.T);
    if (pos0 > ((int64_t)1 << 61)) return fail(LL_ERR_POSITION, "pos0=%lld is too large", (long long)pos0);
    const int64_t end = pos0 + r.T;
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

  // the caller's tensors in the run shape
  char* ws = static_cast<char*>(workspace);
  const int esz = p->io == LL_BF16 ? 2 : 4;
  const int D = r.dk;
  const int64_t mats = (int64_t)p->B * p->H * p->L;
  const void *qr = q, *kr = k, *vr = v;
  const float *gr = log_gate, *lr = lambda, *br = beta, *sr = state_in;
  void* or_ = o;
  void* sor = state_out;
  hipError_t e = hipSuccess;
  auto step = [&](auto fn) {
    if (e == hipSuccess) e = fn();
  };
  if (pl.pad_qk) {
    if (q) {
      step([&] { return pad_rows(esz, q, p->B, p->T, p->H, p->dk, ws + pl.qp_off, r.T, D, stream); });
      qr = ws + pl.qp_off;
    }
    step([&] { return pad_rows(esz, k, p->B, p->T, p->H, p->dk, ws + pl.kp_off, r.T, D, stream); });
    kr = ws + pl.kp_off;
  }
  if (pl.pad_v) {
    step([&] { return pad_rows(esz, v, p->B, p->T, p->H, p->dv, ws + pl.vp_off, r.T, D, stream); });
    vr = ws + pl.vp_off;
    if (o) or_ = ws + pl.op_off;
  }
  if (pl.pad_t) {
    step([&] { return pad_rows(4, log_gate, p->B, p->T, p->H, 1, ws + pl.gp_off, r.T, 1, stream); });
    gr = reinterpret_cast<const float*>(ws + pl.gp_off);
    if (lambda) {
      step([&] { return pad_rows(4, lambda, p->B, p->T, p->H, p->L, ws + pl.lp_off, r.T, p->L, stream); });
      lr = reinterpret_cast<const float*>(ws + pl.lp_off);
    }
    if (beta) {
      step([&] { return pad_rows(4, beta, p->B, p->T, p->H, 1, ws + pl.bp_off, r.T, 1, stream); });
      br = reinterpret_cast<const float*>(ws + pl.bp_off);
    }
  }
  if (pl.pad_state) {
    if (pos0 > 0) {
      step([&] { return pad_state(state_in, p->dk, p->dv, ws + pl.sin_off, D, D, mats, stream); });
      sr = reinterpret_cast<const float*>(ws + pl.sin_off);
    }
    if (state_out) sor = ws + pl.sout_off;
  }
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));

  st = run_core(pl, pos0, sr, qr, kr, vr, gr, lr, br, or_, sor, workspace, stream, reuse_states, mlp);
  if (st != LL_OK) return st;

  // the outputs in the caller's shape
  if (o && or_ != o) step([&] { return pad_rows(esz, or_, p->B, r.T, p->H, D, o, p->T, p->dv, stream); });
  if (state_out && sor != state_out)
    step([&] { return pad_state(sor, D, D, state_out, p->dk, p->dv, mats, stream); });
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
  if (!accepted_head(dk) || !accepted_head(dv))
    return fail(LL_ERR_UNSUPPORTED, "head sizes dk=%d, dv=%d: each must be 16, 32, 64 or 128", dk, dv);
  return LL_OK;
}

ll_status launch_decode(int B, int H, int dk, int dv, int L, ll_dtype io, ll_rule rule, int64_t pos, const int64_t* pos_dev,
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
  hipError_t e = timed(K_DECODE_STEP, stream, [&] { return llattn::launch_decode_step(code, dk, dv, a, stream); });
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
  return launch_decode(B, H, dk, dv, L, io, rule, pos, nullptr, q, k, v, log_gate, lambda, beta, o, state, stream);
}

ll_status ll_decode_step_ragged(int B, int H, int dk, int dv, int L, ll_dtype io, ll_rule rule, const int64_t* pos,
                                const void* q, const void* k, const void* v, const float* log_gate,
                                const float* lambda, const float* beta, void* o, void* state, hipStream_t stream) {
  ll_status st = check_decode(B, H, dk, dv, L, io, rule, q, k, v, log_gate, lambda, beta, o, state);
  if (st != LL_OK) return st;
  if (!pos) return fail(LL_ERR_NULL, "pos must not be NULL");
  return launch_decode(B, H, dk, dv, L, io, rule, 0, pos, q, k, v, log_gate, lambda, beta, o, state, stream);
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

// The prefill with its level weights from the MLP: whether the read makes
// them itself, and the workspace (the prefill's, plus the weights when a
// separate ll_lambda_mlp launch makes them).
struct MlpPlan {
  bool fused;
  size_t lam_off, bytes;
};

ll_status plan_mlp_prefill(const ll_problem* p, int hidden, bool want_state, MlpPlan* mp) {
  if (!p) return fail(LL_ERR_NULL, "problem is NULL");
  if (hidden < 1) return fail(LL_ERR_SHAPE, "hidden=%d must be >= 1", hidden);
  if (hidden > 64 || p->L > 32)
    return fail(LL_ERR_UNSUPPORTED, "L=%d, hidden=%d: at most 32 levels and 64 hidden units are supported", p->L,
                hidden);
  // the read that runs the MLP has the plain prefill's blocks; a read that
  // cannot runs the plain prefill after ll_lambda_mlp
  Plan pl;
  ll_status st = plan_prefill(p, want_state, &pl);
  if (st != LL_OK) return st;
  mp->fused = llattn::read_runs_mlp(pl.r.io == LL_BF16 ? 1 : 0, pl.r.dk, pl.Cr, p->L, hidden);
  mp->lam_off = (pl.bytes + 255) & ~(size_t)255;
  mp->bytes = mp->fused ? pl.bytes : mp->lam_off + (size_t)p->B * p->T * p->H * p->L * sizeof(float);
  return LL_OK;
}

}  // namespace

ll_status ll_attn_fwd_lambda_mlp_workspace_bytes(const ll_problem* p, int hidden, size_t* bytes) {
  if (!bytes) return fail(LL_ERR_NULL, "bytes is NULL");
  MlpPlan mp;
  ll_status st = plan_mlp_prefill(p, hidden, false, &mp);  // the workspace does not depend on exporting
  if (st != LL_OK) return st;
  *bytes = mp.bytes;
  return ok();
}

ll_status ll_attn_fwd_lambda_mlp(const ll_problem* p, const void* q, const void* k, const void* v,
                                 const float* log_gate, const float* d, int hidden, const float* w1, const float* w2,
                                 const float* bias, const float* beta, void* o, void* state_out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  MlpPlan mp;
  ll_status st = plan_mlp_prefill(p, hidden, state_out != nullptr, &mp);
  if (st != LL_OK) return st;
  if (!o) return fail(LL_ERR_NULL, "o must not be NULL: the level weights only serve the read");
  if (!d || !w1 || !w2 || !bias) return fail(LL_ERR_NULL, "d, w1, w2 and bias must not be NULL");
  if (workspace_bytes < mp.bytes)
    return fail(LL_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, mp.bytes);
  if (mp.bytes > 0 && !workspace) return fail(LL_ERR_WORKSPACE, "workspace is NULL");
  if (mp.fused) {
    const ReadMlp mlp{hidden, w1, w2, bias};
    return run_prefill(p, 0, nullptr, q, k, v, log_gate, d, beta, o, state_out, workspace, workspace_bytes, stream,
                       false, false, &mlp);
  }
  // a read that does not run the MLP: the weights first, into the workspace
  float* lam = reinterpret_cast<float*>(static_cast<char*>(workspace) + mp.lam_off);
  st = ll_lambda_mlp((int64_t)p->B * p->T * p->H, p->L, hidden, d, w1, w2, bias, lam, stream);
  if (st != LL_OK) return st;
  return run_prefill(p, 0, nullptr, q, k, v, log_gate, lam, beta, o, state_out, workspace, mp.lam_off, stream);
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
  if (!accepted_head(dk))
    return fail(LL_ERR_UNSUPPORTED, "head size %d not supported (16, 32, 64 or 128)", dk);
  const size_t esz = io == LL_BF16 ? 2 : 4;
  const int D = run_head(dk, dk, io);
  int C = 0;
  for (int c : {64, 32, 16})
    if (!C && T % c == 0) C = c;
  if (!C) return fail(LL_ERR_UNSUPPORTED, "T=%d is not a multiple of 16", T);
  const int CW = run_chunk(C, D, io, LL_MAMBA2);
  const int T_run = (T + CW - 1) / CW * CW;
  CcqPlan c;
  c.p.B = B;
  c.p.T = T;
  c.p.H = H;
  c.p.dk = c.p.dv = dk;
  c.p.L = bit_length((int64_t)T_run - 1) + 1;  // levels for the run length (all weights are 1)
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
  // the prefill's inputs, and sum_{j<=t} k_j as chunk sums with their prefix over the chunks (the
  // rest in the combine)
  hipError_t e = timed(K_CCQ, stream, [&] {
    return llattn::launch_ccq_prepare(code, dk, B, T, H, c.p.C, k, csum, (int64_t)B * T * H, c.p.L, ones, zeros, stream);
  });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  // sum_{j<=t} (k_j . q_t) k_j
  st = run_prefill(&c.p, 0, nullptr, q, k, k, zeros, ones, nullptr, kkq, nullptr, ws + c.fwd_off, c.fwd_bytes, stream);
  if (st != LL_OK) return st;
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
  size_t fwd_off, doo_off, din_off, w_off, bt_off, scratch_off;
  // run-shape copies of dO and of the gradients, where the run shape differs
  size_t dop_off, dqp_off, dkp_off, dvp_off, dgp_off, dlp_off;
  size_t bytes;
};

ll_status plan_bwd(const ll_problem* p, BwdPlan* out) {
  Plan pl;
  // the backward's walks keep up to 2^max_block_depth chunks a block
  const int depth = llattn::max_block_depth(p ? p->dk : 0);
  ll_status st = plan_prefill(p, false, &pl, depth);
  if (st != LL_OK) return st;
  // fp32 runs 32-token chunks where 64 are asked for: the gradients do not
  // depend on the chunk size, and the walks' fp32 fragments of 64 tokens do not
  // fit two waves per SIMD
  if (p->io == LL_F32 && pl.r.C == 64) {
    ll_problem q = *p;
    q.C = 32;
    st = plan_prefill(&q, false, &pl, depth);
    if (st != LL_OK) return st;
  }
  if (p->rule != LL_MAMBA2) return fail(LL_ERR_UNSUPPORTED, "the backward pass is implemented for the Mamba-2 write");
  const ll_problem& r = pl.r;
  BwdPlan c;
  c.pl = pl;
  c.nbl = bit_length((int64_t)pl.nb - 1);
  const size_t bh = (size_t)r.B * r.H, rows = (size_t)r.B * r.T * r.H;
  const size_t dd = (size_t)r.dk * r.dv;
  const size_t esz = p->io == LL_BF16 ? 2 : 4;
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
  c.bt_off = take(bh * pl.nb * 4);
  c.scratch_off = take(llattn::bwd_states_in_lds(r.dk) ? 0
                                                        : bh * pl.nb * (size_t)llattn::max_block_depth(r.dk) * dd * 4);
  c.dop_off = c.dqp_off = c.dkp_off = c.dvp_off = c.dgp_off = c.dlp_off = 0;
  if (pl.pad_qk) {
    c.dqp_off = take(rows * r.dk * esz);
    c.dkp_off = take(rows * r.dk * esz);
  }
  if (pl.pad_v) {
    c.dop_off = take(rows * r.dv * esz);
    c.dvp_off = take(rows * r.dv * esz);
  }
  if (pl.pad_t) {
    c.dgp_off = take(rows * 4);
    c.dlp_off = take(rows * (size_t)r.L * 4);
  }
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
  const ll_problem& r = pl.r;
  char* fws = ws + c.fwd_off;  // the prefill workspace: block states, nodes and run-shape input copies
  const int io = p->io == LL_BF16 ? 1 : 0;
  const int esz = io ? 2 : 4;
  const int D = r.dk;
  hipError_t e = hipSuccess;
  auto step = [&](auto fn) {
    if (e == hipSuccess) e = fn();
  };

  // the inputs in the run shape
  const void *qr = q, *kr = k, *vr = v, *dor = dO;
  const float *gr = log_gate, *lr = lambda;
  void *dqr = dq, *dkr = dk, *dvr = dv;
  float *dgr = dlog_gate, *dlr = dlambda;
  if (pl.pad_qk) {
    step([&] { return pad_rows(esz, q, p->B, p->T, p->H, p->dk, fws + pl.qp_off, r.T, D, stream); });
    step([&] { return pad_rows(esz, k, p->B, p->T, p->H, p->dk, fws + pl.kp_off, r.T, D, stream); });
    qr = fws + pl.qp_off;
    kr = fws + pl.kp_off;
    dqr = ws + c.dqp_off;
    dkr = ws + c.dkp_off;
  }
  if (pl.pad_v) {
    step([&] { return pad_rows(esz, v, p->B, p->T, p->H, p->dv, fws + pl.vp_off, r.T, D, stream); });
    step([&] { return pad_rows(esz, dO, p->B, p->T, p->H, p->dv, ws + c.dop_off, r.T, D, stream); });
    vr = fws + pl.vp_off;
    dor = ws + c.dop_off;
    dvr = ws + c.dvp_off;
  }
  if (pl.pad_t) {
    step([&] { return pad_rows(4, log_gate, p->B, p->T, p->H, 1, fws + pl.gp_off, r.T, 1, stream); });
    step([&] { return pad_rows(4, lambda, p->B, p->T, p->H, p->L, fws + pl.lp_off, r.T, p->L, stream); });
    gr = reinterpret_cast<const float*>(fws + pl.gp_off);
    lr = reinterpret_cast<const float*>(fws + pl.lp_off);
    dgr = reinterpret_cast<float*>(ws + c.dgp_off);
    dlr = reinterpret_cast<float*>(ws + c.dlp_off);
  }

  // the forward's block states and Fenwick nodes of (v, k): the transposed
  // states of (k, v), which the forward walk reads as S dO
  PrefillArgs f;
  f.B = r.B;
  f.T = r.T;
  f.H = r.H;
  f.L = r.L;
  f.LS = pl.LS;
  f.P = pl.P;
  f.nb = pl.nb;
  f.nF = pl.nF;
  f.q = nullptr;
  f.k = vr;
  f.v = kr;
  f.g = gr;
  f.lam = lr;
  f.o = nullptr;
  f.S = reinterpret_cast<float*>(fws + pl.s_off);
  f.GS = reinterpret_cast<float*>(fws + pl.gs_off);
  f.F = reinterpret_cast<float*>(fws + pl.f_off);
  f.GF = reinterpret_cast<float*>(fws + pl.gf_off);
  f.N16 = nullptr;
  f.state = nullptr;
  f.state_in = nullptr;
  f.pos0 = 0;
  if (e == hipSuccess) e = timed(K_BWD, stream, [&] { return llattn::launch_block_state(io, D, pl.Cr, f, stream); });
  if (e == hipSuccess && pl.nb > 1) e = timed(K_BWD, stream, [&] { return llattn::launch_fenwick_scan(D, f, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));

  llattn::BwdArgs a;
  a.B = r.B;
  a.T = r.T;
  a.H = r.H;
  a.D = D;
  a.L = r.L;
  a.q = qr;
  a.k = kr;
  a.v = vr;
  a.g = gr;
  a.lam = lr;
  a.dO = dor;
  a.dq = dqr;
  a.dk = dkr;
  a.dv = dvr;
  a.dlog_gate = dgr;
  a.dlambda = dlr;
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
  w.BT = reinterpret_cast<float*>(ws + c.bt_off);
  w.nbl = c.nbl;
  w.scratch = llattn::bwd_states_in_lds(D) ? nullptr : reinterpret_cast<float*>(ws + c.scratch_off);
  // the forward walk; the reverse bucket states; the reverse walk; the gate's later blocks
  for (int pass = 0; pass < 4 && e == hipSuccess; ++pass)
    e = timed(K_BWD, stream, [&] { return llattn::launch_bwd_native(io, D, pl.Cr, a, n, w, pass, stream); });

  // the gradients in the caller's shape
  if (dqr != dq) step([&] { return pad_rows(esz, dqr, p->B, r.T, p->H, D, dq, p->T, p->dk, stream); });
  if (dkr != dk) step([&] { return pad_rows(esz, dkr, p->B, r.T, p->H, D, dk, p->T, p->dk, stream); });
  if (dvr != dv) step([&] { return pad_rows(esz, dvr, p->B, r.T, p->H, D, dv, p->T, p->dv, stream); });
  if (dgr != dlog_gate) step([&] { return pad_rows(4, dgr, p->B, r.T, p->H, 1, dlog_gate, p->T, 1, stream); });
  if (dlr != dlambda) step([&] { return pad_rows(4, dlr, p->B, r.T, p->H, p->L, dlambda, p->T, p->L, stream); });
  if (e != hipSuccess) return fail(LL_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
