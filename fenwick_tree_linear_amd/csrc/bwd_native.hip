// bwd_native.hip -- the backward pass of the Mamba-2 log-linear read
// ("Log-Linear Attention", section 2.3: the masked form evaluated chunk by
// chunk; section 3: training at scale) as kernels of its own.
//
// With pair weights M[t,s] = lambda_t^{lev(t,s)} e^{G_t - G_s} (s <= t, G the
// inclusive prefix of log a) and E[t,s] = e^{G_t - G_s} (q_t . k_s)(dO_t . v_s):
//   dq_t        = sum_s M[t,s] (dO_t . v_s) k_s        (the forward read with
//                                                      (q,k,v) := (dO,v,k))
//   dlambda_t^l = sum_{s: lev(t,s) = l} E[t,s]                   (ll_bwd_levels)
//   dv_s        = sum_{t >= s} M[t,s] (q_t . k_s) dO_t           (ll_bwd_revread)
//   dk_s        = sum_{t >= s} M[t,s] (dO_t . v_s) q_t           (the same, roles swapped)
//   dlog_gate_r = sum_{s < r <= t} E[t,s] lambda_t^{lev(t,s)}   (the pairs the gate of r decays)
// The gate gradient splits by pairs: those inside one chunk give, per chunk,
// sum_{t >= r} (row sum of t) - sum_{s >= r} (column sum of s) over the chunk's
// exact fp32 pair terms (ll_bwd_levels); those across chunks give the suffix
// sum over all later tokens of dO_t . o_t^x - v_t . dv_t^x, the parts of
// dO . o and v . dv (= k . dk) that come from other chunks (ll_bwd_gate).  Only
// the cross-chunk parts, small where the gates decay within a chunk, run
// through the long suffix sum.
//
// The reverse sums: for a source s, the targets t at level l >= 1 form one
// aligned bucket X, the sibling right after the aligned group of s, and every
// aligned bucket is read at exactly one level (log2 |X| + 1).  So each bucket
// keeps one state R_X = sum_{t in X} lambda_t^{lev(X)} e^{G_t - G_{X0-1}} q_t dO_t^T
// (X0 its first token), and dv_s = sum_X e^{G_{X0-1} - G_s} R_X^T k_s plus
// the in-chunk part.  Inside a block of chunks, a walk over the chunks from
// the last to the first keeps the chunk-level buckets (ll_bwd_revread); above
// it, ll_bwd_rev_state forms each block's share of the buckets it belongs to
// and ll_bwd_rev_scan sums the shares into bucket states.
#include <type_traits>

#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

namespace {

// Staged chunk of the backward kernels: four [C][D] io tiles (row-major,
// swizzled), the gates and the level weights of the chunk's rows.
template <typename T, int D, int C>
struct BwdStage {
  typedef Tile<T, C, D> TL;
  static constexpr int NWT = 8;  // weight rows
  static constexpr int A = 0, B = TL::BYTES, X = 2 * TL::BYTES, Y = 3 * TL::BYTES;
  static constexpr int G = 4 * TL::BYTES;   // gates [C]
  static constexpr int GP = G + C * 4;      // in-chunk inclusive prefix of the gates [C]
  static constexpr int WT = GP + C * 4;     // per-token weight rows [NWT][C]
  static constexpr int LAM = WT + NWT * C * 4;  // level weights [C][kLevelsMax]
  static constexpr int XIN = LAM + C * kLevelsMax * 4;  // in-chunk column sums per wave [C/16][C]
  static constexpr int DOI = XIN + (C / 16) * C * 4;    // in-chunk row sums [C]
  static constexpr int BYTES = DOI + C * 4;
};

// Stages the gate prefix: wave 0 scans, every thread may read it after the
// caller's next barrier.  Returns the chunk's gate sum (every wave).
template <int C>
__device__ __forceinline__ float stage_prefix(const float* gl, float* gp, int wv, int lane) {
  const float G = chunk_scan<C>(lane < C ? gl[lane] : 0.f);
  if (wv == 0 && lane < C) gp[lane] = G;
  return __shfl(G, C - 1, 64);
}

// Loads rows row0 .. row0 + (C-1) H of a [*, D] io tensor into a swizzled tile
// (16-byte pieces; all threads of the workgroup take part).
template <typename T, int D, int C>
__device__ __forceinline__ void stage_tile(const void* src, int64_t row0, int H, char* lds, int tid, int nthreads) {
  typedef Tile<T, C, D> TL;
  constexpr int EPP = 16 / (int)sizeof(T);
  for (int x = tid; x < TL::BYTES / 16; x += nthreads) {
    const int r = x / TL::NCH, c = x % TL::NCH;
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const T*>(src) + (row0 + (int64_t)r * H) * D + c * EPP);
    *reinterpret_cast<uint4*>(lds + r * TL::RB + (TL::pos(r, c) << 4)) = v;
  }
}

// Gates and the first LS level weights of the chunk's rows.
template <int C>
__device__ __forceinline__ void stage_gates(const float* g, const float* lam, int64_t row0, int H, int L, int LS,
                                            float* gl, float* ll, int tid, int nthreads) {
  for (int x = tid; x < C; x += nthreads) gl[x] = g[row0 + (int64_t)x * H];
  for (int x = tid; x < C * LS; x += nthreads) {
    const int r = x / LS, l = x % LS;
    ll[r * kLevelsMax + l] = lam[(row0 + (int64_t)r * H) * L + l];
  }
}

// Sum over the four lane groups (lanes q, q + 16, q + 32, q + 48).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// The block a (head, item) pair walks: first [B,T,H] row and its chunks.
struct BlockOf {
  int J, bh, h, b;
  int64_t row;
  __device__ __forceinline__ void set(int wg, const BwdArgs& a, int nb, int P, int C) {
    J = wg % nb;
    bh = wg / nb;
    h = bh % a.H;
    b = bh / a.H;
    row = ((int64_t)b * a.T + (int64_t)J * P * C) * a.H + h;
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// ll_bwd_levels: one workgroup per (block J, head), C/16 waves, wave rt owns
// the 16 target rows rt of each chunk and every level.  Walks the block's
// chunks in order, keeping the chunk-level Fenwick states of (k, v) (states
// of earlier chunks of the block, merged by the recurrent form's rule) in
// fp32; the states of earlier blocks are the forward's Fenwick nodes.
//   dlambda_t^l = sum_{s in bucket l of t} e^{G_t - G_s} (q_t . k_s)(dO_t . v_s)
//     in-chunk levels: from the score tiles (q.k and dO.v per pair, exact
//       products of the io values, fp32 sums);
//     other levels:    e^{...} q_t^T S_l dO_t, the state read Z^T = S^T Q^T on
//       the matrix cores and its rows dotted with dO in fp32.
// Writes dlambda (every level of every row, zero where the bucket is empty),
// the cross-chunk part of dO_t . o_t (sum over levels above the chunk of
// lambda_t^l dlambda_t^l) and, into dlog_gate, the in-chunk pairs' share of
// the gate gradient.
template <typename T, int D, int C, int MAXB>
__global__ void __launch_bounds__(64 * (C / 16)) ll_bwd_levels(BwdArgs a, BwdFwdNodes n, float* dOo, float* wstates) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef BwdStage<T, D, C> SG;
  constexpr int NW = C / 16, DT = D / 16, KSD = D / M::KS;
  constexpr int LOGC = (C == 16) ? 4 : (C == 32) ? 5 : 6;
  constexpr int SB = D * D;  // floats of one state
  __shared__ __attribute__((aligned(1024))) char smem[SG::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, q16 = lane & 15;
  const int rt = wv;  // this wave's 16 target rows
  BlockOf bk;
  bk.set(blockIdx.x, a, n.nb, n.P, C);
  const int logP = ilog2c(n.P);
  // chunk-level states of the block: MAXB levels, fp32 in the tile layout
  float* st = wstates + (int64_t)blockIdx.x * MAXB * SB;
  float sig[MAXB + 1];  // lazy log-scales of the chunk-level states
#pragma unroll
  for (int m = 0; m <= MAXB; ++m) sig[m] = 0.f;
  float gw = 0.f;  // log-decay from the block start to the current chunk's start
  float* gl = reinterpret_cast<float*>(smem + SG::G);
  float* gp = reinterpret_cast<float*>(smem + SG::GP);
  float* wt = reinterpret_cast<float*>(smem + SG::WT);
  const float* ll = reinterpret_cast<const float*>(smem + SG::LAM);
  const char* sq = smem + SG::A;   // q
  const char* sk = smem + SG::B;   // k
  const char* sv = smem + SG::X;   // v
  const char* sdo = smem + SG::Y;  // dO

  // A fragments (rows = state column n of column tile nt, k = d) of an fp32
  // state in the tile layout
  auto state_frags = [&](Frag (&nf)[KSD], __amdgpu_buffer_rsrc_t S, int nt) __attribute__((always_inline)) {
    f32x4 t[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) t[dt] = load_state_tile<D>(S, dt, nt, lane);
#pragma unroll
    for (int s = 0; s < KSD; ++s) nf[s] = M::acc_frag(t, s);
  };

  for (int j = 0; j < n.P; ++j) {
    const int64_t row0 = bk.row + (int64_t)j * C * a.H;
    __syncthreads();  // the previous chunk's tiles and state writes are done everywhere
    stage_tile<T, D, C>(a.q, row0, a.H, smem + SG::A, tid, 64 * NW);
    stage_tile<T, D, C>(a.k, row0, a.H, smem + SG::B, tid, 64 * NW);
    stage_tile<T, D, C>(a.v, row0, a.H, smem + SG::X, tid, 64 * NW);
    stage_tile<T, D, C>(a.dO, row0, a.H, smem + SG::Y, tid, 64 * NW);
    stage_gates<C>(a.g, a.lam, row0, a.H, a.L, n.LS, gl, reinterpret_cast<float*>(smem + SG::LAM), tid, 64 * NW);
    __syncthreads();
    const float gsum = stage_prefix<C>(gl, gp, wv, lane);
    __syncthreads();
    // decay of each source row to the chunk's end, for this chunk's own state
    for (int x = tid; x < C; x += 64 * NW) wt[x] = __expf(gsum - gp[x]);
    const int r = 16 * rt + q16;  // this lane's target row
    const float Gr = gp[r];
    float lamr[LOGC + 1];  // in-chunk level weights of row r
#pragma unroll
    for (int l = 0; l <= LOGC; ++l) lamr[l] = ll[r * kLevelsMax + l];

    // --- in-chunk levels 0..LOGC: per pair (s, r), s <= r, level bit_length(r ^ s);
    // the weighted pair terms are also summed per source (column) for the gate
    float bin[LOGC + 1];
#pragma unroll
    for (int l = 0; l <= LOGC; ++l) bin[l] = 0.f;
    float* xin = reinterpret_cast<float*>(smem + SG::XIN) + rt * C;
    for (int ct = 0; ct <= rt; ++ct) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f}, y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
        x = M::mma(frag_row<T, C, D>(sk, 16 * ct + q16, s, g4), frag_row<T, C, D>(sq, r, s, g4), x);
        y = M::mma(frag_row<T, C, D>(sv, 16 * ct + q16, s, g4), frag_row<T, C, D>(sdo, r, s, g4), y);
      }
      // lane: sources s = 16 ct + 4 (lane/16) + e of target r
      const f32x4 gs = *reinterpret_cast<const f32x4*>(gp + 16 * ct + 4 * g4);
      f32x4 col;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 16 * ct + 4 * g4 + e;
        col[e] = 0.f;
        if (s <= r) {
          const int lev = (s == r) ? 0 : 32 - __clz(r ^ s);
          const float v = x[e] * y[e] * __expf(Gr - gs[e]);
#pragma unroll
          for (int l = 0; l <= LOGC; ++l)
            if (l == lev) {
              bin[l] += v;
              col[e] = lamr[l] * v;
            }
        }
      }
      // column sums over this wave's 16 targets (the lanes of a 16-lane group)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) col[e] += __shfl_xor(col[e], m, 64);
      if (q16 == 0) *reinterpret_cast<f32x4*>(xin + 16 * ct + 4 * g4) = col;
    }
    float dlam[kLevelsMax];
#pragma unroll
    for (int l = 0; l < kLevelsMax; ++l) dlam[l] = 0.f;
#pragma unroll
    for (int l = 0; l <= LOGC; ++l) dlam[l] = sum_groups(bin[l]);
    if (g4 == 0) {  // row sum of the in-chunk pair terms of row r
      float rs = 0.f;
#pragma unroll
      for (int l = 0; l <= LOGC; ++l) rs += lamr[l] * dlam[l];
      reinterpret_cast<float*>(smem + SG::DOI)[r] = rs;
    }

    // --- other levels: e^{G_r + D} q_r^T S dO_r for every non-empty level of the chunk
    auto level_dot = [&](const float* S, float scale) __attribute__((always_inline)) {
      // Z^T[n][r] = sum_d S[d][n] q[r][d]; lane: n = 16 nt + 4 (lane/16) + e, row r
      Frag qf[KSD];
#pragma unroll
      for (int s = 0; s < KSD; ++s) qf[s] = frag_row<T, C, D>(sq, r, s, g4);
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(S, SB * 4);
      float acc = 0.f;
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) {
        Frag nf[KSD];
        state_frags(nf, rs, nt);
        f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSD; ++s) z = M::mma(nf[s], qf[s], z);
        const T* drow = reinterpret_cast<const T*>(sdo + Tile<T, C, D>::off(r, 16 * nt + 4 * g4));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += z[e] * to_f32(drow[e]);
      }
      return sum_groups(acc) * scale;
    };
    // within-block levels LOGC+1 .. LOGC+logP: states of earlier chunks of the block
#pragma unroll
    for (int m = 1; m <= MAXB; ++m)
      if (m <= logP && ((j >> (m - 1)) & 1)) dlam[LOGC + m] = level_dot(st + (m - 1) * SB, __expf(Gr + sig[m]));
    // earlier blocks: one Fenwick node per set bit of J, most recent first
    {
      int rest = bk.J;
      float dd = 0.f;
      while (rest > 0) {
        const int e = rest - 1;
        const int lev = LOGC + 1 + logP + __ffs(rest) - 1;
        const float* node = (e & 1) ? n.F + ((int64_t)bk.bh * n.nF + (e >> 1)) * SB : n.S + ((int64_t)bk.bh * n.nb + e) * SB;
        const float val = level_dot(node, __expf(Gr + gw + dd));
#pragma unroll
        for (int l = 0; l < kLevelsMax; ++l)
          if (l == lev) dlam[l] = val;
        dd += (e & 1) ? n.GF[(int64_t)bk.bh * n.nF + (e >> 1)] : n.GS[(int64_t)bk.bh * n.nb + e];
        rest &= rest - 1;
      }
    }

    // --- outputs of row r (lane group 0 writes)
    if (g4 == 0) {
      const int64_t orow = row0 + (int64_t)r * a.H;
      const float* lr = ll + r * kLevelsMax;
      float dot = 0.f;  // dO_r . o_r^x: the levels above the chunk
      for (int l = 0; l < a.L; ++l) {
        float v = 0.f;
#pragma unroll
        for (int x = 0; x < kLevelsMax; ++x)
          if (x == l) v = dlam[x];
        if (l > LOGC && l < n.LS) dot += lr[l] * v;
        a.dlambda[orow * a.L + l] = l < n.LS ? v : 0.f;
      }
      dOo[orow] = dot;
    }

    // --- this chunk's state K_w^T V (keys scaled by e^{G[C-1] - G_s}) and the
    // merge rule of the chunk-level states (levels 1..c and the chunk become
    // level c+1, c = ctz(j+1)); each wave makes the state tiles dt = wave,
    // wave + NW, ... of every column tile
    __syncthreads();  // every wave has read the states of this chunk
    // in-chunk share of the gate gradient: sum_{t >= p} (row sum t - column sum t)
    if (wv == 0) {
      float u = 0.f;
      if (lane < C) {
        const float* xs = reinterpret_cast<const float*>(smem + SG::XIN);
        u = reinterpret_cast<const float*>(smem + SG::DOI)[lane];
        for (int w = lane / 16; w < NW; ++w) u -= xs[w * C + lane];  // waves of targets >= the column's tile
      }
      const float pre = chunk_scan<C>(u);
      if (lane < C) a.dlog_gate[row0 + (int64_t)lane * a.H] = __shfl(pre, C - 1, 64) - pre + u;
    }
#pragma unroll
    for (int m = 1; m <= MAXB; ++m) sig[m] += gsum;
    gw += gsum;
    if (j + 1 < n.P) {
      const int c = __ffs(j + 1) - 1;
      // per-lane decay of the source rows to the chunk's end, k-step order
      for (int dt = wv; dt < DT; dt += NW) {
        Frag kf[C / M::KS];
#pragma unroll
        for (int s = 0; s < C / M::KS; ++s) kf[s] = frag_col<T, C, D>(sk, 16 * dt, s, lane);
        for (int nt = 0; nt < DT; ++nt) {
          Frag vf[C / M::KS];
#pragma unroll
          for (int s = 0; s < C / M::KS; ++s) vf[s] = frag_col<T, C, D>(sv, 16 * nt, s, lane);
          lds_wait(kf, vf);
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 1; m <= MAXB; ++m)
            if (m <= c) {
              const f32x4 old = *reinterpret_cast<const f32x4*>(st + (m - 1) * SB + state_tile_offset<D>(dt, nt, lane));
              acc += __expf(sig[m]) * old;
            }
#pragma unroll
          for (int s = 0; s < C / M::KS; ++s) acc = M::mma(kf[s], scale_tokens<T>(vf[s], wt, s, g4), acc);
          *reinterpret_cast<f32x4*>(st + c * SB + state_tile_offset<D>(dt, nt, lane)) = acc;
        }
      }
#pragma unroll
      for (int m = 1; m <= MAXB; ++m)
        if (m == c + 1) sig[m] = 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// ll_bwd_rev_state: one workgroup per (block J, head, group of NLB block
// levels), D/16 waves (one per 16 value columns).  For every block level b of
// the group with bit b of J set (J lies in a right bucket of 2^b blocks), the
// block's share of that bucket's state,
//   W[J][b] = sum_{t in J} lambda_t^{l_b} e^{G_t - G_{J0-1}} kr_t vr_t^T,
// l_b = log2(C P) + 1 + b, in the tile layout; (kr, vr) = (q, dO) for dv and
// (dO, q) for dk.
template <typename T, int D, int C, int NLB>
__global__ void __launch_bounds__(64 * (D / 16)) ll_bwd_rev_state(BwdArgs a, BwdFwdNodes n, const void* kr,
                                                                  const void* vr, float* W, int nbl) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef BwdStage<T, D, C> SG;
  constexpr int NW = D / 16, DT = D / 16, KSC = C / M::KS;
  constexpr int LOGC = (C == 16) ? 4 : (C == 32) ? 5 : 6;
  constexpr int SB = D * D;
  __shared__ __attribute__((aligned(1024))) char smem[SG::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;
  BlockOf bk;
  bk.set(blockIdx.x, a, n.nb, n.P, C);
  const int logP = ilog2c(n.P);
  const int b0 = blockIdx.y * NLB;  // first block level of this group
  // this group's levels that J takes part in (bit b0 + b of J set)
  const int bits = (bk.J >> b0) & ((1 << NLB) - 1) & ((1 << (nbl > b0 ? nbl - b0 : 0)) - 1);
  if (bits == 0) return;
  f32x4 acc[NLB][DT];
#pragma unroll
  for (int b = 0; b < NLB; ++b)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[b][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float* gl = reinterpret_cast<float*>(smem + SG::G);
  float* gp = reinterpret_cast<float*>(smem + SG::GP);
  float* wt = reinterpret_cast<float*>(smem + SG::WT);
  const float* ll = reinterpret_cast<const float*>(smem + SG::LAM);
  static_assert(NLB <= SG::NWT, "a weight row per block level");
  float pre = 0.f;  // G_{chunk start - 1} - G_{J0 - 1}
  for (int j = 0; j < n.P; ++j) {
    const int64_t row0 = bk.row + (int64_t)j * C * a.H;
    __syncthreads();
    stage_tile<T, D, C>(kr, row0, a.H, smem + SG::A, tid, 64 * NW);
    stage_tile<T, D, C>(vr, row0, a.H, smem + SG::B, tid, 64 * NW);
    stage_gates<C>(a.g, a.lam, row0, a.H, a.L, n.LS, gl, reinterpret_cast<float*>(smem + SG::LAM), tid, 64 * NW);
    __syncthreads();
    const float gsum = stage_prefix<C>(gl, gp, wv, lane);
    __syncthreads();
    // weight rows lambda_t^{l_b} e^{G_t - G_{J0-1}} of the block levels J lies in
    for (int x = tid; x < NLB * C; x += 64 * NW) {
      const int b = x / C, t = x % C;
      if ((bits >> b) & 1) wt[x] = ll[t * kLevelsMax + LOGC + logP + 1 + b0 + b] * __expf(pre + gp[t]);
    }
    __syncthreads();
    Frag kf[DT][KSC], vf[KSC];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int s = 0; s < KSC; ++s) kf[dt][s] = frag_col<T, C, D>(smem + SG::A, 16 * dt, s, lane);
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(smem + SG::B, 16 * wv, s, lane);
    lds_wait(kf, vf);
#pragma unroll
    for (int b = 0; b < NLB; ++b) {
      if (!((bits >> b) & 1)) continue;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        const Frag vw = scale_tokens<T>(vf[s], wt + b * C, s, g4);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[b][dt] = M::mma(kf[dt][s], vw, acc[b][dt]);
      }
    }
    pre += gsum;
  }
#pragma unroll
  for (int b = 0; b < NLB; ++b) {
    if (!((bits >> b) & 1)) continue;
    float* dst = W + (((int64_t)bk.bh * n.nb + bk.J) * nbl + b0 + b) * SB;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + state_tile_offset<D>(dt, wv, lane)) = acc[b][dt];
  }
}

// ---------------------------------------------------------------------------
// ll_bwd_rev_scan: for every head, block level b and right bucket X of 2^b
// blocks (X = blocks x 2^b .. (x+1) 2^b - 1, x odd), the bucket state
//   R_X = sum_{J in X} e^{G_{J0-1} - G_{X0-1}} W[J][b],
// written in place of W[x 2^b][b].  One thread per four state elements.
__global__ void __launch_bounds__(256) ll_bwd_rev_scan(BwdFwdNodes n, int BH, int DD, float* W, int nbl) {
  const int n4 = DD / 4;
  const int64_t total = (int64_t)BH * nbl * n.nb * n4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int e4 = (int)(i % n4);
    int64_t rest = i / n4;
    const int first = (int)(rest % n.nb);  // candidate first block of a bucket
    rest /= n.nb;
    const int b = (int)(rest % nbl);
    const int bh = (int)(rest / nbl);
    if (((first >> b) & 1) == 0 || (first & ((1 << b) - 1)) != 0) continue;  // not the first block of a right bucket
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    float dec = 0.f;
    for (int J = first; J < first + (1 << b) && J < n.nb; ++J) {
      const f32x4 w = reinterpret_cast<const f32x4*>(W + (((int64_t)bh * n.nb + J) * nbl + b) * DD)[e4];
      sum += __expf(dec) * w;
      dec += n.GS[(int64_t)bh * n.nb + J];
    }
    reinterpret_cast<f32x4*>(W + (((int64_t)bh * n.nb + first) * nbl + b) * DD)[e4] = sum;
  }
}

// ---------------------------------------------------------------------------
// ll_bwd_revread: one workgroup per (block J, head), C/16 waves, wave rt owns
// the 16 source rows rt of each chunk and every output column.  Walks the
// block's chunks from the last to the first:
//   out_s = sum_{t >= s in chunk} P[t,s] vr_t,  P[t,s] = lambda_t^{lev} e^{G_t - G_s} (kr_t . qr_s)
//         + sum over the buckets X after s: e^{G_{X0-1} - G_s} R_X^T qr_s
// with (qr, kr, vr) = (k, q, dO) for dv and (v, dO, q) for dk.  Chunk-level
// buckets are kept in fp32 (one per within-block level, built from the
// chunks already walked); block-level buckets come from ll_bwd_rev_scan.
// With xdot given, also writes xdot_s . (the buckets' part of out_s) in fp32:
// v . dv^x, the cross-chunk part of v . dv (= k . dk).
template <typename T, int D, int C, int MAXB>
__global__ void __launch_bounds__(64 * (C / 16)) ll_bwd_revread(BwdArgs a, BwdFwdNodes n, const void* qr, const void* kr,
                                                                const void* vr, const float* W, int nbl, void* out,
                                                                const void* xdot, float* dot_out, float* rstates) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef BwdStage<T, D, C> SG;
  typedef Tile<T, C, D> TL;
  typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type Vec4;
  constexpr int NW = C / 16, CT = C / 16, DT = D / 16, KSD = D / M::KS, KSC = C / M::KS;
  constexpr int LOGC = (C == 16) ? 4 : (C == 32) ? 5 : 6;
  constexpr int SB = D * D;
  __shared__ __attribute__((aligned(1024))) char smem[SG::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, q16 = lane & 15;
  const int st_ = wv;  // this wave's 16 source rows
  BlockOf bk;
  bk.set(blockIdx.x, a, n.nb, n.P, C);
  const int logP = ilog2c(n.P);
  float* Rm = rstates + (int64_t)blockIdx.x * MAXB * SB;  // chunk-level bucket states, fp32 tile layout
  float sufX[MAXB + 1];  // gate sum of the walked chunks from each level's bucket start to the block end
#pragma unroll
  for (int m = 0; m <= MAXB; ++m) sufX[m] = 0.f;
  float suf = 0.f;  // gate sum of the chunks after the current one, to the block end
  float* gl = reinterpret_cast<float*>(smem + SG::G);
  float* gp = reinterpret_cast<float*>(smem + SG::GP);
  float* wt = reinterpret_cast<float*>(smem + SG::WT);
  const float* ll = reinterpret_cast<const float*>(smem + SG::LAM);
  static_assert(MAXB <= SG::NWT, "a weight row per chunk level");
  const char* sq = smem + SG::A;  // qr (readers)
  const char* sk = smem + SG::B;  // kr
  const char* sv = smem + SG::X;  // vr
  const char* sx = smem + SG::Y;  // xdot rows

  // A fragments (rows = state column n of column tile nt, k = d) of an fp32 state
  auto state_frags = [&](Frag (&nf)[KSD], __amdgpu_buffer_rsrc_t S, int nt) __attribute__((always_inline)) {
    f32x4 t[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) t[dt] = load_state_tile<D>(S, dt, nt, lane);
#pragma unroll
    for (int s = 0; s < KSD; ++s) nf[s] = M::acc_frag(t, s);
  };

  // block gate sums of the blocks strictly between J and block x (exclusive)
  auto gap_blocks = [&](int x) {
    float d = 0.f;
    for (int y = bk.J + 1; y < x; ++y) d += n.GS[(int64_t)bk.bh * n.nb + y];
    return d;
  };

  for (int j = n.P - 1; j >= 0; --j) {
    const int64_t row0 = bk.row + (int64_t)j * C * a.H;
    __syncthreads();  // the previous chunk's tiles and bucket updates are done everywhere
    stage_tile<T, D, C>(qr, row0, a.H, smem + SG::A, tid, 64 * NW);
    stage_tile<T, D, C>(kr, row0, a.H, smem + SG::B, tid, 64 * NW);
    stage_tile<T, D, C>(vr, row0, a.H, smem + SG::X, tid, 64 * NW);
    if (xdot) stage_tile<T, D, C>(xdot, row0, a.H, smem + SG::Y, tid, 64 * NW);
    stage_gates<C>(a.g, a.lam, row0, a.H, a.L, n.LS, gl, reinterpret_cast<float*>(smem + SG::LAM), tid, 64 * NW);
    __syncthreads();
    const float gsum = stage_prefix<C>(gl, gp, wv, lane);
    __syncthreads();
    // weight rows lambda_t^{LOGC+m} e^{G_t} of the chunk-level buckets this chunk joins
    for (int x = tid; x < MAXB * C; x += 64 * NW) {
      const int m = x / C + 1, t = x % C;
      if (m <= logP && ((j >> (m - 1)) & 1)) wt[x] = ll[t * kLevelsMax + LOGC + m] * __expf(gp[t]);
    }
    const int s = 16 * st_ + q16;  // this lane's source row
    const float Gs = gp[s];

    // --- buckets after this chunk: Out^T[n][s] = sum_X e^{G_{X0-1} - G_s} R_X^T qr_s
    f32x4 o[DT];
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag qf[KSD];
#pragma unroll
    for (int k = 0; k < KSD; ++k) qf[k] = frag_row<T, C, D>(sq, s, k, g4);
    auto bucket_read = [&](const float* R, float scale) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(R, SB * 4);
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) {
        Frag nf[KSD];
        state_frags(nf, rs, nt);
        f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KSD; ++k) z = M::mma(nf[k], qf[k], z);
        o[nt] += scale * z;
      }
    };
    const float dec_end = gsum - Gs;  // G_{chunk end} - G_s
    // chunk-level buckets: the sibling after this chunk's group at level m (bit m-1 of j clear)
#pragma unroll
    for (int m = 1; m <= MAXB; ++m)
      if (m <= logP && !((j >> (m - 1)) & 1)) bucket_read(Rm + (m - 1) * SB, __expf(dec_end + suf - sufX[m]));
    // block-level buckets: the sibling after J's group of 2^b blocks (bit b of J clear)
    {
      const float base = dec_end + suf;  // to the end of block J
      for (int b = 0; b < nbl; ++b) {
        if ((bk.J >> b) & 1) continue;
        const int first = ((bk.J >> b) + 1) << b;
        if (first >= n.nb) continue;
        bucket_read(W + (((int64_t)bk.bh * n.nb + first) * nbl + b) * SB, __expf(base + gap_blocks(first)));
      }
    }

    // the cross-chunk part's dot with xdot_s, before the in-chunk terms join
    float dot = 0.f;
    if (xdot) {
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) {
        const T* xr = reinterpret_cast<const T*>(sx + TL::off(s, 16 * nt + 4 * g4));
#pragma unroll
        for (int e = 0; e < 4; ++e) dot += o[nt][e] * to_f32(xr[e]);
      }
      dot = sum_groups(dot);
    }

    // --- in chunk: Out^T[n][s] = sum_t vr^T[n][t] P[t][s] for t >= s; P tiles with
    // lanes holding rows t = 16 tt + 4 (lane/16) + e of column s (the k operand order)
    f32x4 pt[CT];
#pragma unroll
    for (int tt = 0; tt < CT; ++tt) {
      pt[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (tt < st_) continue;
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSD; ++k) x = M::mma(frag_row<T, C, D>(sk, 16 * tt + q16, k, g4), frag_row<T, C, D>(sq, s, k, g4), x);
      const f32x4 gt = *reinterpret_cast<const f32x4*>(gp + 16 * tt + 4 * g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tt + 4 * g4 + e;
        const int lev = (t == s) ? 0 : 32 - __clz(t ^ s);
        pt[tt][e] = (t >= s) ? x[e] * ll[t * kLevelsMax + lev] * __expf(gt[e] - Gs) : 0.f;
      }
    }
    Frag pf[KSC];
#pragma unroll
    for (int k = 0; k < KSC; ++k) pf[k] = M::acc_frag(pt, k);
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      Frag vf[KSC];
#pragma unroll
      for (int k = 0; k < KSC; ++k) vf[k] = frag_col<T, C, D>(sv, 16 * nt, k, lane);
      lds_wait(vf);
#pragma unroll
      for (int k = 0; k < KSC; ++k) o[nt] = M::mma(vf[k], pf[k], o[nt]);
    }

    // --- outputs of row s: lanes hold columns 16 nt + 4 (lane/16) + e
    {
      const int64_t orow = row0 + (int64_t)s * a.H;
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) {
        Vec4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (T)o[nt][e];
        *reinterpret_cast<Vec4*>(static_cast<T*>(out) + orow * D + 16 * nt + 4 * g4) = ov;
      }
      if (xdot && g4 == 0) dot_out[orow] = dot;
    }

    // --- this chunk joins the chunk-level buckets it lies in (bit m-1 of j set):
    // R_m = e^{g_j} R_m + sum_t lambda_t^{LOGC+m} e^{G_t} kr_t vr_t^T, a fresh
    // bucket when j is its last chunk; each wave makes the tiles dt = wave, ...
    __syncthreads();  // every wave has read the buckets
    const float carry = __expf(gsum);
    for (int dt = wv; dt < DT; dt += NW) {
      Frag kf[KSC];
#pragma unroll
      for (int k = 0; k < KSC; ++k) kf[k] = frag_col<T, C, D>(sk, 16 * dt, k, lane);
      for (int nt = 0; nt < DT; ++nt) {
        Frag vf[KSC];
#pragma unroll
        for (int k = 0; k < KSC; ++k) vf[k] = frag_col<T, C, D>(sv, 16 * nt, k, lane);
        lds_wait(kf, vf);
#pragma unroll
        for (int m = 1; m <= MAXB; ++m) {
          if (m > logP || !((j >> (m - 1)) & 1)) continue;
          const float* w = wt + (m - 1) * C;
          float* dst = Rm + (m - 1) * SB + state_tile_offset<D>(dt, nt, lane);
          const bool fresh = ((j + 1) & ((1 << (m - 1)) - 1)) == 0;
          f32x4 acc = fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : carry * *reinterpret_cast<const f32x4*>(dst);
#pragma unroll
          for (int k = 0; k < KSC; ++k) acc = M::mma(kf[k], scale_tokens<T>(vf[k], w, k, g4), acc);
          *reinterpret_cast<f32x4*>(dst) = acc;
        }
      }
    }
    suf += gsum;
#pragma unroll
    for (int m = 1; m <= MAXB; ++m)
      if (m <= logP && ((j >> (m - 1)) & 1)) sufX[m] = suf;
  }
}

// ---------------------------------------------------------------------------
// ll_bwd_gate: one workgroup per head, adds to the in-chunk share in dlog_gate
// the cross-chunk pairs' share sum_{t >= r} (dOo_t - xdv_t), walking the tokens
// from the end in tiles of 256 with the running sum carried.
__global__ void __launch_bounds__(256) ll_bwd_gate_suffix(BwdArgs a, const float* dOo, const float* xdv) {
  __shared__ float sbuf[256];
  const int bh = blockIdx.x, h = bh % a.H, b = bh / a.H;
  const int tid = threadIdx.x;
  float carry = 0.f;
  for (int t0 = a.T - 256; t0 > -256; t0 -= 256) {
    const int t = t0 + (255 - tid);  // thread 0 takes the latest token of the tile
    const int64_t r = ((int64_t)b * a.T + t) * a.H + h;
    sbuf[tid] = (t >= 0) ? dOo[r] - xdv[r] : 0.f;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const float add = tid >= off ? sbuf[tid - off] : 0.f;
      __syncthreads();
      sbuf[tid] += add;
      __syncthreads();
    }
    if (t >= 0) a.dlog_gate[r] += carry + sbuf[tid];
    carry += sbuf[255];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, int C>
static hipError_t launch_native_t(const BwdArgs& a, const BwdFwdNodes& n, const BwdWork& w, int pass, hipStream_t s) {
  constexpr int MAXB = max_block_depth(D);
  constexpr int NLB = D >= 128 ? 4 : 8;  // block levels per rev_state workgroup: NLB x D/16 accumulator tiles
  const int grid = a.B * a.H * n.nb;
  if (pass == 0) {
    hipLaunchKernelGGL((ll_bwd_levels<T, D, C, MAXB>), dim3(grid), dim3(64 * (C / 16)), 0, s, a, n, w.dOo, w.scratch);
  } else if (pass == 1 || pass == 3) {
    // the reverse bucket states of (kr, vr): (q, dO) for dv, (dO, q) for dk
    const void* kr = pass == 1 ? a.q : a.dO;
    const void* vr = pass == 1 ? a.dO : a.q;
    if (w.nbl == 0) return hipSuccess;  // one block per head: no block-level buckets
    hipLaunchKernelGGL((ll_bwd_rev_state<T, D, C, NLB>), dim3(grid, (w.nbl + NLB - 1) / NLB), dim3(64 * (D / 16)), 0,
                       s, a, n, kr, vr, w.W, w.nbl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)a.B * a.H * w.nbl * n.nb * (D * D / 4);
    const int sgrid = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    hipLaunchKernelGGL(ll_bwd_rev_scan, dim3(sgrid), dim3(256), 0, s, n, a.B * a.H, D * D, w.W, w.nbl);
  } else if (pass == 2) {
    // dv: readers k, states of (q, dO), in-chunk values dO; v . dv for the gate
    hipLaunchKernelGGL((ll_bwd_revread<T, D, C, MAXB>), dim3(grid), dim3(64 * (C / 16)), 0, s, a, n, a.k,
                       a.q, a.dO, (const float*)w.W, w.nbl, a.dv, a.v, w.xdv, w.scratch);
  } else if (pass == 4) {
    // dk: readers v, states of (dO, q), in-chunk values q
    hipLaunchKernelGGL((ll_bwd_revread<T, D, C, MAXB>), dim3(grid), dim3(64 * (C / 16)), 0, s, a, n, a.v,
                       a.dO, a.q, (const float*)w.W, w.nbl, a.dk, (const void*)nullptr, (float*)nullptr, w.scratch);
  } else {
    hipLaunchKernelGGL(ll_bwd_gate_suffix, dim3(a.B * a.H), dim3(256), 0, s, a, w.dOo, w.xdv);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_native(int io, int D, int C, const BwdArgs& a, const BwdFwdNodes& n, const BwdWork& w, int pass,
                             hipStream_t s) {
  if (io == 1) {
    switch (D * 1000 + C) {
      case 32032: return launch_native_t<bf16, 32, 32>(a, n, w, pass, s);
      case 32064: return launch_native_t<bf16, 32, 64>(a, n, w, pass, s);
      case 64032: return launch_native_t<bf16, 64, 32>(a, n, w, pass, s);
      case 64064: return launch_native_t<bf16, 64, 64>(a, n, w, pass, s);
      case 128032: return launch_native_t<bf16, 128, 32>(a, n, w, pass, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (D * 1000 + C) {
    case 16016: return launch_native_t<float, 16, 16>(a, n, w, pass, s);
    case 16032: return launch_native_t<float, 16, 32>(a, n, w, pass, s);
    case 16064: return launch_native_t<float, 16, 64>(a, n, w, pass, s);
    case 32016: return launch_native_t<float, 32, 16>(a, n, w, pass, s);
    case 32032: return launch_native_t<float, 32, 32>(a, n, w, pass, s);
    case 32064: return launch_native_t<float, 32, 64>(a, n, w, pass, s);
    case 64016: return launch_native_t<float, 64, 16>(a, n, w, pass, s);
    case 64032: return launch_native_t<float, 64, 32>(a, n, w, pass, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace llattn
