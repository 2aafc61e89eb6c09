// bwd_native.hip -- the backward pass of the Mamba-2 log-linear read
// ("Log-Linear Attention", section 2.3: the masked form evaluated chunk by
// chunk; section 3: training at scale) as kernels of its own.
//
// With pair weights M[t,s] = lambda_t^{lev(t,s)} e^{G_t - G_s} (s <= t, G the
// inclusive prefix of log a) and E[t,s] = e^{G_t - G_s} (q_t . k_s)(dO_t . v_s):
//   dlambda_t^l = sum_{s: lev(t,s) = l} E[t,s]
//   dq_t        = sum_s M[t,s] (dO_t . v_s) k_s
//   dv_s        = sum_{t >= s} M[t,s] (q_t . k_s) dO_t
//   dk_s        = sum_{t >= s} M[t,s] (dO_t . v_s) q_t
//   dlog_gate_r = sum_{s < r <= t} lambda_t^{lev(t,s)} E[t,s]   (the pairs the gate of r decays)
//
// Forward walk (ll_bwd_fwalk): with S the Fenwick state of a bucket of
// sources (sum e^{..} k_s v_s^T), one product u = S dO_t per level gives both
// dlambda_t^l = e^{..} q_t . u and the level's share lambda_t^l e^{..} u of
// dq_t.  The states are kept transposed (S^T, sum v_s k_s^T), so that the
// product is a plain read of the tile layout; the block-level nodes are the
// forward's block states and Fenwick nodes built from (v, k).
//
// Reverse walk (ll_bwd_rwalk): for a source s, the targets t at level l >= 1
// form one aligned bucket X, the sibling right after the aligned group of s,
// and every bucket is read at exactly one level (log2 |X| + 1).  One state per
// bucket, R_X = sum_{t in X} lambda_t^{lev(X)} e^{G_t - G_{X0-1}} q_t dO_t^T
// (X0 its first token), gives both dv_s += e^{G_{X0-1} - G_s} R_X^T k_s and
// dk_s += e^{G_{X0-1} - G_s} R_X v_s.  Chunk-level buckets are built during
// the walk (from the last chunk to the first); block-level buckets come from
// ll_bwd_rev_state (each block's share) and ll_bwd_rev_scan (their sums).
//
// The gate gradient splits by pairs: those inside one chunk give, per chunk,
// sum_{t >= r} (row sum of t) - sum_{s >= r} (column sum of s) over the
// chunk's exact fp32 pair terms (forward walk); those across chunks give the
// suffix sum over later tokens of dO_t . o_t^x - v_t . dv_t^x, the parts of
// dO . o and v . dv (= k . dk) that come from other chunks (the reverse walk
// sums within the block, ll_bwd_gate_add adds the later blocks).  Only the
// cross-chunk parts, small where the gates decay within a chunk, run through
// the long suffix sum.
#include <mutex>
#include <type_traits>

#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

namespace {

constexpr int logc_of(int C) { return C == 16 ? 4 : C == 32 ? 5 : 6; }

// An fp32 D x D state in LDS: the tile layout (16x16 tiles, accumulator order)
// with 4 floats of padding after every 16 lanes of a tile, so that reading a
// tile across (one float per lane, ds_read_b32) touches distinct banks.
template <int D>
struct PadState {
  static constexpr int DT = D / 16;
  static constexpr int TS = 4 * 68;  // floats per tile
  static constexpr int FLOATS = DT * DT * TS;
  // float offset of the four floats lane `ln` holds in tile (tr, tc)
  __device__ __forceinline__ static int off(int tr, int tc, int ln) { return (tr * DT + tc) * TS + 4 * ln + 4 * (ln >> 4); }
};

// A fragments of a state X in the tile layout: rows = column 16 tc + lane%16
// of X, k = the rows of X.  ld(tr, tc) returns this lane's four floats of
// tile (tr, tc).
template <typename T, int D, typename Ld>
__device__ __forceinline__ void col_frags(typename Mma<T>::Frag (&nf)[D / Mma<T>::KS], int tc, Ld ld) {
  f32x4 t[D / 16];
#pragma unroll
  for (int tr = 0; tr < D / 16; ++tr) t[tr] = ld(tr, tc);
#pragma unroll
  for (int s = 0; s < D / Mma<T>::KS; ++s) nf[s] = Mma<T>::acc_frag(t, s);
}

// A fragments of a state X: rows = row 16 tr + lane%16 of X, k = the columns
// of X, one float per lane and k index.  ld(tile_r, tile_c, lane, slot)
// returns an element of X.
template <typename T, int D, typename Ld>
__device__ __forceinline__ void row_frags(typename Mma<T>::Frag (&nf)[D / Mma<T>::KS], int tr, int lane, Ld ld) {
  using M = Mma<T>;
  const int g = lane >> 4, ar = lane & 15;
#pragma unroll
  for (int s = 0; s < D / M::KS; ++s) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int b = M::kidx(s, g, e);
        nf[s][e] = (bf16)ld(tr, b >> 4, 16 * (ar >> 2) + (b & 15), ar & 3);
      }
    } else {
      const int b = M::kidx(s, g, 0);
      nf[s] = ld(tr, b >> 4, 16 * (ar >> 2) + (b & 15), ar & 3);
    }
  }
}

// Sum over the four lane groups (lanes q, q + 16, q + 32, q + 48).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Stages the gate prefix: every wave scans, wave 0 writes it to LDS for the
// others (visible after the caller's next barrier).  Returns the chunk's gate
// sum.
template <int C>
__device__ __forceinline__ float stage_prefix(const float* gl, float* gp, int wv, int lane) {
  const float G = chunk_scan<C>(lane < C ? gl[lane] : 0.f);
  if (wv == 0 && lane < C) gp[lane] = G;
  return __shfl(G, C - 1, 64);
}

// The block a workgroup walks: (block J, head) from a logical id, and the
// [B,T,H] row of the block's first token.
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

// LDS of the two walks: two staging buffers (each: the q, k, v and dO tiles,
// the gates, two more per-row values and the level weights [C][LS] of one
// chunk, loaded straight into LDS one chunk ahead), per-chunk scratch, and
// the chunk-level states when they fit.  FW: the forward walk's dlambda rows
// and level part of dq, handed from one wave group to the other.
template <typename T, int D, int C, int MAXB, bool SLDS, bool FW>
struct WalkSmem {
  typedef Tile<T, C, D> TL;
  static constexpr int NW = C / 16;
  static constexpr int NWT = 8;  // per-token weight rows
  static constexpr int TQ = 0, TK = TL::BYTES, TV = 2 * TL::BYTES, TD = 3 * TL::BYTES;
  static constexpr int GOFF = 4 * TL::BYTES;   // gates [C]
  static constexpr int R1OFF = GOFF + C * 4;   // a per-row value [C]
  static constexpr int R2OFF = R1OFF + C * 4;  // another [C]
  static constexpr int LOFF = R2OFF + C * 4;   // level weights [C][LS]
  static constexpr int BUF = LOFF + C * kLevelsMax * 4;
  static constexpr int GP = 2 * BUF;            // in-chunk prefix of the gates [C]
  static constexpr int WT = GP + C * 4;         // per-token weight rows [NWT][C]
  static constexpr int XIN = WT + NWT * C * 4;  // per-wave column sums [NW][C]
  static constexpr int DOI = XIN + NW * C * 4;  // row sums [C]
  static constexpr int DL = DOI + C * 4;        // dlambda of the chunk's rows [C][kLevelsMax]
  static constexpr int DQS = DL + (FW ? C * kLevelsMax * 4 : 0);  // dq of the levels above the chunk [C][D]
  static constexpr int ST = DQS + (FW ? C * D * 4 : 0);           // chunk-level states [MAXB] (padded layout)
  static constexpr int BYTES = ST + (SLDS ? MAXB * PadState<D>::FLOATS * 4 : 0);
};

// Fragment registers of one state, the budget for the nodes a walk holds.
template <typename T, int D>
constexpr int state_frag_vgprs() {
  return (D / 16) * (D / Mma<T>::KS) * (int)(sizeof(typename Mma<T>::Frag) / 4);
}

}  // namespace

// ---------------------------------------------------------------------------
// ll_bwd_fwalk: one workgroup per (block J, head), two groups of C/16 waves;
// wave rt of each group owns the target rows 16 rt .. 16 rt + 15 of every
// chunk.  Walks the block's chunks in order.
//   Group A, the chunk itself: the score tiles q.k and dO.v per pair (exact
//     products of the io values, fp32 sums) give the in-chunk dlambda bins,
//     the in-chunk dq and the gate's in-chunk share; and the block's shares
//     of the reverse bucket states of the first NLBF block levels,
//       W[J][b] = sum_{t in J} lambda_t^{l_b} e^{G_t - G_{J0-1}} q_t dO_t^T.
//   Group B, the levels above the chunk: u = S dO_r on the matrix cores for
//     every state S the chunk reads (chunk-level states S^T of earlier chunks
//     of the block, merged by the recurrent form's rule and kept in fp32;
//     Fenwick nodes of earlier blocks, the forward's of (v, k), the first
//     MAXH held in registers), dlambda = e^{..} q_r . u and the level part of
//     dq, lambda_r^l e^{..} u; then the merge of this chunk's state.
// Writes dlambda (every level, zero where no bucket exists), dq, the
// cross-chunk part of dO . o, the gate's in-chunk share and the shares W.
template <typename T, int D, int C, int MAXB, int MAXH, int NLBF, bool SLDS>
__global__ void __launch_bounds__(128 * (C / 16)) ll_bwd_fwalk(BwdArgs a, BwdFwdNodes n, BwdWork w) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef WalkSmem<T, D, C, MAXB, SLDS, true> SM;
  typedef Tile<T, C, D> TL;
  typedef PadState<D> PS;
  typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type Vec4;
  constexpr int NW = C / 16, NWA = 2 * NW, DT = D / 16, KSD = D / M::KS, KSC = C / M::KS, CT = C / 16;
  constexpr int LOGC = logc_of(C);
  constexpr int NTW = (DT + NW - 1) / NW;  // column tiles of the shares per wave of group A
  constexpr int SB = D * D;
  constexpr int NH = MAXH > 0 ? MAXH : 1;
  constexpr int NL = NLBF > 0 ? NLBF : 1;
  static_assert(1 + NLBF <= SM::NWT, "a weight row per held block level");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool gb = wv >= NW;  // group B
  const int rt = gb ? wv - NW : wv;
  const int g4 = lane >> 4, q16 = lane & 15;
  const int r = 16 * rt + q16;  // this lane's target row
  BlockOf bk;
  bk.set(xcd_logical_id(blockIdx.x, gridDim.x), a, n.nb, n.P, C);
  const int logP = ilog2c(n.P);
  const int LS = n.LS;
  const int nbl = w.nbl;
  // block levels b < NLBF that J lies in (bit b of J set): this walk makes J's share
  const int sbits = NLBF > 0 ? bk.J & ((1 << (nbl < NLBF ? nbl : NLBF)) - 1) : 0;
  float* gp = reinterpret_cast<float*>(smem + SM::GP);
  float* wt = reinterpret_cast<float*>(smem + SM::WT);
  float* dl = reinterpret_cast<float*>(smem + SM::DL);
  float* dqs = reinterpret_cast<float*>(smem + SM::DQS);
  float* stl = reinterpret_cast<float*>(smem + SM::ST);
  float* stg = SLDS ? nullptr : w.scratch + (int64_t)blockIdx.x * MAXB * SB;

  ChunkLoads<T, D, C, NWA> cl;
  cl.init(wv, lane, a.H, a.L, LS);
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int64_t row0 = bk.row + (int64_t)j * C * a.H;
    char* buf = smem + (j & 1) * SM::BUF;
    cl.tiles(a.q, row0, buf + SM::TQ, wv);
    cl.tiles(a.k, row0, buf + SM::TK, wv);
    cl.tiles(a.v, row0, buf + SM::TV, wv);
    cl.tiles(a.dO, row0, buf + SM::TD, wv);
    cl.gates(a.g, row0, reinterpret_cast<float*>(buf + SM::GOFF), wv, lane);
    cl.lambda(a.lam, row0, a.L, reinterpret_cast<float*>(buf + SM::LOFF), wv, lane);
  };
  issue(0);
  for (int x = tid; x < C * kLevelsMax; x += 64 * NWA) dl[x] = 0.f;

  // group B: Fenwick nodes of earlier blocks, one per set bit of J, most recent first
  auto node_ptr = [&](int e) {
    return (e & 1) ? n.F + ((int64_t)bk.bh * n.nF + (e >> 1)) * SB : n.S + ((int64_t)bk.bh * n.nb + e) * SB;
  };
  auto node_gamma = [&](int e) {
    return (e & 1) ? n.GF[(int64_t)bk.bh * n.nF + (e >> 1)] : n.GS[(int64_t)bk.bh * n.nb + e];
  };
  // Registers held for the whole walk, shared by the groups: group B's node
  // fragments (node x, tile dt, step k at (x DT + dt) KSD + k) or group A's
  // share accumulators (level b, column tile nt = rt + i NW, row tile dt at
  // (b NTW + i) DT + dt, one f32x4 each).
  constexpr int FPV = (int)(sizeof(Frag) / 4);  // floats per fragment
  constexpr int NHOLD_N = MAXH * DT * KSD, NHOLD_W = NL * NTW * DT * 4 / FPV;
  Frag hold[NHOLD_N > NHOLD_W ? NHOLD_N : NHOLD_W];
  auto wacc_get = [&](int idx) __attribute__((always_inline)) {
    if constexpr (FPV == 4) {
      return __builtin_bit_cast(f32x4, hold[idx]);
    } else {
      return f32x4{hold[4 * idx], hold[4 * idx + 1], hold[4 * idx + 2], hold[4 * idx + 3]};
    }
  };
  auto wacc_set = [&](int idx, f32x4 v) __attribute__((always_inline)) {
    if constexpr (FPV == 4) {
      hold[idx] = __builtin_bit_cast(Frag, v);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) hold[4 * idx + e] = v[e];
    }
  };
  int hlv[NH];
  float hdd[NH];
  int rest_far = bk.J;
  float dd_far = 0.f;
#pragma unroll
  for (int x = 0; x < NH; ++x) {
    hlv[x] = -1;
    hdd[x] = 0.f;
  }
  if (gb) {
#pragma unroll
    for (int x = 0; x < MAXH; ++x) {
      if (rest_far > 0) {
        const int e = rest_far - 1;
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(node_ptr(e), SB * 4);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          Frag nf[KSD];
          col_frags<T, D>(nf, dt, [&](int tr, int tc) { return load_state_tile<D>(rs, tr, tc, lane); });
#pragma unroll
          for (int k = 0; k < KSD; ++k) hold[(x * DT + dt) * KSD + k] = nf[k];
        }
        hlv[x] = LOGC + 1 + logP + __ffs(rest_far) - 1;
        hdd[x] = dd_far;
        dd_far += node_gamma(e);
        rest_far &= rest_far - 1;
      }
    }
  } else {
#pragma unroll
    for (int x = 0; x < NHOLD_W; ++x) wacc_set(x, f32x4{0.f, 0.f, 0.f, 0.f});
  }

  float sig[MAXB + 1];  // lazy log-scales of the chunk-level states
#pragma unroll
  for (int m = 0; m <= MAXB; ++m) sig[m] = 0.f;
  float gw = 0.f;  // log-decay from the block start to the current chunk's start

  // outputs of a chunk, stored during the next one
  float odo = 0.f, odin = 0.f;
  Vec4 odq[DT];
  auto store_out = [&](int jj) __attribute__((always_inline)) {
    const int64_t row0 = bk.row + (int64_t)jj * C * a.H;
    const int64_t orow = row0 + (int64_t)r * a.H;
    if (!gb) {
      // lane group g writes levels g, g + 4, ... and clears them for the next chunk
      for (int l = g4; l < a.L; l += 4) {
        float v = 0.f;
        if (l < kLevelsMax) {
          v = dl[r * kLevelsMax + l];
          dl[r * kLevelsMax + l] = 0.f;
        }
        a.dlambda[orow * a.L + l] = v;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<Vec4*>(static_cast<T*>(a.dq) + orow * D + 16 * dt + 4 * g4) = odq[dt];
      if (wv == 0 && lane < C) w.din[row0 + (int64_t)lane * a.H] = odin;
    } else if (g4 == 0) {
      w.dOo[orow] = odo;
    }
  };

  for (int j = 0; j < n.P; ++j) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk j and stores of chunk j-2 are done
    lds_barrier();                  // chunk j has landed everywhere; chunk j-1 is done with
    if (j > 0) store_out(j - 1);
    if (j + 1 < n.P) issue(j + 1);
    const char* buf = smem + (j & 1) * SM::BUF;
    const char* sq = buf + SM::TQ;
    const char* sk = buf + SM::TK;
    const char* sv = buf + SM::TV;
    const char* sdo = buf + SM::TD;
    const float* ll = reinterpret_cast<const float*>(buf + SM::LOFF);  // [C][LS]
    const float gsum = stage_prefix<C>(reinterpret_cast<const float*>(buf + SM::GOFF), gp, wv, lane);
    lds_barrier();
    // weight rows: 0, the decay of each source to the chunk's end (merge); 1 + b,
    // lambda_t^{l_b} e^{G_t - G_{J0-1}} for the share of block level b
    for (int x = tid; x < (1 + NLBF) * C; x += 64 * NWA) {
      const int row = x / C, t = x % C;
      if (row == 0) wt[x] = __expf(gsum - gp[t]);
      else if ((sbits >> (row - 1)) & 1) wt[x] = ll[t * LS + LOGC + logP + row] * __expf(gw + gp[t]);
    }
    lds_barrier();
    const float Gr = gp[r];
    const float* lr = ll + r * LS;  // level weights of row r
    Frag dofr[KSD];                 // row r of dO (k = head dim)
#pragma unroll
    for (int k = 0; k < KSD; ++k) dofr[k] = frag_row<T, C, D>(sdo, r, k, g4);

    f32x4 dq[DT];  // group A: in-chunk dq; group B: the levels' dq
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!gb) {
      Frag qfr[KSD];
#pragma unroll
      for (int k = 0; k < KSD; ++k) qfr[k] = frag_row<T, C, D>(sq, r, k, g4);
      // --- in-chunk levels 0..LOGC.  Lanes hold sources s = 16 ct + 4 (lane/16) + e
      // of target r; a tile ct < rt lies at the one level 4 + bit_length(rt ^ ct),
      // the diagonal tile at levels bit_length((r ^ s) % 16) <= 4.
      float bin[LOGC + 1];
#pragma unroll
      for (int l = 0; l <= LOGC; ++l) bin[l] = 0.f;
      f32x4 ptl[CT];  // in-chunk dq weights lambda_r^lev e^{G_r - G_s} (dO_r . v_s), rows s
      float* xin = reinterpret_cast<float*>(smem + SM::XIN) + rt * C;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        ptl[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (ct > rt) continue;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f}, y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KSD; ++k) {
          x = M::mma(frag_row<T, C, D>(sk, 16 * ct + q16, k, g4), qfr[k], x);
          y = M::mma(frag_row<T, C, D>(sv, 16 * ct + q16, k, g4), dofr[k], y);
        }
        const f32x4 gs = *reinterpret_cast<const f32x4*>(gp + 16 * ct + 4 * g4);
        f32x4 col;
        if (ct < rt) {
          const int lev = 4 + 32 - __clz(rt ^ ct);
          const float lam = lr[lev];
          float sxy = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ey = y[e] * __expf(Gr - gs[e]);
            sxy += x[e] * ey;
            ptl[ct][e] = lam * ey;
            col[e] = lam * x[e] * ey;
          }
#pragma unroll
          for (int l = 5; l <= LOGC; ++l)
            if (l == lev) bin[l] += sxy;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s4 = 4 * g4 + e;  // source within the tile
            float ey = 0.f, lam = 0.f;
            int lev = 0;
            if (s4 <= q16) {
              lev = 32 - __clz(q16 ^ s4);
              lam = lr[lev];
              ey = y[e] * __expf(Gr - gs[e]);
            }
            const float v = x[e] * ey;
#pragma unroll
            for (int l = 0; l <= 4; ++l)
              if (l == lev) bin[l] += v;
            ptl[ct][e] = lam * ey;
            col[e] = lam * v;
          }
        }
        // column sums over this wave's 16 targets: a prefix within each 16-lane row, total at lane 15
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          col[e] += dpp_f32<0x111, 0xf, true>(col[e]);
          col[e] += dpp_f32<0x112, 0xf, true>(col[e]);
          col[e] += dpp_f32<0x114, 0xf, true>(col[e]);
          col[e] += dpp_f32<0x118, 0xf, true>(col[e]);
        }
        if (q16 == 15) *reinterpret_cast<f32x4*>(xin + 16 * ct + 4 * g4) = col;
      }
      float rsum = 0.f;  // row sum of the in-chunk pair terms
#pragma unroll
      for (int l = 0; l <= LOGC; ++l) {
        const float v = sum_groups(bin[l]);
        rsum += lr[l] * v;
        if (g4 == 0) dl[r * kLevelsMax + l] = v;
      }
      if (g4 == 0) reinterpret_cast<float*>(smem + SM::DOI)[r] = rsum;

      // --- in-chunk dq: dq^T[d][r] = sum_s k^T[d][s] P[s][r]
      {
        Frag pf[KSC];
#pragma unroll
        for (int k = 0; k < KSC; ++k) pf[k] = M::acc_frag(ptl, k);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          Frag kf[KSC];
#pragma unroll
          for (int k = 0; k < KSC; ++k) kf[k] = frag_col<T, C, D>(sk, 16 * dt, k, lane);
          lds_wait(kf);
#pragma unroll
          for (int k = 0; k < KSC; ++k)
            if (M::first_tile(k) <= rt) dq[dt] = M::mma(kf[k], pf[k], dq[dt]);
        }
      }

      // --- the shares: tile (dt, nt) += sum_t q_t[d] w_b(t) dO_t[n]
      if (sbits) {
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
          const int nt = rt + i * NW;
          if (nt >= DT) continue;
          Frag vw[NL][KSC];
          {
            Frag vf[KSC];
#pragma unroll
            for (int k = 0; k < KSC; ++k) vf[k] = frag_col<T, C, D>(sdo, 16 * nt, k, lane);
            lds_wait(vf);
#pragma unroll
            for (int b = 0; b < NL; ++b)
#pragma unroll
              for (int k = 0; k < KSC; ++k) vw[b][k] = scale_tokens<T>(vf[k], wt + (1 + b) * C, k, g4);
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            Frag qf[KSC];
#pragma unroll
            for (int k = 0; k < KSC; ++k) qf[k] = frag_col<T, C, D>(sq, 16 * dt, k, lane);
            lds_wait(qf);
#pragma unroll
            for (int b = 0; b < NL; ++b) {
              if (!((sbits >> b) & 1)) continue;
              f32x4 acc = wacc_get((b * NTW + i) * DT + dt);
#pragma unroll
              for (int k = 0; k < KSC; ++k) acc = M::mma(qf[k], vw[b][k], acc);
              wacc_set((b * NTW + i) * DT + dt, acc);
            }
          }
        }
      }
    } else {
      // --- levels above the chunk: u = S dO_r (lanes: rows d = 16 dt + 4 (lane/16) + e)
      f32x4 qv[DT];  // q_r at those rows
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const T* p = reinterpret_cast<const T*>(sq + TL::off(r, 16 * dt + 4 * g4));
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[dt][e] = to_f32(p[e]);
      }
      odo = 0.f;
      // one level: scale = e^{G_r + decay from the state's end to the chunk start}
      auto level = [&](auto get, float scale, int lev) __attribute__((always_inline)) {
        const float lamw = lr[lev];
        float acc = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          Frag nf[KSD];
          get(dt, nf);
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < KSD; ++k) z = M::mma(nf[k], dofr[k], z);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc += z[e] * qv[dt][e];
          dq[dt] += (lamw * scale) * z;
        }
        const float v = sum_groups(acc) * scale;
        odo += lamw * v;
        if (g4 == 0) dl[r * kLevelsMax + lev] = v;
      };
      // within-block levels LOGC+1 .. LOGC+logP: states of earlier chunks of the block
#pragma unroll
      for (int m = 1; m <= MAXB; ++m)
        if (m <= logP && ((j >> (m - 1)) & 1)) {
          if constexpr (SLDS) {
            const float* X = stl + (m - 1) * PS::FLOATS;
            level(
                [&](int dt, Frag(&nf)[KSD]) {
                  col_frags<T, D>(nf, dt, [&](int tr, int tc) {
                    return *reinterpret_cast<const f32x4*>(X + PS::off(tr, tc, lane));
                  });
                },
                __expf(Gr + sig[m]), LOGC + m);
          } else {
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(stg + (m - 1) * SB, SB * 4);
            level(
                [&](int dt, Frag(&nf)[KSD]) {
                  col_frags<T, D>(nf, dt, [&](int tr, int tc) { return load_state_tile<D>(rs, tr, tc, lane); });
                },
                __expf(Gr + sig[m]), LOGC + m);
          }
        }
      // earlier blocks: the nodes held in registers, then the rest from memory
#pragma unroll
      for (int x = 0; x < MAXH; ++x)
        if (hlv[x] >= 0)
          level(
              [&](int dt, Frag(&nf)[KSD]) {
#pragma unroll
                for (int k = 0; k < KSD; ++k) nf[k] = hold[(x * DT + dt) * KSD + k];
              },
              __expf(Gr + gw + hdd[x]), hlv[x]);
      {
        int rest = rest_far;
        float dd = dd_far;
        while (rest > 0) {
          const int e = rest - 1;
          const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(node_ptr(e), SB * 4);
          level(
              [&](int dt, Frag(&nf)[KSD]) {
                col_frags<T, D>(nf, dt, [&](int tr, int tc) { return load_state_tile<D>(rs, tr, tc, lane); });
              },
              __expf(Gr + gw + dd), LOGC + 1 + logP + __ffs(rest) - 1);
          dd += node_gamma(e);
          rest &= rest - 1;
        }
      }
      // hand the levels' dq to group A
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dqs + ((rt * DT + dt) * 64 + lane) * 4) = dq[dt];
    }

    lds_barrier();  // sums, dlambda rows and the levels' dq are in; every wave has read the states of this chunk
    if (!gb) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 o = dq[dt] + *reinterpret_cast<const f32x4*>(dqs + ((rt * DT + dt) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) odq[dt][e] = (T)o[e];
      }
      // in-chunk share of the gate gradient: sum_{t >= p} (row sum t - column sum t)
      if (wv == 0) {
        float u = 0.f;
        if (lane < C) {
          const float* xs = reinterpret_cast<const float*>(smem + SM::XIN);
          u = reinterpret_cast<const float*>(smem + SM::DOI)[lane];
          for (int v = lane / 16; v < NW; ++v) u -= xs[v * C + lane];  // waves of targets >= the column's tile
        }
        const float pre = chunk_scan<C>(u);
        odin = __shfl(pre, C - 1, 64) - pre + u;
      }
    }

    // --- group B: this chunk's state and the merge rule of the chunk-level
    // states (levels 1..c and the chunk become level c+1, c = ctz(j+1)), kept
    // as S^T: tile (nt, dt) = sum_s e^{G[C-1] - G_s} v_s[n] k_s[d]; wave rt
    // makes the row tiles nt = rt, rt + NW, ...
#pragma unroll
    for (int m = 1; m <= MAXB; ++m) sig[m] += gsum;
    gw += gsum;
    if (gb && j + 1 < n.P) {
      const int c = __ffs(j + 1) - 1;
      for (int nt = rt; nt < DT; nt += NW) {
        Frag vf[KSC];
#pragma unroll
        for (int k = 0; k < KSC; ++k) vf[k] = frag_col<T, C, D>(sv, 16 * nt, k, lane);
        lds_wait(vf);
#pragma unroll
        for (int k = 0; k < KSC; ++k) vf[k] = scale_tokens<T>(vf[k], wt, k, g4);
        for (int dt = 0; dt < DT; ++dt) {
          Frag kf[KSC];
#pragma unroll
          for (int k = 0; k < KSC; ++k) kf[k] = frag_col<T, C, D>(sk, 16 * dt, k, lane);
          lds_wait(kf);
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
          float* dst = SLDS ? stl + c * PS::FLOATS + PS::off(nt, dt, lane) : stg + c * SB + state_tile_offset<D>(nt, dt, lane);
#pragma unroll
          for (int m = 1; m <= MAXB; ++m)
            if (m <= c) {
              const float* src = SLDS ? stl + (m - 1) * PS::FLOATS + PS::off(nt, dt, lane)
                                      : stg + (m - 1) * SB + state_tile_offset<D>(nt, dt, lane);
              acc += __expf(sig[m]) * *reinterpret_cast<const f32x4*>(src);
            }
#pragma unroll
          for (int k = 0; k < KSC; ++k) acc = M::mma(vf[k], kf[k], acc);
          *reinterpret_cast<f32x4*>(dst) = acc;
        }
      }
    }
    if (j + 1 < n.P) {
      const int c = __ffs(j + 1) - 1;
#pragma unroll
      for (int m = 1; m <= MAXB; ++m)
        if (m == c + 1) sig[m] = 0.f;
    }
  }
  lds_barrier();  // the last chunk's dlambda rows are in
  store_out(n.P - 1);
  if (!gb) {
#pragma unroll
    for (int b = 0; b < NL; ++b) {
      if (!((sbits >> b) & 1)) continue;
      float* dst = w.W + (((int64_t)bk.bh * n.nb + bk.J) * nbl + b) * SB;
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int nt = rt + i * NW;
        if (nt >= DT) continue;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4*>(dst + state_tile_offset<D>(dt, nt, lane)) = wacc_get((b * NTW + i) * DT + dt);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// ll_bwd_rev_state: the shares W[J][b] of the block levels b >= bfirst (those
// the forward walk does not make): one workgroup per (block J, head, group of
// NLB block levels), D/16 waves (one per 16 value columns).  For every block
// level b of the group with bit b of J set (J lies in a right bucket of 2^b
// blocks), the block's share of that bucket's state,
//   W[J][b] = sum_{t in J} lambda_t^{l_b} e^{G_t - G_{J0-1}} q_t dO_t^T,
// l_b = log2(C P) + 1 + b, in the tile layout.  The chunks are loaded straight
// into LDS one chunk ahead.
template <typename T, int D, int C>
struct RevSmem {
  typedef Tile<T, C, D> TL;
  static constexpr int TQ = 0, TD = TL::BYTES;
  static constexpr int GOFF = 2 * TL::BYTES;
  static constexpr int LOFF = GOFF + C * 4;
  static constexpr int BUF = LOFF + C * kLevelsMax * 4;
  static constexpr int GP = 2 * BUF;
  static constexpr int WT = GP + C * 4;  // weight rows [NLB][C]
};

template <typename T, int D, int C, int NLB>
__global__ void __launch_bounds__(64 * (D / 16)) ll_bwd_rev_state(BwdArgs a, BwdFwdNodes n, BwdWork w, int bfirst) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef RevSmem<T, D, C> SM;
  constexpr int NW = D / 16, DT = D / 16, KSC = C / M::KS, LOGC = logc_of(C);
  constexpr int SB = D * D;
  __shared__ __attribute__((aligned(1024))) char smem[SM::WT + NLB * C * 4];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;
  BlockOf bk;
  bk.set(xcd_logical_id(blockIdx.x, gridDim.x), a, n.nb, n.P, C);
  const int logP = ilog2c(n.P);
  const int nbl = w.nbl;
  const int b0 = bfirst + blockIdx.y * NLB;  // first block level of this group
  // this group's levels that J takes part in (bit b0 + b of J set)
  const int bits = (bk.J >> b0) & ((1 << NLB) - 1) & ((1 << (nbl > b0 ? nbl - b0 : 0)) - 1);
  if (bits == 0) return;
  const int LS = n.LS;
  float* gp = reinterpret_cast<float*>(smem + SM::GP);
  float* wt = reinterpret_cast<float*>(smem + SM::WT);
  ChunkLoads<T, D, C, NW> cl;
  cl.init(wv, lane, a.H, a.L, LS);
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int64_t row0 = bk.row + (int64_t)j * C * a.H;
    char* buf = smem + (j & 1) * SM::BUF;
    cl.tiles(a.q, row0, buf + SM::TQ, wv);
    cl.tiles(a.dO, row0, buf + SM::TD, wv);
    cl.gates(a.g, row0, reinterpret_cast<float*>(buf + SM::GOFF), wv, lane);
    cl.lambda(a.lam, row0, a.L, reinterpret_cast<float*>(buf + SM::LOFF), wv, lane);
  };
  issue(0);
  f32x4 acc[NLB][DT];
#pragma unroll
  for (int b = 0; b < NLB; ++b)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[b][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float pre = 0.f;  // G_{chunk start - 1} - G_{J0 - 1}
  for (int j = 0; j < n.P; ++j) {
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (j + 1 < n.P) issue(j + 1);
    const char* buf = smem + (j & 1) * SM::BUF;
    const float* ll = reinterpret_cast<const float*>(buf + SM::LOFF);
    const float gsum = stage_prefix<C>(reinterpret_cast<const float*>(buf + SM::GOFF), gp, wv, lane);
    lds_barrier();
    // weight rows lambda_t^{l_b} e^{G_t - G_{J0-1}} of the block levels J lies in
    for (int x = tid; x < NLB * C; x += 64 * NW) {
      const int b = x / C, t = x % C;
      if ((bits >> b) & 1) wt[x] = ll[t * LS + LOGC + logP + 1 + b0 + b] * __expf(pre + gp[t]);
    }
    lds_barrier();
    Frag kf[DT][KSC], vf[KSC];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int s = 0; s < KSC; ++s) kf[dt][s] = frag_col<T, C, D>(buf + SM::TQ, 16 * dt, s, lane);
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(buf + SM::TD, 16 * wv, s, lane);
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
    float* dst = w.W + (((int64_t)bk.bh * n.nb + bk.J) * nbl + b0 + b) * SB;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + state_tile_offset<D>(dt, wv, lane)) = acc[b][dt];
  }
}

// ---------------------------------------------------------------------------
// ll_bwd_rev_scan: for every head, block level b and right bucket X of 2^b
// blocks (blocks x 2^b .. (x+1) 2^b - 1, x odd), the bucket state
//   R_X = sum_{J in X} e^{G_{J0-1} - G_{X0-1}} W[J][b],
// written in place of W[x 2^b][b].  One thread per four state elements.
__global__ void __launch_bounds__(256) ll_bwd_rev_scan(BwdFwdNodes n, int BH, int D, BwdWork w) {
  const int DD = D * D, n4 = DD / 4;
  const int nbl = w.nbl;
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
      const f32x4 v = reinterpret_cast<const f32x4*>(w.W + (((int64_t)bh * n.nb + J) * nbl + b) * DD)[e4];
      sum += __expf(dec) * v;
      dec += n.GS[(int64_t)bh * n.nb + J];
    }
    reinterpret_cast<f32x4*>(w.W + (((int64_t)bh * n.nb + first) * nbl + b) * DD)[e4] = sum;
  }
}

// ---------------------------------------------------------------------------
// ll_bwd_rwalk: one workgroup per (block J, head), two groups of C/16 waves;
// wave rt of each group owns the source rows 16 rt .. 16 rt + 15 of every
// chunk.  Walks the block's chunks from the last to the first:
//   group A: dv_s = sum_{t >= s in chunk} P1[t,s] dO_t + sum_X e^{G_{X0-1} - G_s} R_X^T k_s
//   group B: dk_s = sum_{t >= s in chunk} P2[t,s] q_t  + sum_X e^{G_{X0-1} - G_s} R_X v_s
//   P1[t,s] = M[t,s] (q_t . k_s),  P2[t,s] = M[t,s] (dO_t . v_s)
// over the buckets X after s.  Chunk-level buckets are built from the chunks
// already walked (all waves) and kept in fp32, read as R by group A and
// across (one float per lane and k index) as R^T by group B; block-level
// buckets come from ll_bwd_rev_scan, the first MAXH held in registers by each
// group in the orientation it reads.  Group A also forms v_s . dv_s^x from the
// buckets (before the in-chunk terms) and wave 0 the gate gradient of every
// row up to the later blocks' share:
//   din_s + sum_{t >= s in the block} (dOo_t - v_t . dv_t^x),
// with the block's total left in BT for ll_bwd_gate_add.
template <typename T, int D, int C, int MAXB, int MAXH, bool SLDS>
__global__ void __launch_bounds__(128 * (C / 16)) ll_bwd_rwalk(BwdArgs a, BwdFwdNodes n, BwdWork w) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef WalkSmem<T, D, C, MAXB, SLDS, false> SM;
  typedef Tile<T, C, D> TL;
  typedef PadState<D> PS;
  typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type Vec4;
  constexpr int NW = C / 16, NWA = 2 * NW, DT = D / 16, KSD = D / M::KS, KSC = C / M::KS, CT = C / 16;
  constexpr int LOGC = logc_of(C);
  constexpr int SB = D * D;
  constexpr int NH = MAXH > 0 ? MAXH : 1;
  static_assert(MAXB <= SM::NWT, "a weight row per chunk level");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool gb = wv >= NW;  // group B: dk
  const int rt = gb ? wv - NW : wv;
  const int g4 = lane >> 4, q16 = lane & 15;
  const int s = 16 * rt + q16;  // this lane's source row
  BlockOf bk;
  bk.set(xcd_logical_id(blockIdx.x, gridDim.x), a, n.nb, n.P, C);
  const int logP = ilog2c(n.P);
  const int LS = n.LS;
  const int nbl = w.nbl;
  float* gp = reinterpret_cast<float*>(smem + SM::GP);
  float* wt = reinterpret_cast<float*>(smem + SM::WT);
  float* ub = reinterpret_cast<float*>(smem + SM::XIN);  // per-row terms of the gate's suffix [C]
  float* stl = reinterpret_cast<float*>(smem + SM::ST);
  float* stg = SLDS ? nullptr : w.scratch + (int64_t)blockIdx.x * MAXB * SB;

  ChunkLoads<T, D, C, NWA> cl;
  cl.init(wv, lane, a.H, a.L, LS);
  auto issue = [&](int j, int bi) __attribute__((always_inline)) {
    const int64_t row0 = bk.row + (int64_t)j * C * a.H;
    char* buf = smem + bi * SM::BUF;
    cl.tiles(a.q, row0, buf + SM::TQ, wv);
    cl.tiles(a.k, row0, buf + SM::TK, wv);
    cl.tiles(a.v, row0, buf + SM::TV, wv);
    cl.tiles(a.dO, row0, buf + SM::TD, wv);
    cl.gates(a.g, row0, reinterpret_cast<float*>(buf + SM::GOFF), wv, lane);
    cl.gates(w.dOo, row0, reinterpret_cast<float*>(buf + SM::R1OFF), wv, lane);
    cl.gates(w.din, row0, reinterpret_cast<float*>(buf + SM::R2OFF), wv, lane);
    cl.lambda(a.lam, row0, a.L, reinterpret_cast<float*>(buf + SM::LOFF), wv, lane);
  };
  issue(n.P - 1, 0);

  // block-level buckets after J: the sibling after J's group of 2^b blocks
  // (bit b of J clear), with the decay from the end of block J to its start
  auto gap_blocks = [&](int x) {
    float d = 0.f;
    for (int y = bk.J + 1; y < x; ++y) d += n.GS[(int64_t)bk.bh * n.nb + y];
    return d;
  };
  auto bucket_at = [&](int b) { return (((int64_t)bk.bh * n.nb + (((bk.J >> b) + 1) << b)) * nbl + b) * SB; };
  // one orientation of a bucket state from memory: rows n of R for group A, rows d for group B
  auto bucket_frags = [&](Frag(&nf)[KSD], const __amdgpu_buffer_rsrc_t& rs, int x) __attribute__((always_inline)) {
    if (!gb) {
      col_frags<T, D>(nf, x, [&](int tr, int tc) { return load_state_tile<D>(rs, tr, tc, lane); });
    } else {
      row_frags<T, D>(nf, x, lane, [&](int tr, int tc, int ln, int sl) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, (state_tile_offset<D>(tr, tc, ln) + sl) * 4, 0, 0));
      });
    }
  };
  Frag hb[NH][DT][KSD];
  float hgap[NH];
  int nheld = 0, bfar = nbl;
#pragma unroll
  for (int x = 0; x < NH; ++x) hgap[x] = 0.f;
  for (int b = 0; b < nbl; ++b) {
    if ((bk.J >> b) & 1) continue;
    const int first = ((bk.J >> b) + 1) << b;
    if (first >= n.nb) continue;
    if (nheld >= MAXH) {
      bfar = b;
      break;
    }
#pragma unroll
    for (int x = 0; x < MAXH; ++x)
      if (x == nheld) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w.W + bucket_at(b), SB * 4);
#pragma unroll
        for (int y = 0; y < DT; ++y) bucket_frags(hb[x][y], rs, y);
        hgap[x] = gap_blocks(first);
      }
    ++nheld;
  }

  float sufX[MAXB + 1];  // gate sum of the walked chunks from each level's bucket start to the block end
#pragma unroll
  for (int m = 0; m <= MAXB; ++m) sufX[m] = 0.f;
  float suf = 0.f;     // gate sum of the chunks after the current one, to the block end
  float bcarry = 0.f;  // sum of the gate's per-row terms of the walked chunks (wave 0)

  Vec4 od[DT];  // dv (group A) or dk (group B) of row s
  float odg = 0.f;
  auto store_out = [&](int jj) __attribute__((always_inline)) {
    const int64_t row0 = bk.row + (int64_t)jj * C * a.H;
    const int64_t orow = row0 + (int64_t)s * a.H;
    T* dst = static_cast<T*>(gb ? a.dk : a.dv);
#pragma unroll
    for (int x = 0; x < DT; ++x) *reinterpret_cast<Vec4*>(dst + orow * D + 16 * x + 4 * g4) = od[x];
    if (wv == 0 && lane < C) a.dlog_gate[row0 + (int64_t)lane * a.H] = odg;
  };

  for (int t = 0; t < n.P; ++t) {
    const int j = n.P - 1 - t;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk j and stores of chunk j+2 are done
    lds_barrier();
    if (t > 0) store_out(j + 1);
    if (j > 0) issue(j - 1, (t + 1) & 1);
    const char* buf = smem + (t & 1) * SM::BUF;
    const char* sq = buf + SM::TQ;
    const char* sk = buf + SM::TK;
    const char* sv = buf + SM::TV;
    const char* sdo = buf + SM::TD;
    const float* ll = reinterpret_cast<const float*>(buf + SM::LOFF);
    const float gsum = stage_prefix<C>(reinterpret_cast<const float*>(buf + SM::GOFF), gp, wv, lane);
    lds_barrier();
    // weight rows lambda_t^{LOGC+m} e^{G_t} of the chunk-level buckets this chunk joins
    for (int x = tid; x < MAXB * C; x += 64 * NWA) {
      const int m = x / C + 1, tk = x % C;
      if (m <= logP && ((j >> (m - 1)) & 1)) wt[x] = ll[tk * LS + LOGC + m] * __expf(gp[tk]);
    }
    const float Gs = gp[s];
    // B operand for the buckets and the in-chunk scores: row s of k (group A) or v (group B)
    const char* sr = gb ? sv : sk;
    Frag bf[KSD];
#pragma unroll
    for (int k = 0; k < KSD; ++k) bf[k] = frag_row<T, C, D>(sr, s, k, g4);

    // --- buckets after this chunk.  Lanes: rows (n of dv / d of dk) 16 x + 4 (lane/16) + e, column s
    f32x4 o[DT];
#pragma unroll
    for (int x = 0; x < DT; ++x) o[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto bucket = [&](auto get, float scale) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < DT; ++x) {
        Frag nf[KSD];
        get(x, nf);
        f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KSD; ++k) z = M::mma(nf[k], bf[k], z);
        o[x] += scale * z;
      }
    };
    const float dec_end = gsum - Gs;  // G_{chunk end} - G_s
    // chunk-level buckets: the sibling after this chunk's group at level m (bit m-1 of j clear)
#pragma unroll
    for (int m = 1; m <= MAXB; ++m)
      if (m <= logP && !((j >> (m - 1)) & 1)) {
        const float sc = __expf(dec_end + suf - sufX[m]);
        if constexpr (SLDS) {
          const float* X = stl + (m - 1) * PS::FLOATS;
          if (!gb)
            bucket(
                [&](int x, Frag(&nf)[KSD]) {
                  col_frags<T, D>(nf, x, [&](int tr, int tc) {
                    return *reinterpret_cast<const f32x4*>(X + PS::off(tr, tc, lane));
                  });
                },
                sc);
          else
            bucket(
                [&](int x, Frag(&nf)[KSD]) {
                  row_frags<T, D>(nf, x, lane, [&](int tr, int tc, int ln, int sl) { return X[PS::off(tr, tc, ln) + sl]; });
                },
                sc);
        } else {
          const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(stg + (m - 1) * SB, SB * 4);
          bucket([&](int x, Frag(&nf)[KSD]) { bucket_frags(nf, rs, x); }, sc);
        }
      }
    // block-level buckets: those held in registers, then any others from memory
    {
      const float base = dec_end + suf;  // to the end of block J
#pragma unroll
      for (int x = 0; x < MAXH; ++x)
        if (x < nheld)
          bucket(
              [&](int y, Frag(&nf)[KSD]) {
#pragma unroll
                for (int k = 0; k < KSD; ++k) nf[k] = hb[x][y][k];
              },
              __expf(base + hgap[x]));
      for (int b = bfar; b < nbl; ++b) {
        if ((bk.J >> b) & 1) continue;
        const int first = ((bk.J >> b) + 1) << b;
        if (first >= n.nb) continue;
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w.W + bucket_at(b), SB * 4);
        bucket([&](int y, Frag(&nf)[KSD]) { bucket_frags(nf, rs, y); }, __expf(base + gap_blocks(first)));
      }
    }

    if (!gb) {
      // v_s . dv_s^x, the cross-chunk part, and the gate's per-row term dOo_s - v_s . dv_s^x
      float dot = 0.f;
#pragma unroll
      for (int x = 0; x < DT; ++x) {
        const T* vr = reinterpret_cast<const T*>(sv + TL::off(s, 16 * x + 4 * g4));
#pragma unroll
        for (int e = 0; e < 4; ++e) dot += o[x][e] * to_f32(vr[e]);
      }
      dot = sum_groups(dot);
      if (g4 == 0) ub[s] = reinterpret_cast<const float*>(buf + SM::R1OFF)[s] - dot;
    }

    // --- in chunk: P tiles (P1 = M (q_t . k_s) for dv, P2 = M (dO_t . v_s) for dk) with
    // lanes holding rows t = 16 tt + 4 (lane/16) + e of column s
    {
      const char* sa = gb ? sdo : sq;  // rows t of the score's other side
      f32x4 p[CT];
#pragma unroll
      for (int tt = 0; tt < CT; ++tt) {
        p[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tt < rt) continue;
        f32x4 xs = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KSD; ++k) xs = M::mma(frag_row<T, C, D>(sa, 16 * tt + q16, k, g4), bf[k], xs);
        const f32x4 gt = *reinterpret_cast<const f32x4*>(gp + 16 * tt + 4 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = 16 * tt + 4 * g4 + e;
          const int lev = (tk == s) ? 0 : 32 - __clz(tk ^ s);
          p[tt][e] = (tk >= s) ? xs[e] * ll[tk * LS + lev] * __expf(gt[e] - Gs) : 0.f;
        }
      }
      Frag pf[KSC];
#pragma unroll
      for (int k = 0; k < KSC; ++k) pf[k] = M::acc_frag(p, k);
      // a k step whose accumulator tiles all lie before this wave's rows holds zeros
      constexpr int TPK = (sizeof(T) == 2) ? 2 : 1;  // accumulator tiles a k step spans
      const char* so = gb ? sq : sdo;                // the values the P tiles weight
#pragma unroll
      for (int x = 0; x < DT; ++x) {
        Frag df[KSC];
#pragma unroll
        for (int k = 0; k < KSC; ++k) df[k] = frag_col<T, C, D>(so, 16 * x, k, lane);
        lds_wait(df);
#pragma unroll
        for (int k = 0; k < KSC; ++k)
          if (M::first_tile(k) + TPK - 1 >= rt) o[x] = M::mma(df[k], pf[k], o[x]);
      }
    }
#pragma unroll
    for (int x = 0; x < DT; ++x)
#pragma unroll
      for (int e = 0; e < 4; ++e) od[x][e] = (T)o[x][e];

    lds_barrier();  // every wave has read the buckets; the gate's per-row terms are in
    // the gate: din_s + the suffix of the per-row terms within the block
    if (wv == 0) {
      const float u = lane < C ? ub[lane] : 0.f;
      const float pre = chunk_scan<C>(u);
      const float tot = __shfl(pre, C - 1, 64);
      if (lane < C) odg = reinterpret_cast<const float*>(buf + SM::R2OFF)[lane] + bcarry + tot - pre + u;
      bcarry += tot;
    }

    // --- this chunk joins the chunk-level buckets it lies in (bit m-1 of j set):
    // R_m = e^{g_j} R_m + sum_t lambda_t^{LOGC+m} e^{G_t} q_t dO_t^T, a fresh
    // bucket when j is its last chunk; the tiles are dealt over all waves
    const float carry = __expf(gsum);
#pragma unroll
    for (int m = 1; m <= MAXB; ++m) {
      if (m > logP || !((j >> (m - 1)) & 1)) continue;
      const float* wm = wt + (m - 1) * C;
      const bool fresh = ((j + 1) & ((1 << (m - 1)) - 1)) == 0;
      for (int ti = wv; ti < DT * DT; ti += NWA) {
        const int dt = ti / DT, nt = ti % DT;
        Frag kf[KSC], vf[KSC];
#pragma unroll
        for (int k = 0; k < KSC; ++k) {
          kf[k] = frag_col<T, C, D>(sq, 16 * dt, k, lane);
          vf[k] = frag_col<T, C, D>(sdo, 16 * nt, k, lane);
        }
        lds_wait(kf, vf);
        float* dst = SLDS ? stl + (m - 1) * PS::FLOATS + PS::off(dt, nt, lane)
                          : stg + (m - 1) * SB + state_tile_offset<D>(dt, nt, lane);
        f32x4 acc = fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : carry * *reinterpret_cast<const f32x4*>(dst);
#pragma unroll
        for (int k = 0; k < KSC; ++k) acc = M::mma(scale_tokens<T>(kf[k], wm, k, g4), vf[k], acc);
        *reinterpret_cast<f32x4*>(dst) = acc;
      }
    }
    suf += gsum;
#pragma unroll
    for (int m = 1; m <= MAXB; ++m)
      if (m <= logP && ((j >> (m - 1)) & 1)) sufX[m] = suf;
  }
  store_out(0);
  if (wv == 0 && lane == 0) w.BT[(int64_t)bk.bh * n.nb + bk.J] = bcarry;
}

// ---------------------------------------------------------------------------
// ll_bwd_gate_add: the gate's share from later blocks; every row of block J
// gets the sum of BT over the blocks after J of its head.
__global__ void __launch_bounds__(256) ll_bwd_gate_add(BwdArgs a, int nb, int block_tokens, const float* BT) {
  const int64_t rows = (int64_t)a.B * a.T * a.H;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += (int64_t)gridDim.x * blockDim.x) {
    const int h = (int)(i % a.H);
    const int64_t bt = i / a.H;
    const int t = (int)(bt % a.T), b = (int)(bt / a.T);
    const float* bh = BT + ((int64_t)b * a.H + h) * nb;
    float later = 0.f;
    for (int J = t / block_tokens + 1; J < nb; ++J) later += bh[J];
    a.dlog_gate[i] += later;
  }
}

// ---------------------------------------------------------------------------
// Raises a kernel's dynamic LDS allowance once (above 64 KiB it must be set).
template <typename K>
static hipError_t allow_lds(std::once_flag& once, hipError_t& result, K kern, int bytes) {
  std::call_once(once, [&] {
    result = bytes > 65536 ? hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, bytes)
                           : hipSuccess;
  });
  return result;
}

template <typename T, int D, int C>
static hipError_t launch_native_t(const BwdArgs& a, const BwdFwdNodes& n, const BwdWork& w, int pass, hipStream_t s) {
  constexpr int MAXB = max_block_depth(D);
  constexpr bool SLDS = bwd_states_in_lds(D);  // chunk-level states in LDS (3 x 17 KiB at d = 64)
  constexpr int FV = state_frag_vgprs<T, D>();
  // held in registers for a whole walk (fewer for fp32 at C = 64: eight waves
  // leave 256 registers per wave, and fp32 fragments of a state take more)
  constexpr int HCAP = (sizeof(T) == 4 && C == 64) ? 1 : 2;
  constexpr int HF = 32 / FV > HCAP ? HCAP : 32 / FV;  // forward walk: nodes
  constexpr int HR = 64 / FV > HCAP ? HCAP : 64 / FV;  // reverse walk: buckets
  constexpr int NW = C / 16, DT = D / 16, NTW = (DT + NW - 1) / NW;
  // block levels whose shares the forward walk makes
  constexpr int NLBF = 8 / (NTW * DT) > HCAP ? HCAP : 8 / (NTW * DT);
  constexpr int NLB = D >= 128 ? 4 : 8;  // block levels per rev_state workgroup: NLB x D/16 accumulator tiles
  const int grid = a.B * a.H * n.nb;
  if (pass == 0) {
    auto kern = ll_bwd_fwalk<T, D, C, MAXB, HF, NLBF, SLDS>;
    constexpr int bytes = WalkSmem<T, D, C, MAXB, SLDS, true>::BYTES;
    static std::once_flag once;
    static hipError_t res = hipSuccess;
    hipError_t e = allow_lds(once, res, kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(128 * NW), bytes, s, a, n, w);
  } else if (pass == 1) {
    if (w.nbl == 0) return hipSuccess;  // one block per head: no block-level buckets
    if (w.nbl > NLBF) {
      hipLaunchKernelGGL((ll_bwd_rev_state<T, D, C, NLB>), dim3(grid, (w.nbl - NLBF + NLB - 1) / NLB),
                         dim3(64 * (D / 16)), 0, s, a, n, w, NLBF);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int64_t total = (int64_t)a.B * a.H * w.nbl * n.nb * (D * D / 4);
    const int sgrid = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    hipLaunchKernelGGL(ll_bwd_rev_scan, dim3(sgrid), dim3(256), 0, s, n, a.B * a.H, D, w);
  } else if (pass == 2) {
    auto kern = ll_bwd_rwalk<T, D, C, MAXB, HR, SLDS>;
    constexpr int bytes = WalkSmem<T, D, C, MAXB, SLDS, false>::BYTES;
    static std::once_flag once;
    static hipError_t res = hipSuccess;
    hipError_t e = allow_lds(once, res, kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(128 * NW), bytes, s, a, n, w);
  } else {
    if (n.nb == 1) return hipSuccess;  // no later blocks
    const int64_t rows = (int64_t)a.B * a.T * a.H;
    const int ggrid = (int)((rows + 255) / 256 < 16384 ? (rows + 255) / 256 : 16384);
    hipLaunchKernelGGL(ll_bwd_gate_add, dim3(ggrid), dim3(256), 0, s, a, n.nb, n.P * C, w.BT);
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
    case 32016: return launch_native_t<float, 32, 16>(a, n, w, pass, s);
    case 32032: return launch_native_t<float, 32, 32>(a, n, w, pass, s);
    case 64016: return launch_native_t<float, 64, 16>(a, n, w, pass, s);
    case 64032: return launch_native_t<float, 64, 32>(a, n, w, pass, s);
    case 128016: return launch_native_t<float, 128, 16>(a, n, w, pass, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace llattn
