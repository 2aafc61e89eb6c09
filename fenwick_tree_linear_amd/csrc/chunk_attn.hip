// chunk_attn.hip -- chunk-parallel prefill kernels ("Log-Linear Attention",
// section 2.3: the hierarchical mask M_H evaluated as matrix products).
//
// The sequence of each head is cut into chunks of C tokens and the chunks into
// aligned blocks of P chunks.  For a token t in chunk i of block J, its
// Fenwick buckets split into three groups by the highest bit where the source
// position differs from t:
//   levels 0..log2 C                 : sources inside chunk i      (intra)
//   levels log2 C + 1 .. + log2 P    : earlier chunks of block J   (within-block)
//   higher levels                    : earlier blocks              (block Fenwick nodes)
//
// ll_chunk_state  : per block, the decayed key-value state
//                   sum_s prod_{r=s+1}^{end} a_r k_s v_s^T over its P*C tokens.
// ll_chunk_attn   : per block, walks its chunks in order and produces o:
//                   intra-chunk (Q K^T * level weights * decay) V on MFMA,
//                   within-block levels from a chunk-granular Fenwick state kept
//                   in registers, and the block-level nodes built by
//                   ll_fenwick_scan, each read as diag(alpha) Q N on MFMA.
//
// Chunks stream through LDS with direct global->LDS loads issued one chunk
// ahead.  Tiles keep the global row-major layout; the operands that contract
// over tokens (V, and K for the state) are read with the transposing LDS
// read, and the per-token decay of the state update is applied to the V
// fragments in registers, so no transposed or rescaled tile is ever written.
#include <mutex>
#include <type_traits>

#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// In-chunk inclusive prefix G of the log-gates (every wave computes it; lane
// r holds G[r]).
template <int C>
__device__ __forceinline__ float chunk_prefix(const float* gates, int lane) {
  return chunk_scan<C>(lane < C ? gates[lane] : 0.f);
}

// j mod 3 for 0 <= j < 16 from a table of 2-bit entries (no division).
__device__ __forceinline__ int mod3_small(int j) {
  constexpr unsigned kTable = 0x24924924u;  // entry j = bits [2j, 2j+1]: 0,1,2,0,1,2,...
  return (int)((kTable >> (2 * j)) & 3u);
}

// ---------------------------------------------------------------------------
// ll_chunk_state: one workgroup per (block J, head), one wave per 16 state
// columns.  Writes S[bh, J] (tile layout) and GS[bh, J].
template <typename T, int D, int C>
struct StateSmem {
  typedef Tile<T, C, D> TL;
  static constexpr int KOFF = 0, VOFF = TL::BYTES, GOFF = 2 * TL::BYTES;
  static constexpr int STAGE = GOFF + C * 4;
  static constexpr int WOFF = 2 * STAGE;  // per-wave decay-to-end weights [NW][C]
  static constexpr int BYTES = WOFF + (D / 16) * C * 4;
};

template <typename T, int D, int C>
__global__ void __launch_bounds__(64 * (D / 16)) ll_chunk_state(PrefillArgs a) {
  using M = Mma<T>;
  typedef StateSmem<T, D, C> L;
  constexpr int NW = D / 16;
  constexpr int DT = D / 16;
  constexpr int KSC = C / M::KS;
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), g4 = lane >> 4;
  float* wl = reinterpret_cast<float*>(smem + L::WOFF) + wv * C;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int J = wg % a.nb, bh = wg / a.nb, h = bh % a.H, b = bh / a.H;
  const int64_t row_blk = ((int64_t)b * a.T + (int64_t)J * a.P * C) * a.H + h;  // first row of the block
  auto row_of = [&](int j) { return row_blk + (int64_t)(j * C * a.H); };
  ChunkLoads<T, D, C, NW> ld;
  ld.init(wv, lane, a.H, a.L, a.LS);
  auto issue = [&](int j) {
    char* st = smem + (j & 1) * L::STAGE;
    ld.tiles(a.k, row_of(j), st + L::KOFF, wv);
    ld.tiles(a.v, row_of(j), st + L::VOFF, wv);
    ld.gates(a.g, row_of(j), reinterpret_cast<float*>(st + L::GOFF), wv, lane);
  };

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float gblk = 0.f;

  issue(0);
  for (int j = 0; j < a.P; ++j) {
    const char* st = smem + (j & 1) * L::STAGE;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk j have landed
    __syncthreads();                // every wave's have; chunk j-1 is done everywhere
    if (j + 1 < a.P) issue(j + 1);
    const float gscan = chunk_prefix<C>(reinterpret_cast<const float*>(st + L::GOFF), lane);
    const float gsum = __shfl(gscan, C - 1, 64);
    if (lane < C) wl[lane] = __expf(gsum - gscan);

    // H_j[:, cols] = sum_r k_r (w_r v_r)^T, w_r = exp(G[C-1] - G[r])
    typename M::Frag vf[KSC], kf[DT][KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(st + L::VOFF, 16 * wv, s, lane);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int s = 0; s < KSC; ++s) kf[dt][s] = frag_col<T, C, D>(st + L::KOFF, 16 * dt, s, lane);
    lds_wait(vf, kf);
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = scale_tokens<T>(vf[s], wl, s, g4);
    const float carry = __expf(gsum);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 x = acc[dt] * carry;
#pragma unroll
      for (int s = 0; s < KSC; ++s) x = M::mma(kf[dt][s], vf[s], x);
      acc[dt] = x;
    }
    gblk += gsum;
  }

  float* dst = a.S + ((int64_t)bh * a.nb + J) * D * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + state_tile_offset<D>(dt, wv, lane)) = acc[dt];
  if (tid == 0) a.GS[(int64_t)bh * a.nb + J] = gblk;
}

// MFMA A fragments (row = state column n of this wave's 16, k = head dim d)
// of a dk x dv state stored in tile layout.
template <typename T, int D>
__device__ __forceinline__ void node_frags(typename Mma<T>::Frag (&nf)[D / Mma<T>::KS], const float* node, int wc,
                                           int lane) {
  using M = Mma<T>;
  constexpr int DT = D / 16, KSD = D / M::KS;
  f32x4 t[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) t[dt] = *reinterpret_cast<const f32x4*>(node + state_tile_offset<D>(dt, wc, lane));
#pragma unroll
  for (int s = 0; s < KSD; ++s) nf[s] = M::acc_frag(t, s);
}

// Wave arrangement of ll_chunk_attn: D/16 column tiles x RH row groups
// (at most 8 waves, so that each keeps up to 256 registers).  With two row
// groups, group wr takes row tiles wr and CT-1-wr, so both get the same
// share of the causal triangle.
template <int D, int C>
struct AttnWaves {
  static constexpr int NCT = D / 16;                        // output column tiles
  static constexpr int CT = C / 16;                         // 16-row tiles of a chunk
  static constexpr int RH = (CT >= 2 && NCT <= 4) ? 2 : 1;  // row groups
  static constexpr int NRT = CT / RH;                       // row tiles per wave
  static constexpr int NW = NCT * RH;                       // waves per workgroup
  static_assert(RH == 1 || NRT <= 2, "row pairing covers up to four row tiles");
  __host__ __device__ static constexpr int row_tile(int i, int wr) {
    return RH == 1 ? i : ((i & 1) ? CT - 1 - wr : wr);
  }
};

// Walks consecutive work items item = (b H + h) nb + J (block J of head
// (b, h)) without dividing per step: one division when it starts, then
// carries.  `row` is the first [B,T,H] row of the item's block.
struct ItemWalk {
  int J, h, b;
  int64_t row;
  __device__ __forceinline__ void set_row(const PrefillArgs& a, int C) {
    row = ((int64_t)b * a.T + (int64_t)J * a.P * C) * a.H + h;
  }
  __device__ __forceinline__ void start(int item, const PrefillArgs& a, int C) {
    J = item % a.nb;
    const int bh = item / a.nb;
    h = bh % a.H;
    b = bh / a.H;
    set_row(a, C);
  }
  __device__ __forceinline__ void next(const PrefillArgs& a, int C) {
    if (++J < a.nb) {
      row += (int64_t)a.P * C * a.H;
      return;
    }
    J = 0;
    if (++h == a.H) {
      h = 0;
      ++b;
    }
    set_row(a, C);
  }
  __device__ __forceinline__ int bh(const PrefillArgs& a) const { return b * a.H + h; }
};

// Dynamic LDS layout of ll_chunk_attn (byte offsets; LS = staged levels):
// three staging buffers of chunk tiles, two buffers of masked scores and two
// of decay-scaled keys (chunk parity), and per-wave prefix arrays.
template <typename T, int D, int C>
struct AttnLayout {
  typedef Tile<T, C, D> TL;
  typedef Tile<T, C, C> PT;
  static constexpr int NS = 3;
  int q, k, v, g, lraw, stage;  // per-stage offsets and stage size
  int p, kw, gw, total;
  __host__ __device__ explicit AttnLayout(int LS) {
    q = 0;
    k = q + TL::BYTES;
    v = k + TL::BYTES;
    g = v + TL::BYTES;
    lraw = g + C * 4;  // lambda rows [C][LS]
    stage = (lraw + C * LS * 4 + 255) & ~255;
    p = NS * stage;             // masked scores P[r][s], [2][C][C]
    kw = p + 2 * PT::BYTES;     // K with rows scaled by e^{G[C-1] - G_s}, [2][C][D]
    gw = kw + 2 * TL::BYTES;    // per wave and chunk parity: G, e^{G[C-1]-G}, e^{G[tile end]-G}
    total = gw + AttnWaves<D, C>::NW * 2 * 3 * C * 4;
  }
};

// ---------------------------------------------------------------------------
// ll_chunk_attn: one workgroup per (block J, head) with D/16 x RH waves: wave
// (wc, wr) owns output columns [16 wc, 16 wc + 16) of NRT row tiles.  The P
// chunks of the block are visited in order as a pipeline: while chunk j is
// read out, the workgroup prepares chunk j+1 (its masked in-chunk scores and
// its decay-scaled keys, each tile made once) and chunk j+2 is in flight
// from HBM.  One barrier per chunk hands all of it over.
//
// Every product is formed transposed, O^T[n][r]: a lane then holds one token
// row r and four output columns, so the per-row weights lambda_r^l e^{G_r}
// are per-lane scalars and the output leaves as 4-element vector stores.  The
// Fenwick nodes of earlier blocks are the same for every chunk of the block:
// up to MAXH of them stay in registers as MFMA fragments for the whole block,
// any further ones are read from the workspace per chunk.
template <typename T, int D, int C, int MAXB, int MAXH>
__global__ void __launch_bounds__((64 * AttnWaves<D, C>::NW)) ll_chunk_attn(PrefillArgs a) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef AttnLayout<T, D, C> Lay;
  typedef AttnWaves<D, C> W;
  typedef Tile<T, C, D> TL;
  typedef Tile<T, C, C> PT;
  typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type Vec4;  // 4 values of T
  constexpr int NW = W::NW, NCT = W::NCT, NRT = W::NRT, CT = W::CT;
  constexpr int DT = D / 16;
  constexpr int KSD = D / M::KS, KSC = C / M::KS;
  constexpr int LOGC = (C == 16) ? 4 : (C == 32) ? 5 : 6;
  constexpr int NS = Lay::NS;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int LS = a.LS;
  const Lay lay(LS);
  // the wave index is made a scalar so that every branch on it is a uniform
  // jump: an MFMA must never sit under a partial or empty EXEC mask
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, q16 = lane & 15;
  const int wc = wv % NCT, wr = wv / NCT;
  // This workgroup's work items: consecutive (block J, head) pairs, item
  // i = head * nb + J, walked as one stream of steps t = (item k) * P + chunk j.
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int nitems = a.B * a.H * a.nb;
  const int item0 = (int)((int64_t)wg * nitems / gridDim.x);
  const int nsteps = ((int)((int64_t)(wg + 1) * nitems / gridDim.x) - item0) * a.P;
  const int logP = ilog2c(a.P);
  const int row_step = C * a.H;  // rows per chunk
  // Steps are loaded, read out and stored in order, each by its own cursor
  // over the items; a cursor moves on at the first chunk of every item after
  // its first.
  ItemWalk load_at, store_at, read_at;
  load_at.start(item0, a, C);
  store_at = load_at;
  read_at = load_at;
  auto row_in = [&](const ItemWalk& w, int t) { return w.row + (int64_t)((t & (a.P - 1)) * row_step); };
  static_assert(NS == 3, "the staging ring is three buffers");
  auto stage_of = [&](int t) { return smem + (t % NS) * lay.stage; };
  // this wave's prefix arrays for step parity: G, e^{G[C-1]-G}, e^{G[end of 16-token tile]-G}
  auto garr = [&](int t) { return reinterpret_cast<float*>(smem + lay.gw) + (wv * 2 + (t & 1)) * 3 * C; };
  ChunkLoads<T, D, C, NW> ld;
  ld.init(wv, lane, a.H, a.L, LS);
  // The loads of a step go out in three parts (q and gates, k and lambda, v),
  // so that inside the chunk loop they can be spread between pieces of compute
  // instead of queueing up at the memory pipeline all at once.
  auto issue_part = [&](int j, int part) __attribute__((always_inline)) {
    char* st = stage_of(j);
    if (part == 0 && j > 0 && (j & (a.P - 1)) == 0) load_at.next(a, C);
    const int64_t row0 = row_in(load_at, j);
    if (part == 0) {
      ld.tiles(a.q, row0, st + lay.q, wv);
      ld.gates(a.g, row0, reinterpret_cast<float*>(st + lay.g), wv, lane);
    } else if (part == 1) {
      ld.tiles(a.k, row0, st + lay.k, wv);
      ld.lambda(a.lam, row0, a.L, reinterpret_cast<float*>(st + lay.lraw), wv, lane);
    } else {
      ld.tiles(a.v, row0, st + lay.v, wv);
    }
  };
  auto issue = [&](int j) __attribute__((always_inline)) {
    issue_part(j, 0);
    issue_part(j, 1);
    issue_part(j, 2);
  };

  // Prepares chunk j for its read-out: the in-chunk prefix G of the log-gates
  // (every wave keeps its own copy), the masked scores
  // P[r][s] = (q_r . k_s) lambda_r^(lev(r,s)) e^{G_r - G_s} for s <= r (each
  // 16x16 tile made by one wave) and the keys scaled by e^{G[C-1] - G_s}.
  // Below the diagonal the decay splits at the end e of the source tile,
  // e^{G_r - G_e} e^{G_e - G_s}: both factors are at most one.
  auto prepare = [&](int j) __attribute__((always_inline)) {
    const char* st = stage_of(j);
    const float* lraw = reinterpret_cast<const float*>(st + lay.lraw);
    float* gl = garr(j);
    float* wl = gl + C;
    float* es = wl + C;
    const float gscan = chunk_prefix<C>(reinterpret_cast<const float*>(st + lay.g), lane);
    const float gsum = __shfl(gscan, C - 1, 64);
    const float gend = __shfl(gscan, lane | 15, 64);
    if (lane < C) {
      gl[lane] = gscan;
      wl[lane] = __expf(gsum - gscan);
      es[lane] = __expf(gend - gscan);
    }
    // The causal 16x16 score tiles, the CT diagonal ones first and then the
    // ones below the diagonal, are dealt to the waves in turn: the costlier
    // tiles land on the first row group, which prepares at the start of a step.
    // Below the diagonal every pair (r, s) of a tile has the same level and the
    // decay splits at the end e of the source tile, e^{G_r - G_e} e^{G_e - G_s}:
    // one weight per lane and one per source column.
    char* pt = smem + lay.p + (j & 1) * PT::BYTES;
    constexpr int NT = CT * (CT + 1) / 2, NSLOT = (NT + NW - 1) / NW;
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) {
      const int item = k * NW + wv;
      if (item >= NT) continue;
      const bool diag = item < CT;
      int rt = item, ct = item;
      if (!diag) {  // below-diagonal tile o = rt (rt-1)/2 + ct, ct < rt
        const int o = item - CT;
        rt = 1;
#pragma unroll
        for (int u = 2; u < CT; ++u) rt += (o >= u * (u - 1) / 2) ? 1 : 0;
        ct = o - rt * (rt - 1) / 2;
      }
      const int r = 16 * rt + q16;  // lane: row r, sources 16 ct + 4 (lane/16) .. + 3
      const float* lr = lraw + r * LS;
      Frag kf[KSD], qf[KSD];
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
        kf[s] = frag_row<T, C, D>(st + lay.k, 16 * ct + q16, s, g4);
        qf[s] = frag_row<T, C, D>(st + lay.q, r, s, g4);
      }
      const float gr = gl[r];
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      Vec4 out;
      if (diag) {
        const f32x4 gs = *reinterpret_cast<const f32x4*>(gl + 16 * ct + 4 * g4);
        float lam[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) lam[e] = lr[32 - __clz(r ^ (16 * ct + 4 * g4 + e))];  // level of (r, s)
#pragma unroll
        for (int s = 0; s < KSD; ++s) x = M::mma(kf[s], qf[s], x);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          out[e] = (T)((4 * g4 + e <= q16) ? x[e] * lam[e] * __expf(gr - gs[e]) : 0.f);
      } else {
        const f32x4 ess = *reinterpret_cast<const f32x4*>(es + 16 * ct + 4 * g4);
        const float wrow = lr[4 + 32 - __clz(rt ^ ct)] * __expf(gr - gl[16 * ct + 15]);
#pragma unroll
        for (int s = 0; s < KSD; ++s) x = M::mma(kf[s], qf[s], x);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (T)(x[e] * wrow * ess[e]);
      }
      *reinterpret_cast<Vec4*>(pt + PT::off(r, 16 * ct + 4 * g4)) = out;
    }
    // decay-scaled keys: the same swizzled positions, each 16-byte piece of a
    // row scaled by that row's weight
    char* kw = smem + lay.kw + (j & 1) * TL::BYTES;
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte piece
    // (by the first row group alone: the other one prepares at the end of a
    // step, where it is the last to reach the next barrier)
    if (W::RH == 2 && wr != 0) return;
    for (int x = tid; x < TL::BYTES / 16; x += 64 * NCT) {
      const int row = x / TL::NCH;
      const float w = wl[row];
      const Vec4* src = reinterpret_cast<const Vec4*>(st + lay.k + x * 16);
      Vec4* dst = reinterpret_cast<Vec4*>(kw + x * 16);
#pragma unroll
      for (int u = 0; u < EPC / 4; ++u) {
        const Vec4 kv = src[u];
        Vec4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (T)((float)kv[e] * w);
        dst[u] = o;
      }
    }
  };

  // masked-score tiles above the diagonal are never written: keep them zero
  for (int x = tid * 16; x < 2 * PT::BYTES; x += 64 * NW * 16)
    *reinterpret_cast<uint4*>(smem + lay.p + x) = uint4{0, 0, 0, 0};
  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  if (nsteps > 1) issue(1);
  lds_barrier();  // step 0 has landed for every wave; the zeroed tiles are visible
  prepare(0);

  // The chunk loop, compiled once per row group so that every row-tile
  // index in it is a constant and the work of a chunk is straight-line code.
  auto run = [&](auto row_group) __attribute__((always_inline)) {
    constexpr int WR = decltype(row_group)::value;
    // (all per-wave state is declared in here, so that it stays in registers)
    // Per item: the first MAXH Fenwick nodes of earlier blocks (most recent
    // first) as A fragments of this wave's columns, with their level and decay
    // offset; the within-block Fenwick states and their log-scales.
    Frag hn[MAXH > 0 ? MAXH : 1][KSD];
    int hlv[MAXH > 0 ? MAXH : 1];
    float hdd[MAXH > 0 ? MAXH : 1];
    int rest_far = 0;  // set bits of J whose nodes are not held in registers
    float dd_far = 0.f;
    int bh = 0;
    bool first_item = true;
    f32x4 nst[MAXB][DT];
    float sig[MAXB + 1];
    float gw = 0.f;  // log-decay from the start of block J to the current chunk
    auto node_of = [&](int e) {
      const float* f = a.F + ((int64_t)bh * a.nF + (e >> 1)) * D * D;
      const float* s = a.S + ((int64_t)bh * a.nb + e) * D * D;
      return (e & 1) ? f : s;
    };
    // MFMA fragments of node e for this wave's columns: from the bf16 copies
    // in fragment order where they exist (one 16-byte load per fragment),
    // else from the fp32 nodes
    auto load_node = [&](Frag(&nf)[KSD], int e) __attribute__((always_inline)) {
      if constexpr (node_copies(sizeof(T) == 2 ? 1 : 0, D)) {
        const bf16x8* src = static_cast<const bf16x8*>(a.N16) + ((int64_t)bh * a.nb + e) * (D * D / 8) + wc * KSD * 64 + lane;
#pragma unroll
        for (int s = 0; s < KSD; ++s) nf[s] = src[s * 64];
      } else {
        node_frags<T, D>(nf, node_of(e), wc, lane);
      }
    };
    auto gamma_of = [&](int e) {
      const float* f = a.GF + (int64_t)bh * a.nF + (e >> 1);
      const float* s = a.GS + (int64_t)bh * a.nb + e;
      return *((e & 1) ? f : s);
    };
    auto start_item = [&]() __attribute__((always_inline)) {
      if (!first_item) read_at.next(a, C);
      first_item = false;
      bh = read_at.bh(a);
      // The held nodes: one per set bit of J, most recent first.  A slot past
      // the last set bit repeats the first node and weighs nothing, so that
      // every node and decay load goes out at once instead of each waiting
      // for the one before.
      const int J = read_at.J;
      int ex[MAXH > 0 ? MAXH : 1];
      rest_far = J;
#pragma unroll
      for (int x = 0; x < MAXH; ++x) {
        hlv[x] = rest_far > 0 ? LOGC + 1 + logP + __ffs(rest_far) - 1 : -1;  // token level of the node
        ex[x] = rest_far > 0 ? rest_far - 1 : J - 1;
        rest_far &= rest_far - 1;
      }
      dd_far = 0.f;
#pragma unroll
      for (int x = 0; x < MAXH; ++x) hdd[x] = 0.f;
      if (MAXH > 0 && J > 0) {
        float gm[MAXH > 0 ? MAXH : 1];
#pragma unroll
        for (int x = 0; x < MAXH; ++x) {
          load_node(hn[x], ex[x]);
          gm[x] = gamma_of(ex[x]);
        }
#pragma unroll
        for (int x = 0; x < MAXH; ++x) {
          hdd[x] = dd_far;
          dd_far += hlv[x] >= 0 ? gm[x] : 0.f;
        }
      }
#pragma unroll
      for (int m = 0; m < MAXB; ++m)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) nst[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m <= MAXB; ++m) sig[m] = 0.f;
      gw = 0.f;
    };

    // Output rows of a step leave during the following step, so the wait at
    // the top of each step finds the stores most of a step old.
    Vec4 ov[NRT];
    auto store_out = [&](int jj) __attribute__((always_inline)) {
      if (jj > 0 && (jj & (a.P - 1)) == 0) store_at.next(a, C);
      const int64_t row0 = row_in(store_at, jj);
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        const int r = 16 * W::row_tile(i, WR) + q16;  // lane: row r, columns 16 wc + 4 (lane/16) .. + 3
        T* o = static_cast<T*>(a.o) + (row0 + (int64_t)r * a.H) * D + 16 * wc + 4 * g4;
        *reinterpret_cast<Vec4*>(o) = ov[i];
      }
    };

    // Every step starts with one barrier.  The two row groups share each SIMD
    // (one wave of each), so they take the step's halves in opposite orders:
    // one prepares step t+1 and then reads out step t, the other the reverse,
    // and the waves of a SIMD are in different phases most of the time.  The
    // read-out issues the rest of step t+2's loads after its first products.
    for (int t = 0; t < nsteps; ++t) {
      const int j = t & (a.P - 1);    // chunk within the item's block
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of step t+1 and stores of step t-2 are done
      lds_barrier();                  // step t prepared and step t+1 landed everywhere; step t-1 done
      if (j == 0) start_item();       // node loads ahead of this step's other memory traffic
      if constexpr (WR == 0) {
        if (t + 1 < nsteps) prepare(t + 1);
      }
      if (t > 0) store_out(t - 1);
      if (t + 2 < nsteps) issue_part(t + 2, 0);

      const char* st = stage_of(t);
      const float* lraw = reinterpret_cast<const float*>(st + lay.lraw);
      const float* gl = garr(t);
      const float gsum = gl[C - 1];

      // per row tile: Q fragments (index r, k = head dim), the row's lambda
      // weights times e^{G_r} for every inter-chunk level this chunk reads
      Frag qf[NRT][KSD];
      const float* lr[NRT];
      float egr[NRT], alw[NRT][MAXB], alh[NRT][MAXH > 0 ? MAXH : 1];
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        const int r = 16 * W::row_tile(i, WR) + q16;
#pragma unroll
        for (int s = 0; s < KSD; ++s) qf[i][s] = frag_row<T, C, D>(st + lay.q, r, s, g4);
        lr[i] = lraw + r * LS;
        egr[i] = __expf(gl[r]);
#pragma unroll
        for (int m = 1; m <= MAXB; ++m) alw[i][m - 1] = lr[i][min(LOGC + m, LS - 1)] * egr[i];
#pragma unroll
        for (int x = 0; x < MAXH; ++x) alh[i][x] = lr[i][max(hlv[x], 0)] * egr[i];
      }

      // --- intra-chunk: O^T += V^T P^T
      Frag vf[KSC];
#pragma unroll
      for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(st + lay.v, 16 * wc, s, lane);
      const char* pt = smem + lay.p + (t & 1) * PT::BYTES;
      Frag pf[NRT][KSC];
#pragma unroll
      for (int i = 0; i < NRT; ++i)
#pragma unroll
        for (int s = 0; s < KSC; ++s) pf[i][s] = frag_row<T, C, C>(pt, 16 * W::row_tile(i, WR) + q16, s, g4);
      lds_wait(vf);
      f32x4 oacc[NRT];
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSC; ++s)
          if (M::first_tile(s) <= W::row_tile(i, WR)) oacc[i] = M::mma(vf[s], pf[i][s], oacc[i]);
      }

      if (t + 2 < nsteps) {
        issue_part(t + 2, 1);
        issue_part(t + 2, 2);
      }

      // --- inter-chunk levels: O^T += diag(alpha) N^T Q^T, alpha_r = lambda_r^l e^{G_r} x scale.
      // A level's product is weighted into O only when the next level comes
      // (or at the end), so no level waits right away for its own products.
      f32x4 pend[NRT];
      float pal[NRT];
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        pend[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        pal[i] = 0.f;
      }
      auto level_read = [&](const Frag(&nf)[KSD], const float(&al)[NRT]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NRT; ++i) {
          oacc[i] += pal[i] * pend[i];
          pal[i] = al[i];
          pend[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KSD; ++s) pend[i] = M::mma(nf[s], qf[i][s], pend[i]);
        }
      };
      // within-block levels LOGC+1 .. LOGC+logP
#pragma unroll
      for (int m = 1; m <= MAXB; ++m) {
        if (m <= logP && ((j >> (m - 1)) & 1)) {
          Frag nf[KSD];
#pragma unroll
          for (int s = 0; s < KSD; ++s) nf[s] = M::acc_frag(nst[m - 1], s);
          const float sc = __expf(sig[m]);
          float al[NRT];
#pragma unroll
          for (int i = 0; i < NRT; ++i) al[i] = alw[i][m - 1] * sc;
          level_read(nf, al);
        }
      }
      // earlier blocks: one Fenwick node per set bit of J, most recent first
#pragma unroll
      for (int x = 0; x < MAXH; ++x) {
        if (hlv[x] >= 0) {
          const float sc = __expf(gw + hdd[x]);
          float al[NRT];
#pragma unroll
          for (int i = 0; i < NRT; ++i) al[i] = alh[i][x] * sc;
          level_read(hn[x], al);
        }
      }
      {
        int rest = rest_far;
        float dd = dd_far;
        while (rest > 0) {
          const int e = rest - 1;
          Frag nf[KSD];
          load_node(nf, e);
          const int lev = LOGC + 1 + logP + __ffs(rest) - 1;
          const float sc = __expf(gw + dd);
          float al[NRT];
#pragma unroll
          for (int i = 0; i < NRT; ++i) al[i] = lr[i][lev] * egr[i] * sc;
          level_read(nf, al);
          dd += gamma_of(e);
          rest &= rest - 1;
        }
      }


      // --- the output rows, stored during the next step
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        oacc[i] += pal[i] * pend[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[i][e] = (T)oacc[i][e];
      }

      // --- this chunk's own decayed key-value state K_w^T V (keys scaled by
      // e^{G[C-1] - G_s}), then the merge rule of the within-block Fenwick
      // levels (levels 1..c and the chunk become level c+1, c = ctz(j+1))
#pragma unroll
      for (int m = 1; m <= MAXB; ++m) sig[m] += gsum;
      gw += gsum;
      if (j + 1 < a.P) {
        const char* kw = smem + lay.kw + (t & 1) * TL::BYTES;
        Frag kf[DT][KSC];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int s = 0; s < KSC; ++s) kf[dt][s] = frag_col<T, C, D>(kw, 16 * dt, s, lane);
        // the merged levels are summed first and enter as the accumulator
        const int c = __ffs(j + 1) - 1;
        f32x4 merged[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) merged[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 1; m <= MAXB; ++m) {
          if (m <= c) {
            const float sc = __expf(sig[m]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) merged[dt] += sc * nst[m - 1][dt];
          }
        }
        lds_wait(kf);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int s = 0; s < KSC; ++s) merged[dt] = M::mma(kf[dt][s], vf[s], merged[dt]);
#pragma unroll
        for (int m = 1; m <= MAXB; ++m) {
          if (m == c + 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) nst[m - 1][dt] = merged[dt];
            sig[m] = 0.f;
          }
        }
      }
      if constexpr (WR != 0) {
        if (t + 1 < nsteps) prepare(t + 1);
      }
    }
    store_out(nsteps - 1);
  };
  if constexpr (W::RH == 1) {
    run(std::integral_constant<int, 0>{});
  } else {
    if (wr == 0) {
      run(std::integral_constant<int, 0>{});
    } else {
      run(std::integral_constant<int, 1>{});
    }
  }
}

// ---------------------------------------------------------------------------
// ll_chunk_attn_split: the same read for bf16 with two row groups, with the
// work of a step divided by role instead of repeated per row group.
//   readers (D/16 column tiles x 2 row groups): load the chunks, read out the
//     intra-chunk product and every Fenwick level of their rows and columns,
//     store o.
//   makers (one per column tile): prepare the next chunk (masked scores and
//     decay-scaled keys, each tile once) and merge this chunk into the
//     within-block Fenwick states of their 16 columns, once for both row
//     groups.  A merged state goes to LDS as bf16 MFMA fragments, which the
//     readers take as they are.
// A reader keeps no within-block state and a maker no output, so each fits
// the register share of three waves per SIMD.
template <int D, int C>
struct SplitWaves {
  static constexpr int NCT = D / 16;     // output column tiles
  static constexpr int CT = C / 16;      // 16-row tiles of a chunk
  static constexpr int NRW = 2 * NCT;    // reader waves
  static constexpr int NMW = NCT;        // maker waves
  static constexpr int NW = NRW + NMW;   // waves per workgroup
  static constexpr int NRT = CT / 2;     // row tiles per reader
  static_assert(CT == 2 || CT == 4, "two row groups of one or two row tiles");
  // row group wr takes row tiles wr and CT-1-wr: the same share of the causal triangle
  __host__ __device__ static constexpr int row_tile(int i, int wr) { return (i & 1) ? CT - 1 - wr : wr; }
};

// LDS of ll_chunk_attn_split: the offsets of SplitLds at this head, chunk and
// within-block depth.
template <int D, int C, int MAXB>
struct SplitLayout : SplitLds {
  typedef Tile<bf16, C, D> TL;
  typedef Tile<bf16, C, C> PT;
  static_assert(TL::BYTES == C * D * 2 && PT::BYTES == C * C * 2, "tile sizes as SplitLds counts them");
  static constexpr int STATE_BYTES = MAXB * (D / 16) * (D / 32) * FRAG_BYTES;
  __host__ __device__ explicit SplitLayout(int LS, int mlp_levels = 0) : SplitLds(D, C, MAXB, LS, mlp_levels > 0) {}
};

template <int D, int C, int MAXB, int MAXH, bool MLP, bool PRIOR = false>
__global__ void __launch_bounds__((64 * SplitWaves<D, C>::NW)) ll_chunk_attn_split(PrefillArgs a) {
  static_assert(!(MLP && PRIOR), "the read that makes its level weights starts sequences at position 0");
  typedef bf16 T;
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef SplitLayout<D, C, MAXB> Lay;
  typedef SplitWaves<D, C> W;
  typedef Tile<T, C, D> TL;
  typedef Tile<T, C, C> PT;
  constexpr int NRW = W::NRW, NMW = W::NMW, NW = W::NW, NCT = W::NCT, NRT = W::NRT, CT = W::CT;
  constexpr int DT = D / 16;
  constexpr int KSD = D / M::KS, KSC = C / M::KS;
  constexpr int LOGC = (C == 32) ? 5 : 6;
  constexpr int NS = Lay::NS;
  static_assert(NS == 3, "the staging ring is three buffers");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int LS = a.LS;
  const Lay lay(LS, MLP ? a.L : 0);
  // the wave index is a scalar, so that every branch on it is a uniform jump
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, q16 = lane & 15;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int nitems = a.B * a.H * a.nb;
  const int item0 = (int)((int64_t)wg * nitems / gridDim.x);
  const int nsteps = ((int)((int64_t)(wg + 1) * nitems / gridDim.x) - item0) * a.P;
  const int logP = ilog2c(a.P);
  auto stage_of = [&](int t) { return smem + (t % NS) * lay.stage; };
  // prefix arrays of step parity: G, e^{G[C-1]-G}, e^{G[end of 16-token tile]-G}
  auto garr = [&](int t) { return reinterpret_cast<float*>(smem + lay.gw) + (t & 1) * 3 * C; };
  // fragment s of the within-block state of level m (1..MAXB), column tile wc
  auto state_frag = [&](int m, int wc, int s) {
    return smem + lay.st + (((m - 1) * NCT + wc) * KSD + s) * Lay::FRAG_BYTES + lane * 16;
  };

  // masked-score tiles above the diagonal are never written: keep them zero
  for (int x = tid * 16; x < 2 * PT::BYTES; x += 64 * NW * 16)
    *reinterpret_cast<uint4*>(smem + lay.p + x) = uint4{0, 0, 0, 0};

  // Preparation of chunk j for its read-out, in pieces that the waves share:
  // the in-chunk prefix G of the log-gates (each preparing wave writes the
  // same values), the masked scores
  // P[r][s] = (q_r . k_s) lambda_r^(lev(r,s)) e^{G_r - G_s} for s <= r in
  // 16x16 tiles (the diagonal ones by the makers, the ones below by the
  // readers) and the keys scaled by e^{G[C-1] - G_s} (by the first row group
  // of readers).  Below the diagonal the decay splits at the end e of the
  // source tile, e^{G_r - G_e} e^{G_e - G_s}: both factors are at most one.
  auto prefix = [&](int j) __attribute__((always_inline)) {
    const char* st = stage_of(j);
    float* gl = garr(j);
    const float gscan = chunk_prefix<C>(reinterpret_cast<const float*>(st + lay.g), lane);
    const float gsum = __shfl(gscan, C - 1, 64);
    const float gend = __shfl(gscan, lane | 15, 64);
    if (lane < C) {
      gl[lane] = gscan;
      gl[C + lane] = __expf(gsum - gscan);
      gl[2 * C + lane] = __expf(gend - gscan);
    }
  };
  // tile `item` of the causal tiles: the CT diagonal ones first, then the
  // ones below the diagonal, o = rt (rt-1)/2 + ct for ct < rt
  auto score_tile = [&](int j, int item) __attribute__((always_inline)) {
    const char* st = stage_of(j);
    const float* lraw = reinterpret_cast<const float*>(st + lay.lraw);
    const float* gl = garr(j);
    const float* es = gl + 2 * C;
    char* pt = smem + lay.p + (j & 1) * PT::BYTES;
    const bool diag = item < CT;
    int rt = item, ct = item;
    if (!diag) {
      const int o = item - CT;
      rt = 1;
#pragma unroll
      for (int u = 2; u < CT; ++u) rt += (o >= u * (u - 1) / 2) ? 1 : 0;
      ct = o - rt * (rt - 1) / 2;
    }
    const int r = 16 * rt + q16;  // lane: row r, sources 16 ct + 4 (lane/16) .. + 3
    const float* lr = lraw + r * LS;
    Frag kf[KSD], qf[KSD];
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      kf[s] = frag_row<T, C, D>(st + lay.k, 16 * ct + q16, s, g4);
      qf[s] = frag_row<T, C, D>(st + lay.q, r, s, g4);
    }
    const float gr = gl[r];
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x4 out;
    if (diag) {
      const f32x4 gs = *reinterpret_cast<const f32x4*>(gl + 16 * ct + 4 * g4);
      float lam[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lam[e] = lr[32 - __clz(r ^ (16 * ct + 4 * g4 + e))];  // level of (r, s)
#pragma unroll
      for (int s = 0; s < KSD; ++s) x = M::mma(kf[s], qf[s], x);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (T)((4 * g4 + e <= q16) ? x[e] * lam[e] * __expf(gr - gs[e]) : 0.f);
    } else {
      const f32x4 ess = *reinterpret_cast<const f32x4*>(es + 16 * ct + 4 * g4);
      const float wrow = lr[4 + 32 - __clz(rt ^ ct)] * __expf(gr - gl[16 * ct + 15]);
#pragma unroll
      for (int s = 0; s < KSD; ++s) x = M::mma(kf[s], qf[s], x);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (T)(x[e] * wrow * ess[e]);
    }
    *reinterpret_cast<bf16x4*>(pt + PT::off(r, 16 * ct + 4 * g4)) = out;
  };
  // decay-scaled keys: the same swizzled positions, each 16-byte piece of a
  // row scaled by that row's weight; pieces x0, x0 + STRIDE, ... (x0 < STRIDE,
  // which divides the piece count: a fixed trip count)
  auto scaled_keys = [&](int j, int x0, auto stride) __attribute__((always_inline)) {
    constexpr int STRIDE = decltype(stride)::value;
    static_assert((TL::BYTES / 16) % STRIDE == 0, "whole rounds of pieces");
    const char* st = stage_of(j);
    const float* wl = garr(j) + C;
    char* kw = smem + lay.kw + (j & 1) * TL::BYTES;
#pragma unroll
    for (int u = 0; u < TL::BYTES / 16 / STRIDE; ++u) {
      const int x = x0 + u * STRIDE;
      const float w = wl[x / TL::NCH];
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(st + lay.k + x * 16);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (T)((float)kv[e] * w);
      *reinterpret_cast<bf16x8*>(kw + x * 16) = o;
    }
  };
  constexpr int NBT = CT * (CT - 1) / 2;  // score tiles below the diagonal

  // The level-weight MLP of chunk j ("Adaptive memory decay for log-linear
  // attention", section "Method", LambdaMLPSoftplus), 16 rows at a time, as
  // in ll_lambda_mlp: lambda = softplus(d Wc + b) with the composite Wc = W1 W2
  // (the two layers are linear), formed once per workgroup with the same
  // operations, and the row product with the same k steps and accumulators,
  // into the chunk's level-weight rows.  The second row group of readers runs
  // it (row tile rt by reader rt mod NCT of the group), in the middle of their
  // step.  This lane's fragments of Wc (step s:
  // Wc[4g + s][c], zero past L) and the bias of level c:
  struct MlpFrags {
    float b[4], bias;
  };
  auto mlp_frags = [&]() __attribute__((always_inline)) {
    const float* w = reinterpret_cast<const float*>(smem + lay.mw);
    MlpFrags f;
#pragma unroll
    for (int s = 0; s < 4; ++s) f.b[s] = w[(4 * g4 + s) * 16 + q16];
    f.bias = w[16 * 16 + q16];
    return f;
  };
  auto mlp_tile = [&](const MlpFrags& f, int j, int rt) __attribute__((always_inline)) {
    // the lane's row and group from an opaque copy of the lane index, so that
    // the addresses below are formed here rather than held across the step
    int l = lane;
    asm volatile("" : "+v"(l));
    const int g4 = l >> 4, q16 = l & 15;
    // levels 4 g4 .. + 3 of the row, one 16-byte read (levels past L read the
    // zeros the ring holds there)
    const f32x4 dv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(smem + lay.dr) + (j % 2) * C * 16 +
                                                     (16 * rt + q16) * 16 + 4 * g4);
    const float bd[4] = {dv[0], dv[1], dv[2], dv[3]};
    const f32x4 z = mlp_tile_product<4>(bd, f.b);
    float* lr = reinterpret_cast<float*>(stage_of(j) + lay.lraw);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (q16 < LS) lr[(16 * rt + 4 * g4 + i) * LS + q16] = softplus_f32(z[i] + f.bias);
  };
  // Its input rows (d) go straight into LDS, into a ring of two chunks (chunk
  // j in slot j % 2), 16 levels a row: instruction u of row tile rt takes rows
  // 16 rt + 4u .. + 3, lane l row + l / 16, level l % 16 (levels past L are
  // not loaded).  With four makers, the makers of the last two column tiles
  // (the lightest step) load them, a chunk at the top of each step for use in
  // the next (chunk t+3 during step t, landed before the barrier of step t+1);
  // otherwise each reader of the second row group loads its own tiles, one
  // chunk ahead of its stage loads.
  constexpr bool D_BY_MAKERS = NMW >= 4;
  auto d_owner = [&](int rt) { return D_BY_MAKERS ? NRW + 2 + rt % 2 : NCT + rt % NCT; };
  auto d_owns = [&]() {
    bool o = false;
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) o = o || wv == d_owner(rt);
    return o;
  };
  ItemWalk dload_at;
  dload_at.start(item0, a, C);
  auto issue_d = [&](int j) __attribute__((always_inline)) {
    if (!MLP || !d_owns()) return;
    if (j > 0 && (j & (a.P - 1)) == 0) dload_at.next(a, C);
    const int64_t row0 = dload_at.row + (int64_t)((j & (a.P - 1)) * C * a.H);
    int l = lane;
    asm volatile("" : "+v"(l));  // the lane offsets are formed here, not held across the step
    const uint32_t off = (uint32_t)((((l >> 4) * a.H) * a.L + (l & 15)) * 4);
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
      if (wv == d_owner(rt)) {
        const __amdgpu_buffer_rsrc_t r =
            buffer_rsrc(a.lam + (row0 + (int64_t)16 * rt * a.H) * a.L, (uint32_t)((15 * a.H * a.L + a.L) * 4));
        char* dst = smem + lay.dr + (j % 2) * C * 16 * 4 + 16 * rt * 64;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if ((l & 15) < a.L)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + u * 256), 4, off, u * 4 * a.H * a.L * 4, 0, 0);
      }
  };
  auto mlp_share = [&](int j) __attribute__((always_inline)) {
    if (!MLP || wv < NCT || wv >= NRW) return;
    const MlpFrags f = mlp_frags();  // read for each use: registers are scarce across the step
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
      if (rt % NCT == wv - NCT) mlp_tile(f, j, rt);
  };
  if constexpr (MLP) {
    // the levels past L of the input ring: zero, and never loaded
    float* dring = reinterpret_cast<float*>(smem + lay.dr);
    for (int x = tid; x < 2 * C * 16; x += 64 * NW)
      if ((x & 15) >= a.L) dring[x] = 0.f;
  }

  if (wv >= NRW) {
    // ------------------------------------------------------------ makers
    const int mw = wv - NRW;  // column tile of the states this wave merges
    // the diagonal score tiles of chunk j
    auto prepare = [&](int j) __attribute__((always_inline)) {
      prefix(j);
#pragma unroll
      for (int d = mw; d < CT; d += NMW) score_tile(j, d);
#pragma unroll
      for (int o = NCT + mw; o < NBT; o += 2 * NCT) score_tile(j, CT + o);
    };

    if constexpr (MLP) {
      // Wc (16 x 16, zero past L) and the bias into LDS while the readers'
      // first chunks load
      float* w = reinterpret_cast<float*>(smem + lay.mw);
      for (int x = tid - 64 * NRW; x < 16 * 16; x += 64 * NMW) w[x] = mlp_composite(a.w1, a.w2, a.L, a.hidden, x / 16, x % 16);
      if (tid - 64 * NRW < 16) w[16 * 16 + lane] = lane < a.L ? a.mlp_bias[lane] : 0.f;
      issue_d(0);
      if (nsteps > 1) issue_d(1);
      __builtin_amdgcn_s_waitcnt(0);
    }
    lds_barrier();  // the zeroed tiles are visible; the readers' first chunks landed
    if constexpr (MLP) {
      lds_barrier();  // the readers made the level weights of chunks 0 and 1
      if (nsteps > 2) issue_d(2);
    }
    prepare(0);

    // the within-block Fenwick states of this wave's 16 columns (levels
    // 1..MAXB, fp32) and their log-scales
    f32x4 nst[MAXB][DT];
    float sig[MAXB + 1];
    for (int t = 0; t < nsteps; ++t) {
      const int j = t & (a.P - 1);
      if constexpr (MLP && D_BY_MAKERS) __builtin_amdgcn_s_waitcnt(0);  // the MLP input of chunk t+2
      lds_barrier();  // step t prepared; the readers' loads of step t+1 landed
      if constexpr (MLP) {
        if (t + 3 < nsteps) issue_d(t + 3);  // into the slot of chunk t+1, whose weights are made
      }
      if (j == 0) {
#pragma unroll
        for (int m = 0; m < MAXB; ++m)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) nst[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m <= MAXB; ++m) sig[m] = 0.f;
      }
      // this chunk's decayed key-value state K_w^T V over the wave's columns
      // (keys scaled by e^{G[C-1] - G_s}), merged by the Fenwick rule: levels
      // 1..c and the chunk become level c+1, c = ctz(j+1)
      const float gsum = garr(t)[C - 1];
#pragma unroll
      for (int m = 1; m <= MAXB; ++m) sig[m] += gsum;
      if (j + 1 < a.P) {
        const char* st = stage_of(t);
        const char* kw = smem + lay.kw + (t & 1) * TL::BYTES;
        // the keys' fragments in groups of DG state row tiles, so that few
        // registers hold them at once
        constexpr int DG = DT >= 4 ? 2 : DT;
        Frag vf[KSC], kf[DG][KSC];
#pragma unroll
        for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(st + lay.v, 16 * mw, s, lane);
#pragma unroll
        for (int u = 0; u < DG; ++u)
#pragma unroll
          for (int s = 0; s < KSC; ++s) kf[u][s] = frag_col<T, C, D>(kw, 16 * u, s, lane);
        const int c = __ffs(j + 1) - 1;
        // Level c+1 is empty (bit c of j is clear): the merged state is formed
        // in its registers, one copy of this code per level, so that no copy
        // of the state is made.
#pragma unroll
        for (int m = 1; m <= MAXB; ++m) {
          if (m == c + 1) {
            f32x4(&merged)[DT] = nst[m - 1];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) merged[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m2 = 1; m2 < m; ++m2) {
              const float sc = __expf(sig[m2]);
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) merged[dt] += sc * nst[m2 - 1][dt];
            }
#pragma unroll
            for (int d0 = 0; d0 < DT; d0 += DG) {
              lds_wait(vf, kf);
#pragma unroll
              for (int u = 0; u < DG; ++u)
#pragma unroll
                for (int s = 0; s < KSC; ++s) merged[d0 + u] = M::mma(kf[u][s], vf[s], merged[d0 + u]);
              if (d0 + DG < DT) {
#pragma unroll
                for (int u = 0; u < DG; ++u)
#pragma unroll
                  for (int s = 0; s < KSC; ++s) kf[u][s] = frag_col<T, C, D>(kw, 16 * (d0 + DG + u), s, lane);
              }
            }
            sig[m] = 0.f;
#pragma unroll
            for (int s = 0; s < KSD; ++s) *reinterpret_cast<Frag*>(state_frag(m, mw, s)) = M::acc_frag(merged, s);
          }
        }
      }
      if (t + 1 < nsteps) prepare(t + 1);
    }
    return;
  }

  // -------------------------------------------------------------- readers
  const int wc = wv % NCT, wr = wv / NCT;
  const int row_step = C * a.H;  // rows per chunk
  // Steps are loaded and read out in order, each by its own cursor over the
  // items; a cursor moves on at the first chunk of every item after its
  // first.  A step's output rows leave during the next step, at the row the
  // read cursor gave.
  ItemWalk load_at, read_at;
  load_at.start(item0, a, C);
  read_at = load_at;
  auto row_in = [&](const ItemWalk& w, int t) { return w.row + (int64_t)((t & (a.P - 1)) * row_step); };
  ChunkLoads<T, D, C, NRW> ld;
  ld.init(wv, lane, a.H, a.L, LS);
  // The loads of a step go out in three parts (q and gates, k and lambda, v),
  // so that they can be spread between pieces of compute.
  auto issue_part = [&](int j, int part) __attribute__((always_inline)) {
    char* st = stage_of(j);
    if (part == 0 && j > 0 && (j & (a.P - 1)) == 0) load_at.next(a, C);
    const int64_t row0 = row_in(load_at, j);
    if (part == 0) {
      ld.tiles(a.q, row0, st + lay.q, wv);
      ld.gates(a.g, row0, reinterpret_cast<float*>(st + lay.g), wv, lane);
    } else if (part == 1) {
      ld.tiles(a.k, row0, st + lay.k, wv);
      if constexpr (!MLP) ld.lambda(a.lam, row0, a.L, reinterpret_cast<float*>(st + lay.lraw), wv, lane);
    } else {
      ld.tiles(a.v, row0, st + lay.v, wv);
    }
  };
  auto issue = [&](int j) __attribute__((always_inline)) {
    issue_part(j, 0);
    issue_part(j, 1);
    issue_part(j, 2);
  };
  issue(0);
  if constexpr (MLP) {
    issue_d(0);
    if (nsteps > 1) issue_d(1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (nsteps > 1) issue(1);
  lds_barrier();  // step 0 has landed for every reader; the zeroed tiles are visible
  if constexpr (MLP) {
    mlp_share(0);
    if (nsteps > 1) mlp_share(1);
    if (!D_BY_MAKERS && nsteps > 2) issue_d(2);  // into the slot of chunk 0, whose weights are made
    lds_barrier();  // the level weights of chunks 0 and 1 are made
  }
  // the first row group's share of preparing chunk j: the scaled keys and
  // the score tiles below the diagonal that the makers do not take (the tiles
  // below the diagonal alternate between the two in runs of NCT)
  auto prepare = [&](int j) __attribute__((always_inline)) {
    if (wv >= NCT) return;
    prefix(j);
#pragma unroll
    for (int o = wv; o < NBT; o += 2 * NCT) score_tile(j, CT + o);
    scaled_keys(j, tid, std::integral_constant<int, 64 * NCT>{});
  };
  prepare(0);

  // The chunk loop, compiled once per row group so that every row-tile index
  // in it is a constant.
  auto run = [&](auto row_group) __attribute__((always_inline)) {
    constexpr int WR = decltype(row_group)::value;
    // Per item: the Fenwick nodes of earlier blocks for bits 0 .. MAXH-1 of
    // the block index J (slot b holds the node of bit b, at token level
    // LOGC + 1 + logP + b, when that bit is set) as A fragments of this wave's
    // columns, with their decay from their end to the start of block J (as a
    // factor); the decay factors of the within-block states.  Decays of whole
    // chunks are kept as running products of the chunks' e^{gate sum}.
    Frag hn[MAXH > 0 ? MAXH : 1][KSD];
    int hJ = 0;  // the block index of the item
    float ehd[MAXH > 0 ? MAXH : 1];
    int rest_far = 0;  // set bits of J whose nodes are not held in registers
    float dd_far = 0.f;
    int bh = 0;
    bool first_item = true;
    float esig[MAXB + 1];
    float egw = 1.f;  // decay from the start of block J to the current chunk
    auto node_of = [&](int e) {
      const float* f = a.F + ((int64_t)bh * a.nF + (e >> 1)) * D * D;
      const float* s = a.S + ((int64_t)bh * a.nb + e) * D * D;
      return (e & 1) ? f : s;
    };
    auto load_node = [&](Frag(&nf)[KSD], int e) __attribute__((always_inline)) {
      node_frags<T, D>(nf, node_of(e), wc, lane);
    };
    auto gamma_of = [&](int e) {
      const float* f = a.GF + (int64_t)bh * a.nF + (e >> 1);
      const float* s = a.GS + (int64_t)bh * a.nb + e;
      return *((e & 1) ? f : s);
    };
    auto start_item = [&]() __attribute__((always_inline)) {
      if (!first_item) read_at.next(a, C);
      first_item = false;
      bh = read_at.bh(a);
      // The held nodes: the node of set bit b of J covers the blocks from J
      // with bits below b cleared, back by 2^b; index e = (J >> b << b) - 1.
      // A slot whose bit is clear loads the node of the lowest set bit again
      // and weighs nothing, so that every node and decay load goes out at once.
      const int J = read_at.J;
      hJ = J;
      int ex[MAXH > 0 ? MAXH : 1];
#pragma unroll
      for (int b = 0; b < MAXH; ++b) ex[b] = ((J >> b) & 1) ? (J >> b << b) - 1 : J - 1;
      rest_far = MAXH > 0 ? J >> MAXH << MAXH : J;
      dd_far = 0.f;
#pragma unroll
      for (int b = 0; b < MAXH; ++b) ehd[b] = 1.f;
      if (MAXH > 0 && J > 0) {
        float gm[MAXH > 0 ? MAXH : 1];
#pragma unroll
        for (int b = 0; b < MAXH; ++b) {
          load_node(hn[b], ex[b]);
          gm[b] = gamma_of(ex[b]);
        }
#pragma unroll
        for (int b = 0; b < MAXH; ++b) {
          ehd[b] = __expf(dd_far);
          dd_far += ((J >> b) & 1) ? gm[b] : 0.f;
        }
      }
#pragma unroll
      for (int m = 0; m <= MAXB; ++m) esig[m] = 1.f;
      egw = 1.f;
    };

    // Output rows of a step leave during the following step.
    bf16x4 ov[NRT];
    int64_t out_row = 0;
    auto store_out = [&]() __attribute__((always_inline)) {
      const int64_t row0 = out_row;
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        const int r = 16 * W::row_tile(i, WR) + q16;  // lane: row r, columns 16 wc + 4 (lane/16) .. + 3
        T* o = static_cast<T*>(a.o) + (row0 + (int64_t)r * a.H) * D + 16 * wc + 4 * g4;
        *reinterpret_cast<bf16x4*>(o) = ov[i];
      }
    };

    for (int t = 0; t < nsteps; ++t) {
      const int j = t & (a.P - 1);    // chunk within the item's block
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of step t+1 and stores of step t-2 are done
      lds_barrier();                  // step t prepared and step t+1 landed everywhere; step t-1 done
      if (j == 0) start_item();       // node loads ahead of this step's other memory traffic
      if (t > 0) store_out();
      if (t + 2 < nsteps) issue_part(t + 2, 0);

      const char* st = stage_of(t);
      const float* lraw = reinterpret_cast<const float*>(st + lay.lraw);
      const float* gl = garr(t);
      const float gsum = gl[C - 1];

      // per row tile: Q fragments (index r, k = head dim), the row's lambda
      // weights times e^{G_r} for every inter-chunk level this chunk reads
      Frag qf[NRT][KSD];
      const float* lr[NRT];
      float egr[NRT], alw[NRT][MAXB], alh[NRT][MAXH > 0 ? MAXH : 1];
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        const int r = 16 * W::row_tile(i, WR) + q16;
#pragma unroll
        for (int s = 0; s < KSD; ++s) qf[i][s] = frag_row<T, C, D>(st + lay.q, r, s, g4);
        lr[i] = lraw + r * LS;
        egr[i] = __expf(gl[r]);
        // (levels LOGC+1 .. LOGC+logP+MAXH, contiguous in the row; the ones past
        // the staged levels read the next row's, within LDS, and are never used)
#pragma unroll
        for (int m = 1; m <= MAXB; ++m) alw[i][m - 1] = lr[i][LOGC + m] * egr[i];
        const float* lrh = lr[i] + LOGC + 1 + logP;
#pragma unroll
        for (int b = 0; b < MAXH; ++b) alh[i][b] = lrh[b] * egr[i];
      }

      // --- intra-chunk: O^T += V^T P^T
      Frag vf[KSC];
#pragma unroll
      for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(st + lay.v, 16 * wc, s, lane);
      const char* pt = smem + lay.p + (t & 1) * PT::BYTES;
      Frag pf[NRT][KSC];
#pragma unroll
      for (int i = 0; i < NRT; ++i)
#pragma unroll
        for (int s = 0; s < KSC; ++s) pf[i][s] = frag_row<T, C, C>(pt, 16 * W::row_tile(i, WR) + q16, s, g4);
      lds_wait(vf);
      f32x4 oacc[NRT];
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSC; ++s)
          if (M::first_tile(s) <= W::row_tile(i, WR)) oacc[i] = M::mma(vf[s], pf[i][s], oacc[i]);
      }

      if (t + 2 < nsteps) {
        issue_part(t + 2, 1);
        issue_part(t + 2, 2);
      }
      if (t + 3 < nsteps) issue_d(t + 3);  // into the slot of chunk t+1, whose weights are made
      // the level weights of chunk t+2 (its stage is being loaded, but not its
      // weight rows), here so that their products overlap this step's reads
      if (t + 2 < nsteps) mlp_share(t + 2);

      // --- inter-chunk levels: O^T += diag(alpha) N^T Q^T, alpha_r = lambda_r^l e^{G_r} x scale.
      // A level's product is weighted into O only when the next level comes
      // (or at the end), so no level waits right away for its own products.
      f32x4 pend[NRT];
      float pal[NRT];
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        pend[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        pal[i] = 0.f;
      }
      auto level_read = [&](const Frag(&nf)[KSD], const float(&al)[NRT]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NRT; ++i) {
          oacc[i] += pal[i] * pend[i];
          pal[i] = al[i];
          pend[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KSD; ++s) pend[i] = M::mma(nf[s], qf[i][s], pend[i]);
        }
      };
      // within-block levels LOGC+1 .. LOGC+logP, from the makers' fragments
#pragma unroll
      for (int m = 1; m <= MAXB; ++m) {
        if (m <= logP && ((j >> (m - 1)) & 1)) {
          Frag nf[KSD];
#pragma unroll
          for (int s = 0; s < KSD; ++s) nf[s] = *reinterpret_cast<const Frag*>(state_frag(m, wc, s));
          const float sc = esig[m];
          float al[NRT];
#pragma unroll
          for (int i = 0; i < NRT; ++i) al[i] = alw[i][m - 1] * sc;
          level_read(nf, al);
        }
      }
      // earlier blocks: one Fenwick node per set bit of J, most recent first
#pragma unroll
      for (int b = 0; b < MAXH; ++b) {
        if ((hJ >> b) & 1) {
          const float sc = egw * ehd[b];
          float al[NRT];
#pragma unroll
          for (int i = 0; i < NRT; ++i) al[i] = alh[i][b] * sc;
          level_read(hn[b], al);
        }
      }
      {
        int rest = rest_far;
        float dd = dd_far;
        while (rest > 0) {
          const int e = rest - 1;
          Frag nf[KSD];
          load_node(nf, e);
          const int lev = LOGC + 1 + logP + __ffs(rest) - 1;
          const float sc = egw * __expf(dd);
          float al[NRT];
#pragma unroll
          for (int i = 0; i < NRT; ++i) al[i] = lr[i][lev] * egr[i] * sc;
          level_read(nf, al);
          dd += gamma_of(e);
          rest &= rest - 1;
        }
        // A segment that continues a sequence from the per-level states of
        // [0, pos0) ("Log-Linear Attention", section 2.2): its tokens also
        // read the bucket of each set bit b of pos0, at level b + 1, above
        // every level inside the segment.  The states come in the decode
        // layout (S_hat row-major, true state e^sigma S_hat, decayed through
        // token pos0 - 1) and reach the row with the segment's gates before
        // it: those of the earlier blocks (dd, now all of them), of this
        // block's earlier chunks and of the row's chunk up to the row.
        if (PRIOR) {
          const float* sh = a.prior + (int64_t)bh * a.L * D * D;
          const float* sgm = a.prior + (int64_t)a.B * a.H * a.L * D * D + (int64_t)bh * a.L;
          uint64_t bits = (uint64_t)a.pos0;
          while (bits) {
            const int lev = __ffsll((unsigned long long)bits);  // bit index + 1
            bits &= bits - 1;
            const float* S = sh + (int64_t)lev * D * D + 16 * wc + q16;
            Frag nf[KSD];
#pragma unroll
            for (int s2 = 0; s2 < KSD; ++s2)
#pragma unroll
              for (int e = 0; e < 8; ++e) nf[s2][e] = (T)S[M::kidx(s2, g4, e) * D];
            const float sc = egw * __expf(sgm[lev] + dd);
            float al[NRT];
#pragma unroll
            for (int i = 0; i < NRT; ++i) al[i] = lr[i][lev] * egr[i] * sc;
            level_read(nf, al);
          }
        }
      }

      // --- the output rows, stored during the next step
      out_row = row_in(read_at, t);
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        oacc[i] += pal[i] * pend[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[i][e] = (T)oacc[i][e];
      }

      // the decay factors follow the makers' merge: every level decays by the
      // chunk, the merged level c+1 starts afresh
      const float egs = __expf(gsum);
#pragma unroll
      for (int m = 1; m <= MAXB; ++m) esig[m] *= egs;
      egw *= egs;
      if (j + 1 < a.P) {
        const int c = __ffs(j + 1) - 1;
#pragma unroll
        for (int m = 1; m <= MAXB; ++m)
          if (m == c + 1) esig[m] = 1.f;
      }
      if (t + 1 < nsteps) prepare(t + 1);
    }
    store_out();
  };
  if (wr == 0) {
    run(std::integral_constant<int, 0>{});
  } else {
    run(std::integral_constant<int, 1>{});
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, int C>
static hipError_t launch_state_t(const PrefillArgs& a, hipStream_t s) {
  const int grid = a.B * a.H * a.nb;
  hipLaunchKernelGGL((ll_chunk_state<T, D, C>), dim3(grid), dim3(64 * (D / 16)), 0, s, a);
  return hipGetLastError();
}

// A persistent launch: as many workgroups as fit on the device at once, each
// walking a run of consecutive (block, head) items.  Per kernel instance the
// dynamic LDS allowed (above 64 KiB it must be raised explicitly) and the
// number of workgroups that fit for that LDS size are kept under a lock
// (calls may come from several threads).
struct PersistentGrid {
  std::mutex mu;
  int configured = 0, slots = 0, slots_lds = -1;
  hipError_t launch(const void* kern, int threads, int lds, const PrefillArgs& a, hipStream_t s) {
    int grid_slots = 0;
    {
      std::lock_guard<std::mutex> lock(mu);
      if (lds > configured) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        configured = lds;
      }
      if (slots_lds != lds) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds);
        if (e != hipSuccess) return e;
        slots = cus * (per_cu > 0 ? per_cu : 1);
        slots_lds = lds;
      }
      grid_slots = slots;
    }
    const int items = a.B * a.H * a.nb;
    const int grid = items < grid_slots ? items : grid_slots;
    void* args[] = {const_cast<PrefillArgs*>(&a)};
    hipError_t e = hipLaunchKernel(kern, dim3(grid), dim3(threads), args, lds, s);
    return e != hipSuccess ? e : hipGetLastError();
  }
};

template <typename T, int D, int C>
static hipError_t launch_attn_t(const PrefillArgs& a, hipStream_t s) {
  if constexpr (C * D * (int)sizeof(T) > kAttnTileBytesMax) {
    return hipErrorInvalidValue;  // rejected by the shape checks before launch
  } else {
    // Fenwick nodes of earlier blocks held in registers (4 cover up to 16 blocks per head; the
    // nodes of further set bits are read at each chunk; a fifth held node costs the registers
    // that keep the read's loop free of spills).  At d = 128 the within-block nodes of
    // 8-chunk blocks already fill the register budget, so every earlier block's node is read
    // from LDS (holding even one spills).
    constexpr int MAXH = (sizeof(T) == 2) ? (D <= 64 ? 4 : 0) : 0;
    static PersistentGrid grid;
    if constexpr (read_split(sizeof(T) == 2 ? 1 : 0, D, C)) {
      constexpr int MAXB = read_block_depth(1, D, C);
      if (a.P > (1 << MAXB)) return hipErrorInvalidValue;  // planned within the depth
      if (a.w1) {
        if (a.L > 16 || a.hidden < 1 || a.prior) return hipErrorInvalidValue;  // checked before launch
        static PersistentGrid grid_mlp;
        auto kern = ll_chunk_attn_split<D, C, MAXB, MAXH, true>;
        const SplitLayout<D, C, MAXB> lay(a.LS, a.L);
        return grid_mlp.launch(reinterpret_cast<const void*>(kern), 64 * SplitWaves<D, C>::NW, lay.total, a, s);
      }
      if (a.prior) {
        // a segment continuing a sequence: the read takes the earlier levels too
        static PersistentGrid grid_prior;
        auto kern = ll_chunk_attn_split<D, C, MAXB, MAXH, false, true>;
        const SplitLayout<D, C, MAXB> lay(a.LS);
        return grid_prior.launch(reinterpret_cast<const void*>(kern), 64 * SplitWaves<D, C>::NW, lay.total, a, s);
      }
      auto kern = ll_chunk_attn_split<D, C, MAXB, MAXH, false>;
      const SplitLayout<D, C, MAXB> lay(a.LS);
      return grid.launch(reinterpret_cast<const void*>(kern), 64 * SplitWaves<D, C>::NW, lay.total, a, s);
    } else {
      if (a.w1) return hipErrorInvalidValue;  // the MLP runs inside the bf16 d <= 64 read only
      if (a.P > (1 << max_block_depth(D))) return hipErrorInvalidValue;  // planned within the depth
      auto kern = ll_chunk_attn<T, D, C, max_block_depth(D), MAXH>;
      const AttnLayout<T, D, C> lay(a.LS);
      return grid.launch(reinterpret_cast<const void*>(kern), 64 * AttnWaves<D, C>::NW, lay.total, a, s);
    }
  }
}

// bf16 MFMA steps contract 32 values, so bf16 needs C >= 32 and D >= 32
#define LL_DISPATCH_C(FN, T, D)                     \
  switch (C) {                                      \
    case 32: return FN<T, D, 32>(a, s);             \
    case 64: return FN<T, D, 64>(a, s);             \
    default: return hipErrorInvalidValue;           \
  }

#define LL_DISPATCH_C_F32(FN, D)                    \
  switch (C) {                                      \
    case 16: return FN<float, D, 16>(a, s);         \
    case 32: return FN<float, D, 32>(a, s);         \
    case 64: return FN<float, D, 64>(a, s);         \
    default: return hipErrorInvalidValue;           \
  }

#define LL_DISPATCH(FN)                                          \
  if (io == 1) {                                                 \
    switch (D) {                                                 \
      case 32: LL_DISPATCH_C(FN, bf16, 32)                       \
      case 64: LL_DISPATCH_C(FN, bf16, 64)                       \
      case 128: LL_DISPATCH_C(FN, bf16, 128)                     \
      default: return hipErrorInvalidValue;                      \
    }                                                            \
  } else {                                                       \
    switch (D) {                                                 \
      case 16: LL_DISPATCH_C_F32(FN, 16)                         \
      case 32: LL_DISPATCH_C_F32(FN, 32)                         \
      case 64: LL_DISPATCH_C_F32(FN, 64)                         \
      case 128: /* a C x 128 fp32 tile fits at C = 16 only */    \
        if (C == 16) return FN<float, 128, 16>(a, s);            \
        return hipErrorInvalidValue;                             \
      default: return hipErrorInvalidValue;                      \
    }                                                            \
  }

hipError_t launch_block_state(int io, int D, int C, const PrefillArgs& a, hipStream_t s) { LL_DISPATCH(launch_state_t) }

hipError_t launch_chunk_attn(int io, int D, int C, const PrefillArgs& a, hipStream_t s) { LL_DISPATCH(launch_attn_t) }

}  // namespace llattn
