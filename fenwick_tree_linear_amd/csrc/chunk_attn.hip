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
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// DPP move of a float within a wave (lanes without a source read 0).
template <int CTRL, int ROW_MASK, bool ZERO_FILL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, ZERO_FILL));
}

// In-chunk inclusive prefix G of the log-gates (every wave computes it; lane
// r holds G[r]).  DPP shifts inside each 16-lane row, then the last lane of
// each row is broadcast to the rows above it: no LDS round trips.
template <int C>
__device__ __forceinline__ float chunk_prefix(const float* gates, int lane) {
  float x = lane < C ? gates[lane] : 0.f;
  x += dpp_f32<0x111, 0xf, true>(x);  // row_shr:1
  x += dpp_f32<0x112, 0xf, true>(x);  // row_shr:2
  x += dpp_f32<0x114, 0xf, true>(x);  // row_shr:4
  x += dpp_f32<0x118, 0xf, true>(x);  // row_shr:8
  if (C > 16) x += dpp_f32<0x142, 0xa, false>(x);  // row_bcast:15 into rows 1 and 3
  if (C > 32) x += dpp_f32<0x143, 0xc, false>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Multiplies element e of a fragment whose k axis is tokens by w[token(e)].
template <typename T>
__device__ __forceinline__ typename Mma<T>::Frag scale_tokens(typename Mma<T>::Frag f, const float* w, int s, int g) {
  if constexpr (sizeof(T) == 2) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(w + 32 * s + 4 * g);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(w + 32 * s + 16 + 4 * g);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (bf16)((float)f[e] * lo[e]);
      r[4 + e] = (bf16)((float)f[4 + e] * hi[e]);
    }
    return r;
  } else {
    return f * w[Mma<float>::kidx(s, g, 0)];
  }
}

// Direct loads of chunk rows [row0, row0 + C) of one head.
template <typename T, int D, int C>
__device__ __forceinline__ void issue_rows(const void* src, const PrefillArgs& a, int64_t row0, char* lds, int wv,
                                           int nw, int lane) {
  tile_load_async<T, C, D>(static_cast<const T*>(src) + row0 * D, (int64_t)a.H * D, lds, wv, nw, lane);
}

template <int C>
__device__ __forceinline__ void issue_gates(const PrefillArgs& a, int64_t row0, float* lds, int wv, int nw, int lane) {
  const float* g = a.g + row0;
  scatter_load_async(lds, C, wv, nw, lane, [&](int f) { return g + (int64_t)f * a.H; });
}

// lambda rows of the chunk, row-major [C][LS]: consecutive lanes read
// consecutive floats of one token's level weights.
// (f / LS uses a multiply-high by ceil(2^32 / LS): exact for f * LS < 2^32.)
template <int C>
__device__ __forceinline__ void issue_lambda(const PrefillArgs& a, int64_t row0, float* lds, int LS, unsigned ls_magic,
                                             int wv, int nw, int lane) {
  const float* lam = a.lam + row0 * a.L;
  const int64_t ls = (int64_t)a.H * a.L;
  scatter_load_async(lds, LS * C, wv, nw, lane, [&](int f) {
    const int r = (int)__umulhi((unsigned)f, ls_magic);
    return lam + r * ls + (f - r * LS);
  });
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

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g4 = lane >> 4;
  float* wl = reinterpret_cast<float*>(smem + L::WOFF) + wv * C;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int J = wg % a.nb, bh = wg / a.nb, h = bh % a.H, b = bh / a.H;
  auto row_of = [&](int j) { return ((int64_t)b * a.T + (int64_t)(J * a.P + j) * C) * a.H + h; };
  auto issue = [&](int j) {
    char* st = smem + (j & 1) * L::STAGE;
    issue_rows<T, D, C>(a.k, a, row_of(j), st + L::KOFF, wv, NW, lane);
    issue_rows<T, D, C>(a.v, a, row_of(j), st + L::VOFF, wv, NW, lane);
    issue_gates<C>(a, row_of(j), reinterpret_cast<float*>(st + L::GOFF), wv, NW, lane);
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
    typename M::Frag vf[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = scale_tokens<T>(frag_col<T, C, D>(st + L::VOFF, 16 * wv, s, lane), wl, s, g4);
    const float carry = __expf(gsum);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 x = acc[dt] * carry;
#pragma unroll
      for (int s = 0; s < KSC; ++s) x = M::mma(frag_col<T, C, D>(st + L::KOFF, 16 * dt, s, lane), vf[s], x);
      acc[dt] = x;
    }
    gblk += gsum;
  }

  float* dst = a.S + ((int64_t)bh * a.nb + J) * D * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + state_tile_offset<D>(dt, wv, lane)) = acc[dt];
  if (tid == 0) a.GS[(int64_t)bh * a.nb + J] = gblk;
}

// Adds diag(alpha) (Q N) to oacc, N given as MFMA B fragments (k = head dim,
// n = this wave's 16 columns), alpha_r = lamT[r] * scale for the rows
// r = 16*rt + 4*(lane/16) + i this lane holds.
template <typename T, int D, int C>
__device__ __forceinline__ void level_read(f32x4 (&oacc)[C / 16],
                                           const typename Mma<T>::Frag (&qf)[C / 16][D / Mma<T>::KS],
                                           const typename Mma<T>::Frag (&nf)[D / Mma<T>::KS], const float* lamT,
                                           float scale, int g4) {
  using M = Mma<T>;
  constexpr int CT = C / 16, KSD = D / M::KS;
#pragma unroll
  for (int rt = 0; rt < CT; ++rt) {
    f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSD; ++s) tmp = M::mma(qf[rt][s], nf[s], tmp);
    const f32x4 al = *reinterpret_cast<const f32x4*>(lamT + 16 * rt + 4 * g4);
    oacc[rt] += (al * scale) * tmp;
  }
}

template <typename T, int D>
__device__ __forceinline__ void node_frags(typename Mma<T>::Frag (&nf)[D / Mma<T>::KS], const float* node, int wv,
                                           int lane) {
  using M = Mma<T>;
  constexpr int DT = D / 16, KSD = D / M::KS;
  f32x4 t[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) t[dt] = *reinterpret_cast<const f32x4*>(node + state_tile_offset<D>(dt, wv, lane));
#pragma unroll
  for (int s = 0; s < KSD; ++s) nf[s] = M::acc_frag(t, s);
}

// Dynamic LDS layout of ll_chunk_attn (byte offsets; LS = staged levels).
template <typename T, int D, int C, int MAXH, bool QDB>
struct AttnLayout {
  typedef Tile<T, C, D> TL;
  typedef Tile<T, C, C> PT;
  static constexpr int NW = D / 16;
  static constexpr int LOGC = (C == 16) ? 4 : (C == 32) ? 5 : 6;
  static constexpr int FRAG_BYTES = 64 * (int)sizeof(typename Mma<T>::Frag);
  static constexpr int NODE_BYTES = NW * (D / Mma<T>::KS) * FRAG_BYTES;
  int k, v, lraw, g, stage;  // per-stage offsets and stage size
  int q, p, lt, gw, h, total;  // q: in the stage when double-buffered (QDB)
  __host__ __device__ explicit AttnLayout(int LS) {
    k = 0;
    v = k + TL::BYTES;
    g = v + TL::BYTES;
    lraw = g + C * 4;                      // lambda rows [C][LS]
    stage = lraw + ((C * LS * 4 + 15) & ~15);
    if (QDB) {
      q = stage;
      stage += TL::BYTES;
      p = 2 * stage;
    } else {
      q = 2 * stage;                       // single q tile, refilled after the mid-chunk barrier
      p = q + TL::BYTES;
    }
    // p: masked scores [C][C]
    lt = p + PT::BYTES;                    // inter-chunk lambda^T, scaled [LS-LOGC-1][C]
    const int nlt = LS > LOGC + 1 ? LS - LOGC - 1 : 0;
    gw = lt + nlt * C * 4;                 // per-wave G and decay-to-end [NW][2][C]
    h = gw + NW * 2 * C * 4;               // MAXH nodes as B fragments
    total = h + MAXH * NODE_BYTES;
  }
};

// ---------------------------------------------------------------------------
// ll_chunk_attn: one workgroup per (block J, head); wave wv owns output
// columns [16 wv, 16 wv + 16); the P chunks of the block are visited in order.
// The Fenwick nodes of earlier blocks are the same for every chunk of the
// block: up to MAXH of them are converted once into MFMA B fragments in LDS,
// any further ones are read from the workspace per chunk.
template <typename T, int D, int C, int MAXB, int MAXH, bool QDB>
__global__ void __launch_bounds__(64 * (D / 16)) __attribute__((amdgpu_waves_per_eu(2, 2)))
ll_chunk_attn(PrefillArgs a) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef AttnLayout<T, D, C, MAXH, QDB> Lay;
  typedef Tile<T, C, C> PT;
  constexpr int NW = D / 16;
  constexpr int DT = D / 16, CT = C / 16;
  constexpr int KSD = D / M::KS, KSC = C / M::KS;
  constexpr int LOGC = Lay::LOGC;
  constexpr int FRAG_BYTES = Lay::FRAG_BYTES;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int LS = a.LS;
  const unsigned ls_magic = (unsigned)((0x100000000ull + LS - 1) / LS);
  const Lay lay(LS);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g4 = lane >> 4, q16 = lane & 15;
  float* gl = reinterpret_cast<float*>(smem + lay.gw) + wv * 2 * C;  // this wave's G
  float* wl = gl + C;                                                // and exp(G[C-1] - G)
  float* lt = reinterpret_cast<float*>(smem + lay.lt);
  char* pt = smem + lay.p;
  char* hbuf = smem + lay.h;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int J = wg % a.nb, bh = wg / a.nb, h = bh % a.H, b = bh / a.H;
  const int logP = ilog2c(a.P);
  auto row_of = [&](int j) { return ((int64_t)b * a.T + (int64_t)(J * a.P + j) * C) * a.H + h; };
  auto node_of = [&](int e) {
    return (e & 1) ? a.F + ((int64_t)bh * a.nF + (e >> 1)) * D * D : a.S + ((int64_t)bh * a.nb + e) * D * D;
  };
  auto gamma_of = [&](int e) { return (e & 1) ? a.GF[(int64_t)bh * a.nF + (e >> 1)] : a.GS[(int64_t)bh * a.nb + e]; };
  auto issue_kvl = [&](int j) {
    char* st = smem + (j & 1) * lay.stage;
    issue_rows<T, D, C>(a.k, a, row_of(j), st + lay.k, wv, NW, lane);
    issue_rows<T, D, C>(a.v, a, row_of(j), st + lay.v, wv, NW, lane);
    issue_gates<C>(a, row_of(j), reinterpret_cast<float*>(st + lay.g), wv, NW, lane);
    issue_lambda<C>(a, row_of(j), reinterpret_cast<float*>(st + lay.lraw), LS, ls_magic, wv, NW, lane);
    if (QDB) issue_rows<T, D, C>(a.q, a, row_of(j), st + lay.q, wv, NW, lane);
  };

  issue_kvl(0);
  if (!QDB) issue_rows<T, D, C>(a.q, a, row_of(0), smem + lay.q, wv, NW, lane);

  // masked-score tiles above the diagonal are never written: keep them zero
  for (int x = tid * 16; x < PT::BYTES; x += 64 * NW * 16) *reinterpret_cast<uint4*>(pt + x) = uint4{0, 0, 0, 0};

  // the first MAXH nodes (most recent first) as B fragments of each wave's columns
  if constexpr (MAXH > 0) {
    int rest = J;
    for (int x = 0; x < MAXH && rest > 0; ++x) {
      Frag nf[KSD];
      node_frags<T, D>(nf, node_of(rest - 1), wv, lane);
#pragma unroll
      for (int s = 0; s < KSD; ++s)
        *reinterpret_cast<Frag*>(hbuf + ((x * NW + wv) * KSD + s) * FRAG_BYTES + lane * (int)sizeof(Frag)) = nf[s];
      rest &= rest - 1;
    }
  }

  f32x4 nst[MAXB][DT];
  float sig[MAXB + 1];
#pragma unroll
  for (int m = 0; m < MAXB; ++m)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) nst[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m <= MAXB; ++m) sig[m] = 0.f;
  float gw = 0.f;  // log-decay from the start of block J to the current chunk

  for (int j = 0; j < a.P; ++j) {
    const char* st = smem + (j & 1) * lay.stage;
    const float* lraw = reinterpret_cast<const float*>(st + lay.lraw);
    const char* qt = QDB ? st + lay.q : smem + lay.q;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk j (and q) have landed
    lds_barrier();                  // every wave's have; chunk j-1 is done everywhere
    if (j + 1 < a.P) issue_kvl(j + 1);

    const float gscan = chunk_prefix<C>(reinterpret_cast<const float*>(st + lay.g), lane);
    const float gsum = __shfl(gscan, C - 1, 64);
    if (lane < C) {
      gl[lane] = gscan;
      wl[lane] = __expf(gsum - gscan);
    }

    Frag qf[CT][KSD];
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
#pragma unroll
      for (int s = 0; s < KSD; ++s) qf[rt][s] = frag_row<T, C, D>(qt, 16 * rt + q16, s, g4);

    // --- intra-chunk scores, this wave's share of the causal tiles:
    // P[r][s] = (q_r . k_s) lambda_r^(lev(r,s)) exp(G[r] - G[s]), s <= r
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
#pragma unroll
      for (int ct = 0; ct <= rt; ++ct) {  // ct: source tile (column of P)
        if ((rt * (rt + 1) / 2 + ct) % NW != wv) continue;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSD; ++s) x = M::mma(frag_row<T, C, D>(st + lay.k, 16 * ct + q16, s, g4), qf[rt][s], x);
        const int r = 16 * rt + q16;
        const float gr = gl[r];
        const f32x4 gs = *reinterpret_cast<const f32x4*>(gl + 16 * ct + 4 * g4);
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int src = 16 * ct + 4 * g4 + i;
          float val = 0.f;
          if (src <= r) {
            const int lev = (src == r) ? 0 : 32 - __clz(r ^ src);
            val = x[i] * lraw[r * LS + lev] * __expf(gr - gs[i]);
          }
          pv[i] = val;
        }
        char* dst = pt + PT::off(r, 16 * ct + 4 * g4);
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)pv[0], (bf16)pv[1], (bf16)pv[2], (bf16)pv[3]};
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{pv[0], pv[1], pv[2], pv[3]};
        }
      }

    // --- lambda of the inter-chunk levels, transposed to [level][r] and
    // pre-multiplied by exp(G[r])
    {
      const float eg = __expf(gl[lane & (C - 1)]);
      const int n = (LS - LOGC - 1) * C;
      for (int x = tid; x < n; x += 64 * NW) {
        const int l = LOGC + 1 + x / C, r = x % C;
        lt[x] = lraw[r * LS + l] * eg;
      }
    }
    lds_barrier();  // P and lambda^T visible; the loads of chunk j+1 keep flying
    if (!QDB && j + 1 < a.P) issue_rows<T, D, C>(a.q, a, row_of(j + 1), smem + lay.q, wv, NW, lane);

    f32x4 oacc[CT];
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) oacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // --- within-block levels LOGC+1 .. LOGC+logP
#pragma unroll
    for (int m = 1; m <= MAXB; ++m) {
      if (m <= logP && ((j >> (m - 1)) & 1)) {
        Frag nf[KSD];
#pragma unroll
        for (int s = 0; s < KSD; ++s) nf[s] = M::acc_frag(nst[m - 1], s);
        level_read<T, D, C>(oacc, qf, nf, lt + (m - 1) * C, __expf(sig[m]), g4);
      }
    }

    // --- earlier blocks: one Fenwick node per set bit of J, most recent first
    {
      int rest = J;
      float dd = 0.f;  // log-decay from the node's end to the start of block J
      for (int x = 0; rest > 0; ++x) {
        const int e = rest - 1, l = __ffs(rest) - 1;
        Frag nf[KSD];
        if (x < MAXH) {
#pragma unroll
          for (int s = 0; s < KSD; ++s)
            nf[s] = *reinterpret_cast<const Frag*>(hbuf + ((x * NW + wv) * KSD + s) * FRAG_BYTES +
                                                   lane * (int)sizeof(Frag));
        } else {
          node_frags<T, D>(nf, node_of(e), wv, lane);
        }
        level_read<T, D, C>(oacc, qf, nf, lt + (logP + l) * C, __expf(gw + dd), g4);
        dd += gamma_of(e);
        rest &= rest - 1;
      }
    }

    // --- intra-chunk: O += P V for this wave's columns
    Frag vf[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(st + lay.v, 16 * wv, s, lane);
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
#pragma unroll
      for (int s = 0; s < KSC; ++s)
        if (M::first_tile(s) <= rt) oacc[rt] = M::mma(frag_row<T, C, C>(pt, 16 * rt + q16, s, g4), vf[s], oacc[rt]);

    // --- store this chunk's output rows (this wave's 16 columns)
    {
      T* o = static_cast<T*>(a.o) + row_of(j) * D + 16 * wv + q16;
      const int64_t rs = (int64_t)a.H * D;
#pragma unroll
      for (int rt = 0; rt < CT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[(16 * rt + 4 * g4 + i) * rs] = from_f32<T>(oacc[rt][i]);
    }

    // --- this chunk's own decayed key-value state, then the merge rule of
    // the within-block Fenwick levels (levels 1..c and the chunk become level
    // c+1, c = ctz(j+1))
#pragma unroll
    for (int m = 1; m <= MAXB; ++m) sig[m] += gsum;
    gw += gsum;
    if (j + 1 < a.P) {
#pragma unroll
      for (int s = 0; s < KSC; ++s) vf[s] = scale_tokens<T>(vf[s], wl, s, g4);
      f32x4 merged[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSC; ++s) x = M::mma(frag_col<T, C, D>(st + lay.k, 16 * dt, s, lane), vf[s], x);
        merged[dt] = x;
      }
      const int c = __ffs(j + 1) - 1;
#pragma unroll
      for (int m = 1; m <= MAXB; ++m) {
        if (m <= c) {
          const float sc = __expf(sig[m]);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) merged[dt] += sc * nst[m - 1][dt];
        }
      }
#pragma unroll
      for (int m = 1; m <= MAXB; ++m) {
        if (m == c + 1) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) nst[m - 1][dt] = merged[dt];
          sig[m] = 0.f;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, int C>
static hipError_t launch_state_t(const PrefillArgs& a, hipStream_t s) {
  const int grid = a.B * a.H * a.nb;
  hipLaunchKernelGGL((ll_chunk_state<T, D, C>), dim3(grid), dim3(64 * (D / 16)), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D, int C>
static hipError_t launch_attn_t(const PrefillArgs& a, hipStream_t s) {
  // node fragments kept in LDS (bf16 heads up to 64: 8 KB per node at d=64)
  constexpr int MAXH = 0;
  constexpr bool QDB = false;
  auto kern = ll_chunk_attn<T, D, C, max_block_depth(D), MAXH, QDB>;
  const AttnLayout<T, D, C, MAXH, QDB> lay(a.LS);
  static int configured = 0;  // dynamic LDS above 64 KiB must be allowed per kernel
  if (lay.total > configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lay.total);
    if (e != hipSuccess) return e;
    configured = lay.total;
  }
  const int grid = a.B * a.H * a.nb;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * (D / 16)), lay.total, s, a);
  return hipGetLastError();
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
      default: return hipErrorInvalidValue;                      \
    }                                                            \
  }

hipError_t launch_block_state(int io, int D, int C, const PrefillArgs& a, hipStream_t s) { LL_DISPATCH(launch_state_t) }

hipError_t launch_chunk_attn(int io, int D, int C, const PrefillArgs& a, hipStream_t s) { LL_DISPATCH(launch_attn_t) }

}  // namespace llattn
