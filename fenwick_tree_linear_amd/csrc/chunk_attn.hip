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
// Both kernels stream their chunks through LDS with direct global->LDS loads,
// double-buffered: chunk j+1 is in flight while chunk j is computed.  Tiles
// keep the global row-major layout; the operands that contract over tokens
// (V, and the decayed K for the state) are read with the transposing LDS
// read, so no transposed copy is ever written.
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// Per-chunk staging area of one pipeline stage.
template <typename T, int D, int C>
struct Stage {
  typedef Tile<T, C, D> Row;  // q, k, v: [C][D]
  static constexpr int QOFF = 0;
  static constexpr int KOFF = QOFF + Row::BYTES;
  static constexpr int VOFF = KOFF + Row::BYTES;
  static constexpr int LOFF = VOFF + Row::BYTES;            // lambda^T [kLevelsMax][C] fp32
  static constexpr int GOFF = LOFF + kLevelsMax * C * 4;    // raw log-gates [C] fp32
  static constexpr int BYTES = GOFF + C * 4;
};

// Shared prologue of one chunk: the in-chunk inclusive prefix G of the
// log-gates (every wave computes it; lane r holds G[r]).
template <int C>
__device__ __forceinline__ float chunk_prefix(const float* gates, int lane) {
  float x = lane < C ? gates[lane] : 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Writes kd[r][:] = k[r][:] * exp(G[C-1] - G[r]) (the key decayed to the chunk
// end) for the rows of wave wv.  Elementwise per row, so it works on LDS
// positions directly (the swizzle is the same in both tiles).
template <typename T, int D, int C, int NW>
__device__ __forceinline__ void decay_keys(const char* k, char* kd, float gscan, int wv, int lane) {
  typedef Tile<T, C, D> TL;
  constexpr int RPW = C / NW;                       // rows per wave
  constexpr int CPL = RPW * TL::NCH / 64;           // 16-byte chunks per lane
  static_assert(CPL >= 1 && (RPW * TL::NCH) % 64 == 0, "decay pass shape");
  const float glast = __shfl(gscan, C - 1, 64);
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int ci = lane + 64 * u;
    const int row = wv * RPW + ci / TL::NCH;
    const int byte = row * TL::RB + (ci % TL::NCH) * 16;
    const float w = __expf(glast - __shfl(gscan, row, 64));
    const uint4 raw = *reinterpret_cast<const uint4*>(k + byte);
    uint4 outv;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
      bf16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (bf16)((float)x[e] * w);
      outv = __builtin_bit_cast(uint4, y);
    } else {
      const f32x4 x = __builtin_bit_cast(f32x4, raw);
      outv = __builtin_bit_cast(uint4, x * w);
    }
    *reinterpret_cast<uint4*>(kd + byte) = outv;
  }
}

template <typename T, int D, int C>
__device__ __forceinline__ void issue_chunk(const PrefillArgs& a, int64_t row0, char* st, bool with_q, bool with_lam,
                                            int wv, int nw, int lane, int LS) {
  typedef Stage<T, D, C> S;
  const int64_t rs = (int64_t)a.H * D;
  if (with_q) tile_load_async<T, C, D>(static_cast<const T*>(a.q) + row0 * D, rs, st + S::QOFF, wv, nw, lane);
  tile_load_async<T, C, D>(static_cast<const T*>(a.k) + row0 * D, rs, st + S::KOFF, wv, nw, lane);
  tile_load_async<T, C, D>(static_cast<const T*>(a.v) + row0 * D, rs, st + S::VOFF, wv, nw, lane);
  const float* g = a.g + row0;
  scatter_load_async(reinterpret_cast<float*>(st + S::GOFF), C, wv, nw, lane,
                     [&](int f) { return g + (int64_t)f * a.H; });
  if (with_lam) {
    // lambda^T[l][r] = lambda[token r][l]
    const float* lam = a.lam + row0 * a.L;
    const int64_t ls = (int64_t)a.H * a.L;
    scatter_load_async(reinterpret_cast<float*>(st + S::LOFF), LS * C, wv, nw, lane,
                       [&](int f) { return lam + (f % C) * ls + f / C; });
  }
}

// ---------------------------------------------------------------------------
// ll_chunk_state: one workgroup per (block J, head), one wave per 16 state
// columns.  Writes S[bh, J] (tile layout) and GS[bh, J].
template <typename T, int D, int C>
__global__ void __launch_bounds__(64 * (D / 16)) ll_chunk_state(PrefillArgs a) {
  using M = Mma<T>;
  typedef Stage<T, D, C> S;
  typedef Tile<T, C, D> TL;
  constexpr int NW = D / 16;
  constexpr int DT = D / 16;
  constexpr int KSC = C / M::KS;
  __shared__ __attribute__((aligned(1024))) char smem[2 * S::BYTES + TL::BYTES];
  char* kd = smem + 2 * S::BYTES;  // decayed keys of the current chunk

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int J = wg % a.nb, bh = wg / a.nb, h = bh % a.H, b = bh / a.H;
  auto row_of = [&](int j) { return ((int64_t)b * a.T + (int64_t)(J * a.P + j) * C) * a.H + h; };

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float gblk = 0.f;

  issue_chunk<T, D, C>(a, row_of(0), smem, false, false, wv, NW, lane, 0);
  for (int j = 0; j < a.P; ++j) {
    char* st = smem + (j & 1) * S::BYTES;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk j have landed
    __syncthreads();                // every wave's loads have; chunk j-1 is done
    if (j + 1 < a.P) issue_chunk<T, D, C>(a, row_of(j + 1), smem + ((j + 1) & 1) * S::BYTES, false, false, wv, NW,
                                          lane, 0);
    const float gscan = chunk_prefix<C>(reinterpret_cast<const float*>(st + S::GOFF), lane);
    const float gsum = __shfl(gscan, C - 1, 64);
    decay_keys<T, D, C, NW>(st + S::KOFF, kd, gscan, wv, lane);
    __syncthreads();

    typename M::Frag vf[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(st + S::VOFF, 16 * wv, s, lane);
    const float carry = __expf(gsum);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 x = acc[dt] * carry;
#pragma unroll
      for (int s = 0; s < KSC; ++s) x = M::mma(frag_col<T, C, D>(kd, 16 * dt, s, lane), vf[s], x);
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
// n = this wave's 16 columns), alpha_r = lamT[lvl][r] * scale for the rows
// r = 16*rt + 4*(lane/16) + i this lane holds.
template <typename T, int D, int C>
__device__ __forceinline__ void level_read(f32x4 (&oacc)[C / 16],
                                           const typename Mma<T>::Frag (&qf)[C / 16][D / Mma<T>::KS],
                                           const typename Mma<T>::Frag (&nf)[D / Mma<T>::KS], const float* lamT,
                                           int lvl, float scale, int g4) {
  using M = Mma<T>;
  constexpr int CT = C / 16, KSD = D / M::KS;
#pragma unroll
  for (int rt = 0; rt < CT; ++rt) {
    f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSD; ++s) tmp = M::mma(qf[rt][s], nf[s], tmp);
    const f32x4 al = *reinterpret_cast<const f32x4*>(lamT + lvl * C + 16 * rt + 4 * g4);
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

// ---------------------------------------------------------------------------
// ll_chunk_attn: one workgroup per (block J, head); wave wv owns output
// columns [16 wv, 16 wv + 16); the P chunks of the block are visited in order.
// The Fenwick nodes of earlier blocks are the same for every chunk of the
// block: up to MAXH of them are converted once into MFMA B fragments in LDS,
// any further ones are read from the workspace per chunk.
template <typename T, int D, int C, int MAXB, int MAXH>
__global__ void __launch_bounds__(64 * (D / 16)) __attribute__((amdgpu_waves_per_eu(2, 2))) ll_chunk_attn(PrefillArgs a) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef Stage<T, D, C> S;
  typedef Tile<T, C, D> TL;
  typedef Tile<T, C, C> PT;  // masked scores P[r][s]
  constexpr int NW = D / 16;
  constexpr int DT = D / 16, CT = C / 16;
  constexpr int KSD = D / M::KS, KSC = C / M::KS;
  constexpr int LOGC = (C == 16) ? 4 : (C == 32) ? 5 : 6;
  constexpr int FRAG_BYTES = 64 * (int)sizeof(Frag);     // one fragment of one wave
  constexpr int NODE_BYTES = NW * KSD * FRAG_BYTES;       // one node, every wave's columns
  constexpr int HOFF = 2 * S::BYTES + TL::BYTES + PT::BYTES;
  constexpr int GOFF = HOFF + (MAXH > 0 ? MAXH : 0) * NODE_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[GOFF + NW * C * 4];
  char* kd = smem + 2 * S::BYTES;
  char* pt = kd + TL::BYTES;
  char* hbuf = smem + HOFF;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g4 = lane >> 4, q16 = lane & 15;
  float* gl = reinterpret_cast<float*>(smem + GOFF) + wv * C;  // this wave's copy of G
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int J = wg % a.nb, bh = wg / a.nb, h = bh % a.H, b = bh / a.H;
  const int logP = ilog2c(a.P);
  const int LS = a.LS;
  auto row_of = [&](int j) { return ((int64_t)b * a.T + (int64_t)(J * a.P + j) * C) * a.H + h; };
  auto node_of = [&](int e) {
    return (e & 1) ? a.F + ((int64_t)bh * a.nF + (e >> 1)) * D * D : a.S + ((int64_t)bh * a.nb + e) * D * D;
  };
  auto gamma_of = [&](int e) { return (e & 1) ? a.GF[(int64_t)bh * a.nF + (e >> 1)] : a.GS[(int64_t)bh * a.nb + e]; };

  issue_chunk<T, D, C>(a, row_of(0), smem, true, true, wv, NW, lane, LS);

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
    char* st = smem + (j & 1) * S::BYTES;
    const float* lamT = reinterpret_cast<const float*>(st + S::LOFF);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < a.P)
      issue_chunk<T, D, C>(a, row_of(j + 1), smem + ((j + 1) & 1) * S::BYTES, true, true, wv, NW, lane, LS);

    const float gscan = chunk_prefix<C>(reinterpret_cast<const float*>(st + S::GOFF), lane);
    if (lane < C) gl[lane] = gscan;
    const float gsum = __shfl(gscan, C - 1, 64);

    Frag qf[CT][KSD];
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
#pragma unroll
      for (int s = 0; s < KSD; ++s) qf[rt][s] = frag_row<T, C, D>(st + S::QOFF, 16 * rt + q16, s, g4);

    // --- intra-chunk scores, this wave's share of the causal tiles:
    // P[r][s] = (q_r . k_s) lambda_r^(lev(r,s)) exp(G[r] - G[s]), s <= r
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
#pragma unroll
      for (int ct = 0; ct <= rt; ++ct) {  // ct: source tile (column of P)
        if ((rt * (rt + 1) / 2 + ct) % NW != wv) continue;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSD; ++s) x = M::mma(frag_row<T, C, D>(st + S::KOFF, 16 * ct + q16, s, g4), qf[rt][s], x);
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
            val = x[i] * lamT[lev * C + r] * __expf(gr - gs[i]);
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

    // --- decayed keys for this chunk's state, and lambda of the inter-chunk
    // levels pre-multiplied by exp(G[r]) (in place; levels <= log2 C untouched)
    decay_keys<T, D, C, NW>(st + S::KOFF, kd, gscan, wv, lane);
    {
      float* lw = reinterpret_cast<float*>(st + S::LOFF);
      const float eg = __expf(gl[lane & (C - 1)]);
      const int n = (LS - LOGC - 1) * C;
      for (int x = tid; x < n; x += 64 * NW) lw[(LOGC + 1) * C + x] *= eg;
    }
    __syncthreads();

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
        level_read<T, D, C>(oacc, qf, nf, lamT, LOGC + m, __expf(sig[m]), g4);
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
        level_read<T, D, C>(oacc, qf, nf, lamT, LOGC + logP + l + 1, __expf(gw + dd), g4);
        dd += gamma_of(e);
        rest &= rest - 1;
      }
    }

    // --- intra-chunk: O += P V for this wave's columns
    Frag vf[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = frag_col<T, C, D>(st + S::VOFF, 16 * wv, s, lane);
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
      f32x4 merged[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSC; ++s) x = M::mma(frag_col<T, C, D>(kd, 16 * dt, s, lane), vf[s], x);
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
  const int grid = a.B * a.H * a.nb;
  // node fragments kept in LDS: bf16 heads up to 64 (8 KB per node at d=64)
  constexpr int MAXH = 0;
  hipLaunchKernelGGL((ll_chunk_attn<T, D, C, max_block_depth(D), MAXH>), dim3(grid), dim3(64 * (D / 16)), 0, s, a);
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
