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
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

template <typename T, int D, int C>
struct AttnSmem {
  ChunkTiles<T, D, C> c;
  T o[C][D + 4];
};

// ---------------------------------------------------------------------------
// ll_chunk_state: one workgroup per (block J, head), one wave per 16 output
// columns.  Writes S[bh, J] (tile layout) and GS[bh, J].
template <typename T, int D, int C>
__global__ void __launch_bounds__(64 * (D / 16)) ll_chunk_state(PrefillArgs a) {
  using M = Mma<T>;
  constexpr int NTH = 64 * (D / 16);
  constexpr int DT = D / 16;
  constexpr int KSC = C / M::KS;
  __shared__ __attribute__((aligned(16))) ChunkTiles<T, D, C> sm;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int J = wg % a.nb, bh = wg / a.nb, h = bh % a.H, b = bh / a.H;
  const int64_t rs = (int64_t)a.H * D;

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float gblk = 0.f;

  for (int j = 0; j < a.P; ++j) {
    const int64_t tok0 = (int64_t)(J * a.P + j) * C;
    const int64_t row0 = ((int64_t)b * a.T + tok0) * a.H + h;  // (b, tok0, h)
    stage_rows<T, D, C, ChunkTiles<T, D, C>::RP, ChunkTiles<T, D, C>::TP>(
        static_cast<const T*>(a.k) + row0 * D, rs, nullptr, sm.kt, tid, NTH);
    stage_rows<T, D, C, ChunkTiles<T, D, C>::RP, ChunkTiles<T, D, C>::TP>(
        static_cast<const T*>(a.v) + row0 * D, rs, nullptr, sm.vt, tid, NTH);
    for (int x = tid; x < C; x += NTH) sm.gcum[x] = a.g[row0 + (int64_t)x * a.H];
    __syncthreads();
    if (wv == 0) chunk_gate_prefix<C>(sm.gcum, sm.wend, lane);
    __syncthreads();

    const float gsum = sm.gcum[C - 1];
    const float carry = __expf(gsum);
    typename M::Frag vf[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = M::row_frag(sm.vt[16 * wv + l16], s, g4);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 x = acc[dt] * carry;
#pragma unroll
      for (int s = 0; s < KSC; ++s) x = M::mma(M::row_frag_scaled(sm.kt[16 * dt + l16], sm.wend, s, g4), vf[s], x);
      acc[dt] = x;
    }
    gblk += gsum;
    __syncthreads();
  }

  float* dst = a.S + ((int64_t)bh * a.nb + J) * D * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + state_tile_offset<D>(dt, wv, lane)) = acc[dt];
  if (tid == 0) a.GS[(int64_t)bh * a.nb + J] = gblk;
}

// Adds diag(alpha) (Q N) to oacc, where N is a dk x dv state given as this
// wave's column of 16x16 accumulator-order tiles, and
// alpha_r = lambda[r][lvl] * exp(G[r] + off).
template <typename T, int D, int C>
__device__ __forceinline__ void level_read(f32x4 (&oacc)[C / 16], const typename Mma<T>::Frag (&qf)[C / 16][D / Mma<T>::KS],
                                           const f32x4 (&node)[D / 16], const float* lam, int LS, const float* gcum,
                                           int lvl, float off, int g4) {
  using M = Mma<T>;
  constexpr int CT = C / 16, KSD = D / M::KS;
  f32x4 tmp[CT];
#pragma unroll
  for (int rt = 0; rt < CT; ++rt) tmp[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KSD; ++s) {
    const typename M::Frag bf = M::acc_frag(node, s);
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) tmp[rt] = M::mma(qf[rt][s], bf, tmp[rt]);
  }
#pragma unroll
  for (int rt = 0; rt < CT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * g4 + i;
      oacc[rt][i] += lam[r * LS + lvl] * __expf(gcum[r] + off) * tmp[rt][i];
    }
  }
}

// ---------------------------------------------------------------------------
// ll_chunk_attn: one workgroup per (block J, head); one wave per 16 output
// columns; the P chunks of the block are visited in order.
template <typename T, int D, int C, int MAXB>
__global__ void __launch_bounds__(64 * (D / 16)) ll_chunk_attn(PrefillArgs a) {
  using M = Mma<T>;
  typedef ChunkTiles<T, D, C> Tiles;
  constexpr int NTH = 64 * (D / 16);
  constexpr int DT = D / 16, CT = C / 16;
  constexpr int KSD = D / M::KS, KSC = C / M::KS;
  constexpr int LOGC = (C == 16) ? 4 : (C == 32) ? 5 : 6;
  __shared__ __attribute__((aligned(16))) AttnSmem<T, D, C> smem;
  Tiles& sm = smem.c;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int J = wg % a.nb, bh = wg / a.nb, h = bh % a.H, b = bh / a.H;
  const int logP = ilog2c(a.P);
  const int LS = a.LS;
  const int64_t rs = (int64_t)a.H * D;

  // within-block Fenwick levels 1..MAXB (chunk granularity) of this wave's
  // output columns; true state = exp(sig[m]) * nst[m-1]
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
    const int64_t tok0 = (int64_t)(J * a.P + j) * C;
    const int64_t row0 = ((int64_t)b * a.T + tok0) * a.H + h;
    stage_rows<T, D, C, Tiles::RP, Tiles::TP>(static_cast<const T*>(a.q) + row0 * D, rs, sm.q, nullptr, tid, NTH);
    stage_rows<T, D, C, Tiles::RP, Tiles::TP>(static_cast<const T*>(a.k) + row0 * D, rs, sm.k, sm.kt, tid, NTH);
    stage_rows<T, D, C, Tiles::RP, Tiles::TP>(static_cast<const T*>(a.v) + row0 * D, rs, nullptr, sm.vt, tid, NTH);
    for (int x = tid; x < C * LS; x += NTH) {
      const int r = x / LS, l = x - r * LS;
      sm.lam[x] = a.lam[(row0 + (int64_t)r * a.H) * a.L + l];
    }
    for (int x = tid; x < C; x += NTH) sm.gcum[x] = a.g[row0 + (int64_t)x * a.H];
    __syncthreads();
    if (wv == 0) chunk_gate_prefix<C>(sm.gcum, sm.wend, lane);
    __syncthreads();

    typename M::Frag qf[CT][KSD];
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
#pragma unroll
      for (int s = 0; s < KSD; ++s) qf[rt][s] = M::row_frag(sm.q[16 * rt + l16], s, g4);
    typename M::Frag vf[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) vf[s] = M::row_frag(sm.vt[16 * wv + l16], s, g4);

    f32x4 oacc[CT];
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) oacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // --- intra-chunk levels 0..LOGC: P = (K Q^T)^T masked, then P V
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) {
      f32x4 st[CT];
      const int r = 16 * rt + l16;
      const float gr = sm.gcum[r];
#pragma unroll
      for (int tt = 0; tt < CT; ++tt) {
        st[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tt <= rt) {
          f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KSD; ++s) x = M::mma(M::row_frag(sm.k[16 * tt + l16], s, g4), qf[rt][s], x);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int src = 16 * tt + 4 * g4 + i;
            float val = 0.f;
            if (src <= r) {
              const int lev = (src == r) ? 0 : 32 - __clz(r ^ src);
              val = x[i] * sm.lam[r * LS + lev] * __expf(gr - sm.gcum[src]);
            }
            st[tt][i] = val;
          }
        }
      }
#pragma unroll
      for (int s = 0; s < KSC; ++s)
        if (M::first_tile(s) <= rt) oacc[rt] = M::mma(M::acc_frag(st, s), vf[s], oacc[rt]);
    }

    // --- within-block levels LOGC+1 .. LOGC+logP
#pragma unroll
    for (int m = 1; m <= MAXB; ++m)
      if (m <= logP && ((j >> (m - 1)) & 1))
        level_read<T, D, C>(oacc, qf, nst[m - 1], sm.lam, LS, sm.gcum, LOGC + m, sig[m], g4);

    // --- earlier blocks: Fenwick nodes of the block index, most recent first
    {
      int rest = J;
      float dd = 0.f;  // log-decay from the node's end to the start of block J
      while (rest > 0) {
        const int e = rest - 1;
        const int l = __ffs(rest) - 1;
        const float* node;
        float gam;
        if (e & 1) {
          node = a.F + ((int64_t)bh * a.nF + (e >> 1)) * D * D;
          gam = a.GF[(int64_t)bh * a.nF + (e >> 1)];
        } else {
          node = a.S + ((int64_t)bh * a.nb + e) * D * D;
          gam = a.GS[(int64_t)bh * a.nb + e];
        }
        f32x4 nt[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) nt[dt] = *reinterpret_cast<const f32x4*>(node + state_tile_offset<D>(dt, wv, lane));
        level_read<T, D, C>(oacc, qf, nt, sm.lam, LS, sm.gcum, LOGC + logP + l + 1, gw + dd, g4);
        dd += gam;
        rest &= rest - 1;
      }
    }

    // --- output tile to LDS
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) smem.o[16 * rt + 4 * g4 + i][16 * wv + l16] = from_f32<T>(oacc[rt][i]);

    // --- this chunk's own decayed key-value state (this wave's columns)
    f32x4 hacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSC; ++s) x = M::mma(M::row_frag_scaled(sm.kt[16 * dt + l16], sm.wend, s, g4), vf[s], x);
      hacc[dt] = x;
    }
    const float gsum = sm.gcum[C - 1];
    __syncthreads();

    // --- store the output rows (16-byte vectors)
    {
      constexpr int EPV = 16 / sizeof(T), VPR = D / EPV;
      T* dst = static_cast<T*>(a.o) + row0 * D;
      for (int vi = tid; vi < C * VPR; vi += NTH) {
        const int r = vi / VPR, c0 = (vi % VPR) * EPV;
        const uint2* s2 = reinterpret_cast<const uint2*>(&smem.o[r][c0]);
        const uint2 lo = s2[0], hi = s2[1];
        *reinterpret_cast<uint4*>(dst + r * rs + c0) = uint4{lo.x, lo.y, hi.x, hi.y};
      }
    }

    // --- advance the within-block Fenwick state past chunk j (merge rule:
    // levels 1..c plus the new chunk become level c+1, c = ctz(j+1))
#pragma unroll
    for (int m = 1; m <= MAXB; ++m) sig[m] += gsum;
    gw += gsum;
    if (j + 1 < a.P) {
      const int c = __ffs(j + 1) - 1;
      f32x4 merged[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) merged[dt] = hacc[dt];
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
    __syncthreads();
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
  hipLaunchKernelGGL((ll_chunk_attn<T, D, C, max_block_depth(D)>), dim3(grid), dim3(64 * (D / 16)), 0, s, a);
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
