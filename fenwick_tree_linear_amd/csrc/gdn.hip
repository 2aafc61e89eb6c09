// gdn.hip -- the Gated DeltaNet write of the log-linear read ("Log-Linear
// Attention", section 3: Gated DeltaNet keeps its own structure and the
// hierarchical mask multiplies the read).
//
// With the gated delta rule every token writes its pseudo-value
//   u_t = beta_t (v_t - sum_{s<t} e^{G_t - G_s} (k_t . k_s) u_s)
// (G the prefix of the log-gates), and the output is the log-linear read of
// (q, k, u): the Mamba-2 pipeline runs unchanged with v replaced by u.  Per
// chunk i of C tokens, with G_r the in-chunk inclusive prefix and
// S_i = sum_{s < iC} e^{G_{iC-1} - G_s} k_s u_s^T the plain gated state at the
// chunk start:
//   (I + L) U = diag(beta) V - diag(beta e^G) K S_i,
//   L[r][s] = beta_r e^{G_r - G_s} (k_r . k_s) for s < r, 0 otherwise,
// so U = U' - W S_i with U' = (I + L)^-1 diag(beta) V and
// W = (I + L)^-1 diag(beta e^G) K (the WY form), and
//   S_{i+1} = e^{g_i} S_i + sum_r e^{g_i - G_r} k_r u_r^T   (g_i = G_{C-1}).
//
// ll_gdn_wy    : one workgroup per (chunk, head): L on MFMA, (I + L)^-1 by
//                16x16 blocks on fp32 MFMA, then U' and W as MFMA products.
// ll_gdn_state : one workgroup per (head, 16 state columns): the serial pass
//                over the chunks, U = U' - W S_i and the state update on MFMA,
//                writing the pseudo-values U.
#include <type_traits>

#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// ---------------------------------------------------------------------------
// ll_gdn_wy: one workgroup of four waves per (chunk, head).
//   1. K rows land in LDS (direct loads); wave 0 scans the gates.  V is
//      loaded only for step 4, into the space of L (at d = 128 and C = 64 this
//      keeps the workgroup at 51 KB of LDS: three per CU instead of two).
//   2. L: the causal 16x16 tiles of K K^T on MFMA, weighted by
//      beta_r e^{G_r - G_s} and masked to s < r, fp32 in LDS.
//   3. T = (I + L)^-1 by blocks of 16: the diagonal blocks by forward
//      substitution (one lane per column), then the blocks below by
//      T_ij = -T_ii sum_{j<=k<i} L_ik T_kj, one block distance at a time, on
//      fp32 MFMA.
//   4. W^T = K^T (T diag(beta e^G))^T and U'^T = V^T (T diag(beta))^T on MFMA,
//      each lane ending with four consecutive features of one token.  For
//      bf16 io the scaled T is split into a bf16 head and a bf16 remainder,
//      so that the products keep T to about 16 bits.
template <typename T, int D, int C>
struct WySmem {
  typedef Tile<T, C, D> TL;
  static constexpr int TS = C + 4;  // fp32 row stride of L and T (16-byte rows, rows 4 banks apart)
  static constexpr int LREG = ((C * TS * 4 > TL::BYTES ? C * TS * 4 : TL::BYTES) + 1023) / 1024 * 1024;
  static constexpr int KOFF = 0;
  static constexpr int LOFF = TL::BYTES;  // L [C][TS] fp32; V lands here once L is no longer read
  static constexpr int VOFF = LOFF;
  static constexpr int TOFF = LOFF + LREG;  // T [C][TS] fp32
  static constexpr int GOFF = TOFF + C * TS * 4;  // G [C]
  static constexpr int BOFF = GOFF + C * 4;        // beta [C]
  static constexpr int SOFF = BOFF + C * 4;        // beta e^G [C]
  static constexpr int BYTES = SOFF + C * 4;
  static constexpr int NW = 4;
};

// C += X Y for 16x16 fp32 blocks X, Y in LDS (row strides in floats), on
// the fp32 MFMA; the result is in accumulator layout (lane: rows 4 (lane/16)
// + e of column lane%16).
__device__ __forceinline__ f32x4 mm16(const float* X, int xs, const float* Y, int ys, f32x4 c, int q16, int g4) {
  const f32x4 xa = *reinterpret_cast<const f32x4*>(X + q16 * xs + 4 * g4);
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[s], Y[(4 * g4 + s) * ys + q16], c, 0, 0, 0);
  return c;
}

template <typename T, int D, int C>
__global__ void __launch_bounds__(256) ll_gdn_wy(GdnArgs a) {
  using M = Mma<T>;
  typedef WySmem<T, D, C> SM;
  typedef Tile<T, C, D> TL;
  typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type Vec4;
  constexpr int NW = SM::NW, CT = C / 16, DT = D / 16, KSD = D / M::KS, TS = SM::TS;
  __shared__ __attribute__((aligned(1024))) char smem[SM::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, q16 = lane & 15;
  const int nc = a.T / C;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int i = wg % nc, bh = wg / nc, h = bh % a.H, b = bh / a.H;
  const int64_t row0 = ((int64_t)b * a.T + (int64_t)i * C) * a.H + h;  // row of the chunk's first token
  float* Lm = reinterpret_cast<float*>(smem + SM::LOFF);
  float* Tm = reinterpret_cast<float*>(smem + SM::TOFF);
  float* gl = reinterpret_cast<float*>(smem + SM::GOFF);
  float* bl = reinterpret_cast<float*>(smem + SM::BOFF);
  float* sl = reinterpret_cast<float*>(smem + SM::SOFF);

  // 1. K and V tiles; gates and write strengths
  {
    ChunkLoads<T, D, C, NW> ld;
    ld.init(wv, lane, a.H, 1, 1);
    ld.tiles(a.k, row0, smem + SM::KOFF, wv);
  }
  if (wv == 0) {
    const float G = chunk_scan<C>(lane < C ? a.g[row0 + (int64_t)lane * a.H] : 0.f);
    if (lane < C) {
      const float bt = a.beta[row0 + (int64_t)lane * a.H];
      gl[lane] = G;
      bl[lane] = bt;
      sl[lane] = bt * __expf(G);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 2. L[r][s] = beta_r e^{G_r - G_s} (k_r . k_s) for s < r; lane: row r =
  // 16 rt + lane%16, sources 16 ct + 4 (lane/16) + e
  for (int t = wv; t < CT * (CT + 1) / 2; t += NW) {
    int rt = 0;
#pragma unroll
    for (int u = 1; u < CT; ++u) rt += (t >= u * (u + 1) / 2) ? 1 : 0;
    const int ct = t - rt * (rt + 1) / 2;
    const int r = 16 * rt + q16;
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSD; ++s)
      x = M::mma(frag_row<T, C, D>(smem + SM::KOFF, 16 * ct + q16, s, g4),
                 frag_row<T, C, D>(smem + SM::KOFF, r, s, g4), x);
    const float br = bl[r], gr = gl[r];
    const f32x4 gs = *reinterpret_cast<const f32x4*>(gl + 16 * ct + 4 * g4);
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (16 * ct + 4 * g4 + e < r) ? br * __expf(gr - gs[e]) * x[e] : 0.f;
    *reinterpret_cast<f32x4*>(Lm + r * TS + 16 * ct + 4 * g4) = y;
  }
  __syncthreads();

  // 3a. diagonal blocks T_ww = (I + L_ww)^-1, lane column c = lane%16 (the
  // four lane groups compute the same column; each writes four rows).  A
  // wave with an even block also zeroes the block to its right, which the
  // 32-wide MFMA steps below read.
  if (wv < CT) {
    const float* Lb = Lm + 16 * wv * TS + 16 * wv;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == q16) ? 1.f : 0.f;
#pragma unroll
      for (int s4 = 0; s4 < r; s4 += 4) {
        const f32x4 l = *reinterpret_cast<const f32x4*>(Lb + r * TS + s4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (s4 + e < r) acc -= l[e] * x[s4 + e];
      }
      x[r] = acc;
    }
    float* Tb = Tm + 16 * wv * TS + 16 * wv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Tb[(4 * g4 + e) * TS + q16] = x[4 * g4 + e];
      if ((wv & 1) == 0 && wv + 1 < CT) Tb[(4 * g4 + e) * TS + 16 + q16] = 0.f;
    }
  }
  __syncthreads();

  // 3b. blocks below the diagonal, by distance d: T_ij = -T_ii sum_k L_ik T_kj
  for (int d = 1; d < CT; ++d) {
    if (wv < CT - d) {
      const int bi = wv + d, bj = wv;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k = bj; k < bi; ++k) acc = mm16(Lm + 16 * bi * TS + 16 * k, TS, Tm + 16 * k * TS + 16 * bj, TS, acc, q16, g4);
      float* Tij = Tm + 16 * bi * TS + 16 * bj;
#pragma unroll
      for (int e = 0; e < 4; ++e) Tij[(4 * g4 + e) * TS + q16] = acc[e];  // the sum, read back just below
      f32x4 y = mm16(Tm + 16 * bi * TS + 16 * bi, TS, Tij, TS, f32x4{0.f, 0.f, 0.f, 0.f}, q16, g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) Tij[(4 * g4 + e) * TS + q16] = -y[e];
    }
    __syncthreads();
  }

  {
    ChunkLoads<T, D, C, NW> ld;
    ld.init(wv, lane, a.H, 1, 1);
    ld.tiles(a.v, row0, smem + SM::VOFF, wv);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 4. outputs: wave w takes token tile w % CT and every (NW/CT)-th column
  // tile; lane: token r = 16 tt + lane%16, features 16 nt + 4 (lane/16) + e
  constexpr int WPT = NW / CT;  // waves per token tile
  const int tt = wv % CT, r = 16 * tt + q16;
  T* Wg = static_cast<T*>(a.W);
  T* Ug = static_cast<T*>(a.Up);
  if constexpr (sizeof(T) == 2) {
    constexpr int KSC = C / 32;
    const int nks = tt / 2 + 1;  // 32-token steps that reach token tile tt
    bf16x8 uh[KSC], ul[KSC], wh[KSC], wl[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) {
      if (s < nks) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int k0 = 32 * s + 16 * half + 4 * g4;
          const f32x4 tv = *reinterpret_cast<const f32x4*>(Tm + r * TS + k0);
          const f32x4 bv = *reinterpret_cast<const f32x4*>(bl + k0);
          const f32x4 sv = *reinterpret_cast<const f32x4*>(sl + k0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float u = tv[e] * bv[e], w = tv[e] * sv[e];
            const bf16 u0 = (bf16)u, w0 = (bf16)w;
            uh[s][4 * half + e] = u0;
            ul[s][4 * half + e] = (bf16)(u - (float)u0);
            wh[s][4 * half + e] = w0;
            wl[s][4 * half + e] = (bf16)(w - (float)w0);
          }
        }
      }
    }
    for (int nt = wv / CT; nt < DT; nt += WPT) {
      bf16x8 kf[KSC], vf[KSC];
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        kf[s] = frag_col<T, C, D>(smem + SM::KOFF, 16 * nt, s, lane);
        vf[s] = frag_col<T, C, D>(smem + SM::VOFF, 16 * nt, s, lane);
      }
      lds_wait(kf, vf);
      f32x4 ow = f32x4{0.f, 0.f, 0.f, 0.f}, ou = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (s < nks) {
          ow = M::mma(kf[s], wh[s], ow);
          ow = M::mma(kf[s], wl[s], ow);
          ou = M::mma(vf[s], uh[s], ou);
          ou = M::mma(vf[s], ul[s], ou);
        }
      }
      const int64_t o = (row0 + (int64_t)r * a.H) * D + 16 * nt + 4 * g4;
      *reinterpret_cast<Vec4*>(Wg + o) = Vec4{(T)ow[0], (T)ow[1], (T)ow[2], (T)ow[3]};
      *reinterpret_cast<Vec4*>(Ug + o) = Vec4{(T)ou[0], (T)ou[1], (T)ou[2], (T)ou[3]};
    }
  } else {
    constexpr int KSC = C / 4;
    const int nks = 4 * (tt + 1);  // 4-token steps that reach token tile tt
    float ub[KSC], wb[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) {
      const int k = M::kidx(s, g4, 0);
      ub[s] = Tm[r * TS + k] * bl[k];
      wb[s] = Tm[r * TS + k] * sl[k];
    }
    for (int nt = wv / CT; nt < DT; nt += WPT) {
      f32x4 ow = f32x4{0.f, 0.f, 0.f, 0.f}, ou = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (s < nks) {
          ow = M::mma(frag_col<T, C, D>(smem + SM::KOFF, 16 * nt, s, lane), wb[s], ow);
          ou = M::mma(frag_col<T, C, D>(smem + SM::VOFF, 16 * nt, s, lane), ub[s], ou);
        }
      }
      const int64_t o = (row0 + (int64_t)r * a.H) * D + 16 * nt + 4 * g4;
      *reinterpret_cast<Vec4*>(Wg + o) = ow;
      *reinterpret_cast<Vec4*>(Ug + o) = ou;
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, int C>
struct GstSmem {
  typedef Tile<T, C, D> TL;
  typedef Tile<T, C, 16> UL;
  typedef typename Mma<T>::Frag Frag;
  static constexpr int NW = C / 16, KSD = D / Mma<T>::KS;
  static constexpr int WOFF = 0, KOFF = TL::BYTES, STAGE = 2 * TL::BYTES;  // W and K tiles, two stages
  static constexpr int UOFF = 2 * STAGE;                                   // U of this slice [C][16]
  static constexpr int SFOFF = UOFF + UL::BYTES;                           // S as B fragments [KSD][64]
  static constexpr int WLOFF = SFOFF + KSD * 64 * (int)sizeof(Frag);        // per wave e^{g - G} [NW][C]
  static constexpr int BYTES = WLOFF + NW * C * 4;
};

template <typename T, int D, int C>
__global__ void __launch_bounds__(64 * (C / 16)) ll_gdn_state(GdnArgs a) {
  using M = Mma<T>;
  typedef GstSmem<T, D, C> SM;
  typedef typename M::Frag Frag;
  typedef Tile<T, C, D> TL;
  typedef Tile<T, C, 16> UL;
  constexpr int NW = SM::NW, DT = D / 16, KSD = SM::KSD, KSC = C / M::KS;
  constexpr int ODT = (DT + NW - 1) / NW;  // state tiles owned per wave (at most)
  __shared__ __attribute__((aligned(1024))) char smem[SM::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, q16 = lane & 15;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int slice = wg % DT, bh = wg / DT, h = bh % a.H, b = bh / a.H;
  const int n0 = 16 * slice;
  const int nc = a.T / C;
  auto row_of = [&](int i) { return ((int64_t)b * a.T + (int64_t)i * C) * a.H + h; };
  Frag* sf = reinterpret_cast<Frag*>(smem + SM::SFOFF);
  float* wl = reinterpret_cast<float*>(smem + SM::WLOFF) + wv * C;
  char* ut = smem + SM::UOFF;

  ChunkLoads<T, D, C, NW> ld;
  ld.init(wv, lane, a.H, 1, 1);
  auto issue = [&](int i) {
    char* st = smem + (i & 1) * SM::STAGE;
    ld.tiles(a.W, row_of(i), st + SM::WOFF, wv);
    ld.tiles(a.k, row_of(i), st + SM::KOFF, wv);
  };
  // this wave's rows 16 wv + 4 (lane/16) + e of U' (column n0 + lane%16), and the gate of row lane
  T upn[4];
  float gn = 0.f;
  auto fetch = [&](int i) {
    const T* up = static_cast<const T*>(a.Up);
#pragma unroll
    for (int e = 0; e < 4; ++e) upn[e] = up[(row_of(i) + (int64_t)(16 * wv + 4 * g4 + e) * a.H) * D + n0 + q16];
    gn = lane < C ? a.g[row_of(i) + (int64_t)lane * a.H] : 0.f;
  };

  // S_0: zero, or after a prior state the plain gated state of [0, pos0),
  // the sum of its levels' true states (the buckets partition the prefix)
  f32x4 st[ODT];
#pragma unroll
  for (int o = 0; o < ODT; ++o) st[o] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.pos0 > 0) {
    const float* Sh = a.state_in + (int64_t)bh * a.L * D * D;
    const float* sg = a.state_in + (int64_t)a.B * a.H * a.L * D * D + (int64_t)bh * a.L;
    for (uint64_t bits = (uint64_t)a.pos0; bits; bits &= bits - 1) {
      const int lvl = __ffsll((unsigned long long)bits);
      const float sc = __expf(sg[lvl]);
#pragma unroll
      for (int o = 0; o < ODT; ++o) {
        const int dt = wv + o * NW;
        if (dt >= DT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) st[o][e] += sc * Sh[(int64_t)lvl * D * D + (16 * dt + 4 * g4 + e) * D + n0 + q16];
      }
    }
  }
  for (int x = tid; x < KSD * 64; x += 64 * NW) sf[x] = Frag{};
  if (a.pos0 > 0) {
    __syncthreads();  // the zero fill is complete before the tiles are published into it
#pragma unroll
    for (int o = 0; o < ODT; ++o) {
      const int dt = wv + o * NW;
      if (dt >= DT) continue;
      if constexpr (sizeof(T) == 2) {
        bf16* f = reinterpret_cast<bf16*>(&sf[(dt >> 1) * 64 + lane]) + 4 * (dt & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = (bf16)st[o][e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) reinterpret_cast<float*>(sf)[(4 * dt + e) * 64 + lane] = st[o][e];
      }
    }
  }

  issue(0);
  fetch(0);
  for (int i = 0; i < nc; ++i) {
    const char* stg = smem + (i & 1) * SM::STAGE;
    T up[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) up[e] = upn[e];
    const float gv = gn;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk i (and its U' rows) have landed
    lds_barrier();                  // every wave's have; S_i is in sf; chunk i-1 is done everywhere
    if (i + 1 < nc) {
      issue(i + 1);
      fetch(i + 1);
    }
    const float G = chunk_scan<C>(gv);
    const float gsum = __shfl(G, C - 1, 64);
    if (lane < C) wl[lane] = __expf(gsum - G);

    // U rows of this wave: U' - W S_i
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSD; ++s) x = M::mma(frag_row<T, C, D>(stg + SM::WOFF, 16 * wv + q16, s, g4), sf[s * 64 + lane], x);
    T* ug = static_cast<T*>(a.U);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * wv + 4 * g4 + e;
      const T u = from_f32<T>(to_f32(up[e]) - x[e]);
      ug[(row_of(i) + (int64_t)r * a.H) * D + n0 + q16] = u;
      *reinterpret_cast<T*>(ut + UL::off(r, q16)) = u;
    }
    lds_barrier();  // U of the chunk complete

    // S_{i+1} = e^{g} S_i + K^T diag(e^{g - G}) U for the state tiles this wave owns
    Frag uf[KSC];
#pragma unroll
    for (int s = 0; s < KSC; ++s) uf[s] = frag_col<T, C, 16>(ut, 0, s, lane);
    Frag kf[ODT][KSC];
#pragma unroll
    for (int o = 0; o < ODT; ++o) {
      const int dt = wv + o * NW;
      if (dt < DT)
#pragma unroll
        for (int s = 0; s < KSC; ++s) kf[o][s] = frag_col<T, C, D>(stg + SM::KOFF, 16 * dt, s, lane);
    }
    lds_wait(uf, kf);
#pragma unroll
    for (int s = 0; s < KSC; ++s) uf[s] = scale_tokens<T>(uf[s], wl, s, g4);
    const float carry = __expf(gsum);
#pragma unroll
    for (int o = 0; o < ODT; ++o) {
      const int dt = wv + o * NW;
      if (dt >= DT) continue;
      f32x4 y = st[o] * carry;
#pragma unroll
      for (int s = 0; s < KSC; ++s) y = M::mma(kf[o][s], uf[s], y);
      st[o] = y;
      // publish the tile as part of the B fragments of S (k = state row d)
      if constexpr (sizeof(T) == 2) {
        bf16* f = reinterpret_cast<bf16*>(&sf[(dt >> 1) * 64 + lane]) + 4 * (dt & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = (bf16)y[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) reinterpret_cast<float*>(sf)[(4 * dt + e) * 64 + lane] = y[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, int C>
static hipError_t launch_wy_t(const GdnArgs& a, hipStream_t s) {
  const int grid = a.B * a.H * (a.T / C);
  hipLaunchKernelGGL((ll_gdn_wy<T, D, C>), dim3(grid), dim3(64 * WySmem<T, D, C>::NW), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D, int C>
static hipError_t launch_gst_t(const GdnArgs& a, hipStream_t s) {
  const int grid = a.B * a.H * (D / 16);
  hipLaunchKernelGGL((ll_gdn_state<T, D, C>), dim3(grid), dim3(64 * (C / 16)), 0, s, a);
  return hipGetLastError();
}

#define LL_GDN_DISPATCH(FN)                                                    \
  if (io == 1) {                                                               \
    switch (D * 1000 + C) {                                                    \
      case 32032: return FN<bf16, 32, 32>(a, s);                               \
      case 32064: return FN<bf16, 32, 64>(a, s);                               \
      case 64032: return FN<bf16, 64, 32>(a, s);                               \
      case 64064: return FN<bf16, 64, 64>(a, s);                               \
      case 128032: return FN<bf16, 128, 32>(a, s);                             \
      case 128064: return FN<bf16, 128, 64>(a, s);                             \
      default: return hipErrorInvalidValue;                                    \
    }                                                                          \
  } else {                                                                     \
    switch (D * 1000 + C) {                                                    \
      case 16016: return FN<float, 16, 16>(a, s);                              \
      case 16032: return FN<float, 16, 32>(a, s);                              \
      case 16064: return FN<float, 16, 64>(a, s);                              \
      case 32016: return FN<float, 32, 16>(a, s);                              \
      case 32032: return FN<float, 32, 32>(a, s);                              \
      case 32064: return FN<float, 32, 64>(a, s);                              \
      case 64016: return FN<float, 64, 16>(a, s);                              \
      case 64032: return FN<float, 64, 32>(a, s);                              \
      case 64064: return FN<float, 64, 64>(a, s);                              \
      default: return hipErrorInvalidValue;                                    \
    }                                                                          \
  }

hipError_t launch_gdn_wy(int io, int D, int C, const GdnArgs& a, hipStream_t s) { LL_GDN_DISPATCH(launch_wy_t) }

hipError_t launch_gdn_state(int io, int D, int C, const GdnArgs& a, hipStream_t s) { LL_GDN_DISPATCH(launch_gst_t) }

}  // namespace llattn
