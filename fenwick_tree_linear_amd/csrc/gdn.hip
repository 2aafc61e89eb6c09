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
// ll_gdn_wy    : one workgroup per (chunk, head): L on MFMA, then U' and W by
//                forward substitution, one thread per column of [V | K].
// ll_gdn_state : one workgroup per (head, 16 state columns): the serial pass
//                over the chunks, U = U' - W S_i and the state update on MFMA,
//                writing the pseudo-values U.
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// ---------------------------------------------------------------------------
template <typename T, int D, int C>
struct WySmem {
  typedef Tile<T, C, D> TL;
  static constexpr int KOFF = 0, VOFF = TL::BYTES;
  static constexpr int LOFF = 2 * TL::BYTES;  // L [C][C] fp32
  static constexpr int GOFF = LOFF + C * C * 4;
  static constexpr int BOFF = GOFF + C * 4;
  static constexpr int BYTES = BOFF + C * 4;
  static constexpr int NT = 2 * D < 64 ? 64 : 2 * D;  // one thread per column of [V | K]
};

template <typename T, int D, int C>
__global__ void __launch_bounds__((WySmem<T, D, C>::NT)) ll_gdn_wy(GdnArgs a) {
  using M = Mma<T>;
  typedef WySmem<T, D, C> SM;
  typedef Tile<T, C, D> TL;
  constexpr int NT = SM::NT, NW = NT / 64, CT = C / 16, KSD = D / M::KS;
  constexpr int EPP = 16 / (int)sizeof(T);  // elements per 16-byte piece
  __shared__ __attribute__((aligned(1024))) char smem[SM::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, q16 = lane & 15;
  const int nc = a.T / C;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int i = wg % nc, bh = wg / nc, h = bh % a.H, b = bh / a.H;
  const int64_t row0 = ((int64_t)b * a.T + (int64_t)i * C) * a.H + h;  // row of the chunk's first token

  // K and V rows into swizzled tiles
  const T* kg = static_cast<const T*>(a.k);
  const T* vg = static_cast<const T*>(a.v);
  for (int x = tid; x < C * TL::NCH; x += NT) {
    const int r = x / TL::NCH, c = x % TL::NCH;
    const int64_t src = (row0 + (int64_t)r * a.H) * D + c * EPP;
    const int dst = r * TL::RB + TL::pos(r, c) * 16;
    *reinterpret_cast<uint4*>(smem + SM::KOFF + dst) = *reinterpret_cast<const uint4*>(kg + src);
    *reinterpret_cast<uint4*>(smem + SM::VOFF + dst) = *reinterpret_cast<const uint4*>(vg + src);
  }
  float* gl = reinterpret_cast<float*>(smem + SM::GOFF);
  float* bl = reinterpret_cast<float*>(smem + SM::BOFF);
  float* Lm = reinterpret_cast<float*>(smem + SM::LOFF);
  if (wv == 0) {
    const float G = chunk_scan<C>(lane < C ? a.g[row0 + (int64_t)lane * a.H] : 0.f);
    if (lane < C) {
      gl[lane] = G;
      bl[lane] = a.beta[row0 + (int64_t)lane * a.H];
    }
  }
  __syncthreads();

  // L: the causal 16x16 tiles of K K^T dealt to the waves; lane holds row
  // r = 16 rt + lane%16 and sources s = 16 ct + 4 (lane/16) + e
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
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 16 * ct + 4 * g4 + e;
      Lm[r * C + s] = s < r ? br * __expf(gr - gl[s]) * x[e] : 0.f;
    }
  }
  __syncthreads();

  // forward substitution (I + L) X = B, one column per thread: columns
  // [0, D) of diag(beta) V give U', columns [D, 2D) of diag(beta e^G) K give W
  if (tid < 2 * D) {
    const bool is_w = tid >= D;
    const int c = is_w ? tid - D : tid;
    const char* src = smem + (is_w ? SM::KOFF : SM::VOFF);
    float x[C];
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float acc = to_f32(*reinterpret_cast<const T*>(src + TL::off(r, c))) * bl[r];
      if (is_w) acc *= __expf(gl[r]);
      const float* Lr = Lm + r * C;
#pragma unroll
      for (int s = 0; s < r; ++s) acc -= Lr[s] * x[s];
      x[r] = acc;
    }
    T* dst = static_cast<T*>(is_w ? a.W : a.Up);
#pragma unroll
    for (int r = 0; r < C; ++r) dst[(row0 + (int64_t)r * a.H) * D + c] = from_f32<T>(x[r]);
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

  f32x4 st[ODT];
#pragma unroll
  for (int o = 0; o < ODT; ++o) st[o] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int x = tid; x < KSD * 64; x += 64 * NW) sf[x] = Frag{};

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
  hipLaunchKernelGGL((ll_gdn_wy<T, D, C>), dim3(grid), dim3(WySmem<T, D, C>::NT), 0, s, a);
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
