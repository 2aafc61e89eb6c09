// prior_read.hip -- the read of the per-level states that precede a prefill
// segment ("Log-Linear Attention", section 2.2: every level l of the Fenwick
// decomposition contributes lambda_t^(l) q_t^T S_t^(l)).
//
// A segment of T tokens starting at position pos0, with T <= lowbit(pos0),
// sees the prefix [0, pos0) as the buckets of the set bits of pos0 -- levels
// above every level inside the segment, unchanged by it: token pos0 + t has
// bits of pos0 above and bits of t below, so its buckets are those of t
// within the segment plus those of pos0.  The prior states arrive in the
// decode layout (S_hat, sigma: true state e^sigma S_hat, decayed through token
// pos0 - 1), and reach token pos0 + t with the gates of tokens pos0..pos0+t:
//   o_t += sum_{l: bit l-1 of pos0} lambda_t^(l) e^{sigma_l + G_t} q_t^T S_hat_l,
// G_t the inclusive sum of the segment's log-gates up to t.  ll_chunk_attn has
// written the segment's own part of o; this kernel adds the rest.
//
// One workgroup per (block of P chunks, head), one wave per 16 tokens of a
// chunk.  The prior levels are staged in LDS as MFMA A fragments of S_hat^T
// (a pass takes as many levels as fit), then the block's chunks are walked:
// per chunk each wave forms O^T = S_hat^T Q^T for its 16 tokens on MFMA (a
// lane holds one token and four output columns, so the per-token weight is a
// lane scalar) and adds it to o.  The gate sum up to the chunk comes from the
// block gate sums of ll_chunk_state and the in-chunk prefix.
#include <type_traits>

#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

constexpr int kPriorLdsBytes = 48 * 1024;

template <typename T, int D, int C>
__global__ void __launch_bounds__(64 * (C / 16)) ll_prior_read(PrefillArgs a) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type Vec4;  // 4 values of T
  constexpr int NW = C / 16, NT = D / 16, KSD = D / M::KS;
  constexpr int FR = NT * KSD * 64;  // fragments of one level
  constexpr int NLF = kPriorLdsBytes / (FR * (int)sizeof(Frag));
  constexpr int NL = NLF < 1 ? 1 : (NLF > 32 ? 32 : NLF);  // levels per pass
  __shared__ Frag fr[NL][FR];

  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, q16 = lane & 15;
  const int wg = xcd_logical_id(blockIdx.x, gridDim.x);
  const int J = wg % a.nb, bh = wg / a.nb, h = bh % a.H, b = bh / a.H;
  const float* Sh = a.state_in + (int64_t)bh * a.L * D * D;
  const float* sig = a.state_in + (int64_t)a.B * a.H * a.L * D * D + (int64_t)bh * a.L;

  // gate sum of the segment before block J
  float off = 0.f;
  for (int e = lane; e < J; e += 64) off += a.GS[(int64_t)bh * a.nb + e];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) off += __shfl_xor(off, m, 64);

  uint64_t bits = (uint64_t)a.pos0;
  while (bits) {  // the same in every thread
    int lv[NL];
    int n = 0;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      lv[i] = bits ? __ffsll((unsigned long long)bits) : 0;  // level = bit index + 1
      if (bits) ++n;
      bits &= bits - 1;
    }
    __syncthreads();  // the previous pass's fragments are no longer read
    // stage: fragment f = (nt KSD + s) 64 + l holds S_hat[kidx(s, l/16, e)][16 nt + l%16]
    for (int x = tid; x < n * FR; x += 64 * NW) {
      const int li = x / FR, f = x % FR;
      const int l = f & 63, s = (f >> 6) % KSD, nt = f / (64 * KSD);
      int lvl = lv[0];
#pragma unroll
      for (int i = 1; i < NL; ++i)
        if (li == i) lvl = lv[i];
      const float* S = Sh + (int64_t)lvl * D * D + 16 * nt + (l & 15);
      Frag v;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (T)S[M::kidx(s, l >> 4, e) * D];
      } else {
        v = S[M::kidx(s, l >> 4, 0) * D];
      }
      fr[li][f] = v;
    }
    __syncthreads();

    float run = off;  // gate sum of the segment before the current chunk
    for (int j = 0; j < a.P; ++j) {
      const int64_t row0 = ((int64_t)b * a.T + (int64_t)(J * a.P + j) * C) * a.H + h;
      const float G = chunk_scan<C>(lane < C ? a.g[row0 + (int64_t)lane * a.H] : 0.f);  // lane r: G[r]
      const float gsum = __shfl(G, C - 1, 64);
      const int r = 16 * wv + q16;  // this lane's token within the chunk
      const float Gr = __shfl(G, r, 64) + run;
      const int64_t row = row0 + (int64_t)r * a.H;
      // Q^T operand: k = head dim, column = token r
      const T* qrow = static_cast<const T*>(a.q) + row * D;
      Frag qf[KSD];
#pragma unroll
      for (int s = 0; s < KSD; ++s) {
        if constexpr (sizeof(T) == 2) {
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(qrow + M::kidx(s, g4, 0));
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(qrow + M::kidx(s, g4, 4));
          qf[s] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          qf[s] = qrow[M::kidx(s, g4, 0)];
        }
      }
      f32x4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int li = 0; li < n; ++li) {
        int lvl = lv[0];
#pragma unroll
        for (int i = 1; i < NL; ++i)
          if (li == i) lvl = lv[i];
        const float w = a.lam[row * a.L + lvl] * __expf(Gr + sig[lvl]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KSD; ++s) p = M::mma(fr[li][(nt * KSD + s) * 64 + lane], qf[s], p);
          acc[nt] += w * p;
        }
      }
      // lane: token r, output columns 16 nt + 4 g4 .. + 3
      T* orow = static_cast<T*>(a.o) + row * D + 4 * g4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        Vec4* p = reinterpret_cast<Vec4*>(orow + 16 * nt);
        const Vec4 cur = *p;
        Vec4 nv;
#pragma unroll
        for (int e = 0; e < 4; ++e) nv[e] = (T)((float)cur[e] + acc[nt][e]);
        *p = nv;
      }
      run += gsum;
    }
  }
}

template <typename T, int D, int C>
static hipError_t launch_prior_t(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((ll_prior_read<T, D, C>), dim3(a.B * a.H * a.nb), dim3(64 * (C / 16)), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prior_read(int io, int D, int C, const PrefillArgs& a, hipStream_t s) {
#define LL_PRIOR_C(T, DV)                                 \
  switch (C) {                                            \
    case 16: if constexpr (sizeof(T) == 4) return launch_prior_t<T, DV, 16>(a, s); break; \
    case 32: return launch_prior_t<T, DV, 32>(a, s);      \
    case 64: return launch_prior_t<T, DV, 64>(a, s);      \
  }                                                       \
  return hipErrorInvalidValue;
  if (io == 1) {
    switch (D) {
      case 32: { LL_PRIOR_C(bf16, 32) }
      case 64: { LL_PRIOR_C(bf16, 64) }
      case 128: { LL_PRIOR_C(bf16, 128) }
    }
  } else {
    switch (D) {
      case 16: { LL_PRIOR_C(float, 16) }
      case 32: { LL_PRIOR_C(float, 32) }
      case 64: { LL_PRIOR_C(float, 64) }
      case 128:  // a C x 128 fp32 tile fits at C = 16 only
        if (C == 16) return launch_prior_t<float, 128, 16>(a, s);
        break;
    }
  }
#undef LL_PRIOR_C
  return hipErrorInvalidValue;
}

}  // namespace llattn
