// lambda_mlp.hip -- level weights from the adaptive-decay MLP
// ("Adaptive memory decay for log-linear attention", section "Method",
// LambdaMLPSoftplus): for every token and head, with d its per-level
// representation,
//   h = d W1,   lambda = softplus(h W2 + b),
// W1 [L][hidden], W2 [hidden][L], b [L] shared by all rows.
//
// One wave per 64 rows.  The rows are a dense [rows][L] fp32 array, so a wave
// copies its 64 L floats with coalesced 256-byte instructions into LDS, and
// stores the weights back the same way.  Both layers run on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32) with L and hidden padded to 16:
//   layer 1, transposed: h^T tile (16 hidden x 16 rows) = W1^T d^T, so that
//     lane l ends up holding row l%16 of h at hidden indices 4(l/16)+i --
//     exactly the k operand layout of layer 2 (no trip through LDS);
//   layer 2: z tile (16 rows x 16 levels) = h W2 (even and odd k steps in two
//     accumulators, then summed), then + b and softplus.
// W1 and W2 are loaded once per wave into fragment registers (zero where the
// padding lies).
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

constexpr int kMlpWaves = 4;  // waves (of 64 rows each) per workgroup


// LT = ceil(L / 16) level tiles, HT = ceil(hidden / 16) hidden tiles
template <int LT, int HT>
__global__ void __launch_bounds__(64 * kMlpWaves) ll_lambda_mlp(int64_t rows, int L, int hidden,
                                                                 const float* __restrict__ d,
                                                                 const float* __restrict__ w1,
                                                                 const float* __restrict__ w2,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ lam) {
  constexpr int LP = 16 * LT;  // padded levels
  typedef Mma<float> M;
  // a straight copy of the wave's rows, [64][L] (odd L: the column reads
  // below hit distinct banks; even L at most two-way)
  __shared__ float tile[kMlpWaves][64 * LP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;  // fragment column and lane group
  float* t = tile[wave];
  const int64_t row0 = ((int64_t)blockIdx.x * kMlpWaves + wave) * 64;
  if (row0 >= rows) return;  // whole waves only; no workgroup barrier below
  const int nel = (rows - row0 < 64 ? (int)(rows - row0) : 64) * L;  // floats of this wave's rows

  // weights as MFMA fragments.  Layer 1 (A = W1^T, k = level): step s of
  // hidden tile n gives lane l W1[4s + g][16n + c].  Layer 2 (B = W2, k =
  // hidden in the accumulator order of layer 1): step s gives lane l
  // W2[M::kidx(s, g)][16lt + c].  Zero in the padding.
  float a1[HT][4 * LT], b2[LT][4 * HT];
#pragma unroll
  for (int n = 0; n < HT; ++n)
#pragma unroll
    for (int s = 0; s < 4 * LT; ++s) {
      const int k = 4 * s + g, j = 16 * n + c;
      a1[n][s] = (k < L && j < hidden) ? w1[k * hidden + j] : 0.f;
    }
#pragma unroll
  for (int lt = 0; lt < LT; ++lt)
#pragma unroll
    for (int s = 0; s < 4 * HT; ++s) {
      const int k = M::kidx(s, g, 0), j = 16 * lt + c;
      b2[lt][s] = (k < hidden && j < L) ? w2[k * L + j] : 0.f;
    }
  float bvec[LT];
#pragma unroll
  for (int lt = 0; lt < LT; ++lt) bvec[lt] = 16 * lt + c < L ? bias[16 * lt + c] : 0.f;

  // the wave's rows: coalesced 256-byte loads (element i = lane + 64 j of the
  // rows' contiguous floats), all issued before the first LDS write.  Rows
  // past the end are left unset: every row of both products depends on its
  // own row of d only, and they are never stored.
  {
    const float* src = d + row0 * L;
    float v[LP];
#pragma unroll
    for (int j = 0; j < LP; ++j) {
      const int i = lane + 64 * j;
      if (j < L && i < nel) v[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < LP; ++j) {
      const int i = lane + 64 * j;
      if (j < L && i < nel) t[i] = v[j];
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();

  f32x4 z[4][LT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    // layer 1: h^T (hidden x rows) = W1^T d^T; B operand lane l = d[16rt + c][4s + g]
    const float* drow = t + (16 * rt + c) * L + g;
    f32x4 h[HT];
#pragma unroll
    for (int n = 0; n < HT; ++n) h[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4 * LT; ++s) {
      const float bd = 4 * s + g < L ? drow[4 * s] : 0.f;
#pragma unroll
      for (int n = 0; n < HT; ++n) h[n] = M::mma(a1[n][s], bd, h[n]);
    }
    // layer 2: z (rows x levels) = h W2; lane l holds h[16rt + c][16n + 4g + i].
    // The even and odd k steps go to two accumulators, summed at the end
    // (two dependent chains of half the length).
#pragma unroll
    for (int lt = 0; lt < LT; ++lt) {
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < 4 * HT; ++s) acc[s & 1] = M::mma(M::acc_frag(h, s), b2[lt][s], acc[s & 1]);
      z[rt][lt] = acc[0] + acc[1];
    }
  }
  __builtin_amdgcn_wave_barrier();  // the staged rows are read before they are overwritten
  __builtin_amdgcn_s_waitcnt(0xc07f);
  // z[rt][lt][i] = z[16rt + 4g + i][16lt + c]: bias, softplus, back into the
  // tile in the rows' own layout
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int lt = 0; lt < LT; ++lt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * lt + c < L) t[(16 * rt + 4 * g + i) * L + 16 * lt + c] = softplus_f32(z[rt][lt][i] + bvec[lt]);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  float* dst = lam + row0 * L;
  float o[LP];
#pragma unroll
  for (int j = 0; j < LP; ++j) {
    const int i = lane + 64 * j;
    if (j < L && i < nel) o[j] = t[i];
  }
#pragma unroll
  for (int j = 0; j < LP; ++j) {
    const int i = lane + 64 * j;
    if (j < L && i < nel) dst[i] = o[j];
  }
}

hipError_t launch_lambda_mlp(int64_t rows, int L, int hidden, const float* d, const float* w1, const float* w2,
                             const float* bias, float* lam, hipStream_t s) {
  const int64_t waves = (rows + 63) / 64;
  const dim3 grid((unsigned)((waves + kMlpWaves - 1) / kMlpWaves)), block(64 * kMlpWaves);
  const int lt = (L + 15) / 16, ht = (hidden + 15) / 16;
#define LL_MLP(LTV, HTV)                                                                                 \
  if (lt == LTV && ht == HTV) {                                                                          \
    hipLaunchKernelGGL((ll_lambda_mlp<LTV, HTV>), grid, block, 0, s, rows, L, hidden, d, w1, w2, bias, lam); \
    return hipGetLastError();                                                                            \
  }
  LL_MLP(1, 1) LL_MLP(1, 2) LL_MLP(1, 3) LL_MLP(1, 4) LL_MLP(2, 1) LL_MLP(2, 2) LL_MLP(2, 3) LL_MLP(2, 4)
#undef LL_MLP
  return hipErrorInvalidValue;
}

}  // namespace llattn
