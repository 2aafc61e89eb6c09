// lambda_mlp.hip -- level weights from the adaptive-decay MLP
// ("Adaptive memory decay for log-linear attention", section "Method",
// LambdaMLPSoftplus): for every token and head, with d its per-level
// representation,
//   h = d W1,   lambda = softplus(h W2 + b),
// W1 [L][hidden], W2 [hidden][L], b [L] shared by all rows.  No activation
// lies between the two layers, so lambda = softplus(d Wc + b) with the
// composite Wc = W1 W2 (L x L), which each workgroup forms first
// (mlp_composite, the same operations as the read that makes the weights
// itself).
//
// One wave per 64 rows.  The rows are a dense [rows][L] fp32 array, so a wave
// copies its 64 L floats with coalesced 256-byte instructions into LDS, and
// stores the weights back the same way.  The product runs on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32) with L padded to 16 (mlp_tile_product), then
// + b and softplus.
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

constexpr int kMlpWaves = 4;  // waves (of 64 rows each) per workgroup


// LT = ceil(L / 16) level tiles
template <int LT>
__global__ void __launch_bounds__(64 * kMlpWaves) ll_lambda_mlp(int64_t rows, int L, int hidden,
                                                                 const float* __restrict__ d,
                                                                 const float* __restrict__ w1,
                                                                 const float* __restrict__ w2,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ lam) {
  constexpr int LP = 16 * LT;  // padded levels
  // a straight copy of the wave's rows, [64][L] (odd L: the column reads
  // below hit distinct banks; even L at most two-way)
  __shared__ float tile[kMlpWaves][64 * LP];
  __shared__ float wc[LP * LP];  // the composite weights, zero past L
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;  // fragment column and lane group
  {
    // W1 and W2 staged in the row tiles (2 L hidden floats: at most half of them), then Wc
    float* sw1 = &tile[0][0];
    float* sw2 = sw1 + L * hidden;
    for (int x = threadIdx.x; x < L * hidden; x += 64 * kMlpWaves) {
      sw1[x] = w1[x];
      sw2[x] = w2[x];
    }
    __syncthreads();
    for (int x = threadIdx.x; x < LP * LP; x += 64 * kMlpWaves)
      wc[x] = mlp_composite(sw1, sw2, L, hidden, x / LP, x % LP);
    __syncthreads();
  }
  float* t = tile[wave];
  const int64_t row0 = ((int64_t)blockIdx.x * kMlpWaves + wave) * 64;
  if (row0 >= rows) return;  // whole waves only; no workgroup barrier below
  const int nel = (rows - row0 < 64 ? (int)(rows - row0) : 64) * L;  // floats of this wave's rows

  // this lane's fragments of Wc: level tile lt, step s gives Wc[4 LT g + s][16lt + c]
  float bw[LT][4 * LT];
#pragma unroll
  for (int lt = 0; lt < LT; ++lt)
#pragma unroll
    for (int s = 0; s < 4 * LT; ++s) bw[lt][s] = wc[(4 * LT * g + s) * LP + 16 * lt + c];
  float bvec[LT];
#pragma unroll
  for (int lt = 0; lt < LT; ++lt) bvec[lt] = 16 * lt + c < L ? bias[16 * lt + c] : 0.f;

  // the wave's rows: coalesced 256-byte loads (element i = lane + 64 j of the
  // rows' contiguous floats), all issued before the first LDS write.  Rows
  // past the end are left unset: every row of the product depends on its own
  // row of d only, and they are never stored.
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
    // A operand: lane l = d[16rt + c][4 LT g + s] (zero past L)
    const float* drow = t + (16 * rt + c) * L + 4 * LT * g;
    float a[4 * LT];
#pragma unroll
    for (int s = 0; s < 4 * LT; ++s) a[s] = 4 * LT * g + s < L ? drow[s] : 0.f;
#pragma unroll
    for (int lt = 0; lt < LT; ++lt) z[rt][lt] = mlp_tile_product<4 * LT>(a, bw[lt]);
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
  const int lt = (L + 15) / 16;
  if (lt == 1) {
    hipLaunchKernelGGL((ll_lambda_mlp<1>), grid, block, 0, s, rows, L, hidden, d, w1, w2, bias, lam);
    return hipGetLastError();
  }
  if (lt == 2) {
    hipLaunchKernelGGL((ll_lambda_mlp<2>), grid, block, 0, s, rows, L, hidden, d, w1, w2, bias, lam);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace llattn
