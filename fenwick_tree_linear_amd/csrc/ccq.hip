// ccq.hip -- the curvature-conditioned query ("Don't read everything:
// curvature-conditioned query for linear attention", section 2, "Mechanism"):
//   q_clean = q_t - gamma_t Sigma_t q_t,   gamma_t = sigmoid(w_h . q_t + b_h),
//   Sigma_t = (1/(t+1)) sum_{j<=t} k_j k_j^T - mu_t mu_t^T,   mu_t = (1/(t+1)) sum_{j<=t} k_j.
//
// The page keeps the running covariance with the same chunked machinery as
// the backbone state.  Here the second-moment term comes from the
// chunk-parallel prefill itself, run with every level weight 1 and no decay
// (the Fenwick buckets then add up to the plain prefix sum):
//   sum_{j<=t} (k_j . q_t) k_j   = prefill(q, k, v = k),
// and the running key sum from a chunked prefix sum in fp32: per-chunk column
// sums (ll_ccq_chunk_sum), their exclusive scan over the chunks of a head
// (ll_ccq_chunk_scan), and within the chunk a running sum kept by the wave
// that forms q_clean row by row (ll_ccq_combine).
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// Fills the inputs of the prefill: level weights 1 and log-gates 0.
__global__ void __launch_bounds__(256) ll_ccq_fill(int64_t rows, int L, float* ones, float* zeros) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * L; i += stride) ones[i] = 1.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride) zeros[i] = 0.f;
}

// One wave per (b, h, chunk of CS tokens): the chunk's column sums of k,
// csum[b][h][c][x] (fp32).
template <typename T, int D>
__global__ void __launch_bounds__(256) ll_ccq_chunk_sum(int B, int T_, int H, int CS, const T* __restrict__ k,
                                                        float* __restrict__ csum) {
  constexpr int E = (D + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int nch = T_ / CS;
  const int64_t item = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (item >= (int64_t)B * H * nch) return;
  const int c = (int)(item % nch);
  const int bh = (int)(item / nch), h = bh % H, b = bh / H;
  const int64_t row0 = ((int64_t)b * T_ + (int64_t)c * CS) * H + h;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int r = 0; r < CS; ++r) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int x = lane + 64 * e;
      if (x < D) acc[e] += to_f32(k[(row0 + (int64_t)r * H) * D + x]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane + 64 * e;
    if (x < D) csum[item * D + x] = acc[e];
  }
}

// One thread per (b, h, column): csum becomes, in place, the exclusive prefix
// over the chunks of the head (the key sum of the tokens before the chunk).
__global__ void __launch_bounds__(256) ll_ccq_chunk_scan(int64_t n_bh, int D, int nch, float* __restrict__ csum) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_bh * D) return;
  const int64_t bh = i / D;
  const int x = (int)(i % D);
  float* p = csum + bh * (int64_t)nch * D + x;
  float run = 0.f;
  int c = 0;
  for (; c + 8 <= nch; c += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[(int64_t)(c + j) * D];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[(int64_t)(c + j) * D] = run;
      run += v[j];
    }
  }
  for (; c < nch; ++c) {
    const float v = p[(int64_t)c * D];
    p[(int64_t)c * D] = run;
    run += v;
  }
}

// One wave per (b, h, chunk): walks the chunk's tokens t in order, keeping
// the running key sum (the chunk's exclusive prefix plus the tokens so far);
// per token mu = ksum / (t+1), Sigma q = kkq / (t+1) - mu (mu . q),
// gamma = sigmoid(w_h . q + b_h).
template <typename T, int D>
__global__ void __launch_bounds__(256) ll_ccq_combine(int B, int T_, int H, int CS, const T* __restrict__ q,
                                                      const T* __restrict__ k, const T* __restrict__ kkq,
                                                      const float* __restrict__ csum, const float* __restrict__ w,
                                                      const float* __restrict__ b_, T* __restrict__ q_clean) {
  constexpr int E = (D + 63) / 64;  // elements per lane
  constexpr int RB = 8;             // rows loaded ahead
  const int lane = threadIdx.x & 63;
  const int nch = T_ / CS;
  const int64_t item = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (item >= (int64_t)B * H * nch) return;
  const int c = (int)(item % nch);
  const int bh = (int)(item / nch), h = bh % H, b = bh / H;
  const int64_t row0 = ((int64_t)b * T_ + (int64_t)c * CS) * H + h;
  float run[E], wv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane + 64 * e;
    run[e] = x < D ? csum[item * D + x] : 0.f;
    wv[e] = x < D ? w[(int64_t)h * D + x] : 0.f;
  }
  const float bias = b_[h];
  for (int r0 = 0; r0 < CS; r0 += RB) {
    float qv[RB][E], kv[RB][E], kq[RB][E];
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int x = lane + 64 * e;
        const int64_t o = (row0 + (int64_t)(r0 + j) * H) * D + x;
        const bool in = x < D && r0 + j < CS;
        qv[j][e] = in ? to_f32(q[o]) : 0.f;
        kv[j][e] = in ? to_f32(k[o]) : 0.f;
        kq[j][e] = in ? to_f32(kkq[o]) : 0.f;
      }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      if (r0 + j >= CS) break;
      const int t = c * CS + r0 + j;
      const float inv = 1.f / (float)(t + 1);
      float mq = 0.f, wq = 0.f, mu[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        run[e] += kv[j][e];
        mu[e] = run[e] * inv;
        mq += mu[e] * qv[j][e];
        wq += wv[e] * qv[j][e];
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        mq += __shfl_xor(mq, m, 64);
        wq += __shfl_xor(wq, m, 64);
      }
      const float gamma = 1.f / (1.f + __expf(-(wq + bias)));
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int x = lane + 64 * e;
        if (x < D)
          q_clean[(row0 + (int64_t)(r0 + j) * H) * D + x] = from_f32<T>(qv[j][e] - gamma * (kq[j][e] * inv - mu[e] * mq));
      }
    }
  }
}

hipError_t launch_ccq_fill(int64_t rows, int L, float* ones, float* zeros, hipStream_t s) {
  const int64_t n = rows * L;
  const int grid = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  hipLaunchKernelGGL(ll_ccq_fill, dim3(grid), dim3(256), 0, s, rows, L, ones, zeros);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_ksum_t(int B, int T_, int H, int CS, const void* k, float* csum, hipStream_t s) {
  const int64_t items = (int64_t)B * H * (T_ / CS);
  hipLaunchKernelGGL((ll_ccq_chunk_sum<T, D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, B, T_, H, CS,
                     static_cast<const T*>(k), csum);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t n = (int64_t)B * H * D;
  hipLaunchKernelGGL(ll_ccq_chunk_scan, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (int64_t)B * H, D,
                     T_ / CS, csum);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_combine_t(int B, int T_, int H, int CS, const void* q, const void* k, const void* kkq,
                                   const float* csum, const float* w, const float* b, void* qc, hipStream_t s) {
  const int64_t items = (int64_t)B * H * (T_ / CS);
  hipLaunchKernelGGL((ll_ccq_combine<T, D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, B, T_, H, CS,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(kkq), csum, w, b,
                     static_cast<T*>(qc));
  return hipGetLastError();
}

#define LL_CCQ_DISPATCH(FN, ...)                                  \
  if (io == 1) {                                                  \
    switch (D) {                                                  \
      case 16: return FN<bf16, 16>(__VA_ARGS__);                  \
      case 32: return FN<bf16, 32>(__VA_ARGS__);                  \
      case 64: return FN<bf16, 64>(__VA_ARGS__);                  \
      case 128: return FN<bf16, 128>(__VA_ARGS__);                \
    }                                                             \
  } else {                                                        \
    switch (D) {                                                  \
      case 16: return FN<float, 16>(__VA_ARGS__);                 \
      case 32: return FN<float, 32>(__VA_ARGS__);                 \
      case 64: return FN<float, 64>(__VA_ARGS__);                 \
      case 128: return FN<float, 128>(__VA_ARGS__);               \
    }                                                             \
  }                                                               \
  return hipErrorInvalidValue;

hipError_t launch_ccq_ksum(int io, int D, int B, int T_, int H, int CS, const void* k, float* csum, hipStream_t s) {
  LL_CCQ_DISPATCH(launch_ksum_t, B, T_, H, CS, k, csum, s)
}

hipError_t launch_ccq_combine(int io, int D, int B, int T_, int H, int CS, const void* q, const void* k,
                              const void* kkq, const float* csum, const float* w, const float* b, void* qc,
                              hipStream_t s) {
  LL_CCQ_DISPATCH(launch_combine_t, B, T_, H, CS, q, k, kkq, csum, w, b, qc, s)
}

}  // namespace llattn
