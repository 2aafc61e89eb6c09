// ccq.hip -- the curvature-conditioned query ("Don't read everything:
// curvature-conditioned query for linear attention", section 2, "Mechanism"):
//   q_clean = q_t - gamma_t Sigma_t q_t,   gamma_t = sigmoid(w_h . q_t + b_h),
//   Sigma_t = (1/(t+1)) sum_{j<=t} k_j k_j^T - mu_t mu_t^T,   mu_t = (1/(t+1)) sum_{j<=t} k_j.
//
// The page keeps the running covariance with the same chunked machinery as
// the backbone state.  Here both running sums come from the chunk-parallel
// prefill itself, run with every level weight 1 and no decay (the Fenwick
// buckets then add up to the plain prefix sum):
//   sum_{j<=t} (k_j . q_t) k_j   = prefill(q, k, v = k)
//   sum_{j<=t} k_j               = prefill(e_0, e_0, v = k)     (e_0 . e_0 = 1)
// and ll_ccq_combine forms q_clean from them, one wave per token-head row.
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// Fills the inputs of the two prefills: level weights 1, log-gates 0, and
// rows e_0 (1 in the first element) in the io dtype.
template <typename T>
__global__ void __launch_bounds__(256) ll_ccq_fill(int64_t rows, int L, int D, float* ones, float* zeros, T* e0) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * L; i += stride) ones[i] = 1.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride) zeros[i] = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * D; i += stride)
    e0[i] = from_f32<T>(i % D == 0 ? 1.f : 0.f);
}

// One wave per row (token t of head h): mu = ksum / (t+1),
// Sigma q = kkq / (t+1) - mu (mu . q), gamma = sigmoid(w_h . q + b_h).
template <typename T, int D>
__global__ void __launch_bounds__(256) ll_ccq_combine(int B, int T_, int H, const T* __restrict__ q,
                                                      const T* __restrict__ kkq, const T* __restrict__ ksum,
                                                      const float* __restrict__ w, const float* __restrict__ b,
                                                      T* __restrict__ q_clean) {
  constexpr int E = (D + 63) / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (row >= (int64_t)B * T_ * H) return;
  const int h = (int)(row % H);
  const int t = (int)((row / H) % T_);
  const float inv = 1.f / (float)(t + 1);
  float qv[E], mu[E], kq[E];
  float mq = 0.f, wq = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane + 64 * e;
    qv[e] = mu[e] = kq[e] = 0.f;
    if (x < D) {
      qv[e] = to_f32(q[row * D + x]);
      mu[e] = to_f32(ksum[row * D + x]) * inv;
      kq[e] = to_f32(kkq[row * D + x]) * inv;
      mq += mu[e] * qv[e];
      wq += w[(int64_t)h * D + x] * qv[e];
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    mq += __shfl_xor(mq, m, 64);
    wq += __shfl_xor(wq, m, 64);
  }
  const float gamma = 1.f / (1.f + __expf(-(wq + b[h])));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane + 64 * e;
    if (x < D) q_clean[row * D + x] = from_f32<T>(qv[e] - gamma * (kq[e] - mu[e] * mq));
  }
}

hipError_t launch_ccq_fill(int io, int64_t rows, int L, int D, float* ones, float* zeros, void* e0, hipStream_t s) {
  const int64_t n = rows * (L > D ? L : D);
  const int grid = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (io == 1)
    hipLaunchKernelGGL(ll_ccq_fill<bf16>, dim3(grid), dim3(256), 0, s, rows, L, D, ones, zeros, static_cast<bf16*>(e0));
  else
    hipLaunchKernelGGL(ll_ccq_fill<float>, dim3(grid), dim3(256), 0, s, rows, L, D, ones, zeros,
                       static_cast<float*>(e0));
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_combine_t(int B, int T_, int H, const void* q, const void* kkq, const void* ksum,
                                   const float* w, const float* b, void* qc, hipStream_t s) {
  const int64_t rows = (int64_t)B * T_ * H;
  hipLaunchKernelGGL((ll_ccq_combine<T, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, B, T_, H,
                     static_cast<const T*>(q), static_cast<const T*>(kkq), static_cast<const T*>(ksum), w, b,
                     static_cast<T*>(qc));
  return hipGetLastError();
}

hipError_t launch_ccq_combine(int io, int D, int B, int T_, int H, const void* q, const void* kkq, const void* ksum,
                              const float* w, const float* b, void* qc, hipStream_t s) {
  if (io == 1) {
    switch (D) {
      case 32: return launch_combine_t<bf16, 32>(B, T_, H, q, kkq, ksum, w, b, qc, s);
      case 64: return launch_combine_t<bf16, 64>(B, T_, H, q, kkq, ksum, w, b, qc, s);
      case 128: return launch_combine_t<bf16, 128>(B, T_, H, q, kkq, ksum, w, b, qc, s);
    }
  } else {
    switch (D) {
      case 16: return launch_combine_t<float, 16>(B, T_, H, q, kkq, ksum, w, b, qc, s);
      case 32: return launch_combine_t<float, 32>(B, T_, H, q, kkq, ksum, w, b, qc, s);
      case 64: return launch_combine_t<float, 64>(B, T_, H, q, kkq, ksum, w, b, qc, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace llattn
