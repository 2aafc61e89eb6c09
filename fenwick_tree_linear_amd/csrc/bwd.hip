// bwd.hip -- helper kernels of the backward pass of the Mamba-2 log-linear
// read ("Log-Linear Attention", sections 2.2-2.3).  The gradients are built
// from the chunk-parallel forward itself (see ll_attn_bwd in api.cpp):
//   dq            = forward(q := dO, k := v, v := k)                     (same weights)
//   dlambda^(l)_t = dO_t . forward(q, k, v; weights one-hot at level l)_t
//   dv, dk        = per level l, forward reads in reversed time, where the
//                   level weight (on the later token) is folded into dO:
//     dv = rev forward(q := rev k, k := rev q, v := rev(lambda^(l) dO))
//     dk = rev forward(q := rev v, k := rev(lambda^(l) dO), v := rev q)
//                   with the reversed gates shifted by one token, and one-hot
//                   weights at level l (levels are preserved when positions are
//                   complemented within a power of two, Tp >= T);
//   dlog_gate_r   = sum_{t >= r} (dO_t . o_t - k_t . dk_t).
// The kernels here do the reversal, the weighting, the accumulation and the
// gate gradient; all are elementwise or per-row.
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

static int grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (int)(g < 65536 ? g : 65536);
}
#define LL_GRID_STRIDE(i, n) \
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (n); i += (int64_t)gridDim.x * blockDim.x)

// qr, kr, vr [B,Tp,H,D] = rows of q, k, v at t = Tp-1-t' (zero past T);
// gr [B,Tp,H] = log a at T_p - t' (the shift that makes a forward decay over
// t'+1..s' equal the original decay over s+1..t), zero where out of range.
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_reverse(BwdArgs a, T* qr, T* kr, T* vr, float* gr) {
  const int64_t n = (int64_t)a.B * a.Tp * a.H * a.D;
  LL_GRID_STRIDE(i, n) {
    const int x = (int)(i % a.D);
    const int64_t row = i / a.D;
    const int h = (int)(row % a.H);
    const int tp = (int)((row / a.H) % a.Tp);
    const int b = (int)(row / ((int64_t)a.H * a.Tp));
    const int t = a.Tp - 1 - tp;
    const int64_t src = (((int64_t)b * a.T + t) * a.H + h) * a.D + x;
    const bool ok = t < a.T;
    qr[i] = ok ? static_cast<const T*>(a.q)[src] : from_f32<T>(0.f);
    kr[i] = ok ? static_cast<const T*>(a.k)[src] : from_f32<T>(0.f);
    vr[i] = ok ? static_cast<const T*>(a.v)[src] : from_f32<T>(0.f);
    if (x == 0) {
      const int tg = a.Tp - tp;
      gr[row] = (tp >= 1 && tg < a.T) ? a.g[((int64_t)b * a.T + tg) * a.H + h] : 0.f;
    }
  }
}

// dOr [B,Tp,H,D] = lambda^(l)_t dO_t at t = Tp-1-t' (zero past T)
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_scale_rev(BwdArgs a, int lvl, T* dOr) {
  const int64_t n = (int64_t)a.B * a.Tp * a.H * a.D;
  LL_GRID_STRIDE(i, n) {
    const int x = (int)(i % a.D);
    const int64_t row = i / a.D;
    const int h = (int)(row % a.H);
    const int tp = (int)((row / a.H) % a.Tp);
    const int b = (int)(row / ((int64_t)a.H * a.Tp));
    const int t = a.Tp - 1 - tp;
    float val = 0.f;
    if (t < a.T) {
      const int64_t r = ((int64_t)b * a.T + t) * a.H + h;
      val = a.lam[r * a.L + lvl] * to_f32(static_cast<const T*>(a.dO)[r * a.D + x]);
    }
    dOr[i] = from_f32<T>(val);
  }
}

// level weights one-hot at lvl for `rows` rows
__global__ void __launch_bounds__(256) ll_bwd_onehot(int64_t rows, int L, int lvl, float* w) {
  LL_GRID_STRIDE(i, rows * L) w[i] = (int)(i % L) == lvl ? 1.f : 0.f;
}

// acc [B,T,H,D] (+)= Y at t' = Tp-1-t
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_accum_rev(BwdArgs a, const T* Y, float* acc, int first) {
  const int64_t n = (int64_t)a.B * a.T * a.H * a.D;
  LL_GRID_STRIDE(i, n) {
    const int x = (int)(i % a.D);
    const int64_t row = i / a.D;
    const int h = (int)(row % a.H);
    const int t = (int)((row / a.H) % a.T);
    const int b = (int)(row / ((int64_t)a.H * a.T));
    const float y = to_f32(Y[(((int64_t)b * a.Tp + (a.Tp - 1 - t)) * a.H + h) * a.D + x]);
    acc[i] = first ? y : acc[i] + y;
  }
}

// dlambda[row][lvl] = Y_row . dO_row (Y: [B,T,H,D]); zero when Y is NULL
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_rowdot(BwdArgs a, const T* Y, int lvl) {
  const int64_t rows = (int64_t)a.B * a.T * a.H;
  LL_GRID_STRIDE(r, rows) {
    float s = 0.f;
    if (Y)
      for (int x = 0; x < a.D; ++x) s += to_f32(Y[r * a.D + x]) * to_f32(static_cast<const T*>(a.dO)[r * a.D + x]);
    a.dlambda[r * a.L + lvl] = s;
  }
}

// dk, dv in the io dtype from their fp32 accumulators
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_cast(BwdArgs a, const float* acc_dk, const float* acc_dv) {
  const int64_t n = (int64_t)a.B * a.T * a.H * a.D;
  LL_GRID_STRIDE(i, n) {
    static_cast<T*>(a.dk)[i] = from_f32<T>(acc_dk[i]);
    static_cast<T*>(a.dv)[i] = from_f32<T>(acc_dv[i]);
  }
}

// One workgroup per head: dG_t = dO_t . o_t - k_t . dk_t, then the suffix sum
// dlog_gate_r = sum_{t >= r} dG_t, walking the tokens from the end in tiles of
// 256 with the running sum carried between tiles.
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_gate(BwdArgs a, const float* acc_dk) {
  __shared__ float sbuf[256];
  const int bh = blockIdx.x, h = bh % a.H, b = bh / a.H;
  const int tid = threadIdx.x;
  float carry = 0.f;
  for (int t0 = a.T - 256; t0 > -256; t0 -= 256) {
    const int t = t0 + (255 - tid);  // thread 0 takes the latest token of the tile
    float dg = 0.f;
    if (t >= 0 && t < a.T) {
      const int64_t r = ((int64_t)b * a.T + t) * a.H + h;
      for (int x = 0; x < a.D; ++x) {
        dg += to_f32(static_cast<const T*>(a.dO)[r * a.D + x]) * to_f32(static_cast<const T*>(a.o)[r * a.D + x]);
        dg -= to_f32(static_cast<const T*>(a.k)[r * a.D + x]) * acc_dk[r * a.D + x];
      }
    }
    // inclusive scan over threads 0..255 (tokens from latest to earliest)
    sbuf[tid] = dg;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const float add = tid >= off ? sbuf[tid - off] : 0.f;
      __syncthreads();
      sbuf[tid] += add;
      __syncthreads();
    }
    if (t >= 0 && t < a.T) a.dlog_gate[((int64_t)b * a.T + t) * a.H + h] = carry + sbuf[tid];
    carry += sbuf[255];
    __syncthreads();
  }
}

#define LL_BWD_IO(io, call) \
  do {                      \
    if (io == 1) {          \
      typedef bf16 TT;      \
      call;                 \
    } else {                \
      typedef float TT;     \
      call;                 \
    }                       \
  } while (0)

hipError_t launch_bwd_reverse(int io, const BwdArgs& a, void* qr, void* kr, void* vr, float* gr, hipStream_t s) {
  const int grid = grid_for((int64_t)a.B * a.Tp * a.H * a.D);
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_reverse<TT>, dim3(grid), dim3(256), 0, s, a, static_cast<TT*>(qr),
                                   static_cast<TT*>(kr), static_cast<TT*>(vr), gr));
  return hipGetLastError();
}

hipError_t launch_bwd_scale_rev(int io, const BwdArgs& a, int lvl, void* dOr, hipStream_t s) {
  const int grid = grid_for((int64_t)a.B * a.Tp * a.H * a.D);
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_scale_rev<TT>, dim3(grid), dim3(256), 0, s, a, lvl, static_cast<TT*>(dOr)));
  return hipGetLastError();
}

hipError_t launch_bwd_onehot(int64_t rows, int L, int lvl, float* w, hipStream_t s) {
  hipLaunchKernelGGL(ll_bwd_onehot, dim3(grid_for(rows * L)), dim3(256), 0, s, rows, L, lvl, w);
  return hipGetLastError();
}

hipError_t launch_bwd_accum_rev(int io, const BwdArgs& a, const void* Y, float* acc, int first, hipStream_t s) {
  const int grid = grid_for((int64_t)a.B * a.T * a.H * a.D);
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_accum_rev<TT>, dim3(grid), dim3(256), 0, s, a, static_cast<const TT*>(Y),
                                   acc, first));
  return hipGetLastError();
}

hipError_t launch_bwd_rowdot(int io, const BwdArgs& a, const void* Y, int lvl, hipStream_t s) {
  const int grid = grid_for((int64_t)a.B * a.T * a.H);
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_rowdot<TT>, dim3(grid), dim3(256), 0, s, a, static_cast<const TT*>(Y), lvl));
  return hipGetLastError();
}

hipError_t launch_bwd_cast(int io, const BwdArgs& a, const float* acc_dk, const float* acc_dv, hipStream_t s) {
  const int grid = grid_for((int64_t)a.B * a.T * a.H * a.D);
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_cast<TT>, dim3(grid), dim3(256), 0, s, a, acc_dk, acc_dv));
  return hipGetLastError();
}

hipError_t launch_bwd_gate(int io, const BwdArgs& a, const float* acc_dk, hipStream_t s) {
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_gate<TT>, dim3(a.B * a.H), dim3(256), 0, s, a, acc_dk));
  return hipGetLastError();
}

}  // namespace llattn
