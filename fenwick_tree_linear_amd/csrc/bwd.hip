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
#include <type_traits>

#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

static int grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (int)(g < 65536 ? g : 65536);
}
#define LL_GRID_STRIDE(i, n) \
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (n); i += (int64_t)gridDim.x * blockDim.x)

// Elementwise kernels take four consecutive values of a row per thread; the
// row index splits into (b, position, h) once per thread.
template <typename T>
using Vec4Of = typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type;

// qr, kr, vr [B,Tp,H,D] = rows of q, k, v at t = Tp-1-t' (zero past T);
// gr [B,Tp,H] = log a at Tp - t' (the shift that makes a forward decay over
// t'+1..s' equal the original decay over s+1..t), zero where out of range.
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_reverse(BwdArgs a, T* qr, T* kr, T* vr, float* gr) {
  typedef Vec4Of<T> V;
  const int G4 = a.D / 4;
  const int64_t n = (int64_t)a.B * a.Tp * a.H * G4;
  LL_GRID_STRIDE(i, n) {
    const int x4 = (int)(i % G4);
    const int64_t row = i / G4;
    const int h = (int)(row % a.H);
    const int64_t bt = row / a.H;
    const int tp = (int)(bt % a.Tp), b = (int)(bt / a.Tp);
    const int t = a.Tp - 1 - tp;
    V zq = {}, zk = {}, zv = {};
    if (t < a.T) {
      const int64_t src = (((int64_t)b * a.T + t) * a.H + h) * G4 + x4;
      zq = static_cast<const V*>(a.q)[src];
      zk = static_cast<const V*>(a.k)[src];
      zv = static_cast<const V*>(a.v)[src];
    }
    reinterpret_cast<V*>(qr)[i] = zq;
    reinterpret_cast<V*>(kr)[i] = zk;
    reinterpret_cast<V*>(vr)[i] = zv;
    if (x4 == 0) {
      const int tg = a.Tp - tp;
      gr[row] = (tp >= 1 && tg < a.T) ? a.g[((int64_t)b * a.T + tg) * a.H + h] : 0.f;
    }
  }
}

// dOr [B,Tp,H,D] = lambda^(l)_t dO_t at t = Tp-1-t' (zero past T)
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_scale_rev(BwdArgs a, int lvl, T* dOr) {
  typedef Vec4Of<T> V;
  const int G4 = a.D / 4;
  const int64_t n = (int64_t)a.B * a.Tp * a.H * G4;
  LL_GRID_STRIDE(i, n) {
    const int x4 = (int)(i % G4);
    const int64_t row = i / G4;
    const int h = (int)(row % a.H);
    const int64_t bt = row / a.H;
    const int tp = (int)(bt % a.Tp), b = (int)(bt / a.Tp);
    const int t = a.Tp - 1 - tp;
    V out = {};
    if (t < a.T) {
      const int64_t r = ((int64_t)b * a.T + t) * a.H + h;
      const float w = a.lam[r * a.L + lvl];
      const V d = static_cast<const V*>(a.dO)[r * G4 + x4];
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = from_f32<T>(w * to_f32(d[e]));
    }
    reinterpret_cast<V*>(dOr)[i] = out;
  }
}

// level weights one-hot at lvl for `rows` rows
__global__ void __launch_bounds__(256) ll_bwd_onehot(int64_t rows, int L, int lvl, float* w) {
  LL_GRID_STRIDE(i, rows * L) w[i] = (int)(i % L) == lvl ? 1.f : 0.f;
}

// Moves the one of a one-hot [rows, L] from level lvl - 1 to level lvl.
__global__ void __launch_bounds__(256) ll_bwd_onehot_next(int64_t rows, int L, int lvl, float* w) {
  LL_GRID_STRIDE(r, rows) {
    w[r * L + lvl - 1] = 0.f;
    w[r * L + lvl] = 1.f;
  }
}

// The reversed-time reads of every level, summed: level l's dv read is the
// buffer Y + 2 l ystride and its dk read Y + (2 l + 1) ystride, each [B,Tp,H,D]
// in reversed time.  Writes dv, dk at t = Tp-1-t' in the io dtype (levels
// added in order in fp32) and the fp32 sum for dk, which the gate uses.
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_sum_rev(BwdArgs a, const T* Y, int64_t ystride, int LS, float* acc_dk) {
  typedef Vec4Of<T> V;
  const int G4 = a.D / 4;
  const int64_t n = (int64_t)a.B * a.T * a.H * G4;
  LL_GRID_STRIDE(i, n) {
    const int x4 = (int)(i % G4);
    const int64_t row = i / G4;
    const int h = (int)(row % a.H);
    const int64_t bt = row / a.H;
    const int t = (int)(bt % a.T), b = (int)(bt / a.T);
    const int64_t src = (((int64_t)b * a.Tp + (a.Tp - 1 - t)) * a.H + h) * G4 + x4;
    f32x4 sv = f32x4{0.f, 0.f, 0.f, 0.f}, sk = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int l = 0; l < LS; ++l) {
      const V yv = reinterpret_cast<const V*>(Y + 2 * l * ystride)[src];
      const V yk = reinterpret_cast<const V*>(Y + (2 * l + 1) * ystride)[src];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[e] += to_f32(yv[e]);
        sk[e] += to_f32(yk[e]);
      }
    }
    V ok, ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ok[e] = from_f32<T>(sk[e]);
      ov[e] = from_f32<T>(sv[e]);
    }
    reinterpret_cast<f32x4*>(acc_dk)[i] = sk;
    static_cast<V*>(a.dk)[i] = ok;
    static_cast<V*>(a.dv)[i] = ov;
  }
}

// Dot products of rows, D/4 lanes per row (four elements a lane, D/4 a power
// of two <= 64, so a row's lanes are an aligned group of the wave):
// out[row * stride + col] = sum_x X1 Y1 (- X2 Y2 when X2 is given; Y2 fp32);
// 0 when X1 is null.
template <typename T>
__global__ void __launch_bounds__(256) ll_bwd_rowdot(int64_t rows, int D, const T* X1, const T* Y1, const T* X2,
                                                     const float* Y2, float* out, int stride, int col) {
  typedef Vec4Of<T> V;
  const int G4 = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / G4;
  const int x4 = (int)(gid % G4);
  float s = 0.f;
  if (row < rows && X1) {
    const int64_t i = row * G4 + x4;
    const V x = reinterpret_cast<const V*>(X1)[i], y = reinterpret_cast<const V*>(Y1)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) s += to_f32(x[e]) * to_f32(y[e]);
    if (X2) {
      const V x2 = reinterpret_cast<const V*>(X2)[i];
      const f32x4 y2 = reinterpret_cast<const f32x4*>(Y2)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) s -= to_f32(x2[e]) * y2[e];
    }
  }
  for (int m = G4 >> 1; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (row < rows && x4 == 0) out[row * stride + col] = s;
}

// One workgroup per head: dlog_gate_r = sum_{t >= r} dG_t, walking the tokens
// from the end in tiles of 256 with the running sum carried between tiles.
__global__ void __launch_bounds__(256) ll_bwd_suffix(BwdArgs a, const float* dG) {
  __shared__ float sbuf[256];
  const int bh = blockIdx.x, h = bh % a.H, b = bh / a.H;
  const int tid = threadIdx.x;
  float carry = 0.f;
  for (int t0 = a.T - 256; t0 > -256; t0 -= 256) {
    const int t = t0 + (255 - tid);  // thread 0 takes the latest token of the tile
    const int64_t r = ((int64_t)b * a.T + t) * a.H + h;
    sbuf[tid] = (t >= 0) ? dG[r] : 0.f;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const float add = tid >= off ? sbuf[tid - off] : 0.f;
      __syncthreads();
      sbuf[tid] += add;
      __syncthreads();
    }
    if (t >= 0) a.dlog_gate[r] = carry + sbuf[tid];
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
  const int grid = grid_for((int64_t)a.B * a.Tp * a.H * a.D / 4);
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_reverse<TT>, dim3(grid), dim3(256), 0, s, a, static_cast<TT*>(qr),
                                   static_cast<TT*>(kr), static_cast<TT*>(vr), gr));
  return hipGetLastError();
}

hipError_t launch_bwd_scale_rev(int io, const BwdArgs& a, int lvl, void* dOr, hipStream_t s) {
  const int grid = grid_for((int64_t)a.B * a.Tp * a.H * a.D / 4);
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_scale_rev<TT>, dim3(grid), dim3(256), 0, s, a, lvl, static_cast<TT*>(dOr)));
  return hipGetLastError();
}

hipError_t launch_bwd_onehot(int64_t rows, int L, int lvl, float* w, hipStream_t s) {
  // the levels are taken in order: after level 0 only two columns change
  if (lvl > 0 && lvl < L)
    hipLaunchKernelGGL(ll_bwd_onehot_next, dim3(grid_for(rows)), dim3(256), 0, s, rows, L, lvl, w);
  else
    hipLaunchKernelGGL(ll_bwd_onehot, dim3(grid_for(rows * L)), dim3(256), 0, s, rows, L, lvl, w);
  return hipGetLastError();
}

hipError_t launch_bwd_sum_rev(int io, const BwdArgs& a, const void* Y, int64_t ystride, int LS, float* acc_dk,
                             hipStream_t s) {
  const int grid = grid_for((int64_t)a.B * a.T * a.H * a.D / 4);
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_sum_rev<TT>, dim3(grid), dim3(256), 0, s, a, static_cast<const TT*>(Y),
                                   ystride, LS, acc_dk));
  return hipGetLastError();
}

static unsigned rowdot_blocks(int64_t rows, int D) { return (unsigned)((rows * (D / 4) + 255) / 256); }

hipError_t launch_bwd_rowdot(int io, const BwdArgs& a, const void* Y, int lvl, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.T * a.H;
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_rowdot<TT>, dim3(rowdot_blocks(rows, a.D)), dim3(256), 0, s, rows, a.D,
                                   static_cast<const TT*>(Y), static_cast<const TT*>(a.dO), (const TT*)nullptr,
                                   (const float*)nullptr, a.dlambda, a.L, lvl));
  return hipGetLastError();
}

hipError_t launch_bwd_gate(int io, const BwdArgs& a, const float* acc_dk, float* dG, hipStream_t s) {
  // dG_t = dO_t . o_t - k_t . dk_t per row, then the suffix sums per head
  const int64_t rows = (int64_t)a.B * a.T * a.H;
  LL_BWD_IO(io, hipLaunchKernelGGL(ll_bwd_rowdot<TT>, dim3(rowdot_blocks(rows, a.D)), dim3(256), 0, s, rows, a.D,
                                   static_cast<const TT*>(a.dO), static_cast<const TT*>(a.o),
                                   static_cast<const TT*>(a.k), acc_dk, dG, 1, 0));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ll_bwd_suffix, dim3(a.B * a.H), dim3(256), 0, s, a, dG);
  return hipGetLastError();
}

}  // namespace llattn
