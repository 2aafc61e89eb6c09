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
// sums (ccq_chunk_sum, in ll_ccq_prepare beside the fill of the prefill's
// inputs), their exclusive scan over the chunks of a head
// (ll_ccq_chunk_scan), and within the chunk the key sums of its earlier groups
// of 8 tokens plus a running sum over the group's own (ll_ccq_combine, one
// wave per group).
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // a 16-byte piece of a row

// The values of a 16-byte piece: 8 bf16 (element 2i in the low half of word
// i) or 4 fp32.
template <typename T>
__device__ __forceinline__ void unpack_piece(u32x4 v, float (&f)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
}

// A 16-byte piece from its values (bf16: rounded to nearest even).
template <typename T>
__device__ __forceinline__ u32x4 pack_piece(const float (&f)[16 / sizeof(T)]) {
  u32x4 v;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (unsigned)__builtin_bit_cast(unsigned short, (bf16)f[2 * i]) |
             ((unsigned)__builtin_bit_cast(unsigned short, (bf16)f[2 * i + 1]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  }
  return v;
}

// Fills the inputs of the prefill: level weights 1 and log-gates 0, thread
// i0 of a grid of `stride` threads.  VEC: the buffers start on 16 bytes and
// take 4 values per store.
template <bool VEC>
__device__ __forceinline__ void ccq_fill(int64_t i0, int64_t stride, int64_t n_ones, int64_t n_zeros, float* ones,
                                         float* zeros) {
  if (VEC) {
    const float4 one4 = make_float4(1.f, 1.f, 1.f, 1.f), zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = i0; i < n_ones / 4; i += stride) reinterpret_cast<float4*>(ones)[i] = one4;
    for (int64_t i = i0; i < n_zeros / 4; i += stride) reinterpret_cast<float4*>(zeros)[i] = zero4;
    if (i0 < n_ones % 4) ones[n_ones / 4 * 4 + i0] = 1.f;
    if (i0 < n_zeros % 4) zeros[n_zeros / 4 * 4 + i0] = 0.f;
  } else {
    for (int64_t i = i0; i < n_ones; i += stride) ones[i] = 1.f;
    for (int64_t i = i0; i < n_zeros; i += stride) zeros[i] = 0.f;
  }
}

// Wave `item` of the chunk sums, one per (b, h, chunk of CS tokens, CS a
// multiple of 16): the chunk's column sums of k, csum[b][h][c][x] (fp32), 16
// rows loaded per round.  Items go along the heads first (the rows in flight
// then cover every head).
template <typename T, int D>
__device__ __forceinline__ void ccq_chunk_sum(int64_t item, int B, int T_, int H, int CS, const T* __restrict__ k,
                                              float* __restrict__ csum) {
  constexpr int E = (D + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int nch = T_ / CS;
  if (item >= (int64_t)B * H * nch) return;
  const int h = (int)(item % H);
  const int64_t bc = item / H;
  const int c = (int)(bc % nch), b = (int)(bc / nch);
  const int64_t row0 = ((int64_t)b * T_ + (int64_t)c * CS) * H + h;
  const int64_t out = ((int64_t)b * H + h) * nch + c;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int r0 = 0; r0 < CS; r0 += 16) {
    float kv[16][E];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool in = lane * E < D;  // lanes past the last column read column 0 and add 0
        const float v = to_f32(k[(row0 + (int64_t)(r0 + r) * H) * D + (in ? lane * E + e : 0)]);
        kv[r][e] = in ? v : 0.f;
      }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += kv[r][e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = lane * E + e;
    if (x < D) csum[out * D + x] = acc[e];
  }
}

// The first sum_blocks workgroups take the chunk sums (four waves each), the
// others the fill: the two are independent, and one launch lets the fill's
// stores and the sums' loads overlap.
template <typename T, int D, bool VEC>
__global__ void __launch_bounds__(256) ll_ccq_prepare(int B, int T_, int H, int CS, const T* __restrict__ k,
                                                      float* __restrict__ csum, int sum_blocks, int64_t n_ones,
                                                      int64_t n_zeros, float* ones, float* zeros) {
  if ((int)blockIdx.x < sum_blocks) {
    ccq_chunk_sum<T, D>((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), B, T_, H, CS, k, csum);
  } else {
    ccq_fill<VEC>((int64_t)(blockIdx.x - sum_blocks) * blockDim.x + threadIdx.x,
                  (int64_t)(gridDim.x - sum_blocks) * blockDim.x, n_ones, n_zeros, ones, zeros);
  }
}

// csum becomes, in place, the exclusive prefix over the chunks of each head
// (the key sum of the tokens before the chunk).  One workgroup of 1024 threads
// per (b, h): thread (s, x) takes column x of the s-th of 1024 / D runs of
// consecutive chunks; run totals meet in LDS.
template <int D>
__global__ void __launch_bounds__(1024) ll_ccq_chunk_scan(int nch, float* __restrict__ csum) {
  constexpr int S = 1024 / D;
  __shared__ float tot[S][D];
  const int x = threadIdx.x % D, s = threadIdx.x / D;
  const int per = (nch + S - 1) / S;
  const int c0 = s * per, c1 = min(nch, c0 + per);
  float* p = csum + (int64_t)blockIdx.x * nch * D + x;
  float sum = 0.f;
  int c = c0;
  for (; c + 16 <= c1; c += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = p[(int64_t)(c + j) * D];
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += v[j];
  }
  for (; c < c1; ++c) sum += p[(int64_t)c * D];
  tot[s][x] = sum;
  __syncthreads();
  float run = 0.f;
  for (int j = 0; j < s; ++j) run += tot[j][x];
  c = c0;
  for (; c + 16 <= c1; c += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = p[(int64_t)(c + j) * D];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[(int64_t)(c + j) * D] = run;
      run += v[j];
    }
  }
  for (; c < c1; ++c) {
    const float v = p[(int64_t)c * D];
    p[(int64_t)c * D] = run;
    run += v;
  }
}

// Tokens per wave of ll_ccq_combine and waves per workgroup (a workgroup
// holds whole chunks of up to 64 tokens).
constexpr int kCombineG = 8, kCombineNW = 8;
static_assert(64 / kCombineG <= kCombineNW, "a chunk of 64 tokens must fit one workgroup");

// One wave per 8 tokens of a chunk (a chunk has 2, 4 or 8 such groups); a
// workgroup of 8 waves holds the same chunk of 8 / (CS / 8) heads, and
// consecutive workgroups go along the heads first, so that the waves in flight
// read rows of every head ([B, T, H, D] puts a token's heads side by side; one
// head's rows alone, 128 bytes every H * D elements, leave most HBM channels
// idle).  Rows come whole in 16-byte pieces: lane l holds piece l % LPR (VW
// elements) of row l / LPR of each load.  Per token t: the running key sum
// (the chunk's exclusive prefix, the key sums of the chunk's earlier groups
// from LDS, the earlier rows of the group by a scan over the lanes),
// mu = ksum / (t+1), Sigma q = kkq / (t+1) - mu (mu . q), gamma =
// sigmoid(w_h . q + b_h); the two dot products are summed over the LPR lanes
// of the row.
template <typename T, int D>
__global__ void __launch_bounds__(64 * kCombineNW) ll_ccq_combine(int B, int T_, int H, int CS, const T* __restrict__ q,
                                                      const T* __restrict__ k, const T* __restrict__ kkq,
                                                      const float* __restrict__ csum, const float* __restrict__ w,
                                                      const float* __restrict__ b_, T* __restrict__ q_clean) {
  constexpr int G = kCombineG, NW = kCombineNW;
  constexpr int VW = 16 / (int)sizeof(T), LPR = D / VW, RW = 64 / LPR;
  constexpr int RL = RW < G ? RW : G;  // rows per load
  constexpr int NL = G / RL;           // loads per tensor
  static_assert(D % VW == 0 && 64 % LPR == 0 && G % RL == 0, "a row is a whole number of 16-byte pieces");
  __shared__ float gsum[NW][D];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gpc = CS / G, nch = T_ / CS, hpw = NW / gpc;
  const int nhb = (H + hpw - 1) / hpw;
  const unsigned blk = blockIdx.x, bc = blk / (unsigned)nhb;
  const int hb = (int)(blk % (unsigned)nhb);
  const int c = (int)(bc % (unsigned)nch), bb = (int)(bc / (unsigned)nch);
  const int sub = wv % gpc, hw = hb * hpw + wv / gpc;
  const bool live = hw < H;
  const int h = live ? hw : 0;
  const int64_t chunk = ((int64_t)bb * H + h) * nch + c;
  const int t0 = c * CS + sub * G;
  const int64_t row0 = ((int64_t)bb * T_ + t0) * H + h;
  const int cp = lane % LPR, rl = lane / LPR;
  // Every load is in bounds (a wave past the last head reads head 0, a lane
  // past the last row of a load reads that row again), so that none waits
  // behind a branch; such lanes and waves store nothing.
  const bool lane_in = rl < RL;
  const int rlc = lane_in ? rl : RL - 1;
  u32x4 rq[NL], rk[NL], rz[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int64_t o = (row0 + (int64_t)(i * RL + rlc) * H) * D + cp * VW;
    rq[i] = *reinterpret_cast<const u32x4*>(q + o);
    rk[i] = *reinterpret_cast<const u32x4*>(k + o);
    rz[i] = *reinterpret_cast<const u32x4*>(kkq + o);
  }
  float pre[VW], wx[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) {
    pre[e] = csum[chunk * D + cp * VW + e];
    wx[e] = w[(int64_t)h * D + cp * VW + e];
  }
  const float bias = b_[h];
  // k summed over the rows of each load up to the lane's own (a scan over the
  // lanes, RL / 2, ..., 1 rows apart), and each load's total from its last row
  float kc[NL][VW], gt[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) gt[e] = 0.f;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    unpack_piece<T>(rk[i], kc[i]);
#pragma unroll
    for (int s = 1; s < RL; s <<= 1)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const float up = __shfl_up(kc[i][e], s * LPR, 64);
        kc[i][e] = rl >= s ? kc[i][e] + up : kc[i][e];
      }
  }
  float base[NL][VW];  // key sum of the group's rows before load i
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      base[i][e] = gt[e];
      gt[e] += __shfl(kc[i][e], (RL - 1) * LPR + cp, 64);
    }
  if (rl == 0)
#pragma unroll
    for (int e = 0; e < VW; ++e) gsum[wv][cp * VW + e] = gt[e];
  __syncthreads();
  float run0[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) run0[e] = pre[e];
  for (int s = 0; s < sub; ++s)
#pragma unroll
    for (int e = 0; e < VW; ++e) run0[e] += gsum[wv - sub + s][cp * VW + e];
  if (!live) return;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    float qv[VW], kq[VW], run[VW];
    unpack_piece<T>(rq[i], qv);
    unpack_piece<T>(rz[i], kq);
    float a = 0.f, bq = 0.f;
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      run[e] = run0[e] + base[i][e] + kc[i][e];
      a += run[e] * qv[e];
      bq += wx[e] * qv[e];
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      a += __shfl_xor(a, m, 64);
      bq += __shfl_xor(bq, m, 64);
    }
    const float inv = 1.f / (float)(t0 + i * RL + rlc + 1);
    const float mq = a * inv, gamma = 1.f / (1.f + __expf(-(bq + bias)));
    float out[VW];
#pragma unroll
    for (int e = 0; e < VW; ++e) out[e] = qv[e] - gamma * inv * (kq[e] - run[e] * mq);
    if (lane_in)
      *reinterpret_cast<u32x4*>(q_clean + (row0 + (int64_t)(i * RL + rl) * H) * D + cp * VW) = pack_piece<T>(out);
  }
}

template <typename T, int D>
static hipError_t launch_prepare_t(int B, int T_, int H, int CS, const void* k, float* csum, int64_t rows, int L,
                                   float* ones, float* zeros, hipStream_t s) {
  const int64_t items = (int64_t)B * H * (T_ / CS), n = rows * L;
  const int64_t sum_blocks = (items + 3) / 4, fill_blocks = (n / 4 + 255) / 256 < 8192 ? (n / 4 + 255) / 256 + 1 : 8192;
  if (sum_blocks + fill_blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(sum_blocks + fill_blocks));
  if ((reinterpret_cast<uintptr_t>(ones) | reinterpret_cast<uintptr_t>(zeros)) % 16 == 0)
    hipLaunchKernelGGL((ll_ccq_prepare<T, D, true>), grid, dim3(256), 0, s, B, T_, H, CS, static_cast<const T*>(k),
                       csum, (int)sum_blocks, n, rows, ones, zeros);
  else
    hipLaunchKernelGGL((ll_ccq_prepare<T, D, false>), grid, dim3(256), 0, s, B, T_, H, CS, static_cast<const T*>(k),
                       csum, (int)sum_blocks, n, rows, ones, zeros);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(ll_ccq_chunk_scan<D>, dim3((unsigned)(B * H)), dim3(1024), 0, s, T_ / CS, csum);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_combine_t(int B, int T_, int H, int CS, const void* q, const void* k, const void* kkq,
                                   const float* csum, const float* w, const float* b, void* qc, hipStream_t s) {
  const int hpw = kCombineNW / (CS / kCombineG);
  const int64_t blocks = (int64_t)B * (T_ / CS) * ((H + hpw - 1) / hpw);
  hipLaunchKernelGGL((ll_ccq_combine<T, D>), dim3((unsigned)blocks), dim3(64 * kCombineNW), 0, s, B, T_, H, CS,
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

hipError_t launch_ccq_prepare(int io, int D, int B, int T_, int H, int CS, const void* k, float* csum, int64_t rows,
                              int L, float* ones, float* zeros, hipStream_t s) {
  LL_CCQ_DISPATCH(launch_prepare_t, B, T_, H, CS, k, csum, rows, L, ones, zeros, s)
}

hipError_t launch_ccq_combine(int io, int D, int B, int T_, int H, int CS, const void* q, const void* k,
                              const void* kkq, const float* csum, const float* w, const float* b, void* qc,
                              hipStream_t s) {
  LL_CCQ_DISPATCH(launch_combine_t, B, T_, H, CS, q, k, kkq, csum, w, b, qc, s)
}

}  // namespace llattn
