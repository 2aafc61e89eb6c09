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
// (ll_ccq_chunk_scan), and within the chunk the key sums of its earlier groups
// of 8 tokens plus a running sum over the group's own (ll_ccq_combine, one
// wave per group).
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// Fills the inputs of the prefill: level weights 1 and log-gates 0.  VEC: the
// buffers start on 16 bytes and take 4 values per store.
template <bool VEC>
__global__ void __launch_bounds__(256) ll_ccq_fill(int64_t n_ones, int64_t n_zeros, float* ones, float* zeros) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

// One wave per (b, h, chunk of CS tokens, CS a multiple of 16): the chunk's
// column sums of k, csum[b][h][c][x] (fp32), 16 rows loaded per round.  Waves
// go along the heads first (the rows in flight then cover every head).
template <typename T, int D>
__global__ void __launch_bounds__(256) ll_ccq_chunk_sum(int B, int T_, int H, int CS, const T* __restrict__ k,
                                                        float* __restrict__ csum) {
  constexpr int E = (D + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int nch = T_ / CS;
  const int64_t item = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
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

// Sums v[r] (r = 0..G-1, G a power of two up to 64) over the 64 lanes of the
// wave, halving the vector at each exchange (lanes with bit 5, 4, ... set keep
// the upper half): lane l ends with the total of v[l >> (6 - log2 G)].  Both
// halves are exchanged and the kept one chosen after the adds (a choice
// between two array slots would become an indexed read of the array).
template <int G>
__device__ __forceinline__ float wave_sum_rows(const float (&v)[G], int lane) {
  float a[G];
#pragma unroll
  for (int i = 0; i < G; ++i) a[i] = v[i];
  int m = 32;
#pragma unroll
  for (int n = G; n > 1; n >>= 1, m >>= 1) {
    const bool up = lane & m;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float lo = a[i] + __shfl_xor(a[i], m, 64), hi = a[n / 2 + i] + __shfl_xor(a[n / 2 + i], m, 64);
      a[i] = up ? hi : lo;
    }
  }
#pragma unroll
  for (; m >= 1; m >>= 1) a[0] += __shfl_xor(a[0], m, 64);
  return a[0];
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // a 16-byte piece of a row

// Orders the wave's LDS accesses around it: what a lane wrote before is seen
// by the other lanes of the wave after (a wave's LDS operations run in order;
// this waits for them and keeps the compiler from moving memory accesses
// across, without waiting for the wave's global loads in flight).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16-byte pieces of a G x D tile (one per lane and step, the last piece
// again past the end) through the wave's LDS tile into one column per lane:
// out[r][e] = tile[r][xl + e], or 0 on lanes past the last column.
template <typename T, int D, int G, int E, int NL, int CPW>
__device__ __forceinline__ void stage_columns(const u32x4 (&rr)[NL], u32x4* tw, const T* tile, int lane, int xl,
                                              bool lane_in, float (&out)[G][E]) {
#pragma unroll
  for (int i = 0; i < NL; ++i) tw[min(lane + 64 * i, CPW - 1)] = rr[i];
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float v = to_f32(tile[r * D + xl + e]);
      out[r][e] = lane_in ? v : 0.f;
    }
  wave_lds_sync();
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Tokens per wave of ll_ccq_combine (and their log2), waves per workgroup
// (a workgroup holds whole chunks of up to 64 tokens).
constexpr int kCombineLG = 3, kCombineG = 1 << kCombineLG, kCombineNW = 8;
static_assert(64 / kCombineG <= kCombineNW, "a chunk of 64 tokens must fit one workgroup");

// One wave per 8 tokens of a chunk (a chunk has 2, 4 or 8 such groups); a
// workgroup of 8 waves holds the same chunk of 8 / (CS / 8) heads, and consecutive
// workgroups go along the heads first, so that the waves in flight read rows
// of every head ([B, T, H, D] puts a token's heads side by side; one head's
// rows alone, 128 bytes every H * D elements, leave most HBM channels idle).  Lane l holds columns
// l*E .. l*E+E-1.  Per token t: the running key sum (the chunk's exclusive
// prefix, the key sums of the chunk's earlier groups from LDS, and the
// group's tokens so far), mu = ksum / (t+1), Sigma q = kkq / (t+1) - mu (mu . q),
// gamma = sigmoid(w_h . q + b_h).  Rows are read and written in 16-byte
// pieces through an LDS tile per wave.  The two dot products of the 8 tokens are
// summed over the lanes together (wave_sum_rows), one token per 8 lanes, and
// taken back from those lanes as wave-uniform values.
template <typename T, int D>
__global__ void __launch_bounds__(64 * kCombineNW) ll_ccq_combine(int B, int T_, int H, int CS, const T* __restrict__ q,
                                                      const T* __restrict__ k, const T* __restrict__ kkq,
                                                      const float* __restrict__ csum, const float* __restrict__ w,
                                                      const float* __restrict__ b_, T* __restrict__ q_clean) {
  constexpr int E = (D + 63) / 64;
  constexpr int G = kCombineG, NW = kCombineNW, LG = kCombineLG;
  constexpr int VW = 16 / (int)sizeof(T), LPR = D / VW, CPW = G * LPR, NL = (CPW + 63) / 64;
  static_assert(D % VW == 0 && 64 % LPR == 0, "a row is a whole number of 16-byte pieces");
  __shared__ float gsum[NW][64 * E];
  __shared__ __align__(16) T tile[NW][G * D];
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
  // The group's rows of q, k and kkq come in 16-byte pieces (piece p: row
  // p / LPR, elements VW * (p % LPR) onward; a lane past the last piece takes
  // the last one again) and are turned to one column per lane through the
  // wave's LDS tile.  Every load is in bounds (a wave past the last head reads
  // head 0, a lane past the last column reads column 0), so that none waits
  // behind a branch; lanes past the last column then take zeros, and such
  // waves store nothing.
  const bool lane_in = lane * E < D;
  const int xl = lane_in ? lane * E : 0;
  u32x4 rq[NL], rk[NL], rz[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int pc = min(lane + 64 * i, CPW - 1);
    const int64_t o = (row0 + (int64_t)(pc / LPR) * H) * D + (pc % LPR) * VW;
    rq[i] = *reinterpret_cast<const u32x4*>(q + o);
    rk[i] = *reinterpret_cast<const u32x4*>(k + o);
    rz[i] = *reinterpret_cast<const u32x4*>(kkq + o);
  }
  u32x4* tw = reinterpret_cast<u32x4*>(&tile[wv][0]);
  float qv[G][E], kv[G][E], kq[G][E];
  stage_columns<T, D, G, E, NL, CPW>(rq, tw, &tile[wv][0], lane, xl, lane_in, qv);
  stage_columns<T, D, G, E, NL, CPW>(rk, tw, &tile[wv][0], lane, xl, lane_in, kv);
  stage_columns<T, D, G, E, NL, CPW>(rz, tw, &tile[wv][0], lane, xl, lane_in, kq);
  float run[E], wx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float a = csum[chunk * D + xl + e], b = w[(int64_t)h * D + xl + e];
    run[e] = lane_in ? a : 0.f;
    wx[e] = lane_in ? b : 0.f;
    float g = 0.f;
#pragma unroll
    for (int r = 0; r < G; ++r) g += kv[r][e];
    gsum[wv][lane * E + e] = g;
  }
  __syncthreads();
  for (int s = 0; s < sub; ++s)
#pragma unroll
    for (int e = 0; e < E; ++e) run[e] += gsum[wv - sub + s][lane * E + e];
  // The bias joins lane 0's share of w . q, so that its load goes out with
  // the others rather than after the sums over the lanes.
  const float bh_ = b_[h];
  const float bias = lane == 0 ? bh_ : 0.f;
  float mq[G], wq[G], run0[E];
#pragma unroll
  for (int e = 0; e < E; ++e) run0[e] = run[e];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const float inv = 1.f / (float)(t0 + r + 1);
    mq[r] = 0.f;
    wq[r] = bias;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      run[e] += kv[r][e];
      mq[r] += run[e] * inv * qv[r][e];
      wq[r] += wx[e] * qv[r][e];
    }
  }
  const float mq_l = wave_sum_rows<G>(mq, lane);
  const float gamma_l = 1.f / (1.f + __expf(-wave_sum_rows<G>(wq, lane)));
  if (!live) return;
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const float inv = 1.f / (float)(t0 + r + 1);
    const float m = lane_value(mq_l, r << (6 - LG)), g = lane_value(gamma_l, r << (6 - LG));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      run0[e] += kv[r][e];  // the running key sum again, as in the first pass
      if (lane_in) tile[wv][r * D + xl + e] = from_f32<T>(qv[r][e] - g * (kq[r][e] * inv - run0[e] * inv * m));
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int pc = min(lane + 64 * i, CPW - 1);
    *reinterpret_cast<u32x4*>(q_clean + (row0 + (int64_t)(pc / LPR) * H) * D + (pc % LPR) * VW) = tw[pc];
  }
}

hipError_t launch_ccq_fill(int64_t rows, int L, float* ones, float* zeros, hipStream_t s) {
  const int64_t n = rows * L;
  const int grid = (int)((n / 4 + 255) / 256 < 8192 ? (n / 4 + 255) / 256 + 1 : 8192);
  if ((reinterpret_cast<uintptr_t>(ones) | reinterpret_cast<uintptr_t>(zeros)) % 16 == 0)
    hipLaunchKernelGGL(ll_ccq_fill<true>, dim3(grid), dim3(256), 0, s, n, rows, ones, zeros);
  else
    hipLaunchKernelGGL(ll_ccq_fill<false>, dim3(grid), dim3(256), 0, s, n, rows, ones, zeros);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_ksum_t(int B, int T_, int H, int CS, const void* k, float* csum, hipStream_t s) {
  const int64_t items = (int64_t)B * H * (T_ / CS);
  hipLaunchKernelGGL((ll_ccq_chunk_sum<T, D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, B, T_, H, CS,
                     static_cast<const T*>(k), csum);
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

hipError_t launch_ccq_ksum(int io, int D, int B, int T_, int H, int CS, const void* k, float* csum, hipStream_t s) {
  LL_CCQ_DISPATCH(launch_ksum_t, B, T_, H, CS, k, csum, s)
}

hipError_t launch_ccq_combine(int io, int D, int B, int T_, int H, int CS, const void* q, const void* k,
                              const void* kkq, const float* csum, const float* w, const float* b, void* qc,
                              hipStream_t s) {
  LL_CCQ_DISPATCH(launch_combine_t, B, T_, H, CS, q, k, kkq, csum, w, b, qc, s)
}

}  // namespace llattn
