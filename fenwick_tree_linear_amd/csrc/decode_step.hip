// decode_step.hip -- one recurrent decode step ("Log-Linear Attention",
// section 2.3: O(log T) state and work per generated token).
//
// Per head the state keeps one dk x dv fp32 matrix per level plus a log-scale
// sigma (true state = exp(sigma) * S_hat), so the per-token decay of every
// level costs one scalar add instead of a pass over the matrices.  At position
// pos:
//   sigma_l += log a_pos                                   (all levels)
//   o = lambda_0 (q.k) v + sum_{l: bit l-1 of pos} lambda_l exp(sigma_l) S_hat_l^T q
//   c = ctz(pos+1):  S_hat_{c+1} = k v^T + sum_{l=1..c} exp(sigma_l) S_hat_l,  sigma_{c+1} = 0
// For the Gated DeltaNet write the token writes its pseudo-value
//   u = beta (v - sum_l exp(sigma_l) S_hat_l^T k)
// (the levels partition the prefix, so their sum is the plain gated state) in
// place of v, in the level-0 term of o and in the merge.
// Levels 1..c are exactly the low set bits of pos, so the merge reuses the rows
// loaded for the read; they become empty (bit clear in pos+1) and are not
// rewritten.  Traffic per head: popcount(pos) level reads + one level write.
// Sequences of a batch may sit at different positions (read per sequence from
// device memory): each workgroup is one head of one sequence, so nothing else
// changes.
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

constexpr int kDecodeLevelsMax = 32;

template <typename T, int DK, int DV>
__global__ void __launch_bounds__(256) ll_decode_step(DecodeArgs a) {
  constexpr int NTH = (DK * DV / 4 < 256) ? DK * DV / 4 : 256;
  constexpr int CG = DV / 4;     // column groups of 4 floats
  constexpr int RG = NTH / CG;   // row groups
  constexpr int RPT = DK / RG;   // rows per thread
  static_assert(RG * RPT == DK && NTH >= 64 && NTH >= DV, "a state row group per thread");
  // levels whose rows are in flight together (at most 20 f32x4 rows per
  // thread, so that four workgroups fit a CU: all heads of the 32K decode
  // workload in one round)
  constexpr int kDecodeBatch = RPT >= 20 ? 1 : (20 / RPT < 5 ? 20 / RPT : 5);
  __shared__ float qs[DK], ks[DK], vs[DV], us[DV];
  __shared__ float lam[kDecodeLevelsMax], sig[kDecodeLevelsMax];
  __shared__ float qk_s;
  __shared__ __attribute__((aligned(16))) float red[RG][DV];
  __shared__ __attribute__((aligned(16))) float redk[RG][DV];  // Gated DeltaNet: the levels read by k

  const int bh = blockIdx.x;
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  const int L = a.L;
  float* Sh = a.state + (int64_t)bh * L * DK * DV;
  float* sigma = a.state + (int64_t)a.B * a.H * L * DK * DV + (int64_t)bh * L;
  // one position for the batch (checked by the host), or one per sequence
  // from device memory: a position whose successor state would not fit in L
  // levels (or a negative one) gives NaN outputs and leaves the state as it is
  const int64_t pos = a.pos_dev ? a.pos_dev[bh / a.H] : a.pos;
  if (pos < 0 || pos + 1 >= ((int64_t)1 << (L - 1))) {
    for (int x = tid; x < DV; x += NTH) static_cast<T*>(a.o)[(int64_t)bh * DV + x] = from_f32<T>(__builtin_nanf(""));
    return;  // the whole workgroup: pos is the same for every thread
  }
  const int c = __ffsll((unsigned long long)(pos + 1)) - 1;
  const bool gdn = a.beta != nullptr;

  // Non-empty levels l >= 1 are the set bits l-1 of pos.  The rows of the
  // first kDecodeBatch of them are put in flight before anything else, so
  // their latency overlaps the loads of the token's q, k, v and weights.
  uint64_t bits = (uint64_t)pos & ((L - 1 >= 64) ? ~0ull : ((1ull << (L - 1)) - 1));
  int lv[kDecodeBatch];
  f32x4 rows[kDecodeBatch][RPT];
#pragma unroll
  for (int u = 0; u < kDecodeBatch; ++u) {
    lv[u] = bits ? __ffsll((unsigned long long)bits) : 0;  // level = bit index + 1; 0 = none
    bits &= bits - 1;
    if (lv[u] == 0) continue;
    const float* lev = Sh + (int64_t)lv[u] * DK * DV + 4 * cg;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) rows[u][rr] = *reinterpret_cast<const f32x4*>(lev + (rr * RG + rg) * DV);
  }

  const T* q = static_cast<const T*>(a.q) + (int64_t)bh * DK;
  const T* k = static_cast<const T*>(a.k) + (int64_t)bh * DK;
  const T* v = static_cast<const T*>(a.v) + (int64_t)bh * DV;
  if (tid < 64) {
    // q.k by one wave: lane x holds q_x k_x (+ q_{x+64} k_{x+64}), then a butterfly
    float pk = 0.f;
    for (int x = tid; x < DK; x += 64) {
      const float qx = to_f32(q[x]), kx = to_f32(k[x]);
      qs[x] = qx;
      ks[x] = kx;
      pk += qx * kx;
    }
    for (int x = tid; x < DV; x += 64) vs[x] = to_f32(v[x]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) pk += __shfl_xor(pk, m, 64);
    if (tid == 0) qk_s = pk;
  }
  const float loga = a.g[bh];
  for (int x = tid; x < L; x += NTH) {
    lam[x] = a.lam[(int64_t)bh * L + x];
    sig[x] = sigma[x] + loga;
  }
  __syncthreads();

  f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 kpart = f32x4{0.f, 0.f, 0.f, 0.f};  // Gated DeltaNet: sum_l e^{sigma_l} S_hat_l^T k
  f32x4 msum[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) msum[rr] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (;;) {
#pragma unroll
    for (int u = 0; u < kDecodeBatch; ++u) {
      if (lv[u] == 0) continue;
      const int l = lv[u];
      const float decay = __expf(sig[l]);
      const float coef = lam[l] * decay;
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) part += (coef * qs[rr * RG + rg]) * rows[u][rr];
      if (gdn) {
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr) kpart += (decay * ks[rr * RG + rg]) * rows[u][rr];
      }
      if (l <= c) {
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr) msum[rr] += decay * rows[u][rr];
      }
    }
    if (!bits) break;
    // further levels (more than kDecodeBatch set bits), a batch at a time
#pragma unroll
    for (int u = 0; u < kDecodeBatch; ++u) {
      lv[u] = bits ? __ffsll((unsigned long long)bits) : 0;
      bits &= bits - 1;
      if (lv[u] == 0) continue;
      const float* lev = Sh + (int64_t)lv[u] * DK * DV + 4 * cg;
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) rows[u][rr] = *reinterpret_cast<const f32x4*>(lev + (rr * RG + rg) * DV);
    }
  }

  *reinterpret_cast<f32x4*>(&red[rg][4 * cg]) = part;
  if (gdn) *reinterpret_cast<f32x4*>(&redk[rg][4 * cg]) = kpart;
  __syncthreads();
  if (tid < DV) {
    float acc = 0.f;
    for (int r = 0; r < RG; ++r) acc += red[r][tid];
    // the value this token writes: v, or for Gated DeltaNet its pseudo-value
    // u = beta (v - S^T k) with S the decayed plain state (the sum of all levels)
    float u = vs[tid];
    if (gdn) {
      float sk = 0.f;
      for (int r = 0; r < RG; ++r) sk += redk[r][tid];
      u = a.beta[bh] * (vs[tid] - sk);
      us[tid] = u;
    }
    static_cast<T*>(a.o)[(int64_t)bh * DV + tid] = from_f32<T>(lam[0] * qk_s * u + acc);
  }
  if (gdn) __syncthreads();

  // merge into level c+1 (c + 1 <= L - 1 by the position check above)
  float* dst = Sh + (int64_t)(c + 1) * DK * DV + 4 * cg;
  const f32x4 vv = *reinterpret_cast<const f32x4*>(gdn ? &us[4 * cg] : &vs[4 * cg]);
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int d = rr * RG + rg;
    *reinterpret_cast<f32x4*>(dst + d * DV) = ks[d] * vv + msum[rr];
  }
  for (int x = tid; x < L; x += NTH) sigma[x] = (x == c + 1) ? 0.f : sig[x];
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int NTH = (DK * DV / 4 < 256) ? DK * DV / 4 : 256;
  hipLaunchKernelGGL((ll_decode_step<T, DK, DV>), dim3(a.B * a.H), dim3(NTH), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_decode_dv(int DV, const DecodeArgs& a, hipStream_t s) {
  switch (DV) {
    case 16: return launch_decode_t<T, DK, 16>(a, s);
    case 32: return launch_decode_t<T, DK, 32>(a, s);
    case 64: return launch_decode_t<T, DK, 64>(a, s);
    case 128: return launch_decode_t<T, DK, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_dk(int DK, int DV, const DecodeArgs& a, hipStream_t s) {
  switch (DK) {
    case 16: return launch_decode_dv<T, 16>(DV, a, s);
    case 32: return launch_decode_dv<T, 32>(DV, a, s);
    case 64: return launch_decode_dv<T, 64>(DV, a, s);
    case 128: return launch_decode_dv<T, 128>(DV, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_step(int io, int DK, int DV, const DecodeArgs& a, hipStream_t s) {
  return io == 1 ? launch_decode_dk<bf16>(DK, DV, a, s) : launch_decode_dk<float>(DK, DV, a, s);
}

}  // namespace llattn
