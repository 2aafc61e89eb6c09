// fenwick_scan.hip -- Fenwick combination of block states and state export
// ("Log-Linear Attention", section 2.2: the prefix is covered by power-of-two
// buckets of the Fenwick tree).
//
// Input: per head, the decayed key-value state S[e] of every block e and its
// gate sum GS[e] (from ll_chunk_state).  The Fenwick node stored at block
// index e covers blocks [e + 1 - 2^z, e], z = ctz(e+1):
//   node(e) = sum over those blocks b of exp(gates after b up to e) * S[b].
// z = 0 nodes are S[e] itself; ll_fenwick_scan builds the others (odd e) into
// F[e/2], GF[e/2].  A block J then reads, for each set bit of J, the node at
// e = (J with its lower bits cleared) - 1, exactly the buckets of section 2.2
// at block granularity.
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

constexpr int kScanDepth = 20;  // up to 2^20 blocks per head

// One thread per (head, four consecutive state elements, segment): the
// blocks of a head are split into NS aligned segments of 2^seg_log blocks, and
// each thread walks its segment in order, keeping the pending node of every
// level in registers (the same merge rule as a decode step, at block
// granularity).  The block states are read in batches of BATCH, all in flight
// at once: consecutive lanes read consecutive 16-byte pieces of one state, so
// every load and store instruction moves 1 KiB.
//
// A node whose run of blocks stays inside one segment is finished by that
// segment's thread.  The node at the last block of segment s covers
// 2^ctz(s+1) whole segments: the segment totals meet in LDS and the thread of
// segment s combines them, newest first, with the same merge rule.  Splitting
// into segments puts NS times more loads in flight when there are few heads.
constexpr int kScanThreads = 256;

template <int D, int NS, int BATCH>
__global__ void __launch_bounds__(kScanThreads) ll_fenwick_scan(PrefillArgs a, int seg_log) {
  constexpr int G = D * D / 4;  // 16-byte pieces per state
  constexpr int PW = kScanThreads / NS;  // pieces per workgroup, a multiple of the wave size
  static_assert(PW % 64 == 0, "a wave must stay inside one segment");
  __shared__ f32x4 tot[NS > 1 ? NS : 1][PW];
  __shared__ float gtot[NS > 1 ? NS : 1][PW];
  const int seg = threadIdx.x / PW, wl = threadIdx.x % PW;
  // the same head-to-XCD placement as ll_chunk_state (consecutive logical
  // workgroups on one XCD), so block states are read where they were written
  const int64_t piece = (int64_t)xcd_logical_id(blockIdx.x, gridDim.x) * PW + wl;
  const bool active = piece < (int64_t)a.B * a.H * G;
  const int bh = active ? (int)(piece / G) : 0, w = active ? (int)(piece % G) : 0;
  // With the bf16 copy (below) threads are ordered by its layout, w = ((nt
  // KSD + s) 64 + l) 2 + h: the thread takes lane l of tile (2s + h, nt) of
  // the state tile layout, so a wave reads and writes fp32 as two runs of 512
  // bytes and writes its bf16 copy as one run of 512 bytes.  Without it, w is
  // the tile layout itself (runs of 1 KiB).
  int el = w;
  if (D >= 32 && a.N16) {
    constexpr int NCT = D / 16, KSD = D >= 32 ? D / 32 : 1;
    const int h = w & 1, l = (w >> 1) & 63, f = w >> 7, nt = f / KSD, st = f % KSD;
    el = ((2 * st + h) * NCT + nt) * 64 + l;
  }
  const f32x4* __restrict__ S = reinterpret_cast<const f32x4*>(a.S) + (int64_t)bh * a.nb * G + el;
  const float* __restrict__ GS = a.GS + (int64_t)bh * a.nb;
  f32x4* __restrict__ F = reinterpret_cast<f32x4*>(a.F) + (int64_t)bh * a.nF * G + el;
  float* __restrict__ GF = a.GF + (int64_t)bh * a.nF;
  // bf16 copy of every node in MFMA fragment order: this thread's four values
  // are half h of lane l's fragment s for wave column nt
  bf16x4* N16 = nullptr;
  if constexpr (D >= 32) {
    if (a.N16) N16 = static_cast<bf16x4*>(a.N16) + (int64_t)bh * a.nb * G + w;
  }

  f32x4 stack[kScanDepth];
  float gstack[kScanDepth];
#pragma unroll
  for (int l = 0; l < kScanDepth; ++l) {
    stack[l] = f32x4{0.f, 0.f, 0.f, 0.f};
    gstack[l] = 0.f;
  }

  // this thread's blocks [e_begin, e_end); with one segment, all of them
  const int e_begin = NS > 1 ? seg << seg_log : 0;
  const int e_last = NS > 1 ? e_begin + (1 << seg_log) - 1 : -1;  // the segment's last block
  const int e_end = NS > 1 ? min(e_last + 1, a.nb) : a.nb;
  f32x4 total = f32x4{0.f, 0.f, 0.f, 0.f};
  float gtotal = 0.f;
  for (int e0 = e_begin; active && e0 < e_end; e0 += BATCH) {
    f32x4 in[BATCH];
    float gin[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int e = e0 + u;
      in[u] = e < e_end ? S[(int64_t)e * G] : f32x4{0.f, 0.f, 0.f, 0.f};
      gin[u] = e < e_end ? GS[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int e = e0 + u;
      if (e >= e_end) break;
      f32x4 cur = in[u];
      float gc = gin[u];
      // e0 is a multiple of the batch, so below its last step ctz(e+1) is a
      // compile-time constant and the level updates are straight-line code
      const int z = (u + 1 < BATCH) ? __builtin_ctz(u + 1) : __ffs(e + 1) - 1;
#pragma unroll
      for (int l = 0; l < kScanDepth; ++l) {
        if (l < z) {
          cur = __expf(gc) * stack[l] + cur;
          gc += gstack[l];
        }
      }
      if (e == e_last) {  // the whole segment: finished across segments below
        total = cur;
        gtotal = gc;
        break;
      }
      if (z > 0) {
        F[(int64_t)(e >> 1) * G] = cur;
        if (el == 0) GF[e >> 1] = gc;
      }
      if (N16) N16[(int64_t)e * G] = bf16x4{(bf16)cur[0], (bf16)cur[1], (bf16)cur[2], (bf16)cur[3]};
#pragma unroll
      for (int l = 0; l < kScanDepth; ++l) {
        if (l == z) {
          stack[l] = cur;
          gstack[l] = gc;
        }
      }
    }
  }
  if constexpr (NS > 1) {
    tot[seg][wl] = total;
    gtot[seg][wl] = gtotal;
    __syncthreads();
    if (active && e_last < a.nb) {
      // node at e_last: segments seg + 1 - 2^m .. seg, m = ctz(seg + 1)
      const int first = seg + 1 - (1 << __builtin_ctz(seg + 1));
      f32x4 cur = total;
      float gc = gtotal;
      for (int j = seg - 1; j >= first; --j) {
        cur = __expf(gc) * tot[j][wl] + cur;
        gc += gtot[j][wl];
      }
      F[(int64_t)(e_last >> 1) * G] = cur;
      if (el == 0) GF[e_last >> 1] = gc;
      if (N16) N16[(int64_t)e_last * G] = bf16x4{(bf16)cur[0], (bf16)cur[1], (bf16)cur[2], (bf16)cur[3]};
    }
  }
}

// Export of the per-level states in the decode layout.  Segment from
// position 0: for each set bit z of nb the node covering the aligned run of
// blocks ending at (nb with bits below z cleared) - 1, decayed to the last
// token; token level log2(C) + log2(P) + z + 1.  After a prior state (pos0 >
// 0, T <= lowbit(pos0)): the levels of pos0 + T -- the prior levels decayed
// through the segment (e^{sigma + segment gate sum} S_hat), and when
// T == lowbit(pos0) the carry: the segment's bucket merged with the run of
// prior levels from level log2(T) + 1 up into the next free level.  Every
// written level is a true state (its log-scale is 0, written by
// ll_sigma_zero after this kernel, since other workgroups still read the
// prior log-scales); the other levels are zeroed.  Each thread reads all its
// prior elements before it writes any, so the prior state may be the output.
template <int D>
__global__ void __launch_bounds__(256) ll_state_export(PrefillArgs a, int logCP) {
  constexpr int G = D * D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)a.B * a.H * G) return;
  const int bh = (int)(gid / G), grp = (int)(gid % G);
  const int lane = grp & 63, tile = grp >> 6;
  const int dt = tile / (D / 16), nt = tile % (D / 16);
  const int d0 = 16 * dt + 4 * (lane >> 4), n = 16 * nt + (lane & 15);
  float* out = a.state + (int64_t)bh * a.L * D * D;
  auto put = [&](int lvl, f32x4 v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(int64_t)lvl * D * D + (d0 + i) * D + n] = v[i];
  };
  auto node = [&](int e, f32x4& val, float& gam) {
    if (e & 1) {
      val = reinterpret_cast<const f32x4*>(a.F)[((int64_t)bh * a.nF + (e >> 1)) * G + grp];
      gam = a.GF[(int64_t)bh * a.nF + (e >> 1)];
    } else {
      val = reinterpret_cast<const f32x4*>(a.S)[((int64_t)bh * a.nb + e) * G + grp];
      gam = a.GS[(int64_t)bh * a.nb + e];
    }
  };

  // the segment's gate sum (over the set bits of nb: the nodes tile the blocks)
  float gseg = 0.f;
  for (int rest = a.nb; rest > 0; rest &= rest - 1) {
    const int e = rest - 1;
    gseg += (e & 1) ? a.GF[(int64_t)bh * a.nF + (e >> 1)] : a.GS[(int64_t)bh * a.nb + e];
  }

  uint64_t written = 0;
  const int segtop = logCP + 31 - __clz(a.nb) + 1;  // level of the segment's largest bucket
  const uint64_t prior = (uint64_t)a.pos0;
  // carry: T == lowbit(pos0), i.e. bit segtop - 1 of pos0 is set (nb is then a power of two)
  const bool carry = prior != 0 && ((prior >> (segtop - 1)) & 1);
  f32x4 merged = f32x4{0.f, 0.f, 0.f, 0.f};
  int carry_lvl = 0;
  if (prior != 0) {
    const float* Sp = a.state_in + (int64_t)bh * a.L * D * D;
    const float* sp = a.state_in + (int64_t)a.B * a.H * a.L * D * D + (int64_t)bh * a.L;
    int run_end = 0;  // levels segtop .. run_end - 1 are the carried run
    if (carry) {
      run_end = segtop;
      while (run_end <= 62 && ((prior >> (run_end - 1)) & 1)) ++run_end;
      carry_lvl = run_end;
    }
    for (uint64_t bits = prior; bits; bits &= bits - 1) {
      const int lvl = __ffsll((unsigned long long)bits);
      const float sc = __expf(sp[lvl] + gseg);
      f32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = sc * Sp[(int64_t)lvl * D * D + (d0 + i) * D + n];
      if (carry && lvl >= segtop && lvl < run_end) {
        merged += v;
      } else {
        put(lvl, v);
        written |= 1ull << lvl;
      }
    }
  }

  float dd = 0.f;
  for (int rest = a.nb; rest > 0; rest &= rest - 1) {
    const int e = rest - 1;
    const int z = __ffs(rest) - 1;
    f32x4 val;
    float gam;
    node(e, val, gam);
    const int lvl = logCP + z + 1;
    const float sc = __expf(dd);
    if (carry) {
      merged += sc * val;  // the only bucket: nb is a power of two
    } else {
      put(lvl, sc * val);
      written |= 1ull << lvl;
    }
    dd += gam;
  }
  if (carry) {
    put(carry_lvl, merged);
    written |= 1ull << carry_lvl;
  }
  for (int lvl = 0; lvl < a.L; ++lvl) {
    if ((written >> lvl) & 1) continue;
    put(lvl, f32x4{0.f, 0.f, 0.f, 0.f});
  }
}

// Log-scales of an exported state: all zero (true states).
__global__ void __launch_bounds__(256) ll_sigma_zero(float* sigma, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) sigma[i] = 0.f;
}

// Segments per head: enough threads to keep every CU loading (up to 2^17),
// each segment at least 8 blocks.  With segments the batch is 8 blocks (a
// segment takes several): the larger batches of the one-segment walk do not
// fit in registers next to the segment bookkeeping and spill.
template <int D>
hipError_t launch_scan_d(const PrefillArgs& a, hipStream_t s) {
  constexpr int G = D * D / 4;
  const int64_t pieces = (int64_t)a.B * a.H * G;
  int ns = 1;
  while (ns < 4 && pieces * ns < ((int64_t)1 << 17) && (a.nb + 2 * ns - 1) / (2 * ns) >= 8) ns *= 2;
  int seg_log = 0;
  while ((int64_t)ns << seg_log < a.nb) ++seg_log;
  const int grid = (int)((pieces + kScanThreads / ns - 1) / (kScanThreads / ns));
  const dim3 g(grid), b(kScanThreads);
  if (ns == 1) {
    hipLaunchKernelGGL((ll_fenwick_scan<D, 1, 32>), g, b, 0, s, a, 30);
  } else if (ns == 2) {
    hipLaunchKernelGGL((ll_fenwick_scan<D, 2, 8>), g, b, 0, s, a, seg_log);
  } else {
    hipLaunchKernelGGL((ll_fenwick_scan<D, 4, 8>), g, b, 0, s, a, seg_log);
  }
  return hipGetLastError();
}

hipError_t launch_fenwick_scan(int D, const PrefillArgs& a, hipStream_t s) {
  switch (D) {
    case 16: return launch_scan_d<16>(a, s);
    case 32: return launch_scan_d<32>(a, s);
    case 64: return launch_scan_d<64>(a, s);
    case 128: return launch_scan_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_state_export(int D, int C, const PrefillArgs& a, hipStream_t s) {
  const int64_t threads = (int64_t)a.B * a.H * D * D / 4;
  const int grid = (int)((threads + 255) / 256);
  const int logCP = ilog2_host(C) + ilog2_host(a.P);
  switch (D) {
    case 16: hipLaunchKernelGGL((ll_state_export<16>), dim3(grid), dim3(256), 0, s, a, logCP); break;
    case 32: hipLaunchKernelGGL((ll_state_export<32>), dim3(grid), dim3(256), 0, s, a, logCP); break;
    case 64: hipLaunchKernelGGL((ll_state_export<64>), dim3(grid), dim3(256), 0, s, a, logCP); break;
    case 128: hipLaunchKernelGGL((ll_state_export<128>), dim3(grid), dim3(256), 0, s, a, logCP); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ns = (int64_t)a.B * a.H * a.L;
  float* sigma = a.state + (int64_t)a.B * a.H * a.L * D * D;
  hipLaunchKernelGGL(ll_sigma_zero, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, s, sigma, ns);
  return hipGetLastError();
}

}  // namespace llattn
