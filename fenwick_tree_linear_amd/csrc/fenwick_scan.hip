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

// One thread per (head, four consecutive state elements); walks the blocks
// of its head in order, keeping the pending node of every level in registers
// (the same merge rule as a decode step, at block granularity).  The block
// states are read in batches of kScanBatch, all in flight at once:
// consecutive lanes read consecutive 16-byte pieces of one state, so every
// load and store instruction moves 1 KiB.
constexpr int kScanBatch = 32;  // a power of two

template <int D>
__global__ void __launch_bounds__(256) ll_fenwick_scan(PrefillArgs a) {
  constexpr int G = D * D / 4;  // 16-byte pieces per state
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)a.B * a.H * G) return;
  const int bh = (int)(gid / G), w = (int)(gid % G);
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

  for (int e0 = 0; e0 < a.nb; e0 += kScanBatch) {
    f32x4 in[kScanBatch];
    float gin[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const int e = e0 + u;
      in[u] = e < a.nb ? S[(int64_t)e * G] : f32x4{0.f, 0.f, 0.f, 0.f};
      gin[u] = e < a.nb ? GS[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const int e = e0 + u;
      if (e >= a.nb) break;
      f32x4 cur = in[u];
      float gc = gin[u];
      // e0 is a multiple of the batch, so below its last step ctz(e+1) is a
      // compile-time constant and the level updates are straight-line code
      const int z = (u + 1 < kScanBatch) ? __builtin_ctz(u + 1) : __ffs(e + 1) - 1;
#pragma unroll
      for (int l = 0; l < kScanDepth; ++l) {
        if (l < z) {
          cur = __expf(gc) * stack[l] + cur;
          gc += gstack[l];
        }
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
}

// Export of the per-level states of [0,T) in the decode layout: for each set
// bit z of nb the node covering the aligned run of blocks ending at
// (nb with bits below z cleared) - 1, decayed to the last token; token level
// log2(C) + log2(P) + z + 1.  Other levels are written as zeros; all
// log-scales are 0.
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

  uint64_t written = 0;
  int rest = a.nb;
  float dd = 0.f;
  while (rest > 0) {
    const int e = rest - 1;
    const int z = __ffs(rest) - 1;
    f32x4 val;
    float gam;
    if (e & 1) {
      val = reinterpret_cast<const f32x4*>(a.F)[((int64_t)bh * a.nF + (e >> 1)) * G + grp];
      gam = a.GF[(int64_t)bh * a.nF + (e >> 1)];
    } else {
      val = reinterpret_cast<const f32x4*>(a.S)[((int64_t)bh * a.nb + e) * G + grp];
      gam = a.GS[(int64_t)bh * a.nb + e];
    }
    const int lvl = logCP + z + 1;
    const float sc = __expf(dd);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(int64_t)lvl * D * D + (d0 + i) * D + n] = sc * val[i];
    written |= 1ull << lvl;
    dd += gam;
    rest &= rest - 1;
  }
  for (int lvl = 0; lvl < a.L; ++lvl) {
    if ((written >> lvl) & 1) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(int64_t)lvl * D * D + (d0 + i) * D + n] = 0.f;
  }
  if (grp == 0) {
    float* sigma = a.state + (int64_t)a.B * a.H * a.L * D * D + (int64_t)bh * a.L;
    for (int lvl = 0; lvl < a.L; ++lvl) sigma[lvl] = 0.f;
  }
}

hipError_t launch_fenwick_scan(int D, const PrefillArgs& a, hipStream_t s) {
  const int64_t threads = (int64_t)a.B * a.H * D * D / 4;
  const int grid = (int)((threads + 255) / 256);
  switch (D) {
    case 16: hipLaunchKernelGGL((ll_fenwick_scan<16>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((ll_fenwick_scan<32>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((ll_fenwick_scan<64>), dim3(grid), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((ll_fenwick_scan<128>), dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
  return hipGetLastError();
}

}  // namespace llattn
