// ll_device.hpp -- device-side building blocks shared by the gfx950 kernels of
// libllattn: matrix-core (MFMA) fragments, chunk staging into LDS, the
// in-chunk gate prefix, and the tile layout of key-value states.
//
// MFMA conventions (CDNA3/CDNA4 16x16 shapes, wave64):
//   accumulator f32x4 of a 16x16 tile: lane l holds rows 4*(l/16)+i (i=0..3)
//   of column l%16.  One MFMA step contracts KS values of the k axis; lane l
//   supplies, for row/column l%16, the k indices kidx(step, l/16, e).
// Every contraction here uses the same k order, chosen so that a 16-row
// accumulator tile can be fed back as the k axis of the next product without
// a trip through LDS: for bf16 (v_mfma_f32_16x16x32_bf16) step s covers the
// rows of accumulator tiles 2s and 2s+1, for fp32 (v_mfma_f32_16x16x4_f32)
// step s covers one row per lane group of tile s/4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ll_launch.hpp"

namespace llattn {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int ilog2c(int x) { return 31 - __clz(x); }

template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KS = 32;  // k values per MFMA step
  typedef bf16x8 Frag;
  __device__ __forceinline__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // k index carried by element e (0..7) of lane group g in step s
  __device__ __forceinline__ static int kidx(int s, int g, int e) {
    return 32 * s + 16 * (e >> 2) + 4 * g + (e & 3);
  }
  // fragment whose k axis runs along a contiguous row (row + kidx(s, g, e))
  __device__ __forceinline__ static Frag row_frag(const bf16* row, int s, int g) {
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * s + 4 * g);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * s + 16 + 4 * g);
    return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // same, each element multiplied by w[kidx] (w in LDS, fp32)
  __device__ __forceinline__ static Frag row_frag_scaled(const bf16* row, const float* w, int s, int g) {
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * s + 4 * g);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * s + 16 + 4 * g);
    f32x4 wl = *reinterpret_cast<const f32x4*>(w + 32 * s + 4 * g);
    f32x4 wh = *reinterpret_cast<const f32x4*>(w + 32 * s + 16 + 4 * g);
    Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = (bf16)((float)lo[e] * wl[e]);
      f[4 + e] = (bf16)((float)hi[e] * wh[e]);
    }
    return f;
  }
  // fragment from accumulator tiles: tiles[t] are 16-row tiles along k
  __device__ __forceinline__ static Frag acc_frag(const f32x4* tiles, int s) {
    const f32x4 a = tiles[2 * s], b = tiles[2 * s + 1];
    return Frag{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  }
  // highest 16-row tile index that step s touches
  __device__ __forceinline__ static constexpr int last_tile(int s) { return 2 * s + 1; }
  __device__ __forceinline__ static constexpr int first_tile(int s) { return 2 * s; }
};

template <>
struct Mma<float> {
  static constexpr int KS = 4;
  typedef float Frag;
  __device__ __forceinline__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static int kidx(int s, int g, int) { return 16 * (s >> 2) + 4 * g + (s & 3); }
  __device__ __forceinline__ static Frag row_frag(const float* row, int s, int g) { return row[kidx(s, g, 0)]; }
  __device__ __forceinline__ static Frag row_frag_scaled(const float* row, const float* w, int s, int g) {
    const int k = kidx(s, g, 0);
    return row[k] * w[k];
  }
  __device__ __forceinline__ static Frag acc_frag(const f32x4* tiles, int s) { return tiles[s >> 2][s & 3]; }
  __device__ __forceinline__ static constexpr int last_tile(int s) { return s >> 2; }
  __device__ __forceinline__ static constexpr int first_tile(int s) { return s >> 2; }
};

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
  return (float)x;
}
template <typename T>
__device__ __forceinline__ T from_f32(float x) {
  return (T)x;
}

// ---------------------------------------------------------------- XCD order
// Workgroup ids are dealt round-robin to the 8 XCDs of the chip; each XCD
// has its own L2.  Renumber so that consecutive logical ids (the blocks of
// one head, which share Fenwick nodes) run on the same XCD.
__device__ __forceinline__ int xcd_logical_id(int hw_id, int n) {
  constexpr int kXcd = 8;
  if (n % kXcd != 0) return hw_id;
  return (hw_id % kXcd) * (n / kXcd) + hw_id / kXcd;
}

// ------------------------------------------------------------ state layout
// A dk x dv fp32 state is stored as 16x16 tiles in accumulator order:
// tile (dt, nt) at ((dt * (dv/16) + nt) * 64 + lane) * 4 floats, so that
// one wave moves a whole tile with one 16-byte access per lane.  Element
// (d, n) lives in tile (d/16, n/16), lane 16*((d%16)/4) + n%16, slot d%4.
template <int D>
__device__ __forceinline__ int state_tile_offset(int dt, int nt, int lane) {
  return ((dt * (D / 16) + nt) * 64 + lane) * 4;
}

// --------------------------------------------------------- chunk staging
// LDS image of one chunk of C tokens of one head.
template <typename T, int D, int C>
struct ChunkTiles {
  static constexpr int RP = D + 4;  // padded row of q / k (k axis = head dim)
  static constexpr int TP = C + 4;  // padded row of k^T / v^T (k axis = tokens)
  T q[C][RP];
  T k[C][RP];
  T kt[D][TP];
  T vt[D][TP];
  float lam[C * kLevelsMax];
  float gcum[C];  // inclusive prefix of log a inside the chunk
  float wend[C];  // exp(G[C-1] - G[r]): decay from token r to the chunk end
};

// Loads rows [t0, t0+C) of head (b,h) of a [B,T,H,D] tensor into LDS.
// Row-major copy into `row` (if non-null) and transposed copy into `col`
// (if non-null).  16-byte global loads, one row segment per thread.
template <typename T, int D, int C, int RP, int TP>
__device__ __forceinline__ void stage_rows(const T* __restrict__ src, int64_t row_stride, T (*row)[RP],
                                           T (*col)[TP], int tid, int nthreads) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int VPR = D / EPV;         // vectors per row
  for (int vi = tid; vi < C * VPR; vi += nthreads) {
    const int r = vi / VPR, c0 = (vi % VPR) * EPV;
    const uint4 raw = *reinterpret_cast<const uint4*>(src + r * row_stride + c0);
    if (row) {
      uint2* dst = reinterpret_cast<uint2*>(&row[r][c0]);
      dst[0] = uint2{raw.x, raw.y};
      dst[1] = uint2{raw.z, raw.w};
    }
    if (col) {
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int j = 0; j < EPV; ++j) col[c0 + j][r] = e[j];
    }
  }
}

// Inclusive prefix sum of the chunk's log-gates (one wave, C <= 64 lanes),
// and the decay of every token to the chunk end.  Reads gcum[] holding the
// raw log-gates, rewrites it in place.  Call from one whole wave.
template <int C>
__device__ __forceinline__ void chunk_gate_prefix(float* gcum, float* wend, int lane) {
  float x = lane < C ? gcum[lane] : 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  const float total = __shfl(x, C - 1, 64);
  if (lane < C) {
    gcum[lane] = x;
    wend[lane] = __expf(total - x);
  }
}

}  // namespace llattn
