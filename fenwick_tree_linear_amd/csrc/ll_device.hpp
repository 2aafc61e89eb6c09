// ll_device.hpp -- device-side building blocks shared by the gfx950 kernels of
// libllattn: matrix-core (MFMA) fragments, asynchronous global->LDS staging of
// chunk tiles, fragment reads from swizzled LDS tiles (including the gfx950
// transposing LDS read), and the tile layout of key-value states.
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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ int ilog2c(int x) { return 31 - __clz(x); }

// Workgroup barrier that orders LDS accesses only.  Unlike __syncthreads()
// it does not wait for this wave's outstanding global loads, so direct
// global->LDS loads of the next chunk stay in flight across it.  (A release
// fence on LDS would wait for them too: the compiler counts direct loads as
// pending LDS writes.)  Only this wave's own LDS operations are drained; the
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
  __device__ __forceinline__ static constexpr int kidx(int s, int g, int e) {
    return 32 * s + 16 * (e >> 2) + 4 * g + (e & 3);
  }
  // fragment from accumulator tiles: tiles[t] are 16-row tiles along k
  __device__ __forceinline__ static Frag acc_frag(const f32x4* tiles, int s) {
    const f32x4 a = tiles[2 * s], b = tiles[2 * s + 1];
    return Frag{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  }
  __device__ __forceinline__ static constexpr int first_tile(int s) { return 2 * s; }
};

template <>
struct Mma<float> {
  static constexpr int KS = 4;
  typedef float Frag;
  __device__ __forceinline__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static constexpr int kidx(int s, int g, int) { return 16 * (s >> 2) + 4 * g + (s & 3); }
  __device__ __forceinline__ static Frag acc_frag(const f32x4* tiles, int s) { return tiles[s >> 2][s & 3]; }
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

// DPP move of a float within a wave (lanes without a source read 0).
template <int CTRL, int ROW_MASK, bool ZERO_FILL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, ZERO_FILL));
}

// Inclusive prefix sum over lanes 0..C-1 of a wave (C <= 64; lanes at or past C
// must hold 0).  DPP shifts inside each 16-lane row, then the last lane of each
// row is broadcast to the rows above it: no LDS round trips.
template <int C>
__device__ __forceinline__ float chunk_scan(float x) {
  x += dpp_f32<0x111, 0xf, true>(x);  // row_shr:1
  x += dpp_f32<0x112, 0xf, true>(x);  // row_shr:2
  x += dpp_f32<0x114, 0xf, true>(x);  // row_shr:4
  x += dpp_f32<0x118, 0xf, true>(x);  // row_shr:8
  if (C > 16) x += dpp_f32<0x142, 0xa, false>(x);  // row_bcast:15 into rows 1 and 3
  if (C > 32) x += dpp_f32<0x143, 0xc, false>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// softplus(z) = log(1 + e^z), as max(z, 0) + log(1 + e^-|z|) so that large |z|
// neither overflows nor cancels; rounding 1 + x (x in (0, 1]) to fp32 costs at
// most 2^-24 in absolute terms, far below the weights' own size.  The
// logarithm's argument lies in (1, 2], so the hardware log2 (v_log_f32) serves
// as is, times ln 2, without the range scaling a general logf needs.
__device__ __forceinline__ float softplus_f32(float z) {
  return fmaxf(z, 0.f) + 0.693147180559945309f * __builtin_amdgcn_logf(1.f + __expf(-fabsf(z)));
}

// The level-weight MLP ("Adaptive memory decay for log-linear attention",
// section "Method", LambdaMLPSoftplus) has no activation between its two
// linear layers: h = d W1, lambda = softplus(h W2 + b).  So lambda =
// softplus(d Wc + b) with the composite Wc = W1 W2 (L x L): every kernel that
// makes level weights forms Wc once, with these same fp32 operations, and
// then one L x L product per row instead of the two layers.
// Element (k, n) of Wc (zero past L), summed over the hidden units in order.
__device__ __forceinline__ float mlp_composite(const float* w1, const float* w2, int L, int hidden, int k, int n) {
  float acc = 0.f;
  if (k < L && n < L)
    for (int j = 0; j < hidden; ++j) acc = fmaf(w1[k * hidden + j], w2[j * L + n], acc);
  return acc;
}
// One 16 x 16 tile of z = d Wc on the fp32 matrix cores over KSTEPS k steps of
// four levels, lane group g = l/16 taking the KSTEPS consecutive levels from
// KSTEPS g (so that a lane reads its row's levels as one run): a[s] =
// d[row l%16][KSTEPS g + s], b[s] = Wc[KSTEPS g + s][column l%16]; the even
// and odd steps in two accumulators, then summed (two dependent chains of half
// the length).  Lane l gets z[4(l/16) + i][l%16].
template <int KSTEPS>
__device__ __forceinline__ f32x4 mlp_tile_product(const float* a, const float* b) {
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) acc[s & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc[s & 1], 0, 0, 0);
  return acc[0] + acc[1];
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A raw buffer resource over `bytes` bytes from `base` (gfx9 descriptor:
// stride 0, range-checked against the byte count).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Tile (dt, nt) of an fp32 state through a buffer resource over the state.
// The tile's byte offset is the scalar offset of the load, so reading many
// tiles needs no 64-bit address per tile.
template <int D>
__device__ __forceinline__ f32x4 load_state_tile(__amdgpu_buffer_rsrc_t r, int dt, int nt, int lane) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, (dt * (D / 16) + nt) * 1024, 0));
}

// ------------------------------------------------------------ LDS tiles
// Row-major [ROWS][COLS] tile of T in LDS.  Rows are stored unpadded and the
// 16-byte chunks of row r are permuted by XOR with a key of r, so that the
// accesses of a fragment read spread over the 64 four-byte banks (256 bytes,
// RP = 256 / row-bytes rows).  The key is x = (r / RP) mod chunks-per-row
// with its bits rotated left by one: x alone keeps the 16 rows of a row-wise
// fragment read apart, and the rotation also keeps apart the rows r and r + 2
// that one 16-lane group of a transposing read takes the same two chunks of
// (with x alone they collided, two-way).
template <typename T, int ROWS, int COLS>
struct Tile {
  static constexpr int ESZ = sizeof(T);
  static constexpr int RB = COLS * ESZ;  // bytes per row
  static constexpr int NCH = RB / 16;    // 16-byte chunks per row
  static constexpr int BYTES = ROWS * RB;
  static constexpr int RP = RB >= 256 ? 1 : 256 / RB;  // rows per bank sweep
  static constexpr int KB = NCH >= 16 ? 4 : NCH >= 8 ? 3 : NCH >= 4 ? 2 : NCH >= 2 ? 1 : 0;  // key bits
  static_assert((NCH & (NCH - 1)) == 0 && NCH >= 1, "rows must be a power-of-two number of 16-byte chunks");
  __device__ __forceinline__ static int key(int row) {
    const int x = (row / RP) & (NCH - 1);
    if constexpr (KB > 1) {
      return ((x << 1) | (x >> (KB - 1))) & (NCH - 1);
    } else {
      return x;
    }
  }
  __device__ __forceinline__ static int pos(int row, int chunk) { return chunk ^ key(row); }
  // byte offset of element (row, col)
  __device__ __forceinline__ static int off(int row, int col) {
    const int byte = col * ESZ;
    return row * RB + (pos(row, byte >> 4) << 4) + (byte & 15);
  }
};

// Fragment whose k axis runs along a row: rows/columns of the MFMA tile are
// LDS rows `row`, k = columns kidx(s, g, .).
template <typename T, int ROWS, int COLS>
__device__ __forceinline__ typename Mma<T>::Frag frag_row(const char* lds, int row, int s, int g) {
  typedef Tile<T, ROWS, COLS> TL;
  if constexpr (sizeof(T) == 2) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(lds + TL::off(row, 32 * s + 4 * g));
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(lds + TL::off(row, 32 * s + 16 + 4 * g));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    return *reinterpret_cast<const float*>(lds + TL::off(row, Mma<float>::kidx(s, g, 0)));
  }
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16), issued as inline
// assembly.  Through the builtin, the compiler makes every such read wait for
// all outstanding direct global->LDS loads, since it cannot tell that they
// fill another buffer; that would serialise the next chunk's loads with the
// current chunk's work.  The compiler does not track this read: call
// lds_wait() on the result before using it.
__device__ __forceinline__ i16x4 ds_read_tr16(const char* lds) {
  i16x4 r;
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// Waits for this wave's LDS reads issued through inline assembly; the
// values passed in (arrays of fragments) are not used before the wait.
template <typename F, int N>
__device__ __forceinline__ void lds_pin(F (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(f[i]));
}
template <typename F, int N, int M>
__device__ __forceinline__ void lds_pin(F (&f)[N][M]) {
#pragma unroll
  for (int i = 0; i < N; ++i) lds_pin(f[i]);
}
template <typename... A>
__device__ __forceinline__ void lds_wait(A&... arrays) {
  asm volatile("s_waitcnt lgkmcnt(0)");
  (lds_pin(arrays), ...);
}

// Fragment whose k axis runs down the rows (tokens): the MFMA row/column is
// LDS column col0 + lane%16, k = rows kidx(s, lane/16, .).  For bf16 this is
// two gfx950 transposing reads: within each 16-lane group, lane q supplies the
// address of row base + q/4, columns col0 + 4*(q%4) .. +3, and receives
// column col0 + q of rows base .. base+3.  The bf16 result must pass through
// lds_wait() before use.
template <typename T, int ROWS, int COLS>
__device__ __forceinline__ typename Mma<T>::Frag frag_col(const char* lds, int col0, int s, int lane) {
  typedef Tile<T, ROWS, COLS> TL;
  const int g = lane >> 4, q = lane & 15;
  if constexpr (sizeof(T) == 2) {
    const int row = 32 * s + 4 * g + (q >> 2), col = col0 + 4 * (q & 3);
    const i16x4 lo = ds_read_tr16(lds + TL::off(row, col));
    const i16x4 hi = ds_read_tr16(lds + TL::off(row + 16, col));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  } else {
    return *reinterpret_cast<const float*>(lds + TL::off(Mma<float>::kidx(s, g, 0), col0 + q));
  }
}

// Multiplies element e of a fragment whose k axis is tokens by w[token(e)].
template <typename T>
__device__ __forceinline__ typename Mma<T>::Frag scale_tokens(typename Mma<T>::Frag f, const float* w, int s, int g) {
  if constexpr (sizeof(T) == 2) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(w + 32 * s + 4 * g);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(w + 32 * s + 16 + 4 * g);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (bf16)((float)f[e] * lo[e]);
      r[4 + e] = (bf16)((float)f[4 + e] * hi[e]);
    }
    return r;
  } else {
    return f * w[Mma<float>::kidx(s, g, 0)];
  }
}

// The direct global->LDS loads one wave issues for a chunk of one head.  The
// per-lane byte offsets (from the chunk's first row) are the same for every
// chunk and are computed once; per chunk only the scalar base pointers move.
//   tiles : C rows of D values at a stride of H*D, 1 KiB per instruction,
//           landing in the swizzled Tile layout (instruction i of the tile is
//           issued by wave i % NW)
//   gates : C floats at a stride of H (wave 0)
//   lambda: the first LS of the L level weights of each row, row-major [C][LS]
//           in LDS, 64 consecutive floats per instruction (instruction k by
//           wave k % NW)
__device__ __forceinline__ void load_lds16(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 16, 0, 0);
}

template <typename T, int D, int C, int NW>
struct ChunkLoads {
  typedef Tile<T, C, D> TL;
  static constexpr int NINST = TL::BYTES / 1024;
  static constexpr int TPW = (NINST + NW - 1) / NW;                        // tile instructions per wave
  static constexpr int LPW = (C * kLevelsMax + 64 * NW - 1) / (64 * NW);   // lambda instructions per wave, at most
  // lambda instructions whose lane offsets are held: those of up to 16 staged
  // levels; the others (more levels) form theirs at each use
  static constexpr int LPH = (C * 16 + 64 * NW - 1) / (64 * NW) < LPW ? (C * 16 + 64 * NW - 1) / (64 * NW) : LPW;
  static_assert(TL::BYTES % 1024 == 0 && 1024 % TL::RB == 0, "tile must be whole 1 KiB instructions");
  uint32_t tile_off[TPW], lam_off[LPH];
  int lam_n;  // lambda floats per chunk, C * LS

  __device__ __forceinline__ void init(int wv, int lane, int H, int L, int LS) {
    constexpr int RPI = 1024 / TL::RB;  // rows per instruction
    const int rl = lane / TL::NCH, p = lane % TL::NCH;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int row = (wv + k * NW) * RPI + rl;
      tile_off[k] = (uint32_t)(row * H * D * (int)sizeof(T) + TL::pos(row, p) * 16);
    }
    lam_n = C * LS;
#pragma unroll
    for (int k = 0; k < LPH; ++k) lam_off[k] = lam_offset((wv + k * NW) * 64 + lane, H, L, LS);
    h_ = H;
  }
  // byte offset of float f of a chunk's staged [C][LS] rows in the [rows][L] tensor
  __device__ __forceinline__ static uint32_t lam_offset(int f, int H, int L, int LS) {
    const int r = f / LS;
    return (uint32_t)((r * H * L + (f - r * LS)) * 4);
  }
  // a lane index formed where it is used (not held across the caller's loop)
  __device__ __forceinline__ static int lane_here() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  }
  // Every load goes through a buffer resource whose base is the chunk's first
  // element, so the per-lane offsets above stay 32-bit registers and moving to
  // another chunk is scalar work only.
  int h_;
  __device__ __forceinline__ void tiles_from(__amdgpu_buffer_rsrc_t rsrc, char* lds, int wv) const {
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int i = wv + k * NW;
      if (i < NINST) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + i * 1024), 16, tile_off[k], 0, 0, 0);
    }
  }
  __device__ __forceinline__ void tiles(const void* tensor, int64_t row0, char* lds, int wv) const {
    tiles_from(buffer_rsrc(static_cast<const char*>(tensor) + row0 * D * (int64_t)sizeof(T),
                           (uint32_t)(((C - 1) * h_ + 1) * D * (int)sizeof(T))),
               lds, wv);
  }
  __device__ __forceinline__ void gates(const float* g, int64_t row0, float* lds, int wv, int lane) const {
    if (wv == 0 && lane < C) {
      // the offset is formed here each time (an opaque copy of the lane keeps the
      // compiler from hoisting it into a register held, or spilled, across a loop)
      int l = lane;
      asm volatile("" : "+v"(l));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(g + row0, (uint32_t)(((C - 1) * h_ + 1) * 4)),
                                               (lds_void*)lds, 4, (uint32_t)(l * h_ * 4), 0, 0, 0);
    }
  }
  __device__ __forceinline__ void lambda_from(__amdgpu_buffer_rsrc_t rsrc, float* lds, int wv, int L) const {
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int first = (wv + k * NW) * 64;
      if (first < lam_n) {
        // the last, partial instruction (never at C = 64) and the offsets
        // that are not held are formed here, from a lane index made here, so
        // that no mask or offset is held (or spilled) across the caller's loop
        const bool held = k < LPH, whole = first + 64 <= lam_n;
        const int l = (held && whole) ? 0 : lane_here();
        const uint32_t off = held ? lam_off[held ? k : 0] : lam_offset(first + l, h_, L, lam_n / C);
        if (whole || l < lam_n - first)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + first), 4, off, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void lambda(const float* lam, int64_t row0, int L, float* lds, int wv, int lane) const {
    (void)lane;
    lambda_from(buffer_rsrc(lam + row0 * L, (uint32_t)(((C - 1) * h_ * L + lam_n / C) * 4)), lds, wv, L);
  }
};

}  // namespace llattn
