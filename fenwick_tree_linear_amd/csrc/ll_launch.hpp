// ll_launch.hpp -- host-side launch interface between the C ABI (api.cpp)
// and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llattn {

constexpr int kLevelsMax = 24;  // levels staged per chunk: positions < 2^23
// Largest chunk tile (C x d values) of the staged prefill pipeline, in bytes.
constexpr int kAttnTileBytesMax = 8192;

// Everything one prefill needs, with the workspace already carved up.
struct PrefillArgs {
  int B, T, H, L;
  int LS;    // levels staged per chunk: min(L, bit_length(T-1) + 1)
  int P;     // chunks per block (power of two)
  int nb;    // blocks per head = T / (C * P)
  int nF;    // Fenwick nodes of level >= 1 per head = nb / 2
  const void* q;
  const void* k;
  const void* v;
  const float* g;    // log-gates [B,T,H]
  const float* lam;  // [B,T,H,L]
  void* o;
  float* S;   // [B*H, nb, D*D] decayed key-value state of each block (tile layout)
  float* GS;  // [B*H, nb] sum of log-gates of each block
  float* F;   // [B*H, nF, D*D] Fenwick nodes of level >= 1 (odd block index e at e/2)
  float* GF;  // [B*H, nF]
  // with node_copies(): every Fenwick node (index e: S[e] for even e, F[e/2]
  // for odd e) as bf16 MFMA A fragments, [B*H, nb, D/16 wave columns, D/32
  // steps, 64 lanes, 8]; NULL otherwise
  void* N16;
  float* state;  // nullable export target [B,H,L,D,D] + sigma [B,H,L]
  // prefill from a state: the per-level states of the positions before the
  // segment in the decode layout, and the segment's first position (0: none)
  const float* state_in;
  int64_t pos0;
  // state_in when the read itself takes the levels of [0, pos0) (the
  // reader/maker read, with those levels among the staged ones; else NULL and
  // ll_prior_read adds them after the read)
  const float* prior = nullptr;
  // The level-weight MLP run inside the read (ll_chunk_attn_split only): when
  // w1 is set, lam holds the MLP's input d [B,T,H,L] instead of the weights,
  // and the read makes lambda = softplus((d W1) W2 + b) per chunk.
  const float* w1 = nullptr;  // [L, hidden]
  const float* w2 = nullptr;  // [hidden, L]
  const float* mlp_bias = nullptr;  // [L]
  int hidden = 0;
};

struct DecodeArgs {
  int B, H, L;
  int64_t pos;             // the position of every sequence, unless pos_dev is given
  const int64_t* pos_dev;  // nullable: device [B], one position per sequence
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* lam;
  const float* beta;  // Gated DeltaNet write strength [B,H]; NULL for the Mamba-2 write
  void* o;
  float* state;
};

// The Gated DeltaNet pseudo-value pass of a prefill (rows [B,T,H,D] in io dtype).
struct GdnArgs {
  int B, T, H;
  const void* k;
  const void* v;
  const float* g;     // log-gates [B,T,H]
  const float* beta;  // [B,T,H]
  void* W;            // (I + L)^-1 diag(beta e^G) K per chunk
  void* Up;           // (I + L)^-1 diag(beta) V per chunk
  void* U;            // pseudo-values, the values the log-linear read uses
  // a segment continuing a sequence: the per-level states of [0, pos0) in the
  // decode layout (L levels); the chunk recurrence starts from their sum
  int L;
  const float* state_in;
  int64_t pos0;
};

// Inputs and outputs of the backward pass.
struct BwdArgs {
  int B, T, H, D, L;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* lam;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  float* dlog_gate;
  float* dlambda;
};

// The forward's block decomposition of (k, v) that the backward reads: block
// states S/GS and Fenwick nodes F/GF as PrefillArgs holds them.
struct BwdFwdNodes {
  int nb, nF, P, LS;
  const float* S;
  const float* GS;
  const float* F;
  const float* GF;
};

// Scratch of the backward kernels.
struct BwdWork {
  float* dOo;      // [B,T,H] the cross-chunk part of dO_t . o_t
  float* din;      // [B,T,H] the in-chunk pairs' share of the gate gradient
  float* W;        // [B*H, nb, nbl, D*D] block shares of the reverse bucket states, then the bucket states
  float* BT;       // [B*H, nb] per block: sum of dO.o - v.dv over its cross-chunk pairs, then the sum over later blocks
  int nbl;         // block levels: bit_length(nb - 1)
  float* scratch;  // [B*H*nb, max_block_depth, D*D] chunk-level states of a walk, where they do not fit in LDS
};

// io: 0 = fp32, 1 = bf16.  Each returns hipSuccess or the launch error.
hipError_t launch_block_state(int io, int D, int C, const PrefillArgs& a, hipStream_t s);
hipError_t launch_chunk_attn(int io, int D, int C, const PrefillArgs& a, hipStream_t s);
hipError_t launch_fenwick_scan(int D, const PrefillArgs& a, hipStream_t s);
hipError_t launch_state_export(int D, int C, const PrefillArgs& a, hipStream_t s);
hipError_t launch_prior_read(int io, int D, int C, const PrefillArgs& a, hipStream_t s);
// pass: 0 the forward walk (dlambda, dq, the gate's in-chunk share; needs n
// built from (v, k)), 1 the reverse bucket states, 2 the reverse walk (dv, dk),
// 3 the gate's sum over later blocks
hipError_t launch_bwd_native(int io, int D, int C, const BwdArgs& a, const BwdFwdNodes& n, const BwdWork& w, int pass,
                             hipStream_t s);
// the prefill's level weights (1) and log-gates (0) for rows x L, and the
// exclusive per-chunk key sums of each head in csum
hipError_t launch_ccq_prepare(int io, int D, int B, int T, int H, int CS, const void* k, float* csum, int64_t rows,
                              int L, float* ones, float* zeros, hipStream_t s);
hipError_t launch_ccq_combine(int io, int D, int B, int T, int H, int CS, const void* q, const void* k,
                              const void* kkq, const float* csum, const float* w, const float* b, void* qc,
                              hipStream_t s);
hipError_t launch_decode_step(int io, int DK, int DV, const DecodeArgs& a, hipStream_t s);
// dst[i0][i1][i2][i3] = src[..] inside src's extents (s1, s2, s3), else 0; esz 2 or 4 bytes
hipError_t launch_pad_copy(int esz, const void* src, void* dst, int64_t n0, int s1, int s2, int s3, int d1, int d2,
                           int d3, hipStream_t s);
hipError_t launch_gdn_wy(int io, int D, int C, const GdnArgs& a, hipStream_t s);
hipError_t launch_gdn_state(int io, int D, int C, const GdnArgs& a, hipStream_t s);
hipError_t launch_lambda_mlp(int64_t rows, int L, int hidden, const float* d, const float* w1, const float* w2,
                             const float* bias, float* lam, hipStream_t s);

inline int ilog2_host(int x) {
  int r = 0;
  while (x > 1) {
    x >>= 1;
    ++r;
  }
  return r;
}

// largest within-block Fenwick depth the chunk kernels hold in registers
constexpr int max_block_depth(int /*D*/) { return 3; }
// The reader/maker read (bf16, square head D <= 64, chunks of at least 32)
// keeps four within-block levels, so its blocks hold up to 16 chunks (also
// when it runs the level-weight MLP); every other read and the backward up to
// 2^max_block_depth.
constexpr bool read_split(int io, int D, int C) { return io == 1 && D <= 64 && C >= 32; }
constexpr int read_block_depth(int io, int D, int C) { return read_split(io, D, C) ? 4 : max_block_depth(D); }
// Whether the read takes the levels of [0, pos0) of a segment that continues a
// sequence itself (the reader/maker read, while levels 0 .. bit_length(pos0)
// can be staged), so that no ll_prior_read follows it.
inline bool read_takes_prior(int io, int D, int C, int64_t pos0) {
  int bl = 0;
  while (bl < 63 && (pos0 >> bl) != 0) ++bl;
  return pos0 > 0 && read_split(io, D, C) && bl + 1 <= kLevelsMax;
}
// Whether the read runs the level-weight MLP itself (PrefillArgs::w1): bf16 in
// the run shape, square head D <= 64, chunk C >= 32, L <= 16 (any hidden size:
// the read applies the composite W1 W2).
inline bool read_runs_mlp(int io, int D, int C, int L, int hidden) {
  return read_split(io, D, C) && L <= 16 && hidden >= 1;
}

// LDS of the reader/maker read (bf16, head D, chunk C, within-block depth
// maxb, LS staged levels), byte offsets: the chunk staging ring (three stages
// of q, k and v tiles, gates and level-weight rows), the masked scores and the
// decay-scaled keys of two chunk parities, the in-chunk prefix arrays of two
// parities, the within-block states as bf16 MFMA fragments ([level][column
// tile][k step][lane], 1 KiB each); with the level-weight MLP, its composite
// weights and bias ([16][16], [16]) and a ring of two chunks of its input
// [C][16].
struct SplitLds {
  static constexpr int NS = 3;
  static constexpr int FRAG_BYTES = 64 * 16;
  static constexpr int MLP_W_BYTES = (16 * 16 + 16) * 4;
  int q = 0, k = 0, v = 0, g = 0, lraw = 0, stage = 0;
  int p = 0, kw = 0, gw = 0, st = 0, mw = 0, dr = 0, total = 0;
  __host__ __device__ constexpr SplitLds(int D, int C, int maxb, int LS, bool mlp) {
    const int tile = C * D * 2, scores = C * C * 2;
    q = 0;
    k = q + tile;
    v = k + tile;
    g = v + tile;
    lraw = g + C * 4;
    stage = (lraw + C * LS * 4 + 255) & ~255;
    p = NS * stage;
    kw = p + 2 * scores;
    gw = kw + 2 * tile;
    st = (gw + 2 * 3 * C * 4 + 255) & ~255;
    total = st + maxb * (D / 16) * (D / 32) * FRAG_BYTES;
    mw = dr = total;
    if (mlp) {
      dr = mw + MLP_W_BYTES;
      total = dr + 2 * C * 16 * 4;
    }
  }
};
constexpr int kLdsBytesMax = 160 * 1024;  // per workgroup on gfx950
// The largest reader/maker reads fit: 24 staged levels without the MLP, 16
// with it (the MLP takes L <= 16), both with four within-block levels.
static_assert(SplitLds(64, 64, 4, kLevelsMax, false).total <= kLdsBytesMax, "the split read fits LDS");
static_assert(SplitLds(64, 64, 4, 16, true).total <= kLdsBytesMax, "the split read with the MLP fits LDS");

// Whether the backward walks keep their chunk-level states in LDS (else in
// BwdWork::scratch).
constexpr bool bwd_states_in_lds(int D) { return D <= 64; }

// Whether the read takes the block-level Fenwick nodes from bf16 copies in
// fragment order (PrefillArgs::N16): for bf16 io at head sizes where no node
// is held in registers across a block, so that every chunk reads its nodes.
constexpr bool node_copies(int io, int D) { return io == 1 && D > 64; }

}  // namespace llattn
