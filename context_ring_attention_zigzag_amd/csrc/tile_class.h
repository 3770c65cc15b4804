// Classification of (query tile, key tile) pairs from position ranges, shared
// by the bf16 forward kernel and the tile census kernel, so that the census
// counts exactly the tiles the forward pass computes.
//
// A key is allowed for a query when its position lies in the query's window
// [qlow, qlim]: the causal bound (key position <= query position, by global
// position: "Context Parallelism v.s. Sequence Parallelism (Megatron-LM)",
// "Implementation quirk: symmetric chunk assignment", where the allowed
// region of causal attention is lower-triangular) and the optional per-query
// key window; pad tokens (position -1) are never allowed. A key tile is
//   skipped  when no query of the workgroup may attend any of its keys,
//   full     when every live query may attend every key (no element mask),
//   masked   otherwise (kept, with the element mask).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "mfma_util.h"

namespace cpring {
namespace tiles {

// Tile sizes of the bf16 forward pass: a workgroup of 8 waves owns 256
// queries, keys stream in tiles of 64.
constexpr int kWaves = 8;
constexpr int kQueryTile = 32 * kWaves;
constexpr int kKeyTile = 64;
constexpr int kSegTiles = 4096;   // key tiles classified per segment of a block

// Window [qlow, qlim] of key positions query q_idx may attend; empty
// (qlow > qlim) for a pad query or an empty window. qlow >= 0, so pad keys
// always fall outside.
__device__ __forceinline__ void query_window(const int32_t* q_pos, const int32_t* kw_lo, const int32_t* kw_hi,
                                             int32_t causal, int q_idx, bool q_in, int32_t& qlow, int32_t& qlim) {
  const int32_t qp = q_in ? q_pos[q_idx] : -1;
  qlow = 0;
  qlim = -1;
  if (qp >= 0) {
    qlow = kw_lo ? max(kw_lo[q_idx], 0) : 0;
    qlim = causal ? qp : INT_MAX;
    if (kw_hi) qlim = min(qlim, kw_hi[q_idx]);
  }
}

// Bounds over the workgroup's live queries: the lowest and highest key
// position any query may attend (lb_min, ub_max) and every query may attend
// (lb_max, ub_min). Every thread of the NW-wave workgroup calls it; qrange
// holds 4 * NW ints of LDS scratch.
struct QBounds {
  int lb_min, lb_max, ub_min, ub_max;
};

template <int NW>
__device__ __forceinline__ QBounds workgroup_bounds(bool q_live, int32_t qlow, int32_t qlim, int32_t (*qrange)[NW]) {
  using namespace mfma;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w0 = wave_min(q_live ? qlow : INT_MAX), w1 = wave_max(q_live ? qlow : -1);
  const int w2 = wave_min(q_live ? qlim : INT_MAX), w3 = wave_max(q_live ? qlim : -1);
  if (lane == 0) {
    qrange[0][wave] = w0;
    qrange[1][wave] = w1;
    qrange[2][wave] = w2;
    qrange[3][wave] = w3;
  }
  __syncthreads();
  QBounds r{INT_MAX, -1, INT_MAX, -1};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    r.lb_min = min(r.lb_min, qrange[0][w]);
    r.lb_max = max(r.lb_max, qrange[1][w]);
    r.ub_min = min(r.ub_min, qrange[2][w]);
    r.ub_max = max(r.ub_max, qrange[3][w]);
  }
  return r;
}

// Flags of key tiles seg0 .. seg0 + nseg - 1 (kBN keys each) of a block of Lk
// keys with positions posb: flags8[t] bit 0 = kept, bit 1 = needs the element
// mask (a tile holding pads or keys past Lk, or one only some queries may
// attend fully). 16 lanes per tile, 4 positions each; every thread of the
// kThreads-thread workgroup calls it.
template <int kThreads, int kBN>
__device__ __forceinline__ void classify_key_tiles(const int32_t* posb, int seg0, int nseg, int Lk, const QBounds& qb,
                                                   uint8_t* flags8) {
  static_assert(kBN == 64, "16 lanes x 4 positions per tile");
  const int tid = threadIdx.x;
  for (int base = 0; base < nseg; base += kThreads / 16) {
    const int tt = base + (tid >> 4);
    const int g16 = tid & 15;
    int kmin = INT_MAX, kmax = -1, pad = 0;
    if (tt < nseg) {
      const int k0 = (seg0 + tt) * kBN + 4 * g16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = k0 + e;
        if (j < Lk) {
          const int p = posb[j];
          pad |= p < 0;
          kmin = (p >= 0 && p < kmin) ? p : kmin;
          kmax = p > kmax ? p : kmax;
        } else {
          pad = 1;
        }
      }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      kmin = min(kmin, __shfl_xor(kmin, o));
      kmax = max(kmax, __shfl_xor(kmax, o));
      pad |= __shfl_xor(pad, o);
    }
    if (g16 == 0 && tt < nseg) {
      // kept when the tile's positions meet some query's allowed range; full
      // when every live query may attend every key of the tile
      const bool keep = kmax >= 0 && kmax >= qb.lb_min && kmin <= qb.ub_max;
      const bool full = !pad && kmin >= qb.lb_max && kmax <= qb.ub_min;
      flags8[tt] = (uint8_t)((keep ? 1 : 0) | ((keep && !full) ? 2 : 0));
    }
  }
}

}  // namespace tiles
}  // namespace cpring
