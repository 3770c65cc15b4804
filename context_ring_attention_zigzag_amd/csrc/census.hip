// Tile census of the bf16 forward pass: for every 256-query tile, how many
// 64-key tiles of all the ring's blocks the pass computes (kept) and how many
// of those need the element mask (masked); the rest are skipped, neither
// loaded nor computed. It runs the forward kernel's own classification
// (tile_class.h) with the forward kernel's thread-to-query mapping, so its
// counts are the forward pass's. Under the head-tail layout every rank keeps
// the same number of tiles ("Context Parallelism v.s. Sequence Parallelism
// (Megatron-LM)", "Implementation quirk: symmetric chunk assignment": the
// chunk pairing balances the lower-triangular causal work).
#include "common.h"
#include "tile_class.h"

namespace cpring {
namespace {

constexpr int kNW = tiles::kWaves;
constexpr int kThreads = 64 * kNW;

__global__ void __launch_bounds__(kThreads) tile_census_kernel(CensusArgs a) {
  __shared__ __attribute__((aligned(8))) uint8_t flags8[tiles::kSegTiles];
  __shared__ int32_t qrange[4][kNW];
  __shared__ int32_t wsum[2][kNW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qt = blockIdx.x;
  // the forward kernel's mapping: wave w, lane l owns query 32 * w + l % 32
  const int q_idx = qt * tiles::kQueryTile + wave * 32 + (lane & 31);
  const bool q_in = q_idx < a.Lq;
  int32_t qlow, qlim;
  tiles::query_window(a.q_pos, a.kw_lo, a.kw_hi, a.causal, q_idx, q_in, qlow, qlim);
  const tiles::QBounds qb = tiles::workgroup_bounds<kNW>(qlow <= qlim, qlow, qlim, qrange);

  int kept = 0, masked = 0;
  const int n_kt = (a.Lk + tiles::kKeyTile - 1) / tiles::kKeyTile;
  for (int t = 0; t < a.nblocks && qb.ub_max >= 0; ++t) {
    const int32_t* posb = a.kv_pos + (int64_t)t * a.Lk;
    for (int seg0 = 0; seg0 < n_kt; seg0 += tiles::kSegTiles) {
      const int nseg = min(tiles::kSegTiles, n_kt - seg0);
      __syncthreads();
      tiles::classify_key_tiles<kThreads, tiles::kKeyTile>(posb, seg0, nseg, a.Lk, qb, flags8);
      __syncthreads();
      for (int i = tid; i < nseg; i += kThreads) {
        const int f = flags8[i];
        kept += f & 1;
        masked += (f >> 1) & 1;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kept += __shfl_xor(kept, o);
    masked += __shfl_xor(masked, o);
  }
  if (lane == 0) {
    wsum[0][wave] = kept;
    wsum[1][wave] = masked;
  }
  __syncthreads();
  if (tid == 0) {
    int k = 0, m = 0;
    for (int w = 0; w < kNW; ++w) {
      k += wsum[0][w];
      m += wsum[1][w];
    }
    a.kept[qt] = k;
    a.masked[qt] = m;
  }
}

}  // namespace

hipError_t launch_tile_census(const CensusArgs& a, hipStream_t st) {
  const int nqt = (a.Lq + tiles::kQueryTile - 1) / tiles::kQueryTile;
  hipLaunchKernelGGL(tile_census_kernel, dim3((unsigned)nqt), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace cpring
