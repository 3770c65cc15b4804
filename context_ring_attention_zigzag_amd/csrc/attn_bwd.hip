// Backward ring pass, bf16 on CDNA4 matrix cores (gfx950), plus the
// preprocessing shared with the fp32 path.
//
// What it computes: the gradients of the rank's attention output with respect
// to its queries and to every KV block it saw ("Context Parallelism", section
// "Practical use and trade-offs": the example differentiates the
// context-parallel output). With P = exp(scale * Q K^T - LSE) recomputed from
// the LSE the forward pass saved (exact, so no running max is needed), Dvec =
// rowsum(dO * O), dP = dO V^T and dS = P * (dP - Dvec):
//   dQ = scale * dS K      (stays on the rank; summed over the ring's blocks)
//   dK = scale * dS^T Q,  dV = P^T dO   (the rank's share of each block's
//   gradient, which travels around the ring with the block, "Sequence
//   Parallelism and Ring Attention", "Deep dive").
// Masking is the forward's: causal by global position, optional per-query key
// window, pads never attended.
//
// Mapping to the hardware:
//  * a preprocessing pass turns (O, dO, LSE) into per-row lse2 = LSE * log2(e)
//    and Dvec, and the positions into a per-query allowed window {lo, hi};
//  * every streamed tile is 32 rows, stored once in LDS, row-major with a
//    16-byte-chunk XOR swizzle chosen so that both access patterns are free of
//    bank conflicts: the row reads of an A operand (an LDS pass serves 16
//    lanes: 16 rows at one chunk) and the transposed reads (ds_read_b64_tr_b16,
//    a pass serves 32 lanes: 4 aligned rows at 4 aligned chunks) that give the
//    tile's transpose as an A operand;
//  * the dQ kernel: a workgroup owns 128 queries of one (b, h), each wave 32 of
//    them with Q and dO resident in VGPRs in the B-operand layout of
//    v_mfma_f32_32x32x16_bf16. Keys stream through LDS in tiles of 32 with
//    direct buffer->LDS loads, double-buffered. S^T = K Q^T and dP^T = V dO^T
//    put one query and 16 keys in each lane, so P^T and dS^T are lane-local and
//    leave the accumulators already in the B-operand layout of
//    dQ^T += K^T dS^T (v_cvt_pk_bf16_f32, round to nearest even), whose first
//    K^T fragments are read before the tile's vector work; two workgroups
//    share a CU;
//  * the dK/dV kernel: a workgroup owns 128 keys of one (b, kv head) as four
//    pairs of waves, 32 keys per pair, and streams query tiles (Q, dO, lse2,
//    Dvec, windows) of every query head of the grouped-query group through
//    four LDS buffers. The two waves of a pair share a SIMD and split the work
//    of each tile: role A computes S = Q K^T and P (masked) and dV^T += dO^T P
//    with K resident; role B computes dP = dO V^T and dS = P * (dP - Dvec) with
//    P handed over through LDS in float32, and dK^T += Q^T dS with V resident.
//    The roles alternate between matrix and vector work phase by phase, so one
//    wave's MFMAs run beside the other's exponentials or dS products;
//  * both kernels classify the streamed tiles against the rows they own from
//    position ranges (skip / full / masked) and walk an ordered list of the
//    kept ones, as the forward kernel does; the grid keeps the workgroups of
//    one head on one XCD.
#include <math.h>

#include "common.h"
#include "mfma_util.h"

namespace cpring {
namespace {

using namespace mfma;

constexpr int kT = 32;        // rows per streamed tile
constexpr int kListPad = 2;   // end markers after the last kept tile

template <int D>
struct BCfg {
  static constexpr int kKSteps = D / 16;   // MFMA steps over the head dim
  static constexpr int kDTiles = D / 32;   // 32-row tiles of a transposed gradient
  static constexpr int kChunks = D / 8;    // 16-byte chunks per row
  static constexpr int kTileLoads = kT * kChunks / 64;   // wave loads per tile
};

// Physical 16-byte chunk of logical chunk c in row r of a streamed tile. The
// XOR value is a permutation of the row's low bits: bits (r1, r0, r3, r2) for
// D = 128, whose rows are one 256-byte bank sweep each, so that the two low row
// bits pick the chunk quad; for D = 64, whose rows are half a sweep, a bit
// rotation of (r >> 1) & 7. Either way the 16 rows of a row-read pass at one
// chunk hit 16 distinct 16-byte bank groups, and so do the 4 aligned rows x 4
// aligned chunks of a 32-lane transposed pass.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    const int k = (r >> 1) & 7;
    return c ^ (((k & 1) << 2) | (k >> 1));
  }
}

// Element offset of (row r, column col) in a streamed tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * D + swz<D>(r, col >> 3) * 8 + (col & 7);
}

// Byte offset, within a 32-row tile of row stride `sl` elements, of the global
// 16-byte chunk that LDS chunk slot `sidx` of the tile holds.
template <int D>
__device__ __forceinline__ uint32_t dma_off(unsigned sidx, int64_t sl) {
  constexpr int kChunks = D / 8;
  const unsigned r = sidx / kChunks;
  return r * (uint32_t)sl * 2u + (uint32_t)swz<D>((int)r, (int)(sidx % kChunks)) * 16u;
}

// A-operand fragments of a tile: row ql, logical chunk 2 * kk + hh (8 columns
// of the contraction dim). The offsets are kept in bytes, so that a read is
// the lane register plus the array's address as an immediate, with no vector
// instruction in front of it (in a matrix phase those would wait behind the
// other wave's vector stream on the same SIMD).
template <int D>
struct RowFrags {
  int off[BCfg<D>::kKSteps];
  __device__ __forceinline__ void init(int ql, int hh) {
#pragma unroll
    for (int kk = 0; kk < BCfg<D>::kKSteps; ++kk) off[kk] = 2 * tile_off<D>(ql, 16 * kk + 8 * hh);
  }
  __device__ __forceinline__ bf16x8 get(const __bf16* tile, int kk) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + off[kk]);
  }
  // move every offset by d elements (to another tile buffer of the same array)
  __device__ __forceinline__ void shift(int d) {
#pragma unroll
    for (int kk = 0; kk < BCfg<D>::kKSteps; ++kk) off[kk] += 2 * d;
  }
};

// A-operand fragments of the transposed tile through two transposed reads:
// lane (column d = 32 * dt + lane % 32, half hh) gets rows 16c + 4hh + {0..3}
// and 16c + 8 + 4hh + {0..3}, the rows whose values a B operand packed from an
// accumulator chunk c holds for k = 8 * hh + {0..7}. Lane l reads row
// 4 * hh + ((l % 16) >> 2) and the 4 columns at 16 * ((l / 16) & 1) + 4 * (l % 4)
// of its d tile.
// Row r + 16 has the swizzle of row r, so chunk c = 1 sits 16 rows further.
template <int D>
struct TrFrags {
  int off[2][BCfg<D>::kDTiles];   // bytes, as in RowFrags
  __device__ __forceinline__ void init(int lane) {
    const int r = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < BCfg<D>::kDTiles; ++dt) {
      off[0][dt] = 2 * tile_off<D>(r, 32 * dt + col);
      off[1][dt] = 2 * tile_off<D>(r + 8, 32 * dt + col);
    }
  }
  __device__ __forceinline__ bf16x8 get(const __bf16* tile, int c, int dt) const {
    const char* t = reinterpret_cast<const char*>(tile);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + off[0][dt] + 32 * c * D));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + off[1][dt] + 32 * c * D));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  // see RowFrags::shift
  __device__ __forceinline__ void shift(int d) {
#pragma unroll
    for (int dt = 0; dt < BCfg<D>::kDTiles; ++dt) {
      off[0][dt] += 2 * d;
      off[1][dt] += 2 * d;
    }
  }
};

// 8 bf16 values of a 32x32 accumulator's chunk c (elements 8c .. 8c+7) as a B operand
__device__ __forceinline__ bf16x8 pack_chunk(const float (&x)[16], int c) {
  uint32_t w4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {(__bf16)x[8 * c + 2 * i], (__bf16)x[8 * c + 2 * i + 1]};
    w4[i] = __builtin_bit_cast(uint32_t, pr);
  }
  return __builtin_bit_cast(bf16x8, w4);
}

// A stream of N MFMAs whose A operands come from LDS: fragment m is read
// kPf MFMAs ahead of its use through a ring of kPf + 1 registers, and the
// read / MFMA order is pinned with scheduling-group barriers, so every MFMA
// finds its operand loaded instead of waiting out the LDS latency.
// fetch(m) returns fragment m (kReads LDS reads); mma(m, frag) issues MFMA m.
constexpr int kPf = 4;
template <int N, int kReads, typename Fetch, typename Mma>
__device__ __forceinline__ void mfma_stream(Fetch&& fetch, Mma&& mma) {
  bf16x8 fr[kPf + 1];
#pragma unroll
  for (int m = 0; m < kPf && m < N; ++m) fr[m] = fetch(m);
#pragma unroll
  for (int m = 0; m < N; ++m) {
    if (m + kPf < N) fr[(m + kPf) % (kPf + 1)] = fetch(m + kPf);
    mma(m, fr[m % (kPf + 1)]);
  }
#pragma unroll
  for (int m = 0; m < kPf && m < N; ++m) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReads, 0);
#pragma unroll
  for (int m = 0; m < N; ++m) {
    if (m + kPf < N) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReads, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
  }
}

// mfma_stream whose first kPf fragments the caller has already read into fr
// (before the barrier that opens the phase, so that the first MFMA does not
// wait out the LDS latency)
template <int N, int kReads, typename Fetch, typename Mma>
__device__ __forceinline__ void mfma_stream_pre(bf16x8 (&fr)[kPf + 1], Fetch&& fetch, Mma&& mma) {
  static_assert(N >= kPf, "the prefetched fragments belong to this stream");
#pragma unroll
  for (int m = 0; m < N; ++m) {
    if (m + kPf < N) fr[(m + kPf) % (kPf + 1)] = fetch(m + kPf);
    mma(m, fr[m % (kPf + 1)]);
  }
#pragma unroll
  for (int m = 0; m < N; ++m) {
    if (m + kPf < N) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReads, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
  }
}

// mfma_stream_pre with side(m) called after MFMA m
template <int N, int kReads, typename Fetch, typename Mma, typename Side>
__device__ __forceinline__ void mfma_stream_side_pre(bf16x8 (&fr)[kPf + 1], Fetch&& fetch, Mma&& mma, Side&& side) {
  static_assert(N >= kPf, "the prefetched fragments belong to this stream");
#pragma unroll
  for (int m = 0; m < N; ++m) {
    if (m + kPf < N) fr[(m + kPf) % (kPf + 1)] = fetch(m + kPf);
    mma(m, fr[m % (kPf + 1)]);
    side(m);
  }
}

// mfma_stream with side(m) called after MFMA m (e.g. to issue loads between MFMAs)
template <int N, int kReads, typename Fetch, typename Mma, typename Side>
__device__ __forceinline__ void mfma_stream_side(Fetch&& fetch, Mma&& mma, Side&& side) {
  bf16x8 fr[kPf + 1];
#pragma unroll
  for (int m = 0; m < kPf && m < N; ++m) fr[m] = fetch(m);
#pragma unroll
  for (int m = 0; m < N; ++m) {
    if (m + kPf < N) fr[(m + kPf) % (kPf + 1)] = fetch(m + kPf);
    mma(m, fr[m % (kPf + 1)]);
    side(m);
  }
}

// workgroup index -> logical index with the workgroups of one head on one XCD
__device__ __forceinline__ int xcd_logical(int w, int ntiles) {
  const int xcd = w % kXcds, idx = w / kXcds;
  const int per = ntiles / kXcds, rem = ntiles % kXcds;
  return xcd * per + min(xcd, rem) + idx;
}

// ---------------------------------------------------------------- prep pass

// One group of D*esize/16 lanes per query row: Dvec = sum over d of dO * O in
// fp32, lse2 = LSE * log2(e) (+inf when LSE = -inf); rows of head 0, batch 0
// also write the query's window.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdPrepArgs a) {
  constexpr int kPer = 16 / sizeof(T);   // elements per lane
  constexpr int kLanes = D / kPer;       // lanes per row
  const int64_t rows = (int64_t)a.B * a.H * a.Lq;
  const int64_t row = (int64_t)blockIdx.x * (256 / kLanes) + threadIdx.x / kLanes;
  const int sub = threadIdx.x % kLanes;
  float acc = 0.f;
  int64_t bh = 0, i = 0;
  if (row < rows) {
    bh = row / a.Lq;
    i = row - bh * a.Lq;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    const T* o = static_cast<const T*>(a.o) + b * a.o_sb + h * a.o_sh + i * a.o_sl + sub * kPer;
    const T* g = static_cast<const T*>(a.dout) + b * a.do_sb + h * a.do_sh + i * a.do_sl + sub * kPer;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(o);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(g);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
    } else {
      const float4 x = *reinterpret_cast<const float4*>(o);
      const float4 y = *reinterpret_cast<const float4*>(g);
      acc = fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, x.w * y.w)));
    }
  }
#pragma unroll
  for (int o = kLanes / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, kLanes);
  if (row >= rows || sub != 0) return;
  const float l = a.lse[row];
  a.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  a.dvec[row] = acc;
  if (bh == 0) {
    const int32_t qp = a.q_pos[i];
    int32_t lo = 1, hi = 0;   // empty
    if (qp >= 0) {
      lo = a.kw_lo ? max(a.kw_lo[i], 0) : 0;
      hi = a.causal ? qp : INT_MAX;
      if (a.kw_hi) hi = min(hi, a.kw_hi[i]);
    }
    a.qwin[i] = make_int2(lo, hi);
  }
}

// ---------------------------------------------------------------- dQ kernel

constexpr int kQWaves = 4;                    // 32 queries each
constexpr int kQThreads = 64 * kQWaves;
constexpr int kQOwn = 32 * kQWaves;           // queries per workgroup
constexpr int kQMaxTiles = 8 * kQThreads;     // key tiles classified per segment

template <int D, bool SPLIT>
__global__ void __launch_bounds__(kQThreads, 2) bwd_dq_kernel(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int kLoads = C::kTileLoads / kQWaves;   // per wave per tensor
  static_assert(kLoads >= 1 && C::kTileLoads % kQWaves == 0, "tile/waves mismatch");

  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kT * D];   // K tiles (S^T A operand, K^T reads)
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kT * D];   // V tiles (dP^T A operand)
  __shared__ __attribute__((aligned(16))) int32_t pos_lds[2][64];
  __shared__ __attribute__((aligned(8))) uint8_t flags8[kQMaxTiles];
  __shared__ uint16_t klist[kQMaxTiles + kListPad];
  __shared__ int32_t qrange[4][kQWaves];
  __shared__ int32_t wcount[kQWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31;
  const int hh = lane >> 5;

  const int nqt = (a.Lq + kQOwn - 1) / kQOwn;
  int logical = xcd_logical(blockIdx.x, gridDim.x);
  int slice = 0;   // key slice of a split launch; the slices of one query tile are adjacent
  if constexpr (SPLIT) {
    slice = logical % a.q_split;
    logical /= a.q_split;
  }
  const int bh = logical / nqt;
  const int qt = nqt - 1 - (logical - bh * nqt);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int q_idx = qt * kQOwn + wave * 32 + ql;
  const bool q_in = q_idx < a.Lq;
  const int64_t srow = (int64_t)bh * a.Lq + q_idx;

  int32_t qlow = 1, qlim = 0;
  float lse2 = INFINITY, dvec = 0.f;
  if (q_in) {
    const int2 w = a.qwin[q_idx];
    qlow = w.x;
    qlim = w.y;
    lse2 = a.lse2[srow];
    dvec = a.dvec[srow];
  }
  const bool q_live = qlow <= qlim;

  // bounds over the workgroup's live queries: the lowest and highest allowed
  // key position any query may attend (lb_min, ub_max) and every query may
  // attend (lb_max, ub_min)
  int lb_min, lb_max, ub_min, ub_max;
  {
    const int w0 = wave_min(q_live ? qlow : INT_MAX), w1 = wave_max(q_live ? qlow : -1);
    const int w2 = wave_min(q_live ? qlim : INT_MAX), w3 = wave_max(q_live ? qlim : -1);
    if (lane == 0) {
      qrange[0][wave] = w0;
      qrange[1][wave] = w1;
      qrange[2][wave] = w2;
      qrange[3][wave] = w3;
    }
    __syncthreads();
    lb_min = INT_MAX;
    lb_max = -1;
    ub_min = INT_MAX;
    ub_max = -1;
#pragma unroll
    for (int w = 0; w < kQWaves; ++w) {
      lb_min = min(lb_min, qrange[0][w]);
      lb_max = max(lb_max, qrange[1][w]);
      ub_min = min(ub_min, qrange[2][w]);
      ub_max = max(ub_max, qrange[3][w]);
    }
  }

  // resident Q and dO (B operands): d = 16 * kk + 8 * hh + e
  bf16x8 qf[C::kKSteps], gf[C::kKSteps];
  {
    const __bf16* qg = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)q_idx * a.q_sl;
    const __bf16* gg = static_cast<const __bf16*>(a.dout) + b * a.do_sb + h * a.do_sh + (int64_t)q_idx * a.do_sl;
    const s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk) {
      qf[kk] = q_in ? *reinterpret_cast<const bf16x8*>(qg + 16 * kk + 8 * hh) : __builtin_bit_cast(bf16x8, z);
      gf[kk] = q_in ? *reinterpret_cast<const bf16x8*>(gg + 16 * kk + 8 * hh) : __builtin_bit_cast(bf16x8, z);
    }
    ready(qf);
    ready(gf);
  }

  // dQ^T[d = 32 * dt + 8 * i + 4 * hh + j][query] in dqt[dt][4 * i + j]
  f32x16 dqt[C::kDTiles];
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqt[dt][i] = 0.f;

  const float c2 = a.scale * kLog2e;
  const int hk = h / (a.H / a.H_kv);
  const __bf16* kbh = static_cast<const __bf16*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const __bf16* vbh = static_cast<const __bf16*>(a.v) + b * a.v_sb + hk * a.v_sh;
  const int n_kt = (a.Lk + kT - 1) / kT;
  // key tiles of every block that this workgroup walks: all, or its slice
  int kt_lo = 0, kt_hi = n_kt;
  if constexpr (SPLIT) {
    kt_lo = (int)((int64_t)slice * n_kt / a.q_split);
    kt_hi = (int)((int64_t)(slice + 1) * n_kt / a.q_split);
  }
  // this wave's share of a tile: LDS chunk slots (wave * kLoads + i) * 64 + lane
  uint32_t k_off[kLoads], v_off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const unsigned sidx = (unsigned)((wave * kLoads + i) * 64 + lane);
    k_off[i] = dma_off<D>(sidx, a.k_sl);
    v_off[i] = dma_off<D>(sidx, a.v_sl);
  }
  RowFrags<D> rowf;
  rowf.init(ql, hh);
  TrFrags<D> trf;
  trf.init(lane);

  for (int t = 0; t < a.nblocks && ub_max >= 0; ++t) {
    int src = (a.rank - t) % a.cp;
    if (src < 0) src += a.cp;
    const int64_t row0 = (int64_t)src * a.Lk;
    const int32_t* posb = a.kv_pos + row0;
    const __bf16* kb = kbh + row0 * a.k_sl;
    const __bf16* vb = vbh + row0 * a.v_sl;

    for (int seg0 = kt_lo; seg0 < kt_hi; seg0 += kQMaxTiles) {
      const int nseg = min(kQMaxTiles, kt_hi - seg0);
      // ---- classify the segment's key tiles: 8 lanes per tile, 4 positions each
      bar();
      for (int base = 0; base < nseg; base += kQThreads / 8) {
        const int tt = base + (tid >> 3);
        const int g8 = tid & 7;
        int kmin = INT_MAX, kmax = -1, pad = 0;
        if (tt < nseg) {
          const int k0 = (seg0 + tt) * kT + 4 * g8;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = k0 + e;
            if (j < a.Lk) {
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
        for (int o = 4; o >= 1; o >>= 1) {
          kmin = min(kmin, __shfl_xor(kmin, o));
          kmax = max(kmax, __shfl_xor(kmax, o));
          pad |= __shfl_xor(pad, o);
        }
        if (g8 == 0 && tt < nseg) {
          const bool keep = kmax >= 0 && kmax >= lb_min && kmin <= ub_max;
          const bool full = !pad && kmin >= lb_max && kmax <= ub_min;
          flags8[tt] = (uint8_t)((keep ? 1 : 0) | ((keep && !full) ? 2 : 0));
        }
      }
      bar();
      const int nk = build_tile_list<kQWaves, kListPad>(flags8, nseg, klist, wcount);
      bar();
      if (nk == 0) continue;

      // ---- the wave's share of the loads of kept tile j into buffer `slot`
      auto issue = [&](int j, int slot) __attribute__((always_inline)) {
        const int r0 = (seg0 + j) * kT;
        const uint32_t rows = (uint32_t)min(kT, a.Lk - r0);
        const i32x4 rk = make_rsrc(kb + (int64_t)r0 * a.k_sl, rows * (uint32_t)a.k_sl * 2u);
        const i32x4 rv = make_rsrc(vb + (int64_t)r0 * a.v_sl, rows * (uint32_t)a.v_sl * 2u);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
          dma_b128(rk, k_off[i], lds_addr(&k_lds[slot][(wave * kLoads + i) * 512]));
          dma_b128(rv, v_off[i], lds_addr(&v_lds[slot][(wave * kLoads + i) * 512]));
        }
        if (wave == 0) dma_b32(make_rsrc(posb + r0, rows * 4u), (uint32_t)lane * 4u, lds_addr(&pos_lds[slot][0]));
      };

      // one kept tile u in buffer `slot`; the buffer index is a compile-time constant of each copy
      // of the body (the loop below takes two tiles per turn), so that every operand read is the
      // lane's offset plus the buffer's address as an immediate
      auto tile = [&](int u, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        const int e = __builtin_amdgcn_readfirstlane((int)klist[u]);
        const int en = __builtin_amdgcn_readfirstlane((int)klist[u + 1]);
        vm_wait<0>();
        bar();   // tile u is in LDS; every wave is done with buffer (u + 1) & 1
        if (u + 1 < nk) issue(en & 0x7fff, slot ^ 1);
        const __bf16* kl = &k_lds[slot][0];
        const __bf16* vl = &v_lds[slot][0];

        // S^T = K Q^T and dP^T = V dO^T for this tile's 32 keys, alternating
        f32x16 st = {}, pt = {};
        mfma_stream<2 * C::kKSteps, 1>(
            [&](int m) { return rowf.get((m & 1) ? vl : kl, m >> 1); },
            [&](int m, const bf16x8& a) {
              if (m & 1) pt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf[m >> 1], pt, 0, 0, 0);
              else st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[m >> 1], st, 0, 0, 0);
            });

        // the first fragments of the dQ stream (K^T of this tile) go out now and land during the
        // vector work below
        bf16x8 qfr[kPf + 1];
#pragma unroll
        for (int m = 0; m < kPf; ++m) qfr[m] = trf.get(kl, m / C::kDTiles, m % C::kDTiles);

        // lane: query ql, keys 8 * i + 4 * hh + jj of the tile (element 4 * i + jj)
        float s[16], ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = st[i];
        if (e & 0x8000) {
          const int32_t* pl = &pos_lds[slot][4 * hh];
          const int remh = a.Lk - (seg0 + (e & 0x7fff)) * kT - 4 * hh;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int4 p = *reinterpret_cast<const int4*>(pl + 8 * i);
            const int pk[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const bool ok = 8 * i + jj < remh && pk[jj] >= qlow && pk[jj] <= qlim;
              s[4 * i + jj] = ok ? s[4 * i + jj] : -INFINITY;
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lse2));
          ds[i] = p * (pt[i] - dvec);
        }
        const bf16x8 d0 = pack_chunk(ds, 0), d1 = pack_chunk(ds, 1);

        // dQ^T += K^T dS^T
        mfma_stream_pre<2 * C::kDTiles, 2>(
            qfr, [&](int m) { return trf.get(kl, m / C::kDTiles, m % C::kDTiles); },
            [&](int m, const bf16x8& a) {
              const int dt = m % C::kDTiles;
              dqt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, m < C::kDTiles ? d0 : d1, dqt[dt], 0, 0, 0);
            });
      };

      issue(klist[0] & 0x7fff, 0);
      for (int u = 0; u < nk; u += 2) {
        tile(u, ic<0>{});
        if (u + 1 < nk) tile(u + 1, ic<1>{});
      }
    }
  }

  if (!q_in) return;
  // a split launch writes its slice's partial dQ
  float* out = SPLIT ? a.dq_part + ((int64_t)slice * a.B * a.H * a.Lq + srow) * D : a.dq + srow * D;
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 x = make_float4(a.scale * dqt[dt][4 * i + 0], a.scale * dqt[dt][4 * i + 1], a.scale * dqt[dt][4 * i + 2],
                             a.scale * dqt[dt][4 * i + 3]);
      float4* p = reinterpret_cast<float4*>(out + 32 * dt + 8 * i + 4 * hh);
      if (!SPLIT && a.accumulate) {
        const float4 y = *p;
        x.x += y.x;
        x.y += y.y;
        x.z += y.z;
        x.w += y.w;
      }
      *p = x;
    }
}

// ------------------------------------------------------------- dK/dV kernel
//
// A workgroup owns 128 keys of one (b, kv head): eight waves, four pairs of 32
// keys. Wave s (role A, K resident, dV accumulated) and wave s + 4 (role B, V
// resident, dK accumulated) own the same keys and share SIMD s. Query tiles
// (items) run in phases separated by workgroup barriers, and in every phase one
// role works the matrix cores while the other works the vector ALU:
//   phase 2k:   A: S(k) = Q(k) K^T, then dV^T += dO(k-1)^T P(k-1),
//                  with the loads of item k + 2 between the MFMAs    [MFMA]
//               B: dS(k-1) = P(k-1) * (dP(k-1) - Dvec(k-1))          [VALU]
//   phase 2k+1: A: P(k) = 2^(S(k) c - lse2(k)), masked, handed to B
//                  through LDS in float32                            [VALU]
//               B: dP(k) = dO(k) V^T, then dK^T += Q(k-1)^T dS(k-1)  [MFMA]
// Items rotate through four LDS buffers. Phase 2k reads items k - 1 and k and
// loads item k + 2 into the buffer of item k - 2, whose last reader was phase
// 2k - 1; role A waits for those loads at the end of phase 2k + 1, so item
// k + 2 is visible from phase 2k + 2 on, two phases before its first reader.
// That slack lets each role read the first operand fragments of its next
// matrix phase before the barrier that opens it (role A at the start of its
// vector phase, role B at the end of its own), so that the first MFMA of a
// phase does not wait out the LDS latency.
constexpr int kKvWaves = 8;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvOwn = 128;                   // keys per workgroup, 32 per pair
constexpr int kKvMaxTiles = 8 * kKvThreads;   // query tiles classified per segment

template <int D, bool SPLIT>
__global__ void __launch_bounds__(kKvThreads, 1) bwd_dkv_kernel(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int kTileElems = kT * D;   // elements of one streamed tile buffer
  constexpr int kLoads = C::kTileLoads / 2;   // per role-A wave: two waves per tensor
  static_assert(kLoads >= 1 && C::kTileLoads % 2 == 0, "tile/waves mismatch");

  constexpr int kBufs = 4;   // item buffers: loads go out two items ahead
  __shared__ __attribute__((aligned(16))) __bf16 q_lds[kBufs][kT * D];   // Q tiles (S A operand, Q^T reads)
  __shared__ __attribute__((aligned(16))) __bf16 g_lds[kBufs][kT * D];   // dO tiles (dP A operand, dO^T reads)
  __shared__ __attribute__((aligned(16))) float l2_lds[kBufs][64];       // lse2 of the tile's queries (32 used)
  __shared__ __attribute__((aligned(16))) float dv_lds[kBufs][64];       // Dvec of the tile's queries (32 used)
  __shared__ __attribute__((aligned(16))) int2 qw_lds[kBufs][kT];        // {lo, hi} of the tile's queries
  __shared__ __attribute__((aligned(16))) float4 p_lds[4][4 * 64];   // P from role A to role B, per pair
  __shared__ __attribute__((aligned(8))) uint8_t flags8[kKvMaxTiles];
  __shared__ uint16_t klist[kKvMaxTiles + kListPad];
  __shared__ int32_t krange[3][kKvWaves];
  __shared__ int32_t wcount[kKvWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool role_a = wave < 4;
  const int pair = wave & 3;
  const int ql = lane & 31;   // key column owned by this lane
  const int hh = lane >> 5;

  const int64_t lk_total = (int64_t)a.nblocks * a.Lk;
  const int nkt = (int)((lk_total + kKvOwn - 1) / kKvOwn);
  int logical = xcd_logical(blockIdx.x, gridDim.x);
  int slice = 0;   // query slice of a split launch; the slices of one key tile are adjacent
  if constexpr (SPLIT) {
    slice = logical % a.kv_split;
    logical /= a.kv_split;
  }
  const int bhk = logical / nkt;
  const int kt = logical - bhk * nkt;
  const int b = bhk / a.H_kv;
  const int hk = bhk - b * a.H_kv;
  const int64_t k_idx = (int64_t)kt * kKvOwn + pair * 32 + ql;
  const bool k_in = k_idx < lk_total;
  const int32_t kp = k_in ? a.kv_pos[k_idx] : -1;

  // the workgroup's key range and whether it holds pads
  int kmin, kmax, anypad;
  {
    const int w0 = wave_min(kp >= 0 ? kp : INT_MAX), w1 = wave_max(kp);
    const int w2 = wave_max(kp < 0 ? 1 : 0);
    if (lane == 0) {
      krange[0][wave] = w0;
      krange[1][wave] = w1;
      krange[2][wave] = w2;
    }
    __syncthreads();
    kmin = INT_MAX;
    kmax = -1;
    anypad = 0;
#pragma unroll
    for (int w = 0; w < kKvWaves; ++w) {
      kmin = min(kmin, krange[0][w]);
      kmax = max(kmax, krange[1][w]);
      anypad |= krange[2][w];
    }
  }

  // resident B operands: K rows (role A) or V rows (role B), d = 16 * kk + 8 * hh + e
  bf16x8 rf[C::kKSteps];
  {
    const __bf16* src = role_a ? static_cast<const __bf16*>(a.k) + b * a.k_sb + hk * a.k_sh + k_idx * a.k_sl
                               : static_cast<const __bf16*>(a.v) + b * a.v_sb + hk * a.v_sh + k_idx * a.v_sl;
    const s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk)
      rf[kk] = k_in ? *reinterpret_cast<const bf16x8*>(src + 16 * kk + 8 * hh) : __builtin_bit_cast(bf16x8, z);
    ready(rf);
  }

  // dV^T (role A) or dK^T (role B) [d = 32 * dt + 8 * i + 4 * hh + j][key] in acc[dt][4 * i + j]
  f32x16 acc[C::kDTiles];
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  const float c2 = a.scale * kLog2e;
  const int group = a.H / a.H_kv;
  const int n_qt = (a.Lq + kT - 1) / kT;
  // query tiles this workgroup walks: all, or its slice
  int qt_lo = 0, qt_hi = n_qt;
  if constexpr (SPLIT) {
    qt_lo = (int)((int64_t)slice * n_qt / a.kv_split);
    qt_hi = (int)((int64_t)(slice + 1) * n_qt / a.kv_split);
  }
  // role A's share of an item's loads: Q (waves 0, 1) or dO (waves 2, 3), LDS
  // chunk slots ((wave & 1) * kLoads + i) * 64 + lane
  const bool load_q = wave < 2;
  uint32_t ld_off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
    ld_off[i] = dma_off<D>((unsigned)(((wave & 1) * kLoads + i) * 64 + lane), load_q ? a.q_sl : a.do_sl);
  RowFrags<D> rowf;
  rowf.init(ql, hh);
  TrFrags<D> trf;
  trf.init(lane);

  // The two roles run disjoint copies of the loop (a compile-time role), so
  // the register allocator never has to hold one role's temporaries while
  // the other's are live; both copies pass the same sequence of barriers.
  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool kA = decltype(role)::value;
    for (int seg0 = qt_lo; seg0 < qt_hi && kmax >= 0; seg0 += kKvMaxTiles) {
      const int nseg = min(kKvMaxTiles, qt_hi - seg0);
      // ---- classify the segment's query tiles: 8 lanes per tile, 4 queries each
      bar();
      for (int base = 0; base < nseg; base += kKvThreads / 8) {
        const int tt = base + (tid >> 3);
        const int g8 = tid & 7;
        int lbmin = INT_MAX, lbmax = -1, ubmin = INT_MAX, ubmax = -1, dead = 0;
        if (tt < nseg) {
          const int q0 = (seg0 + tt) * kT + 4 * g8;
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = q0 + e;
            if (j < a.Lq) {
              const int2 w = a.qwin[j];
              if (w.x <= w.y) {
                lbmin = min(lbmin, w.x);
                lbmax = max(lbmax, w.x);
                ubmin = min(ubmin, w.y);
                ubmax = max(ubmax, w.y);
              } else {
                dead = 1;
              }
            } else {
              dead = 1;
            }
          }
        }
  #pragma unroll
        for (int o = 4; o >= 1; o >>= 1) {
          lbmin = min(lbmin, __shfl_xor(lbmin, o));
          lbmax = max(lbmax, __shfl_xor(lbmax, o));
          ubmin = min(ubmin, __shfl_xor(ubmin, o));
          ubmax = max(ubmax, __shfl_xor(ubmax, o));
          dead |= __shfl_xor(dead, o);
        }
        if (g8 == 0 && tt < nseg) {
          // kept when some query of the tile may attend some key of the workgroup;
          // full when every query may attend every key (and there are no pads)
          const bool keep = ubmax >= 0 && kmax >= lbmin && kmin <= ubmax;
          const bool full = !dead && !anypad && kmin >= lbmax && kmax <= ubmin;
          flags8[tt] = (uint8_t)((keep ? 1 : 0) | ((keep && !full) ? 2 : 0));
        }
      }
      bar();
      const int nk = build_tile_list<kKvWaves, kListPad>(flags8, nseg, klist, wcount);
      bar();
      if (nk == 0) continue;
      const int nitems = nk * group;   // (kept tile, query head of the group), head fastest

      // role A's loads of item `item` into buffer item % kBufs, one at a time
      // (load n = 0 .. kLoads of this wave), so that they can go out between
      // the MFMAs of its matrix phase. They are issued whether or not the item
      // exists, so that the matrix phase is one branch-free block
      struct Plan {
        i32x4 rs, rx;
        uint32_t dst, dx;
      };
      // valid false: there is no such item; the descriptors are empty (the loads write zeros into its
      // buffer, which nothing reads), and the addresses come from item 0's list entry
      auto plan = [&](int item, bool valid) __attribute__((always_inline)) -> Plan {
        Plan pl;
        const int slot = item % kBufs;
        const int ia = valid ? item : 0;
        const int u = ia / group;
        const int h = hk * group + (ia - u * group);
        const int j = klist[u] & 0x7fff;
        const int q0 = (seg0 + j) * kT;
        const uint32_t rows = valid ? (uint32_t)min(kT, a.Lq - q0) : 0u;
        const __bf16* base = load_q
            ? static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)q0 * a.q_sl
            : static_cast<const __bf16*>(a.dout) + b * a.do_sb + h * a.do_sh + (int64_t)q0 * a.do_sl;
        pl.rs = make_rsrc(base, rows * (uint32_t)(load_q ? a.q_sl : a.do_sl) * 2u);
        pl.dst = lds_addr(load_q ? &q_lds[slot][0] : &g_lds[slot][0]) + (uint32_t)((wave & 1) * kLoads) * 1024u;
        const int64_t qrow = (int64_t)(b * a.H + h) * a.Lq + q0;
        if (wave == 0) {
          pl.rx = make_rsrc(a.lse2 + qrow, rows * 4u);
          pl.dx = lds_addr(&l2_lds[slot][0]);
        } else if (wave == 1) {
          pl.rx = make_rsrc(a.dvec + qrow, rows * 4u);
          pl.dx = lds_addr(&dv_lds[slot][0]);
        } else {
          pl.rx = make_rsrc(a.qwin + q0, rows * 8u);
          pl.dx = lds_addr(&qw_lds[slot][0]);
        }
        return pl;
      };
      auto load_n = [&](const Plan& pl, int n) __attribute__((always_inline)) {
        if (n < kLoads) dma_b128(pl.rs, ld_off[n], pl.dst + (uint32_t)n * 1024u);
        else if (wave < 3) dma_b32(pl.rx, (uint32_t)lane * 4u, pl.dx);
      };

      // One wave plays one role, so the roles share their per-item state:
      // sx holds S(k) (role A) or dP(k) (role B); bx0, bx1 the bf16 P of the
      // previous item (B operand of dV) or its bf16 dS (B operand of dK).
      f32x16 sx = {};
      bf16x8 bx0 = {}, bx1 = {};
      bf16x8 bfr[kPf + 1];   // the leading stream's first fragments, read before its phase opens

      // role A on the matrix cores: S(k) when WS, then dV(k - 1) when WV
      auto a_mfma = [&](int k, auto ws, auto wv) __attribute__((always_inline)) {
        constexpr bool kS = decltype(ws)::value, kV = decltype(wv)::value;
        constexpr int kNs = kS ? C::kKSteps : 0;
        constexpr int kN = kNs + (kV ? 2 * C::kDTiles : 0);
        // rowf points at buffer k % kBufs (Q(k)), trf at buffer (k - 1) % kBufs (dO(k - 1))
        const __bf16* qt_l = &q_lds[0][0];
        const __bf16* gt_l = &g_lds[0][0];
        const Plan pl = plan(k + 2, k + 2 < nitems);
        // load n of item k + 2 goes out after MFMA 1 + 3n: the address unit
        // drains while the matrix cores work instead of stalling a vector phase
        auto fetch = [&](int m) {
          if (m < kNs) return rowf.get(qt_l, m);
          const int mm = m - kNs;
          return trf.get(gt_l, mm / C::kDTiles, mm % C::kDTiles);
        };
        auto mma = [&](int m, const bf16x8& f) {
          if (m < kNs) {
            sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, rf[m], m == 0 ? f32x16{} : sx, 0, 0, 0);
          } else {
            const int mm = m - kNs, dt = mm % C::kDTiles;
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, mm < C::kDTiles ? bx0 : bx1, acc[dt], 0, 0, 0);
          }
        };
        auto side = [&](int m) {
          if (m % 3 == 1 && m / 3 <= kLoads) load_n(pl, m / 3);
        };
        if constexpr (kS) mfma_stream_side_pre<kN, kV ? 2 : 1>(bfr, fetch, mma, side);
        else mfma_stream_side<kN, kV ? 2 : 1>(fetch, mma, side);
        // the loads a short stream had no room for
#pragma unroll
        for (int n = 0; n <= kLoads; ++n)
          if (3 * n + 1 >= kN) load_n(pl, n);
      };

      // role A: P(k) = 2^(S(k) c - lse2(k)), masked; to LDS for role B, bf16 kept for dV(k).
      // Lane: key ql, queries 8 * i + 4 * hh + jj of the tile (element 4 * i + jj). The lse2 reads
      // (and the window reads of a masked tile) go out together before the first exponential, so
      // their latencies overlap; the P stores stay spread over the phase, one per group of four,
      // so that they do not arrive at the LDS as one burst beside role B's operand reads.
      auto a_valu = [&](int k) __attribute__((always_inline)) {
        const int slot = k % kBufs;
        const int e = __builtin_amdgcn_readfirstlane((int)klist[k / group]);
        float4 l2[4];
  #pragma unroll
        for (int i = 0; i < 4; ++i) l2[i] = *reinterpret_cast<const float4*>(&l2_lds[slot][8 * i + 4 * hh]);
        float p[16];
        if (e & 0x8000) {
          int4 w[8];
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            w[2 * i] = *reinterpret_cast<const int4*>(&qw_lds[slot][8 * i + 4 * hh]);
            w[2 * i + 1] = *reinterpret_cast<const int4*>(&qw_lds[slot][8 * i + 4 * hh + 2]);
          }
          const int remq = a.Lq - (seg0 + (e & 0x7fff)) * kT - 4 * hh;
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float l2v[4] = {l2[i].x, l2[i].y, l2[i].z, l2[i].w};
            const int lo[4] = {w[2 * i].x, w[2 * i].z, w[2 * i + 1].x, w[2 * i + 1].z};
            const int hi[4] = {w[2 * i].y, w[2 * i].w, w[2 * i + 1].y, w[2 * i + 1].w};
  #pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const bool ok = 8 * i + jj < remq && kp >= lo[jj] && kp <= hi[jj];
              const float e2 = __builtin_amdgcn_exp2f(fmaf(sx[4 * i + jj], c2, -l2v[jj]));
              p[4 * i + jj] = ok ? e2 : 0.f;
            }
            p_lds[pair][i * 64 + lane] = make_float4(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float l2v[4] = {l2[i].x, l2[i].y, l2[i].z, l2[i].w};
  #pragma unroll
            for (int jj = 0; jj < 4; ++jj) p[4 * i + jj] = __builtin_amdgcn_exp2f(fmaf(sx[4 * i + jj], c2, -l2v[jj]));
            p_lds[pair][i * 64 + lane] = make_float4(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        bx0 = pack_chunk(p, 0);
        bx1 = pack_chunk(p, 1);
      };

      // role B on the matrix cores: dP(k) when WP, then dK(k - 1) when WK
      auto b_mfma = [&](int k, auto wp, auto wk) __attribute__((always_inline)) {
        constexpr bool kP = decltype(wp)::value, kK = decltype(wk)::value;
        constexpr int kNp = kP ? C::kKSteps : 0;
        // rowf points at buffer k % kBufs (dO(k)), trf at buffer (k - 1) % kBufs (Q(k - 1))
        const __bf16* gt_l = &g_lds[0][0];
        const __bf16* qt_l = &q_lds[0][0];
        auto fetch = [&](int m) {
          if (m < kNp) return rowf.get(gt_l, m);
          const int mm = m - kNp;
          return trf.get(qt_l, mm / C::kDTiles, mm % C::kDTiles);
        };
        auto mma = [&](int m, const bf16x8& f) {
          if (m < kNp) {
            sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, rf[m], m == 0 ? f32x16{} : sx, 0, 0, 0);
          } else {
            const int mm = m - kNp, dt = mm % C::kDTiles;
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, mm < C::kDTiles ? bx0 : bx1, acc[dt], 0, 0, 0);
          }
        };
        if constexpr (kP) mfma_stream_pre<kNp + (kK ? 2 * C::kDTiles : 0), kK ? 2 : 1>(bfr, fetch, mma);
        else mfma_stream<kNp + (kK ? 2 * C::kDTiles : 0), kK ? 2 : 1>(fetch, mma);
      };
      // the first fragments of the next matrix phase's leading stream, read before the barrier that opens
      // it: role A's S(k + 1) (Q(k + 1), visible since the barrier that opened phase 2k), role B's
      // dP(k) (dO(k), visible since the barrier that opened phase 2k - 2); rowf already points at them
      auto prefetch = [&]() __attribute__((always_inline)) {
        const __bf16* t = kA ? &q_lds[0][0] : &g_lds[0][0];
#pragma unroll
        for (int m = 0; m < kPf; ++m) bfr[m] = rowf.get(t, m);
      };

      // role B: dS(k) = P(k) * (dP(k) - Dvec(k))
      auto b_valu = [&](int k) __attribute__((always_inline)) {
        const int slot = k % kBufs;
        float ds[16];
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 dv = *reinterpret_cast<const float4*>(&dv_lds[slot][8 * i + 4 * hh]);
          const float dvv[4] = {dv.x, dv.y, dv.z, dv.w};
          const float4 pv = p_lds[pair][i * 64 + lane];
          const float pp[4] = {pv.x, pv.y, pv.z, pv.w};
  #pragma unroll
          for (int jj = 0; jj < 4; ++jj) ds[4 * i + jj] = pp[jj] * (sx[4 * i + jj] - dvv[jj]);
        }
        bx0 = pack_chunk(ds, 0);
        bx1 = pack_chunk(ds, 1);
      };

      // one pair of phases (see above) for item k; the first (k = 0) and the
      // last (k = nitems) have no previous or no current item
      auto phases = [&](int k, auto first, auto last) __attribute__((always_inline)) {
        constexpr bool kFirst = decltype(first)::value, kLast = decltype(last)::value;
        // advance the fragment offsets one buffer (back by kBufs - 1 at the wrap), so that every
        // operand read of the matrix phases is a lane register plus an immediate offset: trf to
        // (k - 1) % kBufs and, in role B, rowf to k % kBufs (role A moved its rowf when it read
        // ahead in the previous phase pair)
        if (!kFirst) {
          const int sk = k % kBufs;
          if (!kA) rowf.shift(sk == 0 ? -(kBufs - 1) * kTileElems : kTileElems);
          trf.shift(sk == 1 ? -(kBufs - 1) * kTileElems : kTileElems);
        }
        // phase 2k: A on the matrix cores (+ loads of item k + 2), B on the vector ALU
        if (kA) {
          a_mfma(k, std::integral_constant<bool, !kLast>{}, std::integral_constant<bool, !kFirst>{});
        } else {
          if (!kFirst) b_valu(k - 1);
          if (!kLast) prefetch();
        }
        __builtin_amdgcn_sched_barrier(0);
        bar();
        // phase 2k+1: A on the vector ALU, B on the matrix cores
        if (kA) {
          if (k + 1 < nitems) {   // the next phase pair opens with S(k + 1): its first reads go out now
            rowf.shift((k + 1) % kBufs == 0 ? -(kBufs - 1) * kTileElems : kTileElems);
            prefetch();
          }
          if (!kLast) a_valu(k);
          __builtin_amdgcn_sched_barrier(0);
          vm_wait<0>();   // the loads of item k + 2 have landed
        } else {
          b_mfma(k, std::integral_constant<bool, !kLast>{}, std::integral_constant<bool, !kFirst>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        bar();
      };

      // fragment offsets of item 0: rowf at buffer 0, trf at buffer kBufs - 1 (= (0 - 1) mod kBufs)
      rowf.init(ql, hh);
      trf.init(lane);
      trf.shift((kBufs - 1) * kTileElems);
      // prologue: items 0 and 1 in LDS
      if (kA) {
        const Plan p0 = plan(0, true);
        const Plan p1 = plan(1, nitems > 1);
#pragma unroll
        for (int n = 0; n <= kLoads; ++n) {
          load_n(p0, n);
          load_n(p1, n);
        }
      }
      vm_wait<0>();
      bar();
      if (kA) prefetch();   // S(0) opens the first phase
      phases(0, std::true_type{}, std::false_type{});
      for (int k = 1; k < nitems; ++k) phases(k, std::false_type{}, std::false_type{});
      phases(nitems, std::false_type{}, std::true_type{});
    }

    if (!k_in) return;
    const int64_t krow = (int64_t)bhk * lk_total + k_idx;
    // a split launch writes its slice's partial dK / dV
    float* out = SPLIT ? (kA ? a.dv_part : a.dk_part) + ((int64_t)slice * a.B * a.H_kv * lk_total + krow) * D
                       : (kA ? a.dv : a.dk) + krow * D;
    const float sc = kA ? 1.f : a.scale;
  #pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 x = make_float4(sc * acc[dt][4 * i + 0], sc * acc[dt][4 * i + 1], sc * acc[dt][4 * i + 2],
                               sc * acc[dt][4 * i + 3]);
        float4* p = reinterpret_cast<float4*>(out + 32 * dt + 8 * i + 4 * hh);
        if (!SPLIT && a.accumulate) {
          const float4 y = *p;
          x.x += y.x;
          x.y += y.y;
          x.z += y.z;
          x.w += y.w;
        }
        *p = x;
      }

  };
  if (role_a) run(std::true_type{});
  else run(std::false_type{});
}

// Sum of the partial gradients of a split launch, in slice order:
// out[i] = (accumulate ? out[i] : 0) + part[0][i] + part[1][i] + ...
// blockIdx.y picks one of up to three (partials, output) pairs.
struct ReduceArgs {
  const float4* part[3];
  float4* out[3];
  int64_t n4[3];     // float4 elements of one output
  int32_t ns[3];     // slices
  int32_t accumulate;
};

__global__ void __launch_bounds__(256) bwd_reduce_kernel(ReduceArgs r) {
  const int y = blockIdx.y;
  const int64_t n4 = r.n4[y];
  const float4* part = r.part[y];
  float4* out = r.out[y];
  const int ns = r.ns[y];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    float4 s = r.accumulate ? out[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < ns; ++j) {
      const float4 x = part[(int64_t)j * n4 + i];
      s.x += x.x;
      s.y += x.y;
      s.z += x.z;
      s.w += x.w;
    }
    out[i] = s;
  }
}

template <int D>
hipError_t launch_bwd(const BwdArgs& a, int32_t do_dq, int32_t do_dkv, hipStream_t st) {
  const bool qs = do_dq && a.q_split > 1, ks = do_dkv && a.kv_split > 1;
  if (do_dq) {
    const int nqt = (a.Lq + kQOwn - 1) / kQOwn;
    if (qs)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3((unsigned)(nqt * a.B * a.H * a.q_split)), dim3(kQThreads), 0,
                         st, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3((unsigned)(nqt * a.B * a.H)), dim3(kQThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t lk_total = (int64_t)a.nblocks * a.Lk;
  if (do_dkv) {
    const int64_t nkt = (lk_total + kKvOwn - 1) / kKvOwn;
    if (ks)
      hipLaunchKernelGGL((bwd_dkv_kernel<D, true>), dim3((unsigned)(nkt * a.B * a.H_kv * a.kv_split)),
                         dim3(kKvThreads), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dkv_kernel<D, false>), dim3((unsigned)(nkt * a.B * a.H_kv)), dim3(kKvThreads), 0, st,
                         a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!qs && !ks) return hipSuccess;
  ReduceArgs r{};
  int n = 0;
  if (qs) {
    r.part[n] = reinterpret_cast<const float4*>(a.dq_part);
    r.out[n] = reinterpret_cast<float4*>(a.dq);
    r.n4[n] = (int64_t)a.B * a.H * a.Lq * D / 4;
    r.ns[n++] = a.q_split;
  }
  if (ks) {
    const int64_t n4 = (int64_t)a.B * a.H_kv * lk_total * D / 4;
    r.part[n] = reinterpret_cast<const float4*>(a.dk_part);
    r.out[n] = reinterpret_cast<float4*>(a.dk);
    r.n4[n] = n4;
    r.ns[n++] = a.kv_split;
    r.part[n] = reinterpret_cast<const float4*>(a.dv_part);
    r.out[n] = reinterpret_cast<float4*>(a.dv);
    r.n4[n] = n4;
    r.ns[n++] = a.kv_split;
  }
  r.accumulate = a.accumulate;
  int64_t most = 0;
  for (int i = 0; i < n; ++i) most = r.n4[i] > most ? r.n4[i] : most;
  const int64_t blocks = (most + 255) / 256;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024), (unsigned)n), dim3(256), 0,
                     st, r);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_prep_t(const BwdPrepArgs& a, hipStream_t st) {
  constexpr int kLanes = D / (16 / sizeof(T));
  const int64_t rows = (int64_t)a.B * a.H * a.Lq;
  const int64_t per = 256 / kLanes;
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)((rows + per - 1) / per)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// Split only grids that fill at most half of the workgroup slots (the dQ
// kernel runs two workgroups per compute unit, the dK/dV kernel one), into as
// many slices as bring them to about one full round, at most 16.
int32_t bwd_bf16_q_split(int32_t B, int32_t H, int32_t Lq) {
  constexpr int64_t kSlots = 2 * 256, kMaxSplit = 16;
  if (B < 1 || H < 1 || Lq < 1) return 1;
  const int64_t grid = (int64_t)((Lq + kQOwn - 1) / kQOwn) * B * H;
  if (2 * grid > kSlots) return 1;
  return (int32_t)(kSlots / grid < kMaxSplit ? kSlots / grid : kMaxSplit);
}

int32_t bwd_bf16_kv_split(int32_t B, int32_t H_kv, int64_t Lk_total) {
  constexpr int64_t kSlots = 256, kMaxSplit = 16;
  if (B < 1 || H_kv < 1 || Lk_total < 1) return 1;
  const int64_t grid = (Lk_total + kKvOwn - 1) / kKvOwn * B * H_kv;
  if (2 * grid > kSlots) return 1;
  return (int32_t)(kSlots / grid < kMaxSplit ? kSlots / grid : kMaxSplit);
}

hipError_t launch_bwd_prep(int32_t dtype_bf16, const BwdPrepArgs& a, hipStream_t st) {
  if (dtype_bf16) return a.D == 64 ? launch_prep_t<__bf16, 64>(a, st) : launch_prep_t<__bf16, 128>(a, st);
  return a.D == 64 ? launch_prep_t<float, 64>(a, st) : launch_prep_t<float, 128>(a, st);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int32_t do_dq, int32_t do_dkv, hipStream_t st) {
  if (a.D == 64) return launch_bwd<64>(a, do_dq, do_dkv, st);
  return launch_bwd<128>(a, do_dq, do_dkv, st);
}

}  // namespace cpring
