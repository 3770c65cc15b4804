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
//  * a preprocessing pass turns (O, dO, LSE) into per-row {LSE * log2(e),
//    Dvec} and the positions into a per-query allowed window {lo, hi};
//  * the dQ kernel: a workgroup owns 128 queries of one (b, h), each wave 32 of
//    them with Q and dO resident in VGPRs in the B-operand layout of
//    v_mfma_f32_32x32x16_bf16. Keys stream through LDS in tiles of 32 with
//    direct buffer->LDS loads, double-buffered: K twice (rows with a chunk
//    swizzle for S^T = K Q^T; 4-key x 32-column sub-blocks for the transposed
//    reads that give K^T), V once (rows, for dP^T = V dO^T). A lane then holds
//    one query and 16 keys of a 32x32 block, so P^T and dS^T are lane-local
//    and leave the accumulators already in the B-operand layout of
//    dQ^T += K^T dS^T (v_cvt_pk_bf16_f32, round to nearest even);
//  * the dK/dV kernel is the mirror image: a workgroup owns 128 keys of one
//    (b, kv head), each wave 32 keys with K and V resident; queries stream in
//    tiles of 32 (Q and dO, rows and sub-blocks, with their {lse2, Dvec} and
//    windows), for every query head of the grouped-query group; S = Q K^T and
//    dP = dO V^T give one key and 16 queries per lane, and dV^T += dO^T P,
//    dK^T += Q^T dS take dO^T and Q^T from transposed LDS reads;
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

constexpr int kT = 32;                    // rows per streamed tile
constexpr int kNW = 4;                    // waves per workgroup, 32 owned rows each
constexpr int kThreads = 64 * kNW;
constexpr int kOwn = 32 * kNW;            // rows a workgroup owns
constexpr int kMaxTiles = 8 * kThreads;   // tiles classified per segment
constexpr int kListPad = 2;               // end markers after the last kept tile

template <int D>
struct BCfg {
  static constexpr int kKSteps = D / 16;      // MFMA steps over the head dim
  static constexpr int kDTiles = D / 32;      // 32-row tiles of a transposed gradient
  static constexpr int kChunks = D / 8;       // 16-byte chunks per row
  static constexpr int kDq = D / 32;          // 32-column sub-blocks per 4-row group
  static constexpr int kLoads = kT * kChunks / kThreads;   // 16-byte loads per thread per tile copy
  static_assert(kLoads >= 1 && (kT * kChunks) % kThreads == 0, "tile/threads mismatch");
};

// Per-thread byte offsets (within a 32-row tile of row stride `sl` elements)
// of the 16-byte chunks this thread's wave writes to LDS chunk slots
// (wave * kLoads + i) * 64 + lane, for the two tile layouts:
//  rows: slot -> row slot / kChunks, physical chunk slot % kChunks holding
//        logical chunk swz_k(row, physical);
//  sub-blocks: slot -> sub-block slot / 16 (4 rows x 32 columns, 4-row group
//        sb / kDq, column block sb % kDq), chunk (slot % 16) within it.
// Element (row, col) of a sub-block tile sits at
// ((row / 4) * kDq + col / 32) * 128 + (row % 4) * 32 + col % 32.
template <int D>
__device__ __forceinline__ void tile_offsets(int wave, int lane, int64_t sl, uint32_t (&rm)[BCfg<D>::kLoads],
                                             uint32_t (&sb)[BCfg<D>::kLoads]) {
  using C = BCfg<D>;
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    const unsigned sidx = (unsigned)((wave * C::kLoads + i) * 64 + lane);
    const unsigned r = sidx / C::kChunks;
    rm[i] = r * (uint32_t)sl * 2u + (uint32_t)swz_k<D>((int)r, (int)(sidx % C::kChunks)) * 16u;
    const unsigned blk = sidx >> 4, q = sidx & 15;
    const unsigned r2 = 4 * (blk / C::kDq) + (q >> 2), ch = 4 * (blk % C::kDq) + (q & 3);
    sb[i] = r2 * (uint32_t)sl * 2u + ch * 16u;
  }
}

// The wave's share of one tile copy: kLoads 16-byte loads into LDS chunk slots
// (wave * kLoads + i) * 64 + lane of `dst`.
template <int D>
__device__ __forceinline__ void load_tile(const i32x4& rsrc, const uint32_t (&off)[BCfg<D>::kLoads], __bf16* dst,
                                          int wave) {
#pragma unroll
  for (int i = 0; i < BCfg<D>::kLoads; ++i) dma_b128(rsrc, off[i], lds_addr(dst + (wave * BCfg<D>::kLoads + i) * 512));
}

// A-operand fragment of a row tile: row `ql`, logical chunk 2 * kk + hh.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const __bf16* tile, int ql, int hh, int kk) {
  return *reinterpret_cast<const bf16x8*>(tile + ql * D + swz_k<D>(ql, 2 * kk + hh) * 8);
}

// A-operand fragment of the transposed tile, from the sub-block copy: lane
// (column d = 32 * dt + lane % 32, half hh) gets rows 16c + 4hh + {0..3} and
// 16c + 8 + 4hh + {0..3}, the rows whose values a B operand packed from the
// accumulators (chunk c) holds for k = 8 * hh + {0..7}.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* tile_sb, int tbase, int c, int dt) {
  constexpr int kDq = BCfg<D>::kDq;
  const __bf16* p = tile_sb + tbase + (4 * c * kDq + dt) * 128;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 2 * kDq * 128));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// lane's base offset for tr_frag: 16-lane group g reads 4 columns of row
// 4 * (g >> 1) + (gi >> 2) of its 4-row group, columns 16 * (g & 1) + 4 * (gi & 3)
__device__ __forceinline__ int tr_base(int lane, int kDq) {
  return (lane >> 5) * kDq * 128 + ((lane & 15) >> 2) * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
}

// 16 bf16 values of one 32x32 accumulator chunk c (elements 8c .. 8c+7) as a
// B operand
__device__ __forceinline__ bf16x8 pack_chunk(const float (&x)[16], int c) {
  uint32_t w4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {(__bf16)x[8 * c + 2 * i], (__bf16)x[8 * c + 2 * i + 1]};
    w4[i] = __builtin_bit_cast(uint32_t, pr);
  }
  return __builtin_bit_cast(bf16x8, w4);
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
  a.qinfo[row] = make_float2(l == -INFINITY ? INFINITY : l * kLog2e, acc);
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

template <int D>
__global__ void __launch_bounds__(kThreads, 2) bwd_dq_kernel(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int kDq = C::kDq;

  __shared__ __attribute__((aligned(16))) __bf16 k_rm[2][kT * D];   // K rows (A operand of S^T)
  __shared__ __attribute__((aligned(16))) __bf16 k_sb[2][kT * D];   // K sub-blocks (K^T fragments)
  __shared__ __attribute__((aligned(16))) __bf16 v_rm[2][kT * D];   // V rows (A operand of dP^T)
  __shared__ __attribute__((aligned(16))) int32_t pos_lds[2][64];
  __shared__ __attribute__((aligned(8))) uint8_t flags8[kMaxTiles];
  __shared__ uint16_t klist[kMaxTiles + kListPad];
  __shared__ int32_t qrange[4][kNW];
  __shared__ int32_t wcount[kNW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31;
  const int hh = lane >> 5;

  const int nqt = (a.Lq + kOwn - 1) / kOwn;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int bh = logical / nqt;
  const int qt = nqt - 1 - (logical - bh * nqt);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int q_idx = qt * kOwn + wave * 32 + ql;
  const bool q_in = q_idx < a.Lq;
  const int64_t srow = (int64_t)bh * a.Lq + q_idx;

  int32_t qlow = 1, qlim = 0;
  float lse2 = INFINITY, dvec = 0.f;
  if (q_in) {
    const int2 w = a.qwin[q_idx];
    qlow = w.x;
    qlim = w.y;
    const float2 qi = a.qinfo[srow];
    lse2 = qi.x;
    dvec = qi.y;
  }
  const bool q_live = qlow <= qlim;

  // bounds over the workgroup's live queries (see the forward kernel)
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
    for (int w = 0; w < kNW; ++w) {
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
  uint32_t k_rm_off[C::kLoads], k_sb_off[C::kLoads], v_rm_off[C::kLoads], v_sb_unused[C::kLoads];
  tile_offsets<D>(wave, lane, a.k_sl, k_rm_off, k_sb_off);
  tile_offsets<D>(wave, lane, a.v_sl, v_rm_off, v_sb_unused);
  const int tb = tr_base(lane, kDq);

  for (int t = 0; t < a.nblocks && ub_max >= 0; ++t) {
    int src = (a.rank - t) % a.cp;
    if (src < 0) src += a.cp;
    const int64_t row0 = (int64_t)src * a.Lk;
    const int32_t* posb = a.kv_pos + row0;
    const __bf16* kb = kbh + row0 * a.k_sl;
    const __bf16* vb = vbh + row0 * a.v_sl;

    for (int seg0 = 0; seg0 < n_kt; seg0 += kMaxTiles) {
      const int nseg = min(kMaxTiles, n_kt - seg0);
      // ---- classify the segment's key tiles: 8 lanes per tile, 4 positions each
      bar();
      for (int base = 0; base < nseg; base += kThreads / 8) {
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
      const int nk = build_tile_list<kNW, kListPad>(flags8, nseg, klist, wcount);
      bar();
      if (nk == 0) continue;

      // ---- the wave's share of the loads of kept tile j into buffer `slot`
      auto issue = [&](int j, int slot) __attribute__((always_inline)) {
        const int r0 = (seg0 + j) * kT;
        const uint32_t rows = (uint32_t)min(kT, a.Lk - r0);
        const i32x4 rk = make_rsrc(kb + (int64_t)r0 * a.k_sl, rows * (uint32_t)a.k_sl * 2u);
        const i32x4 rv = make_rsrc(vb + (int64_t)r0 * a.v_sl, rows * (uint32_t)a.v_sl * 2u);
        load_tile<D>(rk, k_rm_off, &k_rm[slot][0], wave);
        load_tile<D>(rk, k_sb_off, &k_sb[slot][0], wave);
        load_tile<D>(rv, v_rm_off, &v_rm[slot][0], wave);
        if (wave == 0) dma_b32(make_rsrc(posb + r0, rows * 4u), (uint32_t)lane * 4u, lds_addr(&pos_lds[slot][0]));
      };

      issue(klist[0] & 0x7fff, 0);
      for (int u = 0; u < nk; ++u) {
        const int e = __builtin_amdgcn_readfirstlane((int)klist[u]);
        const int en = __builtin_amdgcn_readfirstlane((int)klist[u + 1]);
        const int slot = u & 1;
        vm_wait<0>();
        bar();   // tile u is in LDS; every wave is done with buffer (u + 1) & 1
        if (u + 1 < nk) issue(en & 0x7fff, slot ^ 1);

        // S^T = K Q^T and dP^T = V dO^T for this tile's 32 keys
        f32x16 st = {}, pt = {};
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk)
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(&k_rm[slot][0], ql, hh, kk), qf[kk], st, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk)
          pt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(&v_rm[slot][0], ql, hh, kk), gf[kk], pt, 0, 0, 0);

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
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
          dqt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(&k_sb[slot][0], tb, 0, dt), d0, dqt[dt], 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
          dqt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(&k_sb[slot][0], tb, 1, dt), d1, dqt[dt], 0, 0, 0);
      }
    }
  }

  if (!q_in) return;
  float* out = a.dq + srow * D;
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 x = make_float4(a.scale * dqt[dt][4 * i + 0], a.scale * dqt[dt][4 * i + 1], a.scale * dqt[dt][4 * i + 2],
                             a.scale * dqt[dt][4 * i + 3]);
      float4* p = reinterpret_cast<float4*>(out + 32 * dt + 8 * i + 4 * hh);
      if (a.accumulate) {
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

template <int D>
__global__ void __launch_bounds__(kThreads, D == 128 ? 1 : 2) bwd_dkv_kernel(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int kDq = C::kDq;

  __shared__ __attribute__((aligned(16))) __bf16 q_rm[2][kT * D];   // Q rows (A operand of S)
  __shared__ __attribute__((aligned(16))) __bf16 q_sb[2][kT * D];   // Q sub-blocks (Q^T fragments)
  __shared__ __attribute__((aligned(16))) __bf16 g_rm[2][kT * D];   // dO rows (A operand of dP)
  __shared__ __attribute__((aligned(16))) __bf16 g_sb[2][kT * D];   // dO sub-blocks (dO^T fragments)
  __shared__ __attribute__((aligned(16))) float2 qi_lds[2][kT];     // {lse2, Dvec} of the tile's queries
  __shared__ __attribute__((aligned(16))) int2 qw_lds[2][kT];       // {lo, hi} of the tile's queries
  __shared__ __attribute__((aligned(8))) uint8_t flags8[kMaxTiles];
  __shared__ uint16_t klist[kMaxTiles + kListPad];
  __shared__ int32_t krange[3][kNW];
  __shared__ int32_t wcount[kNW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31;   // key column owned by this lane
  const int hh = lane >> 5;

  const int64_t lk_total = (int64_t)a.nblocks * a.Lk;
  const int nkt = (int)((lk_total + kOwn - 1) / kOwn);
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int bhk = logical / nkt;
  const int kt = logical - bhk * nkt;
  const int b = bhk / a.H_kv;
  const int hk = bhk - b * a.H_kv;
  const int64_t k_idx = (int64_t)kt * kOwn + wave * 32 + ql;
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
    for (int w = 0; w < kNW; ++w) {
      kmin = min(kmin, krange[0][w]);
      kmax = max(kmax, krange[1][w]);
      anypad |= krange[2][w];
    }
  }

  // resident K and V (B operands): d = 16 * kk + 8 * hh + e of key k_idx
  bf16x8 kf[C::kKSteps], vf[C::kKSteps];
  {
    const __bf16* kg = static_cast<const __bf16*>(a.k) + b * a.k_sb + hk * a.k_sh + k_idx * a.k_sl;
    const __bf16* vg = static_cast<const __bf16*>(a.v) + b * a.v_sb + hk * a.v_sh + k_idx * a.v_sl;
    const s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk) {
      kf[kk] = k_in ? *reinterpret_cast<const bf16x8*>(kg + 16 * kk + 8 * hh) : __builtin_bit_cast(bf16x8, z);
      vf[kk] = k_in ? *reinterpret_cast<const bf16x8*>(vg + 16 * kk + 8 * hh) : __builtin_bit_cast(bf16x8, z);
    }
  }

  // dV^T and dK^T[d = 32 * dt + 8 * i + 4 * hh + j][key] in [dt][4 * i + j]
  f32x16 dvt[C::kDTiles], dkt[C::kDTiles];
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dvt[dt][i] = 0.f;
      dkt[dt][i] = 0.f;
    }

  const float c2 = a.scale * kLog2e;
  const int group = a.H / a.H_kv;
  const int n_qt = (a.Lq + kT - 1) / kT;
  uint32_t q_rm_off[C::kLoads], q_sb_off[C::kLoads], g_rm_off[C::kLoads], g_sb_off[C::kLoads];
  tile_offsets<D>(wave, lane, a.q_sl, q_rm_off, q_sb_off);
  tile_offsets<D>(wave, lane, a.do_sl, g_rm_off, g_sb_off);
  const int tb = tr_base(lane, kDq);

  for (int seg0 = 0; seg0 < n_qt && kmax >= 0; seg0 += kMaxTiles) {
    const int nseg = min(kMaxTiles, n_qt - seg0);
    // ---- classify the segment's query tiles: 8 lanes per tile, 4 queries each
    bar();
    for (int base = 0; base < nseg; base += kThreads / 8) {
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
    const int nk = build_tile_list<kNW, kListPad>(flags8, nseg, klist, wcount);
    bar();
    if (nk == 0) continue;
    const int nitems = nk * group;   // (kept tile, query head of the group), head fastest

    auto issue = [&](int item, int slot) __attribute__((always_inline)) {
      const int u = item / group;
      const int h = hk * group + (item - u * group);
      const int j = klist[u] & 0x7fff;
      const int q0 = (seg0 + j) * kT;
      const uint32_t rows = (uint32_t)min(kT, a.Lq - q0);
      const __bf16* qb = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)q0 * a.q_sl;
      const __bf16* gb = static_cast<const __bf16*>(a.dout) + b * a.do_sb + h * a.do_sh + (int64_t)q0 * a.do_sl;
      const i32x4 rq = make_rsrc(qb, rows * (uint32_t)a.q_sl * 2u);
      const i32x4 rg = make_rsrc(gb, rows * (uint32_t)a.do_sl * 2u);
      load_tile<D>(rq, q_rm_off, &q_rm[slot][0], wave);
      load_tile<D>(rq, q_sb_off, &q_sb[slot][0], wave);
      load_tile<D>(rg, g_rm_off, &g_rm[slot][0], wave);
      load_tile<D>(rg, g_sb_off, &g_sb[slot][0], wave);
      if (wave == 0) {
        const float2* qi = a.qinfo + ((int64_t)(b * a.H + h) * a.Lq + q0);
        dma_b32(make_rsrc(qi, rows * 8u), (uint32_t)lane * 4u, lds_addr(&qi_lds[slot][0]));
      } else if (wave == 1) {
        dma_b32(make_rsrc(a.qwin + q0, rows * 8u), (uint32_t)lane * 4u, lds_addr(&qw_lds[slot][0]));
      }
    };

    issue(0, 0);
    for (int it = 0; it < nitems; ++it) {
      const int u = it / group;
      const int e = __builtin_amdgcn_readfirstlane((int)klist[u]);
      const int slot = it & 1;
      vm_wait<0>();
      bar();
      if (it + 1 < nitems) issue(it + 1, slot ^ 1);

      // S = Q K^T and dP = dO V^T for the tile's 32 queries
      f32x16 sa = {}, pa = {};
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk)
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(&q_rm[slot][0], ql, hh, kk), kf[kk], sa, 0, 0, 0);
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk)
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(&g_rm[slot][0], ql, hh, kk), vf[kk], pa, 0, 0, 0);

      // lane: key ql, queries 8 * i + 4 * hh + jj of the tile (element 4 * i + jj)
      float p[16], ds[16];
      const int remq = a.Lq - (seg0 + (e & 0x7fff)) * kT - 4 * hh;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x0 = *reinterpret_cast<const float4*>(&qi_lds[slot][8 * i + 4 * hh]);
        const float4 x1 = *reinterpret_cast<const float4*>(&qi_lds[slot][8 * i + 4 * hh + 2]);
        const float l2[4] = {x0.x, x0.z, x1.x, x1.z};
        const float dv[4] = {x0.y, x0.w, x1.y, x1.w};
        bool ok[4] = {true, true, true, true};
        if (e & 0x8000) {
          const int4 w0 = *reinterpret_cast<const int4*>(&qw_lds[slot][8 * i + 4 * hh]);
          const int4 w1 = *reinterpret_cast<const int4*>(&qw_lds[slot][8 * i + 4 * hh + 2]);
          const int lo[4] = {w0.x, w0.z, w1.x, w1.z};
          const int hi[4] = {w0.y, w0.w, w1.y, w1.w};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) ok[jj] = 8 * i + jj < remq && kp >= lo[jj] && kp <= hi[jj];
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float e2 = __builtin_amdgcn_exp2f(fmaf(sa[4 * i + jj], c2, -l2[jj]));
          p[4 * i + jj] = ok[jj] ? e2 : 0.f;
          ds[4 * i + jj] = p[4 * i + jj] * (pa[4 * i + jj] - dv[jj]);
        }
      }
      const bf16x8 p0 = pack_chunk(p, 0), p1 = pack_chunk(p, 1);
      const bf16x8 d0 = pack_chunk(ds, 0), d1 = pack_chunk(ds, 1);

      // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt)
        dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(&g_sb[slot][0], tb, 0, dt), p0, dvt[dt], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt)
        dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(&g_sb[slot][0], tb, 1, dt), p1, dvt[dt], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt)
        dkt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(&q_sb[slot][0], tb, 0, dt), d0, dkt[dt], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt)
        dkt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(&q_sb[slot][0], tb, 1, dt), d1, dkt[dt], 0, 0, 0);
    }
  }

  if (!k_in) return;
  const int64_t krow = (int64_t)bhk * lk_total + k_idx;
  float* dko = a.dk + krow * D;
  float* dvo = a.dv + krow * D;
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 xk = make_float4(a.scale * dkt[dt][4 * i + 0], a.scale * dkt[dt][4 * i + 1],
                              a.scale * dkt[dt][4 * i + 2], a.scale * dkt[dt][4 * i + 3]);
      float4 xv = make_float4(dvt[dt][4 * i + 0], dvt[dt][4 * i + 1], dvt[dt][4 * i + 2], dvt[dt][4 * i + 3]);
      float4* pk = reinterpret_cast<float4*>(dko + 32 * dt + 8 * i + 4 * hh);
      float4* pv = reinterpret_cast<float4*>(dvo + 32 * dt + 8 * i + 4 * hh);
      if (a.accumulate) {
        const float4 yk = *pk, yv = *pv;
        xk.x += yk.x; xk.y += yk.y; xk.z += yk.z; xk.w += yk.w;
        xv.x += yv.x; xv.y += yv.y; xv.z += yv.z; xv.w += yv.w;
      }
      *pk = xk;
      *pv = xv;
    }
}

template <int D>
hipError_t launch_bwd(const BwdArgs& a, int32_t do_dq, int32_t do_dkv, hipStream_t st) {
  if (do_dq) {
    const int nqt = (a.Lq + kOwn - 1) / kOwn;
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)(nqt * a.B * a.H)), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (do_dkv) {
    const int64_t lk_total = (int64_t)a.nblocks * a.Lk;
    const int64_t nkt = (lk_total + kOwn - 1) / kOwn;
    hipLaunchKernelGGL((bwd_dkv_kernel<D>), dim3((unsigned)(nkt * a.B * a.H_kv)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
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

hipError_t launch_bwd_prep(int32_t dtype_bf16, const BwdPrepArgs& a, hipStream_t st) {
  if (dtype_bf16) return a.D == 64 ? launch_prep_t<__bf16, 64>(a, st) : launch_prep_t<__bf16, 128>(a, st);
  return a.D == 64 ? launch_prep_t<float, 64>(a, st) : launch_prep_t<float, 128>(a, st);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int32_t do_dq, int32_t do_dkv, hipStream_t st) {
  if (a.D == 64) return launch_bwd<64>(a, do_dq, do_dkv, st);
  return launch_bwd<128>(a, do_dq, do_dkv, st);
}

}  // namespace cpring
