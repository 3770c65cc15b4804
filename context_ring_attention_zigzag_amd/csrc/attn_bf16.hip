// bf16 ring-attention pass on CDNA4 matrix cores (gfx950).
//
// What it computes ("Sequence Parallelism and Ring Attention", "Deep dive"
// and "Technical insight"; "Context Parallelism", "How context parallelism
// works"): the rank's local queries stay resident while the KV blocks arrive
// one ring hop at a time; each block's scaled-dot-product scores are folded
// into a running max m, running normaliser l and unnormalised output O, with
// earlier partial sums rescaled whenever a larger score appears. Masking is
// causal by global position ("Context Parallelism v.s. Sequence Parallelism
// (Megatron-LM)", "Implementation quirk: symmetric chunk assignment").
//
// Mapping to the hardware:
//  * a workgroup owns BM = 32*NW queries of one (b, h); each wavefront owns 32
//    of them and keeps their Q rows in VGPRs for the whole pass;
//  * two wave groups (waves [0, NW/2) and [NW/2, NW), one wave of each per
//    SIMD) run the same key-tile sequence one phase apart. Each tile takes two
//    phases: an MFMA phase (S^T = K Q^T of this tile, then P*V of the previous
//    one, with the row max of the new scores and the tile loads beside it) and
//    a VALU phase (mask, rescale decision, exponentials, row sums). While one
//    group is in its MFMA phase the other is in its VALU phase, so the matrix
//    cores and the vector ALUs of every SIMD work at the same time; a
//    workgroup barrier separates consecutive phases;
//  * keys stream through LDS in tiles of BN = 64 with direct buffer->LDS
//    16-byte loads, into three K and three V buffers, issued from the middle of
//    the MFMA phase (the vector phase is the longer one); every wave waits for
//    its own loads at the end of its next MFMA phase, one barrier before their
//    first reader;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: lane l then holds query l%32 and 16 of the 32
//    keys of a 32x32 block, so the per-query max and sum are lane-local plus
//    one exchange between the two half-waves (v_permlane32_swap);
//  * O^T = V^T P^T on the same MFMA: the probabilities leave the score
//    accumulators already in the B-operand layout (v_cvt_pk_bf16_f32, round
//    to nearest even), and V^T comes from the V tile through ds_read_b64_tr_b16;
//    the row sums add the float32 probabilities before rounding (a sum of the
//    rounded values would carry their 2^-9 relative error into the LSE of rows
//    that see few keys);
//  * lazy rescaling: exponents are taken against a reference max that is only
//    raised when a row's max exceeds it by more than kTau (log2 units), so the
//    O/l rescale is almost never executed; the result is unchanged because O
//    and l always share the same reference;
//  * every LDS read of the MFMA phase is one per-lane base register plus a
//    compile-time offset: K is row-major with a 16-byte-chunk XOR swizzle,
//    V is stored as 4-key x 32-column sub-blocks that a 32-lane transposed read
//    covers without bank conflicts;
//  * (query tile, key tile) pairs are classified from their position ranges
//    into skip / full / mixed and the kept ones listed in order in LDS;
//    skipped tiles are neither loaded nor computed, full tiles need no element
//    mask;
//  * the grid is remapped so that the workgroups of one (b, h) land on the
//    same XCD (shared L2), heaviest query tiles first;
//  * a grid too small to fill the chip is split over the keys: each query
//    tile gets several workgroups, each walking one slice of every block's key
//    tiles and writing its partial (O, m, l); a merge pass combines them.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "mfma_util.h"
#include "tile_class.h"

namespace cpring {
namespace {

using namespace mfma;

constexpr float kTau = 8.0f;    // lazy-rescale threshold: probabilities stay below 2^kTau
constexpr float kGuard = 256.0f;   // 2^kTau: a lane's probability sum under it bounds each probability
constexpr int kBN = tiles::kKeyTile;          // keys per tile (64)
constexpr int kMaxTiles = tiles::kSegTiles;   // key tiles classified per segment of a KV block (4096)
constexpr int kListPad = 8;     // end markers after the last kept tile (look-ahead reads)
#ifndef CPR_M_PREFETCH
#define CPR_M_PREFETCH 5
#endif
constexpr int kMPrefetch = CPR_M_PREFETCH;   // MFMAs whose LDS operand reads are in flight
constexpr int kKLoadAt = 8;                  // MFMA of the MFMA phase before which the K loads go out

template <int D, int NW>
struct Cfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBM = 32 * NW;              // queries per workgroup
  static constexpr int kKSteps = D / 16;           // MFMA steps over the head dim
  static constexpr int kDTiles = D / 32;           // 32-row tiles of O^T
  static constexpr int kChunks = D / 8;            // 16-byte chunks per K/V row
  static constexpr int kDq = D / 32;               // 32-column V sub-blocks per 4-key group
  static constexpr int kTileChunks = kBN * kChunks;
  static constexpr int kLoadsPerWave = kTileChunks / (64 * NW);   // 16-byte wave loads per tensor and tile
  static constexpr int kNB = 4 * kDTiles;          // MFMAs of O^T per tile
  static_assert(NW % 2 == 0, "two wave groups");
  static_assert(kLoadsPerWave >= 1 && kTileChunks % (64 * NW) == 0, "tile/threads mismatch");
};


// EXACT: every tile's row max is taken (needed when the launch hands back the
// state (O, m, l) with m the true running max: a ring step). Otherwise (a
// fused run, which finalises, or a split launch, whose partial states the
// merge rescales from any reference) the row max is taken only when a tile's
// probability sum says the reference may be too low, see softmax_guarded.
template <int D, int NW, bool SPLIT, bool EXACT>
__global__ void __launch_bounds__(NW * 64, 1) attn_bf16_kernel(AttnArgs a) {
  using C = Cfg<D, NW>;
  constexpr int kThreads = C::kThreads;
  constexpr int kDq = C::kDq;

  // Three K and three V tile buffers, a separate array each so that every
  // MFMA-phase access names its buffer statically; four position buffers
  // (positions are read one phase later than K).
  __shared__ __attribute__((aligned(16))) __bf16 k_lds0[kBN * D];
  __shared__ __attribute__((aligned(16))) __bf16 k_lds1[kBN * D];
  __shared__ __attribute__((aligned(16))) __bf16 k_lds2[kBN * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds0[kBN * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds1[kBN * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds2[kBN * D];
  __shared__ __attribute__((aligned(16))) int32_t pos_lds[4][kBN];
  __shared__ __attribute__((aligned(8))) uint8_t flags8[kMaxTiles];
  __shared__ uint16_t klist[kMaxTiles + kListPad];
  __shared__ int32_t qrange[4][NW];
  __shared__ int32_t wcount[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers and branches
  const int group = wave / (NW / 2);   // 0 leads, 1 trails by one phase
  const int ql = lane & 31;   // query column owned by this lane
  const int hh = lane >> 5;   // half-wave

  // ---- which (b, h, query tile): XCD-aware, heaviest tile first
  const int nqt = (a.Lq + C::kBM - 1) / C::kBM;
  const int ntiles = gridDim.x;
  int logical;
  {
    const int w = blockIdx.x;
    const int xcd = w % kXcds, idx = w / kXcds;
    const int per = ntiles / kXcds, rem = ntiles % kXcds;
    logical = xcd * per + min(xcd, rem) + idx;
  }
  int slice = 0;   // key slice of a split launch; its workgroups of one query tile are adjacent
  if constexpr (SPLIT) {
    slice = logical % a.kv_split;
    logical /= a.kv_split;
  }
  const int bh = logical / nqt;
  const int qt = nqt - 1 - (logical - bh * nqt);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int q_base = qt * C::kBM;
  const int q_idx = q_base + wave * 32 + ql;
  const bool q_in = q_idx < a.Lq;
  // key positions this query may attend, [qlow, qlim]: the causal bound and the
  // optional per-query window; empty for a pad query
  int32_t qlow, qlim;
  tiles::query_window(a.q_pos, a.kw_lo, a.kw_hi, a.causal, q_idx, q_in, qlow, qlim);
  const bool q_live = qlow <= qlim;   // attends some key position

  // ---- bounds over the workgroup's live queries (tile classification)
  const tiles::QBounds qb = tiles::workgroup_bounds<NW>(q_live, qlow, qlim, qrange);

  // ---- resident Q fragments (B operand of S^T = K Q^T): d = 16*kk + 8*hh + e
  bf16x8 qf[C::kKSteps];
  {
    const __bf16* qg = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)q_idx * a.q_sl;
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk) {
      if (q_in) {
        qf[kk] = *reinterpret_cast<const bf16x8*>(qg + 16 * kk + 8 * hh);
      } else {
        s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        qf[kk] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  // ---- running state: O^T[d = 32*dt + 8*i + 4*hh + j][query] in ot[dt][4*i + j]
  // m_ref: reference max (log2 units of the scaled score) the exponents are taken
  // against; m_true: the true running max; lsum0/1: this half-wave's share of l.
  f32x16 ot[C::kDTiles];
  float m_ref = -INFINITY, m_true = -INFINITY, lsum0 = 0.f, lsum1 = 0.f;
  const int64_t srow = (int64_t)bh * a.Lq + q_idx;
  if (!SPLIT && a.load_state && q_in) {   // a split launch always starts from an empty state
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(a.o_acc + srow * D + 32 * dt + 8 * i + 4 * hh);
        ot[dt][4 * i + 0] = x.x;
        ot[dt][4 * i + 1] = x.y;
        ot[dt][4 * i + 2] = x.z;
        ot[dt][4 * i + 3] = x.w;
      }
    const float mn = a.m[srow];
    m_ref = (mn == -INFINITY) ? -INFINITY : mn * kLog2e;
    m_true = m_ref;
    lsum0 = hh == 0 ? a.l[srow] : 0.f;
  } else {
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) ot[dt][i] = 0.f;
  }
  float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;   // finite stand-in while nothing is allowed yet

  const float c2 = a.scale * kLog2e;   // score -> log2 units
  const bool wg_has_queries = qb.ub_max >= 0;

  const int hk = h / (a.H / a.H_kv);   // grouped-query attention: the K/V head of query head h
  const __bf16* kbh = static_cast<const __bf16*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const __bf16* vbh = static_cast<const __bf16*>(a.v) + b * a.v_sb + hk * a.v_sh;
  const int n_kt = (a.Lk + kBN - 1) / kBN;
  // key tiles of every block that this workgroup walks: all, or its slice
  int kt_lo = 0, kt_hi = n_kt;
  if constexpr (SPLIT) {
    kt_lo = (int)((int64_t)slice * n_kt / a.kv_split);
    kt_hi = (int)((int64_t)(slice + 1) * n_kt / a.kv_split);
  }

  // LDS read offsets (elements), loop invariant.
  // K, A operand of S^T: lane (ql, hh) reads row 32*kt + ql, logical chunk 2*kk + hh.
  int koff[C::kKSteps];
#pragma unroll
  for (int kk = 0; kk < C::kKSteps; ++kk) koff[kk] = ql * D + swz_k<D>(ql, 2 * kk + hh) * 8;
  // V, A operand of O^T via the transposed read: lane (g, gi) of 16-lane group g
  // reads 4 columns of key 16*ch + 4*(g>>1) + (gi>>2) (+8 for the second read),
  // columns 32*dt + 16*(g&1) + 4*(gi&3). Element (key, d) of the tile sits at
  // ((key/4)*kDq + d/32)*128 + (key%4)*32 + d%32.
  const int vbase = (lane >> 5) * kDq * 128 + ((lane & 15) >> 2) * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  // Per-lane byte offsets of this wave's share of a tile load (loop invariant):
  // wave load i fills the 16-byte LDS chunks blk*64 + lane, blk = wave*kLoadsPerWave + i,
  // with the global chunk that the tile layout puts there.
  uint32_t ldk[C::kLoadsPerWave], ldv[C::kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    const unsigned sidx = (unsigned)((wave * C::kLoadsPerWave + i) * 64 + lane);
    const int krow = (int)(sidx / C::kChunks);
    ldk[i] = (uint32_t)krow * (uint32_t)a.k_sl * 2u + (uint32_t)swz_k<D>(krow, (int)(sidx % C::kChunks)) * 16u;
    const unsigned sb = sidx >> 4, q = sidx & 15;   // 4-key x 32-column sub-block, chunk within it
    const unsigned vrow = 4 * (sb / kDq) + (q >> 2), vch = 4 * (sb % kDq) + (q & 3);
    ldv[i] = vrow * (uint32_t)a.v_sl * 2u + vch * 16u;
  }
  const uint32_t ldp = (uint32_t)lane * 4u;

  for (int t = 0; t < a.nblocks && wg_has_queries; ++t) {
    int src = (a.rank - t) % a.cp;
    if (src < 0) src += a.cp;
    const int64_t row0 = (int64_t)src * a.Lk;        // first row of this block
    const int32_t* posb = a.kv_pos + row0;
    const __bf16* kb = kbh + row0 * a.k_sl;
    const __bf16* vb = vbh + row0 * a.v_sl;

    for (int seg0 = kt_lo; seg0 < kt_hi; seg0 += kMaxTiles) {
      const int nseg = min(kMaxTiles, kt_hi - seg0);

      // ---- classify the segment's key tiles
      bar();   // the previous segment is done with flags8 / klist / the buffers
      tiles::classify_key_tiles<kThreads, kBN>(posb, seg0, nseg, a.Lk, qb, flags8);
      bar();

      // ---- ordered list of the kept tiles (entry = tile index, | 0x8000 when the
      // tile needs the element mask), then kListPad end markers equal to nseg.
      // Thread tid covers tiles [8*tid, 8*tid + 8): count, scan, scatter.
      static_assert(kMaxTiles == 8 * kThreads, "eight tile flags per thread");
      const int nk = build_tile_list<NW, kListPad>(flags8, nseg, klist, wcount);
      bar();
      if (nk == 0) continue;   // uniform

      auto kbuf = [&](auto slot) __attribute__((always_inline)) -> __bf16* {
        if constexpr (decltype(slot)::value == 0) return k_lds0;
        else if constexpr (decltype(slot)::value == 1) return k_lds1;
        else return k_lds2;
      };
      auto vbuf = [&](auto slot) __attribute__((always_inline)) -> __bf16* {
        if constexpr (decltype(slot)::value == 0) return v_lds0;
        else if constexpr (decltype(slot)::value == 1) return v_lds1;
        else return v_lds2;
      };

      // ---- tile loads, this wave's share. Each goes through a buffer descriptor
      // whose base is the tile's first row and whose size covers the rows that
      // exist: rows past Lk read as zeros (those keys are masked by index, so their
      // P is exactly 0), and a tile index >= nseg (an end marker) gets an empty
      // descriptor, whose loads only zero-fill a buffer no one reads; every wave
      // thus issues the same loads in every VALU phase.
      auto tile_rows = [&](int j) __attribute__((always_inline)) -> uint32_t {
        return j < nseg ? (uint32_t)min(kBN, a.Lk - (seg0 + j) * kBN) : 0u;
      };
      auto load_k = [&](int j, auto i, __bf16* dst) __attribute__((always_inline)) {
        const int r0 = j < nseg ? (seg0 + j) * kBN : 0;
        const i32x4 d = make_rsrc(kb + (int64_t)r0 * a.k_sl, tile_rows(j) * (uint32_t)a.k_sl * 2u);
        dma_b128(d, ldk[decltype(i)::value], lds_addr(dst + (wave * C::kLoadsPerWave + decltype(i)::value) * 512));
      };
      auto load_v = [&](int j, auto i, __bf16* dst) __attribute__((always_inline)) {
        const int r0 = j < nseg ? (seg0 + j) * kBN : 0;
        const i32x4 d = make_rsrc(vb + (int64_t)r0 * a.v_sl, tile_rows(j) * (uint32_t)a.v_sl * 2u);
        dma_b128(d, ldv[decltype(i)::value], lds_addr(dst + (wave * C::kLoadsPerWave + decltype(i)::value) * 512));
      };
      auto load_pos = [&](int j, int slot) __attribute__((always_inline)) {
        const int r0 = j < nseg ? (seg0 + j) * kBN : 0;
        dma_b32(make_rsrc(posb + r0, tile_rows(j) * 4u), ldp, lds_addr(&pos_lds[slot][0]));
      };
      auto load_tile_k = [&](int j, __bf16* dst) __attribute__((always_inline)) {
        if constexpr (C::kLoadsPerWave >= 1) load_k(j, ic<0>{}, dst);
        if constexpr (C::kLoadsPerWave >= 2) load_k(j, ic<1>{}, dst);
        static_assert(C::kLoadsPerWave <= 2, "loads per wave");
      };
      auto load_tile_v = [&](int j, __bf16* dst) __attribute__((always_inline)) {
        if constexpr (C::kLoadsPerWave >= 1) load_v(j, ic<0>{}, dst);
        if constexpr (C::kLoadsPerWave >= 2) load_v(j, ic<1>{}, dst);
      };

      // ---- MFMA phase: one stream of MFMAs, scores of this tile (S^T = K Q^T,
      // two 32-key sub-tiles, kNA MFMAs) then O^T += V^T P^T of the previous tile
      // (kNB MFMAs). Every MFMA's A operand is a 4-register fragment read from LDS
      // kMPrefetch MFMAs ahead through one ring, across the switch from K to V.
      // The read / MFMA order is pinned with scheduling-group barriers.
      // hook(m) runs before MFMA m of the stream and, with m = kN, after the last
      auto mphase = [&](auto kslot, auto vslot, auto with_pv, f32x16 (&s)[2], const bf16x8 (&pb)[4],
                        auto&& hook) __attribute__((always_inline)) {
        constexpr int kNA = 2 * C::kKSteps;
        constexpr int kN = kNA + (decltype(with_pv)::value ? C::kNB : 0);
        constexpr int kPf = kMPrefetch;
        const __bf16* kl = kbuf(kslot);
        const __bf16* vl = vbuf(vslot);
        bf16x8 fr[kPf + 1];
        auto fetch = [&](int m) __attribute__((always_inline)) {
          if (m < kNA) {   // K row 32*kt + ql, logical chunk 2*kk + hh
            const int kk = m >> 1, kt = m & 1;
            fr[m % (kPf + 1)] = *reinterpret_cast<const bf16x8*>(kl + kt * 32 * D + koff[kk]);
          } else {         // V^T fragment through two transposed reads
            const int mm = m - kNA;
            const int ch = mm / C::kDTiles, dt = mm % C::kDTiles;
            const __bf16* p = vl + vbase + (4 * ch * kDq + dt) * 128;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 2 * kDq * 128));
            fr[m % (kPf + 1)] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        };
#pragma unroll
        for (int m = 0; m < kPf; ++m) fetch(m);
#pragma unroll
        for (int m = 0; m < kN; ++m) {
          if (m + kPf < kN) fetch(m + kPf);
          hook(m);
          if (m < kNA) {
            const int kk = m >> 1, kt = m & 1;
            if (kk == 0) {
              const f32x16 z = {};
              s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (kPf + 1)], qf[0], z, 0, 0, 0);
            } else {
              s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (kPf + 1)], qf[kk], s[kt], 0, 0, 0);
            }
          } else {
            const int mm = m - kNA;
            const int ch = mm / C::kDTiles, dt = mm % C::kDTiles;
            ot[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (kPf + 1)], pb[ch], ot[dt], 0, 0, 0);
          }
        }
        hook(kN);
        // pinned order: the first kPf fetches, then per MFMA: its look-ahead fetch, the MFMA
#pragma unroll
        for (int m = 0; m < kPf; ++m) {
          if (m < kNA) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
          else __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
#pragma unroll
        for (int m = 0; m < kN; ++m) {
          if (m + kPf < kNA) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
          else if (m + kPf < kN) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        }
      };

      // ---- VALU phase, first part: mask, max, rescale decision
      // the row max of a tile's scores over this half-wave's keys
      auto row_max = [&](const f32x16 (&s)[2]) __attribute__((always_inline)) -> float {
        float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          m0 = fmaxf(m0, s[0][i]);
          m1 = fmaxf(m1, s[1][i]);
        }
        return fmaxf(m0, m1);
      };
      // mxh: row max of the unmasked scores, taken in the MFMA phase
      // element mask of a tile straddling the causal boundary or holding pads /
      // rows past Lk: scores of keys the query may not attend become -inf
      auto apply_mask = [&](f32x16 (&s)[2], int e, int pslot) __attribute__((always_inline)) {
          const int32_t* pl = &pos_lds[pslot][4 * hh];
          // keys of this tile that exist, less this half-wave's key offset: key
          // kt*32 + 8*i + 4*hh + jj exists when kt*32 + 8*i + jj < remh
          const int remh = a.Lk - (seg0 + (e & 0x7fff)) * kBN - 4 * hh;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int4 p = *reinterpret_cast<const int4*>(pl + kt * 32 + 8 * i);
              const int pk[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const bool ok = kt * 32 + 8 * i + jj < remh && pk[jj] >= qlow && pk[jj] <= qlim;
                s[kt][4 * i + jj] = ok ? s[kt][4 * i + jj] : -INFINITY;
              }
            }
      };
      // raise the reference max of the rows whose max mt (log2 units) outgrew it
      // by more than kTau: O and l are rescaled by 2^(m_ref - m_new)
      auto raise_ref = [&](bool up, float mt) __attribute__((always_inline)) {
        const float m_new = up ? mt : m_ref;
        const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) ot[dt][i] *= alpha;
        lsum0 *= alpha;
        lsum1 *= alpha;
        m_ref = m_new;
        m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      };
      auto softmax_max = [&](f32x16 (&s)[2], int e, int pslot, float mxh) __attribute__((always_inline)) {
        if (e & 0x8000) {
          // the row max is taken again over what the mask leaves
          apply_mask(s, e, pslot);
          mxh = row_max(s);
        }
        const float mx = other_half_max(mxh);
        // raise the reference max where this tile's max outgrew it by more than kTau
        const float mt = mx * c2;
        m_true = fmaxf(m_true, mt);
        const bool need = mt > m_ref + kTau;
        if (__any(need)) raise_ref(need, mt);
      };
      // ---- VALU phase, second part, 16 keys at a time: P = 2^(s*c2 - m_ref)
      // rounded to bf16, in the B-operand layout of O^T += V^T P^T; l accumulates
      // the same values before rounding
      auto softmax_exp = [&](const f32x16 (&s)[2], bf16x8 (&pb)[4], auto chunk, float mu, float& acc0, float& acc1)
          __attribute__((always_inline)) {
        constexpr int c = decltype(chunk)::value;
        uint32_t w4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(s[c >> 1][8 * (c & 1) + 2 * x], c2, -mu));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(s[c >> 1][8 * (c & 1) + 2 * x + 1], c2, -mu));
          const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
          acc0 += e0;
          acc1 += e1;
          w4[x] = __builtin_bit_cast(uint32_t, pr);
        }
        pb[c] = __builtin_bit_cast(bf16x8, w4);
      };
      auto softmax_exp4 = [&](const f32x16 (&s)[2], bf16x8 (&pb)[4], float mu, float& acc0, float& acc1)
          __attribute__((always_inline)) {
        softmax_exp(s, pb, ic<0>{}, mu, acc0, acc1);
        softmax_exp(s, pb, ic<1>{}, mu, acc0, acc1);
        softmax_exp(s, pb, ic<2>{}, mu, acc0, acc1);
        softmax_exp(s, pb, ic<3>{}, mu, acc0, acc1);
      };
      // Exponentials against the current reference, with no row max: the tile's
      // probabilities are summed per lane first. A lane's 32 probabilities all
      // stay below 2^kTau when their sum does, which is the bound the exact rule
      // (raise the reference when the row max outgrows it by kTau) keeps; only
      // when some lane's sum exceeds it, or a row has no reference yet, is the
      // exact rule applied, and the exponentials redone if it raised a reference.
      auto softmax_guarded = [&](f32x16 (&s)[2], bf16x8 (&pb)[4], int e, int pslot) __attribute__((always_inline)) {
        if (e & 0x8000) apply_mask(s, e, pslot);
        float t0 = 0.f, t1 = 0.f;
        softmax_exp4(s, pb, m_use, t0, t1);
        const bool check = m_ref == -INFINITY || !(t0 + t1 <= kGuard);
        if (__any(check)) {
          // the scores pass through an empty asm statement, so that the compiler
          // cannot take the row max ahead of the branch, on the fast path
          f32x16 sx[2] = {s[0], s[1]};
#if defined(__HIP_DEVICE_COMPILE__)
          asm volatile("" : "+v"(sx[0]), "+v"(sx[1]));
#endif
          const float mt = other_half_max(row_max(sx)) * c2;
          const bool up = mt > m_ref + kTau;
          if (__any(up)) {
            raise_ref(up, mt);
            t0 = t1 = 0.f;
            softmax_exp4(sx, pb, m_use, t0, t1);
          }
        }
        lsum0 += t0;
        lsum1 += t1;
      };

      // Empty asm statements that read the given registers: the values must be
      // computed before this point in program order, which keeps the MFMAs of
      // an MFMA phase and the exponentials of a VALU phase from drifting across
      // the phase barrier.
      // (Vector-register constraints exist only in the device pass.)
      auto pin_scores = [&](const f32x16 (&x)[2], const float& m) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
        asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(m));
#endif
      };
      auto pin_probs = [&](const bf16x8 (&x)[4]) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
        asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(lsum0), "v"(lsum1));
#endif
      };

      // Kept tiles 0, 1, ... of the list in order; tile u uses K buffer u%3, V
      // buffer u%3 and position buffer u%4. Global phases: group 0 runs the MFMA
      // phase of tile u in phase 2u and its VALU phase in 2u+1; group 1 runs them
      // in 2u+1 and 2u+2. The MFMA phase of tile u reads K of tile u and V of
      // tile u-1, and loads this wave's share of K of tile u+2 (after the eighth
      // MFMA) and V of tile u+1 (between the score and the P*V MFMAs): those
      // buffers held K of tile u-1 and V of tile u-2, whose last readers (group
      // 1's MFMA phase of tile u-1) ran before the preceding barrier. Each wave
      // waits for these loads at the end of its next MFMA phase, one barrier
      // before the MFMA phase of tile u+2 reads them. The VALU phase of tile u
      // loads (wave NW-1) the positions of tile u+3. The list entries of tiles
      // u .. u+3 ride in e0 .. e3.
      int u = 0;
      int e0 = __builtin_amdgcn_readfirstlane((int)klist[0]);
      int e1 = __builtin_amdgcn_readfirstlane((int)klist[1]);
      int e2 = __builtin_amdgcn_readfirstlane((int)klist[2]);
      int e3 = __builtin_amdgcn_readfirstlane((int)klist[3]);
      auto tix = [](int e) __attribute__((always_inline)) { return e & 0x7fff; };

      f32x16 s[2];
      bf16x8 pb[4];

      auto vphase = [&](bool has, float mxh) __attribute__((always_inline)) {
        const int ahead = klist[u + 4];              // read now, used at the end
        if (has) {
          if constexpr (EXACT) {
            softmax_max(s, e0, u & 3, mxh);
            softmax_exp4(s, pb, m_use, lsum0, lsum1);
          } else {
            softmax_guarded(s, pb, e0, u & 3);
          }
        }
        // (lands by the end of this wave's next MFMA phase, with the tile loads)
        if (wave == NW - 1) load_pos(tix(e3), (u + 3) & 3);
        pin_probs(pb);
        e0 = e1;
        e1 = e2;
        e2 = e3;
        e3 = __builtin_amdgcn_readfirstlane(ahead);
        ++u;
        bar();
      };

      // the MFMA phase's loads of tile u: K of tile u+2 after MFMA kKLoadAt, V of
      // tile u+1 at the switch from the scores to P*V (or at the end of a stream
      // without P*V)
      auto mloads = [&](auto kslot, int m, int n_mfma) __attribute__((always_inline)) {
        constexpr int KS = decltype(kslot)::value;
        constexpr int kNA = 2 * C::kKSteps;
        if (m == min(kKLoadAt, n_mfma)) load_tile_k(tix(e2), kbuf(ic<(KS + 2) % 3>{}));
        if (m == min(kNA, n_mfma)) load_tile_v(tix(e1), vbuf(ic<(KS + 1) % 3>{}));
      };

      // prologue: K of tiles 0 and 1, V of tile 0, positions of tiles 0 .. 2
      load_tile_k(tix(e0), k_lds0);
      load_tile_k(tix(e1), k_lds1);
      load_tile_v(tix(e0), v_lds0);
      if (wave == NW - 1) {
        load_pos(tix(e0), 0);
        load_pos(tix(e1), 1);
        load_pos(tix(e2), 2);
      }
      vm_wait<0>();
      bar();
      if (group == 1) bar();   // group 1 trails by one phase

      // tile 0: no P*V yet
      mphase(ic<0>{}, ic<2>{}, ic<0>{}, s, pb, [&](int m) { mloads(ic<0>{}, m, 2 * C::kKSteps); });
      float mxh = 0.f;
      if constexpr (EXACT) mxh = row_max(s);
      pin_scores(s, mxh);
      vm_wait<2 * C::kLoadsPerWave>();
      bar();
      vphase(true, mxh);

      // tile u >= 1; after the last kept tile one more MFMA phase finishes P*V
      auto tile = [&](auto kslot) __attribute__((always_inline)) -> bool {
        constexpr int KS = decltype(kslot)::value;   // u % 3
        const bool has = tix(e0) < nseg;
        // scores of this tile first (the VALU phase needs them), then P*V of the
        // previous tile; its last MFMAs may still run when the barrier passes,
        // since only the LDS reads have to be complete there
        // (stale K when !has: the scores are never used)
        mphase(ic<KS>{}, ic<(KS + 2) % 3>{}, ic<1>{}, s, pb,
               [&](int m) { mloads(kslot, m, 2 * C::kKSteps + C::kNB); });
        // the row max of the new scores, beside the P*V MFMAs of this phase
        if constexpr (EXACT) mxh = row_max(s);
        pin_scores(s, mxh);
        // this wave's tile loads of the previous MFMA phase have landed
        vm_wait<2 * C::kLoadsPerWave>();
        bar();
        vphase(has, mxh);
        return has;
      };
      while (true) {
        if (!tile(ic<1>{})) break;
        if (!tile(ic<2>{})) break;
        if (!tile(ic<0>{})) break;
      }
      vm_wait<0>();            // the last phases only zero-filled unused buffers; let them land
      if (group == 0) bar();   // group 1 ran one extra barrier at the start
    }
  }

  // ---- epilogue
  const float l_tot = other_half_sum(lsum0 + lsum1);
  if (!q_in) return;
  // a query that may attend no key position (a pad, or an empty window) has no
  // result even if it took part in an unmasked full tile
  const bool has = q_live && l_tot > 0.f;
  if (!SPLIT && a.finalize) {
    const float inv = has ? 1.0f / l_tot : 0.f;
    __bf16* out = static_cast<__bf16*>(a.o_out) + srow * D;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 w0 = {(__bf16)(ot[dt][4 * i + 0] * inv), (__bf16)(ot[dt][4 * i + 1] * inv)};
        const bf16x2 w1 = {(__bf16)(ot[dt][4 * i + 2] * inv), (__bf16)(ot[dt][4 * i + 3] * inv)};
        uint2 w;
        w.x = __builtin_bit_cast(uint32_t, w0);
        w.y = __builtin_bit_cast(uint32_t, w1);
        *reinterpret_cast<uint2*>(out + 32 * dt + 8 * i + 4 * hh) = w;
      }
    if (a.lse && hh == 0) a.lse[srow] = has ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  } else {
    // hand back the state against the true running max (O and l scale by
    // 2^(m_ref - m_true) <= 1); a split launch's partial states keep the
    // reference, which the merge rescales like any other max
    const float m_out = EXACT ? m_true : m_ref;
    const float beta = has ? (EXACT ? __builtin_amdgcn_exp2f(m_ref - m_true) : 1.f) : 0.f;
    const int64_t prow = SPLIT ? srow + (int64_t)slice * a.state_rows : srow;   // this slice's partial state
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = make_float4(ot[dt][4 * i + 0] * beta, ot[dt][4 * i + 1] * beta, ot[dt][4 * i + 2] * beta,
                                     ot[dt][4 * i + 3] * beta);
        *reinterpret_cast<float4*>(a.o_acc + prow * D + 32 * dt + 8 * i + 4 * hh) = x;
      }
    if (hh == 0) {
      a.m[prow] = has ? m_out * kLn2 : -INFINITY;
      a.l[prow] = has ? l_tot * beta : 0.f;
    }
  }
}

// The guarded softmax (no row max per tile) pays off where the vector phase
// sets the pace, at D = 64: 2.4% faster on the non-causal 65,536-token shape.
// At D = 128 the matrix phase is the longer one and the guard measured 0.5%
// slower there and 2.2% slower on the million-token share, so D = 128 keeps
// the row max.
template <int D>
constexpr bool kGuarded = D == 64;

template <int D, int NW>
hipError_t launch(const AttnArgs& a, hipStream_t st) {
  const int nqt = (a.Lq + Cfg<D, NW>::kBM - 1) / Cfg<D, NW>::kBM;
  if (a.kv_split > 1) {
    const dim3 grid((unsigned)(nqt * a.B * a.H * a.kv_split));
    hipLaunchKernelGGL((attn_bf16_kernel<D, NW, true, !kGuarded<D>>), grid, dim3(NW * 64), 0, st, a);
  } else if (a.finalize) {
    const dim3 grid((unsigned)(nqt * a.B * a.H));
    hipLaunchKernelGGL((attn_bf16_kernel<D, NW, false, !kGuarded<D>>), grid, dim3(NW * 64), 0, st, a);
  } else {
    const dim3 grid((unsigned)(nqt * a.B * a.H));
    hipLaunchKernelGGL((attn_bf16_kernel<D, NW, false, true>), grid, dim3(NW * 64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

// Split only a grid that fills at most half of the 256 compute units, into as
// many slices as bring it to about one workgroup per unit; a slice keeps at
// least one key tile of every block.
int32_t attn_bf16_kv_split(int32_t B, int32_t H, int32_t Lq, int32_t Lk) {
  constexpr int64_t kCUs = 256, kMaxSplit = 16;
  constexpr int kBM = Cfg<128, 8>::kBM;
  static_assert(Cfg<64, 8>::kBM == kBM, "one query tile size");
  if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return 1;
  const int64_t grid = (int64_t)((Lq + kBM - 1) / kBM) * B * H;
  const int64_t n_kt = (Lk + kBN - 1) / kBN;
  if (n_kt <= 1 || 2 * grid > kCUs) return 1;
  return (int32_t)std::min(std::min(kCUs / grid, n_kt), kMaxSplit);
}

static_assert(Cfg<128, tiles::kWaves>::kBM == tiles::kQueryTile && Cfg<64, tiles::kWaves>::kBM == tiles::kQueryTile,
              "the tile census describes this kernel's query tiles");

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  if (a.D == 64) return launch<64, tiles::kWaves>(a, st);
  return launch<128, tiles::kWaves>(a, st);
}

}  // namespace cpring
