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
//    phases: an MFMA phase (P*V of the previous tile, then S^T = K Q^T of this
//    one) and a VALU phase (mask, row max, exponentials, row sums). While one
//    group is in its MFMA phase the other is in its VALU phase, so the matrix
//    cores and the vector ALUs of every SIMD work at the same time; a
//    workgroup barrier separates consecutive phases;
//  * keys stream through LDS in tiles of BN = 64 with direct global->LDS
//    16-byte loads (global_load_lds_dwordx4), issued two phases before their
//    first use into double-buffered K and V tiles;
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
//    into skip / full / mixed; skipped tiles are neither loaded nor computed,
//    full tiles need no element mask;
//  * the grid is remapped so that the workgroups of one (b, h) land on the
//    same XCD (shared L2), heaviest query tiles first.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace cpring {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;    // lazy-rescale threshold: probabilities stay below 2^kTau
constexpr int kXcds = 8;        // MI355X: 8 accelerator complex dies, workgroups dealt round-robin
constexpr int kBN = 64;         // keys per tile
constexpr int kMaxTiles = 4096; // key tiles classified per segment of a KV block
#ifndef CPR_M_PREFETCH
#define CPR_M_PREFETCH 5
#endif
constexpr int kMPrefetch = CPR_M_PREFETCH;   // MFMAs whose LDS operand reads are in flight

// Fourth dword of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle, no format conversion).
constexpr int kBufWord3 = 0x00020000;

// scheduling-group masks (AMDGPU sched_group_barrier)
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

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

// K tile: row-major, physical 16-byte chunk = logical chunk XOR a function of
// the row, so the 16 consecutive rows one A-operand read touches per 16 lanes
// hit 16 different bank groups. (An involution: also maps physical to logical.)
template <int D>
__device__ __forceinline__ int swz_k(int row, int chunk) {
  if constexpr (D == 128) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}

__device__ __forceinline__ float other_half_max(float x) {
  // every lane gets max(x of lane l, x of lane l^32)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float other_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Workgroup barrier without a memory fence: this wave's LDS accesses are
// complete, its in-flight global->LDS loads are not waited for (each wave
// waits for its own one phase later, before the barrier that precedes their
// first use). The memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// vmcnt(0), expcnt and lgkmcnt left at their maximum (gfx9 encoding); the
// builtin, unlike inline asm, is visible to the compiler's own wait tracking.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int N>
using ic = std::integral_constant<int, N>;

__device__ __forceinline__ int mod3_next(int x) { return x == 2 ? 0 : x + 1; }

template <int D, int NW>
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
  __shared__ uint64_t keep_w[kMaxTiles / 64];
  __shared__ uint64_t mixed_w[kMaxTiles / 64];
  __shared__ uint8_t flags8[kMaxTiles];
  __shared__ int32_t qrange[2][NW];

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
  const int bh = logical / nqt;
  const int qt = nqt - 1 - (logical - bh * nqt);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int q_base = qt * C::kBM;
  const int q_idx = q_base + wave * 32 + ql;
  const bool q_in = q_idx < a.Lq;
  const int32_t qp = q_in ? a.q_pos[q_idx] : -1;

  // ---- valid-position range of the workgroup's queries
  int qmin, qmax;
  {
    int lo = wave_min(qp >= 0 ? qp : INT_MAX);
    int hi = wave_max(qp);
    if (lane == 0) {
      qrange[0][wave] = lo;
      qrange[1][wave] = hi;
    }
    __syncthreads();
    qmin = INT_MAX;
    qmax = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      qmin = min(qmin, qrange[0][w]);
      qmax = max(qmax, qrange[1][w]);
    }
  }

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
  if (a.load_state && q_in) {
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
  const bool wg_has_queries = qmax >= 0;

  const __bf16* kbh = static_cast<const __bf16*>(a.k) + b * a.k_sb + h * a.k_sh;
  const __bf16* vbh = static_cast<const __bf16*>(a.v) + b * a.v_sb + h * a.v_sh;
  const int n_kt = (a.Lk + kBN - 1) / kBN;

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

  for (int t = 0; t < a.nblocks && wg_has_queries; ++t) {
    int src = (a.rank - t) % a.cp;
    if (src < 0) src += a.cp;
    const int64_t row0 = (int64_t)src * a.Lk;        // first row of this block
    const int32_t* posb = a.kv_pos + row0;
    const __bf16* kb = kbh + row0 * a.k_sl;
    const __bf16* vb = vbh + row0 * a.v_sl;

    for (int seg0 = 0; seg0 < n_kt; seg0 += kMaxTiles) {
      const int nseg = min(kMaxTiles, n_kt - seg0);

      // ---- classify the segment's key tiles: 16 lanes per tile, 4 positions each
      bar();   // the previous segment is done with flags8 / keep_w / the buffers
      for (int base = 0; base < nseg; base += kThreads / 16) {
        const int tt = base + (tid >> 4);
        const int g16 = tid & 15;
        int kmin = INT_MAX, kmax = -1, pad = 0;
        if (tt < nseg) {
          const int k0 = (seg0 + tt) * kBN + 4 * g16;
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
        for (int o = 8; o >= 1; o >>= 1) {
          kmin = min(kmin, __shfl_xor(kmin, o));
          kmax = max(kmax, __shfl_xor(kmax, o));
          pad |= __shfl_xor(pad, o);
        }
        if (g16 == 0 && tt < nseg) {
          const bool keep = kmax >= 0 && (!a.causal || kmin <= qmax);
          const bool full = !pad && (!a.causal || kmax <= qmin);
          flags8[tt] = (uint8_t)((keep ? 1 : 0) | ((keep && !full) ? 2 : 0));
        }
      }
      bar();
      for (int tt = tid; tt < ((nseg + 63) & ~63); tt += kThreads) {
        const int f = tt < nseg ? flags8[tt] : 0;
        const uint64_t kw = __ballot(f & 1);
        const uint64_t mw = __ballot(f & 2);
        if (lane == 0) {
          keep_w[tt >> 6] = kw;
          mixed_w[tt >> 6] = mw;
        }
      }
      bar();

      const int nwords = (nseg + 63) >> 6;
      auto next_kept = [&](int j) __attribute__((always_inline)) -> int {   // first kept tile index > j, or nseg
        if (j >= nseg) return nseg;
        int w = (j + 1) >> 6;
        if (w >= nwords) return nseg;
        uint64_t bits = keep_w[w] & (~0ull << ((j + 1) & 63));
        while (bits == 0) {
          if (++w >= nwords) return nseg;
          bits = keep_w[w];
        }
        return __builtin_amdgcn_readfirstlane(min(nseg, (w << 6) + (int)__builtin_ctzll(bits)));
      };
      auto is_mixed = [&](int j) __attribute__((always_inline)) -> bool { return (mixed_w[j >> 6] >> (j & 63)) & 1ull; };

      // ---- direct global -> LDS loads (this wave's share of a tile): lane
      // `lane` of wave-load `blk` fills the 16-byte LDS chunk blk*64 + lane with
      // the global chunk the layout puts there. Rows past Lk re-read row Lk-1
      // (finite data; those keys are masked, so their P is exactly 0). A tile
      // index >= nseg (past the last kept tile) loads nothing.
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

      // ---- tile loads. Each goes through a buffer descriptor whose base is the
      // tile's first row and whose size covers the rows that exist: rows past Lk
      // read as zeros (those keys are masked by index, so their P is exactly 0),
      // and a tile index past the last kept tile gets an empty descriptor (the
      // load only zero-fills a buffer no one reads), so every wave issues the same
      // number of loads in every MFMA phase. Buffer loads also keep the compiler's
      // LDS wait counting exact, where global->LDS loads make it drain every
      // outstanding LDS read.
      // (three descriptors: K, V and positions; kept as separate values, since
      // buffer-descriptor values cannot be members of a struct in the host pass)
      auto make_desc = [&](int jk, int jv, __amdgpu_buffer_rsrc_t& dk, __amdgpu_buffer_rsrc_t& dv,
                           __amdgpu_buffer_rsrc_t& dp) __attribute__((always_inline)) {
        {
          const bool ok = jk < nseg;
          const int r_base = ok ? (seg0 + jk) * kBN : 0;
          const uint32_t nrows = ok ? (uint32_t)min(kBN, a.Lk - r_base) : 0u;
          dk = __builtin_amdgcn_make_buffer_rsrc((void*)(kb + (int64_t)r_base * a.k_sl), 0,
                                                 nrows * (uint32_t)a.k_sl * 2u, kBufWord3);
          dp = __builtin_amdgcn_make_buffer_rsrc((void*)(posb + r_base), 0, nrows * 4u, kBufWord3);
        }
        {
          const bool ok = jv < nseg;
          const int r_base = ok ? (seg0 + jv) * kBN : 0;
          const uint32_t nrows = ok ? (uint32_t)min(kBN, a.Lk - r_base) : 0u;
          dv = __builtin_amdgcn_make_buffer_rsrc((void*)(vb + (int64_t)r_base * a.v_sl), 0,
                                                 nrows * (uint32_t)a.v_sl * 2u, kBufWord3);
        }
      };
      // load number i (0 .. kDmaPerWave-1) of this wave's share: K, then V, then positions
      auto dma = [&](const __amdgpu_buffer_rsrc_t& dk, const __amdgpu_buffer_rsrc_t& dv,
                     const __amdgpu_buffer_rsrc_t& dp, int i, int ln, __bf16* kdst, __bf16* vdst, int pslot)
          __attribute__((always_inline)) {
        if (i < C::kLoadsPerWave) {
          const int blk = wave * C::kLoadsPerWave + i;
          const unsigned sidx = (unsigned)(blk * 64 + ln);
          const int row = (int)(sidx / C::kChunks);
          const int lch = swz_k<D>(row, (int)(sidx % C::kChunks));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(dk, (lds_void*)(kdst + blk * 512), 16,
                                                   (uint32_t)row * (uint32_t)a.k_sl * 2u + (uint32_t)lch * 16u, 0,
                                                   0, 0);
        } else if (i < 2 * C::kLoadsPerWave) {
          const int blk = wave * C::kLoadsPerWave + (i - C::kLoadsPerWave);
          const unsigned sidx = (unsigned)(blk * 64 + ln);
          const unsigned sb = sidx >> 4, q = sidx & 15;
          const int row = (int)(4 * (sb / kDq) + (q >> 2));
          const int lch = (int)(4 * (sb % kDq) + (q & 3));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(dv, (lds_void*)(vdst + blk * 512), 16,
                                                   (uint32_t)row * (uint32_t)a.v_sl * 2u + (uint32_t)lch * 16u, 0,
                                                   0, 0);
        } else if (wave == NW - 1) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(dp, (lds_void*)&pos_lds[pslot][0], 4, (uint32_t)ln * 4u, 0, 0, 0);
        }
      };
      constexpr int kDmaPerWave = 2 * C::kLoadsPerWave + 1;   // the last one only on wave NW-1
      // this wave's share of K and positions of tile jk, V of tile jv
      auto issue_loads = [&](int jk, int jv, __bf16* kdst, __bf16* vdst, int pslot) __attribute__((always_inline)) {
        __amdgpu_buffer_rsrc_t dk, dv, dp;
        make_desc(jk, jv, dk, dv, dp);
        int ln = lane;
#if defined(__HIP_DEVICE_COMPILE__)
        asm volatile("" : "+v"(ln));   // recompute the load offsets here instead of keeping them live
#endif
#pragma unroll
        for (int i = 0; i < kDmaPerWave; ++i) dma(dk, dv, dp, i, ln, kdst, vdst, pslot);
      };

      // ---- MFMA phase: one stream of MFMAs, scores of this tile (S^T = K Q^T,
      // two 32-key sub-tiles, kNA MFMAs) then O^T += V^T P^T of the previous tile
      // (kNB MFMAs). Every MFMA's A operand is a 4-register fragment read from LDS
      // kMPrefetch MFMAs ahead through one ring, across the switch from K to V;
      // this wave's share of the next tiles' loads is spread over the first
      // MFMAs. The read / load / MFMA order is pinned with scheduling-group
      // barriers.
      auto mphase = [&](auto kslot, auto vslot, auto with_pv, f32x16 (&s)[2], const bf16x8 (&pb)[4])
          __attribute__((always_inline)) {
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
        // pinned order: the first kPf fetches, then per MFMA: its look-ahead fetch, the MFMA, a load
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

      // ---- VALU phase: mask, max, rescale, exponentials, row sums
      auto softmax = [&](f32x16 (&s)[2], bf16x8 (&pb)[4], int j, int pslot) __attribute__((always_inline)) {
        if (is_mixed(j)) {
          // element mask of a tile straddling the causal boundary or holding
          // pads / rows past Lk
          const int32_t* pl = &pos_lds[pslot][0];
          const int rem = a.Lk - (seg0 + j) * kBN;   // keys of this tile that exist
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key0 = kt * 32 + 8 * i + 4 * hh;
              const int4 p = *reinterpret_cast<const int4*>(pl + key0);
              const int pk[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const bool ok = key0 + jj < rem && pk[jj] >= 0 && qp >= 0 && (!a.causal || pk[jj] <= qp);
                s[kt][4 * i + jj] = ok ? s[kt][4 * i + jj] : -INFINITY;
              }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
        mx = other_half_max(mx);
        // raise the reference max where this tile's max outgrew it by more than kTau
        const float mt = mx * c2;
        m_true = fmaxf(m_true, mt);
        const bool need = mt > m_ref + kTau;
        if (__any(need)) {
          const float m_new = need ? mt : m_ref;
          const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
          for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) ot[dt][i] *= alpha;
          lsum0 *= alpha;
          lsum1 *= alpha;
          m_ref = m_new;
          m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
        }
        // P = 2^(s*c2 - m_ref) rounded to bf16, in the B-operand layout of
        // O^T += V^T P^T (16 keys per chunk); l accumulates the same values
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t w4[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const float e0 = __builtin_amdgcn_exp2f(fmaf(s[c >> 1][8 * (c & 1) + 2 * x], c2, -m_use));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(s[c >> 1][8 * (c & 1) + 2 * x + 1], c2, -m_use));
            const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
            lsum0 += e0;
            lsum1 += e1;
            w4[x] = __builtin_bit_cast(uint32_t, pr);
          }
          pb[c] = __builtin_bit_cast(bf16x8, w4);
        }
      };

      // Empty asm statements that read the given registers: the values must be
      // computed before this point in program order, which keeps the MFMAs of
      // an MFMA phase and the exponentials of a VALU phase from drifting across
      // the phase barrier.
      // (Vector-register constraints exist only in the device pass.)
      auto pin_scores = [&](const f32x16 (&x)[2]) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
        asm volatile("" ::"v"(x[0]), "v"(x[1]));
#endif
      };
      auto pin_out = [&]() __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) asm volatile("" ::"v"(ot[dt]));
#endif
      };
      auto pin_probs = [&](const bf16x8 (&x)[4]) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
        asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(lsum0), "v"(lsum1));
#endif
      };

      // Kept tiles j_0, j_1, ... in order. Tile u uses K buffer u%3, V buffer
      // u%3 and position buffer u%4. Global phases: group 0 runs the MFMA phase
      // of tile u in phase 2u and its VALU phase in 2u+1; group 1 runs them in
      // 2u+1 and 2u+2. The VALU phase of tile u also loads this wave's share of
      // K and positions of tile u+2 and V of tile u+1 (the buffers they replace
      // were last read in phase 2u-1); the wave waits for them at the end of its
      // next MFMA phase, before the barrier that ends phase 2u+3, and their first
      // reader runs in phase 2u+4. Loads thus sit in the phases with slack: the
      // VALU phase is shorter than the MFMA phase it overlaps.
      int ju = next_kept(-1);
      if (ju >= nseg) continue;   // uniform: every wave sees the same bitmask
      int ju1 = next_kept(ju);
      int ju2 = next_kept(ju1);

      f32x16 s[2];
      bf16x8 pb[4];

      // prologue: K and positions of tiles 0 and 1, V of tile 0
      issue_loads(ju, ju, k_lds0, v_lds0, 0);
      issue_loads(ju1, nseg, k_lds1, v_lds2, 1);   // (V part: empty descriptor into an unused buffer)
      wait_vmem();
      bar();
      if (group == 1) bar();   // group 1 trails by one phase

      // tile 0: no P*V yet
      mphase(ic<0>{}, ic<2>{}, ic<0>{}, s, pb);
      pin_scores(s);
      bar();
      issue_loads(ju2, ju1, k_lds2, v_lds1, 2);
      softmax(s, pb, ju, 0);
      pin_probs(pb);
      ju = ju1;
      ju1 = ju2;
      ju2 = next_kept(ju2);
      bar();

      // tile u >= 1; after the last kept tile one more MFMA phase finishes P*V
      int pu = 1;   // u % 4
      auto tile = [&](auto kslot) __attribute__((always_inline)) -> bool {
        constexpr int KS = decltype(kslot)::value;   // u % 3
        const bool has = ju < nseg;
        // MFMA phase: scores of this tile first (the VALU phase needs them), then
        // P*V of the previous tile; its last MFMAs may still run when the barrier
        // passes, since only the LDS reads have to be complete there.
        mphase(ic<KS>{}, ic<(KS + 2) % 3>{}, ic<1>{}, s, pb);   // stale K when !has: scores never used
        pin_scores(s);
        wait_vmem();   // this wave's loads from its previous VALU phase
        bar();
        issue_loads(ju2, ju1, kbuf(ic<(KS + 2) % 3>{}), vbuf(ic<(KS + 1) % 3>{}), (pu + 2) & 3);
        if (has) softmax(s, pb, ju, pu);
        pin_probs(pb);
        // advance the tile window here, off the MFMA phase's critical path
        pu = (pu + 1) & 3;
        ju = ju1;
        ju1 = ju2;
        ju2 = next_kept(ju2);
        bar();
        return has;
      };
      while (true) {
        if (!tile(ic<1>{})) break;
        if (!tile(ic<2>{})) break;
        if (!tile(ic<0>{})) break;
      }
      wait_vmem();             // the last phases only zero-filled unused buffers; let them land
      if (group == 0) bar();   // group 1 ran one extra barrier at the start
    }
  }

  // ---- epilogue
  const float l_tot = other_half_sum(lsum0 + lsum1);
  if (!q_in) return;
  const bool has = qp >= 0 && l_tot > 0.f;
  if (a.finalize) {
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
    // hand back the state against the true running max: O and l scale by 2^(m_ref - m_true) <= 1
    const float beta = has ? __builtin_amdgcn_exp2f(m_ref - m_true) : 0.f;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = make_float4(ot[dt][4 * i + 0] * beta, ot[dt][4 * i + 1] * beta, ot[dt][4 * i + 2] * beta,
                                     ot[dt][4 * i + 3] * beta);
        *reinterpret_cast<float4*>(a.o_acc + srow * D + 32 * dt + 8 * i + 4 * hh) = x;
      }
    if (hh == 0) {
      a.m[srow] = has ? m_true * kLn2 : -INFINITY;
      a.l[srow] = has ? l_tot * beta : 0.f;
    }
  }
}

template <int D, int NW>
hipError_t launch(const AttnArgs& a, hipStream_t st) {
  const int nqt = (a.Lq + Cfg<D, NW>::kBM - 1) / Cfg<D, NW>::kBM;
  const dim3 grid((unsigned)(nqt * a.B * a.H));
  hipLaunchKernelGGL((attn_bf16_kernel<D, NW>), grid, dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  if (a.D == 64) return launch<64, 8>(a, st);
  return launch<128, 8>(a, st);
}

}  // namespace cpring
