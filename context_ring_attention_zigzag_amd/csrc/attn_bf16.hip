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
//  * keys stream through LDS in tiles of BN = 64, double-buffered, loaded with
//    coalesced 16-byte global loads and XOR-swizzled against bank conflicts;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: lane l then holds query l%32 and 16 of the 32
//    keys of a 32x32 block, so the per-query max and sum are lane-local plus
//    one exchange between the two half-waves (v_permlane32_swap);
//  * O^T = V^T P^T on the same MFMA: the probabilities leave the score
//    accumulators already in the B-operand layout (rounded to bf16), and V^T
//    comes straight from the row-major V tile through ds_read_b64_tr_b16;
//  * (query tile, key tile) pairs are classified from their position ranges
//    into skip / full / mixed; skipped tiles are neither loaded nor computed,
//    full tiles need no element mask;
//  * the grid is remapped so that the workgroups of one (b, h) land on the
//    same XCD (shared L2), heaviest query tiles first.
#include <math.h>

#include "common.h"

namespace cpring {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;        // MI355X: 8 accelerator complex dies, workgroups dealt round-robin
constexpr int kBN = 64;         // keys per tile
constexpr int kMaxTiles = 4096; // tiles classified per pass (bitmask of kMaxTiles/64 words)

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // round to nearest even (finite inputs)
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a += 0x7fffu + ((a >> 16) & 1u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (a >> 16) | (b & 0xffff0000u);
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

template <int D, int NW>
struct Cfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBM = 32 * NW;          // queries per workgroup
  static constexpr int kKSteps = D / 16;       // MFMA steps over the head dim
  static constexpr int kDTiles = D / 32;       // 32-row tiles of O^T
  static constexpr int kChunksPerRow = D / 8;  // 16-byte chunks per K/V row
  static constexpr int kLoads = kBN * kChunksPerRow / kThreads;  // 16-byte loads per thread per tensor
  static_assert(kLoads >= 1 && kBN * kChunksPerRow % kThreads == 0, "tile/threads mismatch");
};

// LDS swizzles (16-byte chunk index XOR a function of the row).
// K: lanes 0..7 of an A-operand read hit rows r..r+7 at one chunk -> XOR row%8.
// V: a 16-lane transpose read covers 4 consecutive rows x 2 chunks -> XOR 2*(row%4).
__device__ __forceinline__ int swz_k(int row, int chunk) { return chunk ^ (row & 7); }
__device__ __forceinline__ int swz_v(int row, int chunk) { return chunk ^ ((row & 3) << 1); }

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 2) attn_bf16_kernel(AttnArgs a) {
  using C = Cfg<D, NW>;
  constexpr int kThreads = C::kThreads;

  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kBN * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kBN * D];
  __shared__ __attribute__((aligned(16))) int32_t pos_lds[2][kBN];
  __shared__ uint64_t keep_w[kMaxTiles / 64];
  __shared__ uint64_t mixed_w[kMaxTiles / 64];
  __shared__ int32_t qrange[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  f32x16 ot[C::kDTiles];
  float m2 = -INFINITY;   // running max, log2 units of the scaled score
  float lsum = 0.f;       // this half-wave's share of the running sum
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
    m2 = (mn == -INFINITY) ? -INFINITY : mn * kLog2e;
    lsum = hh == 0 ? a.l[srow] : 0.f;
  } else {
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) ot[dt][i] = 0.f;
  }

  const float c2 = a.scale * kLog2e;   // score -> log2 units
  const bool wg_has_queries = qmax >= 0;

  const __bf16* kbh = static_cast<const __bf16*>(a.k) + b * a.k_sb + h * a.k_sh;
  const __bf16* vbh = static_cast<const __bf16*>(a.v) + b * a.v_sb + h * a.v_sh;
  const int n_kt = (a.Lk + kBN - 1) / kBN;

  for (int t = 0; t < a.nblocks && wg_has_queries; ++t) {
    int src = (a.rank - t) % a.cp;
    if (src < 0) src += a.cp;
    const int64_t row0 = (int64_t)src * a.Lk;        // first row of this block
    const int32_t* posb = a.kv_pos + row0;
    const __bf16* kb = kbh + row0 * a.k_sl;
    const __bf16* vb = vbh + row0 * a.v_sl;

    for (int seg0 = 0; seg0 < n_kt; seg0 += kMaxTiles) {
      const int nseg = min(kMaxTiles, n_kt - seg0);

      // ---- classify the segment's key tiles against this query tile
      __syncthreads();
      for (int tt = tid; tt < ((nseg + 63) & ~63); tt += kThreads) {
        bool keep = false, mixed = false;
        if (tt < nseg) {
          const int k0 = (seg0 + tt) * kBN;
          const int k1 = min(k0 + kBN, a.Lk);
          int kmin = INT_MAX, kmax = -1;
          bool pad = (k1 - k0) < kBN;
          for (int j = k0; j < k1; ++j) {
            const int p = posb[j];
            pad |= p < 0;
            kmin = (p >= 0 && p < kmin) ? p : kmin;
            kmax = p > kmax ? p : kmax;
          }
          keep = kmax >= 0 && (!a.causal || kmin <= qmax);
          const bool full = !pad && (!a.causal || kmax <= qmin);
          mixed = keep && !full;
        }
        const uint64_t kw = __ballot(keep);
        const uint64_t mw = __ballot(mixed);
        if (lane == 0) {
          keep_w[tt >> 6] = kw;
          mixed_w[tt >> 6] = mw;
        }
      }
      __syncthreads();

      const int nwords = (nseg + 63) >> 6;
      auto next_kept = [&](int j) -> int {   // first kept tile index > j, or nseg
        int w = (j + 1) >> 6;
        if (w >= nwords) return nseg;
        uint64_t bits = keep_w[w] & (~0ull << ((j + 1) & 63));
        while (bits == 0) {
          if (++w >= nwords) return nseg;
          bits = keep_w[w];
        }
        return min(nseg, (w << 6) + (int)__builtin_ctzll(bits));
      };

      uint4 kreg[C::kLoads], vreg[C::kLoads];
      int32_t preg = -1;
      auto load_tile = [&](int j) {
        const int r_base = (seg0 + j) * kBN;
#pragma unroll
        for (int u = 0; u < C::kLoads; ++u) {
          const int cidx = tid + u * kThreads;
          const int row = cidx / C::kChunksPerRow;
          const int ch = cidx % C::kChunksPerRow;
          if (r_base + row < a.Lk) {
            kreg[u] = *reinterpret_cast<const uint4*>(kb + (int64_t)(r_base + row) * a.k_sl + ch * 8);
            vreg[u] = *reinterpret_cast<const uint4*>(vb + (int64_t)(r_base + row) * a.v_sl + ch * 8);
          } else {
            kreg[u] = make_uint4(0u, 0u, 0u, 0u);
            vreg[u] = make_uint4(0u, 0u, 0u, 0u);
          }
        }
        if (tid < kBN) preg = (r_base + tid < a.Lk) ? posb[r_base + tid] : -1;
      };
      auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < C::kLoads; ++u) {
          const int cidx = tid + u * kThreads;
          const int row = cidx / C::kChunksPerRow;
          const int ch = cidx % C::kChunksPerRow;
          *reinterpret_cast<uint4*>(&k_lds[buf][row * D + swz_k(row, ch) * 8]) = kreg[u];
          *reinterpret_cast<uint4*>(&v_lds[buf][row * D + swz_v(row, ch) * 8]) = vreg[u];
        }
        if (tid < kBN) pos_lds[buf][tid] = preg;
      };

      int j = next_kept(-1);
      if (j < nseg) {
        load_tile(j);
        store_tile(0);
      }
      __syncthreads();
      int buf = 0;
      while (j < nseg) {
        const int jn = next_kept(j);
        const bool has_next = jn < nseg;
        const bool mixed = (mixed_w[j >> 6] >> (j & 63)) & 1ull;
        if (has_next) load_tile(jn);

        // ---- S^T = K Q^T for two 32-key sub-tiles
        const __bf16* kl = k_lds[buf];
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const int row = kt * 32 + ql;
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + row * D + swz_k(row, 2 * kk + hh) * 8);
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[kt], 0, 0, 0);
          }
        }

        // ---- mask (only tiles straddling the causal boundary or holding pads)
        if (mixed) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int4 p = *reinterpret_cast<const int4*>(&pos_lds[buf][kt * 32 + 8 * i + 4 * hh]);
              const int pk[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const bool ok = pk[jj] >= 0 && qp >= 0 && (!a.causal || pk[jj] <= qp);
                s[kt][4 * i + jj] = ok ? s[kt][4 * i + jj] : -INFINITY;
              }
            }
        }

        // ---- online softmax (log2 units)
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
        mx = other_half_max(mx);
        const float m_new = fmaxf(m2, mx * c2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        if (__any(m_new > m2)) {
          const float alpha = __builtin_amdgcn_exp2f(m2 - m_use);
#pragma unroll
          for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) ot[dt][i] *= alpha;
          lsum *= alpha;
        }
        m2 = m_new;

        // probabilities -> bf16 B operand of O^T += V^T P^T (16 keys per chunk)
        bf16x8 pb[4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            float e[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
              e[x] = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * p + x], c2, -m_use));
              lsum += e[x];
            }
            uint32_t w4[4] = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                              pack_bf16x2(e[6], e[7])};
            pb[2 * kt + p] = __builtin_bit_cast(bf16x8, w4);
          }

        // ---- O^T += V^T P^T; V^T rows via the LDS transpose read
        const __bf16* vl = v_lds[buf];
        const int g = lane >> 4, gi = lane & 15;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
          for (int dt = 0; dt < C::kDTiles; ++dt) {
            const int row_a = 16 * ch + 4 * (g >> 1) + (gi >> 2);
            const int row_b = row_a + 8;
            const int col = 32 * dt + 16 * (g & 1) + 4 * (gi & 3);
            const __bf16* pa = vl + row_a * D + swz_v(row_a, col >> 3) * 8 + (col & 7);
            const __bf16* pbp = vl + row_b * D + swz_v(row_b, col >> 3) * 8 + (col & 7);
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pbp);
            const s16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            ot[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pb[ch], ot[dt], 0, 0, 0);
          }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
        buf ^= 1;
        j = jn;
      }
    }
  }

  // ---- epilogue
  const float l_tot = other_half_sum(lsum);
  if (!q_in) return;
  const bool has = qp >= 0 && l_tot > 0.f;
  if (a.finalize) {
    const float inv = has ? 1.0f / l_tot : 0.f;
    __bf16* out = static_cast<__bf16*>(a.o_out) + srow * D;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 w;
        w.x = pack_bf16x2(ot[dt][4 * i + 0] * inv, ot[dt][4 * i + 1] * inv);
        w.y = pack_bf16x2(ot[dt][4 * i + 2] * inv, ot[dt][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(out + 32 * dt + 8 * i + 4 * hh) = w;
      }
    if (a.lse && hh == 0) a.lse[srow] = has ? m2 * kLn2 + logf(l_tot) : -INFINITY;
  } else {
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 x = make_float4(ot[dt][4 * i + 0], ot[dt][4 * i + 1], ot[dt][4 * i + 2], ot[dt][4 * i + 3]);
        if (qp < 0) x = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(a.o_acc + srow * D + 32 * dt + 8 * i + 4 * hh) = x;
      }
    if (hh == 0) {
      a.m[srow] = (qp >= 0 && m2 != -INFINITY) ? m2 * kLn2 : -INFINITY;
      a.l[srow] = qp >= 0 ? l_tot : 0.f;
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
  if (a.D == 64) return launch<64, 4>(a, st);
  const long tiles8 = (long)a.B * a.H * ((a.Lq + 255) / 256);
  if (tiles8 >= 512) return launch<128, 8>(a, st);
  return launch<128, 4>(a, st);
}

}  // namespace cpring
