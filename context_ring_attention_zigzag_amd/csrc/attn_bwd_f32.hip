// float32 backward ring pass (plain FMA, no matrix cores).
//
// Same gradients as the bf16 kernels ("Context Parallelism", "Practical use
// and trade-offs": the context-parallel output is differentiated; block
// handling as in "Sequence Parallelism and Ring Attention", "Deep dive"), at
// float32 accuracy: P = 2^(scale * log2(e) * q.k - lse2) from the saved LSE,
// dS = P * (dO.v - Dvec), dQ = scale * sum dS k, dK = scale * sum dS q,
// dV = sum P dO, with the {lse2, Dvec} and {lo, hi} rows of the
// preprocessing pass.
//
// Work split as in the float32 forward kernel: a workgroup of 256 threads owns
// 64 rows (queries for dQ, keys for dK/dV) of one head, 4 lanes per row with
// D/4 dimensions each; the other side streams through LDS 32 rows at a time.
#include <math.h>

#include "common.h"

namespace cpring {
namespace {

constexpr int kRows = 64;
constexpr int kLanesPerRow = 4;
constexpr int kTile = 32;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

template <int D>
__global__ void __launch_bounds__(256) bwd_dq_f32_kernel(BwdArgs a) {
  constexpr int DS = D / kLanesPerRow;
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  __shared__ int32_t ps[kTile];

  const int tid = threadIdx.x;
  const int nqt = (a.Lq + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int row = qt * kRows + tid / kLanesPerRow;
  const int d0 = (tid % kLanesPerRow) * DS;
  const bool in_range = row < a.Lq;
  const int64_t srow = (int64_t)bh * a.Lq + row;
  int32_t lo = 1, hi = 0;
  float lse2 = INFINITY, dvec = 0.f;
  if (in_range) {
    const int2 w = a.qwin[row];
    lo = w.x;
    hi = w.y;
    lse2 = a.lse2[srow];
    dvec = a.dvec[srow];
  }

  const float* qg = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)row * a.q_sl + d0;
  const float* gg = static_cast<const float*>(a.dout) + b * a.do_sb + h * a.do_sh + (int64_t)row * a.do_sl + d0;
  float q[DS], g[DS], dq[DS];
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    q[i] = in_range ? qg[i] : 0.f;
    g[i] = in_range ? gg[i] : 0.f;
    dq[i] = 0.f;
  }
  const float c2 = a.scale * kLog2e;
  const int hk = h / (a.H / a.H_kv);
  const float* kg = static_cast<const float*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const float* vg = static_cast<const float*>(a.v) + b * a.v_sb + hk * a.v_sh;

  for (int t = 0; t < a.nblocks; ++t) {
    int src = (a.rank - t) % a.cp;
    if (src < 0) src += a.cp;
    const int64_t base = (int64_t)src * a.Lk;
    for (int j0 = 0; j0 < a.Lk; j0 += kTile) {
      __syncthreads();
      for (int e = tid; e < kTile * D; e += 256) {
        const int kr = e / D, kd = e - (e / D) * D;
        const bool ok = j0 + kr < a.Lk;
        const int64_t gr = base + j0 + kr;
        ks[kr][kd] = ok ? kg[gr * a.k_sl + kd] : 0.f;
        vs[kr][kd] = ok ? vg[gr * a.v_sl + kd] : 0.f;
      }
      if (tid < kTile) ps[tid] = (j0 + tid < a.Lk) ? a.kv_pos[base + j0 + tid] : -1;
      __syncthreads();
#pragma unroll 4
      for (int j = 0; j < kTile; ++j) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < DS; ++i) {
          s = fmaf(q[i], ks[j][d0 + i], s);
          dp = fmaf(g[i], vs[j][d0 + i], dp);
        }
        s = quad_sum(s);
        dp = quad_sum(dp);
        const int32_t kp = ps[j];
        const bool allowed = kp >= lo && kp <= hi;   // lo >= 0 also excludes pad keys (-1)
        const float p = allowed ? exp2f(fmaf(s, c2, -lse2)) : 0.f;
        const float ds = p * (dp - dvec);
#pragma unroll
        for (int i = 0; i < DS; ++i) dq[i] = fmaf(ds, ks[j][d0 + i], dq[i]);
      }
    }
  }

  if (!in_range) return;
  float* out = a.dq + srow * D + d0;
#pragma unroll
  for (int i = 0; i < DS; ++i) out[i] = a.scale * dq[i] + (a.accumulate ? out[i] : 0.f);
}

template <int D>
__global__ void __launch_bounds__(256) bwd_dkv_f32_kernel(BwdArgs a) {
  constexpr int DS = D / kLanesPerRow;
  __shared__ float qs[kTile][D];
  __shared__ float gs[kTile][D];
  __shared__ float2 qis[kTile];   // {lse2, dvec}
  __shared__ int2 qws[kTile];

  const int tid = threadIdx.x;
  const int64_t lk_total = (int64_t)a.nblocks * a.Lk;
  const int nkt = (int)((lk_total + kRows - 1) / kRows);
  const int bhk = blockIdx.x / nkt;
  const int kt = blockIdx.x - bhk * nkt;
  const int b = bhk / a.H_kv, hk = bhk - (bhk / a.H_kv) * a.H_kv;
  const int64_t row = (int64_t)kt * kRows + tid / kLanesPerRow;
  const int d0 = (tid % kLanesPerRow) * DS;
  const bool in_range = row < lk_total;
  const int32_t kp = in_range ? a.kv_pos[row] : -1;

  const float* kg = static_cast<const float*>(a.k) + b * a.k_sb + hk * a.k_sh + row * a.k_sl + d0;
  const float* vg = static_cast<const float*>(a.v) + b * a.v_sb + hk * a.v_sh + row * a.v_sl + d0;
  float k[DS], v[DS], dk[DS], dv[DS];
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    k[i] = in_range ? kg[i] : 0.f;
    v[i] = in_range ? vg[i] : 0.f;
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  const float c2 = a.scale * kLog2e;
  const int group = a.H / a.H_kv;

  for (int gi = 0; gi < group; ++gi) {
    const int h = hk * group + gi;
    const float* qg = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh;
    const float* gg = static_cast<const float*>(a.dout) + b * a.do_sb + h * a.do_sh;
    const int64_t qrow0 = (int64_t)(b * a.H + h) * a.Lq;
    for (int i0 = 0; i0 < a.Lq; i0 += kTile) {
      __syncthreads();
      for (int e = tid; e < kTile * D; e += 256) {
        const int r = e / D, c = e - (e / D) * D;
        const bool ok = i0 + r < a.Lq;
        qs[r][c] = ok ? qg[(int64_t)(i0 + r) * a.q_sl + c] : 0.f;
        gs[r][c] = ok ? gg[(int64_t)(i0 + r) * a.do_sl + c] : 0.f;
      }
      if (tid < kTile) {
        const bool ok = i0 + tid < a.Lq;
        qis[tid] = ok ? make_float2(a.lse2[qrow0 + i0 + tid], a.dvec[qrow0 + i0 + tid])
                      : make_float2(INFINITY, 0.f);
        qws[tid] = ok ? a.qwin[i0 + tid] : make_int2(1, 0);
      }
      __syncthreads();
#pragma unroll 4
      for (int j = 0; j < kTile; ++j) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < DS; ++i) {
          s = fmaf(qs[j][d0 + i], k[i], s);
          dp = fmaf(gs[j][d0 + i], v[i], dp);
        }
        s = quad_sum(s);
        dp = quad_sum(dp);
        const int2 w = qws[j];
        const bool allowed = kp >= w.x && kp <= w.y;
        const float2 inf = qis[j];
        const float p = allowed ? exp2f(fmaf(s, c2, -inf.x)) : 0.f;
        const float ds = p * (dp - inf.y);
#pragma unroll
        for (int i = 0; i < DS; ++i) {
          dv[i] = fmaf(p, gs[j][d0 + i], dv[i]);
          dk[i] = fmaf(ds, qs[j][d0 + i], dk[i]);
        }
      }
    }
  }

  if (!in_range) return;
  const int64_t krow = (int64_t)bhk * lk_total + row;
  float* dko = a.dk + krow * D + d0;
  float* dvo = a.dv + krow * D + d0;
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    dko[i] = a.scale * dk[i] + (a.accumulate ? dko[i] : 0.f);
    dvo[i] = dv[i] + (a.accumulate ? dvo[i] : 0.f);
  }
}

template <int D>
hipError_t launch_t(const BwdArgs& a, int32_t do_dq, int32_t do_dkv, hipStream_t st) {
  if (do_dq) {
    const int nqt = (a.Lq + kRows - 1) / kRows;
    hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, dim3((unsigned)(nqt * a.B * a.H)), dim3(256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (do_dkv) {
    const int64_t nkt = ((int64_t)a.nblocks * a.Lk + kRows - 1) / kRows;
    hipLaunchKernelGGL(bwd_dkv_f32_kernel<D>, dim3((unsigned)(nkt * a.B * a.H_kv)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, int32_t do_dq, int32_t do_dkv, hipStream_t st) {
  return a.D == 64 ? launch_t<64>(a, do_dq, do_dkv, st) : launch_t<128>(a, do_dq, do_dkv, st);
}

}  // namespace cpring
