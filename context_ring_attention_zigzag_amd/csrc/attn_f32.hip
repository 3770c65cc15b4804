// float32 ring-attention pass (plain FMA, no matrix cores).
//
// The float32 inputs of the small workloads need ~1e-5 agreement with the
// float64 definition, so nothing here goes through bf16: scores, softmax and
// P*V all run in float32 VALU arithmetic with the accurate expf.
//
// Work split: a workgroup of 256 threads owns 64 query rows of one (b, h);
// 4 consecutive lanes share a row, each holding D/4 of its dimensions.
// K, V and their positions arrive in LDS 32 keys at a time; every lane folds
// the tile into its row's running (O, m, l) with the online-softmax rule of
// "Sequence Parallelism and Ring Attention" ("Deep dive", "Technical
// insight"). Blocks are visited in ring order, block t being the one that
// started on rank (rank - t) mod cp ("Context Parallelism", "How context
// parallelism works").
#include <math.h>

#include "common.h"

namespace cpring {
namespace {

constexpr int kRows = 64;      // query rows per workgroup
constexpr int kLanesPerRow = 4;
constexpr int kKeys = 32;      // keys per LDS tile

template <int D>
__global__ void __launch_bounds__(256) attn_f32_kernel(AttnArgs a) {
  constexpr int DS = D / kLanesPerRow;   // dims per lane
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];
  __shared__ int32_t ps[kKeys];

  const int tid = threadIdx.x;
  const int nqt = (a.Lq + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int row = qt * kRows + tid / kLanesPerRow;
  const int sub = tid % kLanesPerRow;
  const int d0 = sub * DS;
  const bool in_range = row < a.Lq;
  const int32_t qp = in_range ? a.q_pos[row] : -1;
  // allowed key positions [lb, ub]: causal bound, optional per-query window;
  // a pad query gets an empty range
  int32_t lb = 0, ub = -1;
  if (qp >= 0) {
    lb = a.kw_lo ? max(a.kw_lo[row], 0) : 0;
    ub = a.causal ? qp : INT_MAX;
    if (a.kw_hi) ub = min(ub, a.kw_hi[row]);
  }

  const float* qg = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh;
  float q[DS];
#pragma unroll
  for (int i = 0; i < DS; ++i) q[i] = in_range ? qg[(int64_t)row * a.q_sl + d0 + i] : 0.f;

  float o[DS];
  float m = -INFINITY, l = 0.f;
  const int64_t srow = ((int64_t)bh * a.Lq + row);
  if (a.load_state && in_range) {
#pragma unroll
    for (int i = 0; i < DS; ++i) o[i] = a.o_acc[srow * D + d0 + i];
    m = a.m[srow];
    l = a.l[srow];
  } else {
#pragma unroll
    for (int i = 0; i < DS; ++i) o[i] = 0.f;
  }

  const int hk = h / (a.H / a.H_kv);   // grouped-query attention: the K/V head of query head h
  const float* kg = static_cast<const float*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const float* vg = static_cast<const float*>(a.v) + b * a.v_sb + hk * a.v_sh;

  for (int t = 0; t < a.nblocks; ++t) {
    int src = (a.rank - t) % a.cp;
    if (src < 0) src += a.cp;
    const int64_t base = (int64_t)src * a.Lk;
    for (int j0 = 0; j0 < a.Lk; j0 += kKeys) {
      __syncthreads();
      for (int e = tid; e < kKeys * D; e += 256) {
        const int kr = e / D, kd = e - (e / D) * D;
        const bool ok = j0 + kr < a.Lk;
        const int64_t gr = base + j0 + kr;
        ks[kr][kd] = ok ? kg[gr * a.k_sl + kd] : 0.f;
        vs[kr][kd] = ok ? vg[gr * a.v_sl + kd] : 0.f;
      }
      if (tid < kKeys) ps[tid] = (j0 + tid < a.Lk) ? a.kv_pos[base + j0 + tid] : -1;
      __syncthreads();

      float s[kKeys];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < DS; ++i) part = fmaf(q[i], ks[j][d0 + i], part);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        const int32_t kp = ps[j];
        const bool allowed = kp >= lb && kp <= ub;   // lb >= 0 also excludes pad keys (-1)
        s[j] = allowed ? part * a.scale : -INFINITY;
        tmax = fmaxf(tmax, s[j]);
      }
      const float mn = fmaxf(m, tmax);
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - mu);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < DS; ++i) o[i] *= alpha;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) {
        const float p = (s[j] == -INFINITY) ? 0.f : expf(s[j] - mu);
        psum += p;
#pragma unroll
        for (int i = 0; i < DS; ++i) o[i] = fmaf(p, vs[j][d0 + i], o[i]);
      }
      l = alpha * l + psum;
      m = mn;
    }
  }

  if (!in_range) return;
  if (a.finalize) {
    const bool has = l > 0.f && qp >= 0;
    const float inv = has ? 1.0f / l : 0.f;
    float* out = static_cast<float*>(a.o_out) + srow * D + d0;
#pragma unroll
    for (int i = 0; i < DS; ++i) out[i] = o[i] * inv;
    if (a.lse && sub == 0) a.lse[srow] = has ? m + logf(l) : -INFINITY;
  } else {
#pragma unroll
    for (int i = 0; i < DS; ++i) a.o_acc[srow * D + d0 + i] = o[i];
    if (sub == 0) {
      a.m[srow] = m;
      a.l[srow] = l;
    }
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  const int nqt = (a.Lq + kRows - 1) / kRows;
  const dim3 grid((unsigned)(nqt * a.B * a.H));
  if (a.D == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace cpring
