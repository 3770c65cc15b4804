// Running-state kernels: init, merge of two partial states, finalize, and the
// merge of a key-split launch's partial states fused with finalize.
// All three are streaming passes over the float32 state and bound by HBM.
//
// The running max / running normaliser and the rescaling of earlier partial
// sums follow "Sequence Parallelism and Ring Attention", sections "Deep dive"
// and "Technical insight". Finalize produces the normalised output that the
// glossary page ("Context Parallelism", "How context parallelism works") says
// equals full-sequence attention up to rounding.
//
// Thread layout for merge and finalize: D/4 consecutive threads own one row,
// each a float4 of O. 64 is a multiple of D/4, so a row never straddles two
// wavefronts; the row's m and l are read by every thread of the row before the
// first thread writes them back, in the same wavefront instruction order.
#include <math.h>

#include "common.h"

namespace cpring {

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  // round to nearest even; NaN stays NaN
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ void __launch_bounds__(256) state_init_kernel(float4* __restrict__ o, float* __restrict__ m,
                                                         float* __restrict__ l, int64_t rows, int32_t vpr) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * vpr) return;
  o[g] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (g % vpr == 0) {
    const int64_t r = g / vpr;
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
}

hipError_t launch_state_init(int64_t rows, int32_t D, float* o, float* m, float* l, hipStream_t st) {
  const int32_t vpr = D / 4;
  const int64_t total = rows * vpr;
  hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<float4*>(o), m, l, rows, vpr);
  return hipGetLastError();
}

// (o, m, l) <- (o, m, l) (+) (o2, m2, l2)
__global__ void __launch_bounds__(256) merge_kernel(float4* __restrict__ o, float* __restrict__ m,
                                                    float* __restrict__ l, const float4* __restrict__ o2,
                                                    const float* __restrict__ m2, const float* __restrict__ l2,
                                                    int64_t rows, int32_t vpr) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * vpr) return;
  const int64_t r = g / vpr;
  const float ma = m[r], mb = m2[r];
  const float la = l[r], lb = l2[r];
  const float mn = fmaxf(ma, mb);
  const float mu = (mn == -INFINITY) ? 0.f : mn;     // rows with nothing allowed on either side
  const float a = (ma == -INFINITY) ? 0.f : expf(ma - mu);
  const float b = (mb == -INFINITY) ? 0.f : expf(mb - mu);
  const float4 x = o[g], y = o2[g];
  o[g] = make_float4(a * x.x + b * y.x, a * x.y + b * y.y, a * x.z + b * y.z, a * x.w + b * y.w);
  if (g % vpr == 0) {
    m[r] = mn;
    l[r] = a * la + b * lb;
  }
}

hipError_t launch_merge(int64_t rows, int32_t D, float* o, float* m, float* l, const float* o2,
                        const float* m2, const float* l2, hipStream_t st) {
  const int32_t vpr = D / 4;
  const int64_t total = rows * vpr;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<float4*>(o), m, l, reinterpret_cast<const float4*>(o2), m2, l2, rows,
                     vpr);
  return hipGetLastError();
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(256) finalize_kernel(const float4* __restrict__ o, const float* __restrict__ m,
                                                       const float* __restrict__ l, void* __restrict__ out,
                                                       float* __restrict__ lse, int64_t rows, int32_t vpr) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * vpr) return;
  const int64_t r = g / vpr;
  const float lr = l[r];
  const bool has = lr > 0.f;
  const float inv = has ? 1.0f / lr : 0.f;
  const float4 x = o[g];
  const float4 y = make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv);
  if constexpr (OUT_BF16) {
    uint2 p;
    p.x = f32_to_bf16_rne(y.x) | (f32_to_bf16_rne(y.y) << 16);
    p.y = f32_to_bf16_rne(y.z) | (f32_to_bf16_rne(y.w) << 16);
    reinterpret_cast<uint2*>(out)[g] = p;
  } else {
    reinterpret_cast<float4*>(out)[g] = y;
  }
  if (lse && g % vpr == 0) lse[r] = has ? m[r] + logf(lr) : -INFINITY;
}

hipError_t launch_finalize(int out_bf16, int64_t rows, int32_t D, const float* o, const float* m,
                           const float* l, void* out, float* lse, hipStream_t st) {
  const int32_t vpr = D / 4;
  const int64_t total = rows * vpr;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (out_bf16)
    hipLaunchKernelGGL(finalize_kernel<true>, grid, dim3(256), 0, st, reinterpret_cast<const float4*>(o), m, l,
                       out, lse, rows, vpr);
  else
    hipLaunchKernelGGL(finalize_kernel<false>, grid, dim3(256), 0, st, reinterpret_cast<const float4*>(o), m, l,
                       out, lse, rows, vpr);
  return hipGetLastError();
}

// Merge of nsplit partial states over disjoint key sets, then finalize: per
// row, m = max_j m_j, a_j = exp(m_j - m) (0 for an empty partial), l = sum_j
// a_j l_j, O = sum_j a_j O_j / l, LSE = m + ln l; a row with l = 0 gives
// O = 0, LSE = -inf. The same rescale rule as merge_kernel, over nsplit inputs.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) merge_finalize_kernel(const float4* __restrict__ o,
                                                             const float* __restrict__ m,
                                                             const float* __restrict__ l, void* __restrict__ out,
                                                             float* __restrict__ lse, int32_t nsplit, int64_t rows,
                                                             int32_t vpr) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= rows * vpr) return;
  const int64_t r = g / vpr;
  float mx = -INFINITY;
  for (int j = 0; j < nsplit; ++j) mx = fmaxf(mx, m[j * rows + r]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  float lt = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < nsplit; ++j) {
    const float mj = m[j * rows + r];
    const float aj = (mj == -INFINITY) ? 0.f : expf(mj - mu);
    const float4 x = o[j * rows * vpr + g];
    lt += aj * l[j * rows + r];
    acc.x += aj * x.x;
    acc.y += aj * x.y;
    acc.z += aj * x.z;
    acc.w += aj * x.w;
  }
  const bool has = lt > 0.f;
  const float inv = has ? 1.0f / lt : 0.f;
  const float4 y = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if constexpr (OUT_BF16) {
    uint2 p;
    p.x = f32_to_bf16_rne(y.x) | (f32_to_bf16_rne(y.y) << 16);
    p.y = f32_to_bf16_rne(y.z) | (f32_to_bf16_rne(y.w) << 16);
    reinterpret_cast<uint2*>(out)[g] = p;
  } else {
    reinterpret_cast<float4*>(out)[g] = y;
  }
  if (lse && g % vpr == 0) lse[r] = has ? mx + logf(lt) : -INFINITY;
}

hipError_t launch_merge_finalize(int out_bf16, int32_t nsplit, int64_t rows, int32_t D, const float* o,
                                 const float* m, const float* l, void* out, float* lse, hipStream_t st) {
  const int32_t vpr = D / 4;
  const int64_t total = rows * vpr;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (out_bf16)
    hipLaunchKernelGGL(merge_finalize_kernel<true>, grid, dim3(256), 0, st, reinterpret_cast<const float4*>(o), m,
                       l, out, lse, nsplit, rows, vpr);
  else
    hipLaunchKernelGGL(merge_finalize_kernel<false>, grid, dim3(256), 0, st, reinterpret_cast<const float4*>(o), m,
                       l, out, lse, nsplit, rows, vpr);
  return hipGetLastError();
}

}  // namespace cpring
