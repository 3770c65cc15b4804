// Rotary position embedding by global position (HBM-bound, no matrix cores).
//
// "Context Parallelism v.s. Sequence Parallelism (Megatron-LM)",
// "Implementation quirk: symmetric chunk assignment": under the chunk pairing a
// rank's tokens are not a contiguous run, so their rotary embedding must use
// the global position ids the partition produced, not a local 0, 1, 2, ...
// The rotation itself is the standard one: dimension pair (a_j, b_j) turned by
// pos * theta_j, theta_j = base^(-2j/D); pairs are (2j, 2j+1) (interleaved) or
// (j, j + D/2) (half split). Rows with position -1 (pads) are copied unchanged.
//
// Each thread owns one row position and a fixed group of 4 pairs and walks the
// heads, so its 4 sin/cos values are computed once; the frequencies are
// computed once per workgroup. Angles are formed and
// reduced modulo 2*pi in fp64 (positions reach 2^30, where an fp32 angle would
// be off by radians), then sin and cos are taken in fp32 of the reduced angle.
#include <math.h>

#include <algorithm>

#include "common.h"

namespace cpring {
namespace {

constexpr int kThreads = 256;
constexpr double kTwoPiHi = 6.283185307179586;      // 2*pi rounded to double
constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi

template <typename T>
struct Vec;   // 4 and 8 consecutive elements
template <>
struct Vec<__bf16> {
  typedef __bf16 v4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
  typedef __bf16 v8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
};
template <>
struct Vec<float> {
  typedef float v4 __attribute__((__vector_size__(4 * sizeof(float))));
  typedef float v8 __attribute__((__vector_size__(8 * sizeof(float))));
};

// fp32 sin / cos of pos * theta, reduced modulo 2*pi in fp64
__device__ __forceinline__ void angle_sincos(int32_t pos, double theta, float* s, float* c) {
  const double ang = (double)pos * theta;
  const double k = rint(ang * (1.0 / kTwoPiHi));
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
  sincosf((float)r, s, c);
}

// Workgroup (blockIdx.x, blockIdx.y): rows [blockIdx.x * kRowsPer, +kRowsPer) of
// the heads bh = blockIdx.y, blockIdx.y + gridDim.y, ...; D / 8 threads per row,
// thread g of a row rotating pairs 4g .. 4g+3.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads) rope_kernel(RopeArgs a) {
  using V4 = typename Vec<T>::v4;
  using V8 = typename Vec<T>::v8;
  constexpr int kGroups = D / 8;
  constexpr int kRowsPer = kThreads / kGroups;
  __shared__ double theta[D / 2];   // base^(-2j/D), once per workgroup
  if (threadIdx.x < D / 2) theta[threadIdx.x] = pow((double)a.base, -2.0 * (double)threadIdx.x / (double)D);
  __syncthreads();
  const int g = threadIdx.x % kGroups;
  const int i = blockIdx.x * kRowsPer + threadIdx.x / kGroups;
  if (i >= a.L) return;
  const int32_t p = a.pos[i];
  float sn[4], cs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sn[e] = 0.f;
    cs[e] = 1.f;
    if (p >= 0) angle_sincos(p, theta[4 * g + e], &sn[e], &cs[e]);
  }
  const int bh_total = a.B * a.H;
  for (int bh = blockIdx.y; bh < bh_total; bh += gridDim.y) {
    const int b = bh / a.H, h = bh - b * a.H;
    const T* src = static_cast<const T*>(a.x) + b * a.x_sb + h * a.x_sh + (int64_t)i * a.x_sl;
    T* dst = static_cast<T*>(a.out) + ((int64_t)bh * a.L + i) * D;
    float xa[4], xb[4];
    if (a.style == CPR_ROPE_INTERLEAVED) {
      const V8 v = *reinterpret_cast<const V8*>(src + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xa[e] = (float)v[2 * e];
        xb[e] = (float)v[2 * e + 1];
      }
    } else {
      const V4 va = *reinterpret_cast<const V4*>(src + 4 * g);
      const V4 vb = *reinterpret_cast<const V4*>(src + D / 2 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xa[e] = (float)va[e];
        xb[e] = (float)vb[e];
      }
    }
    float ya[4], yb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ya[e] = fmaf(xa[e], cs[e], -xb[e] * sn[e]);
      yb[e] = fmaf(xa[e], sn[e], xb[e] * cs[e]);
    }
    if (p < 0) {   // pad row: unchanged (also exact for inf / nan inputs)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ya[e] = xa[e];
        yb[e] = xb[e];
      }
    }
    if (a.style == CPR_ROPE_INTERLEAVED) {
      V8 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = (T)ya[e];
        v[2 * e + 1] = (T)yb[e];
      }
      *reinterpret_cast<V8*>(dst + 8 * g) = v;
    } else {
      V4 va, vb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        va[e] = (T)ya[e];
        vb[e] = (T)yb[e];
      }
      *reinterpret_cast<V4*>(dst + 4 * g) = va;
      *reinterpret_cast<V4*>(dst + D / 2 + 4 * g) = vb;
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const RopeArgs& a, hipStream_t st) {
  constexpr int kRowsPer = kThreads / (D / 8);
  const unsigned gx = (unsigned)((a.L + kRowsPer - 1) / kRowsPer);
  // enough workgroups to fill the chip several times over; each walks several heads when there are many
  const int64_t want_y = std::max<int64_t>(1, (int64_t)256 * 16 / gx);
  const unsigned gy = (unsigned)std::min<int64_t>({(int64_t)a.B * a.H, want_y, 65535});
  hipLaunchKernelGGL((rope_kernel<T, D>), dim3(gx, gy), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(int32_t dtype_bf16, const RopeArgs& a, hipStream_t st) {
  if (dtype_bf16) return a.D == 64 ? launch_t<__bf16, 64>(a, st) : launch_t<__bf16, 128>(a, st);
  return a.D == 64 ? launch_t<float, 64>(a, st) : launch_t<float, 128>(a, st);
}

}  // namespace cpring
