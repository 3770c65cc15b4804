// Cycle costs on gfx950 that the kernel designs rest on: the bf16 32x32x16
// MFMA (register-fed stream, chip-wide rate), vector instructions per wave64
// instruction, and an MFMA stream co-executing with a vector stream on one
// SIMD. Timing: s_memtime (shader clock) per wave, hipEvent per launch. Every
// kernel writes only its own output slots.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

#define CHECK(x)                                                                 \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));             \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

constexpr int kIters = 8192;
// dynamic LDS per workgroup: more than half of the 160 KB of a compute unit, so
// each unit holds one workgroup and a SIMD runs exactly the waves named below
constexpr size_t kReserve = 96 * 1024;

// MFMA stream: 4 independent accumulators, kIters x 4 MFMAs per wave.
// Waves with (wave & 4) == role_mask run it; with the vector kernel below
// sharing the workgroup, waves w and w + 4 share a SIMD.
__device__ __forceinline__ void mfma_stream(f32x16 (&acc)[4], bf16x8 a, bf16x8 b) {
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
}

// Vector stream: kIters x 8 instructions of one kind over 8 independent chains.
template <int OP>
__device__ __forceinline__ void valu_stream(float (&x)[8]) {
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (OP == 0) asm volatile("v_fma_f32 %0, %0, %0, 1.0" : "+v"(x[j]));
      else if constexpr (OP == 1) asm volatile("v_exp_f32 %0, %0" : "+v"(x[j]));
      else if constexpr (OP == 2) asm volatile("v_max3_f32 %0, %0, %0, 1.0" : "+v"(x[j]));
      else if constexpr (OP == 3) asm volatile("v_add_f32 %0, %0, %0" : "+v"(x[j]));
      else asm volatile("v_cvt_pk_bf16_f32 %0, %0, %0" : "+v"(x[j]));
    }
  }
}

// mode 0: waves 0-3 MFMA only; 1: waves 0-3 vector only (OP); 2: waves 0-3 MFMA, waves 4-7 vector (OP)
template <int OP>
__global__ void __launch_bounds__(512) cycles_kernel(int mode, int nwaves, uint64_t* out, float* sink) {
  extern __shared__ char reserve[];   // sized at launch so that one workgroup fits a compute unit
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x == 0) reserve[0] = 0;
  uint64_t t0 = 0, t1 = 0;
  float res = 0.f;
  const bool do_mfma = (mode == 0 || mode == 2) && wave < 4 && wave < nwaves;
  const bool do_valu = (mode == 1 && wave < 4 && wave < nwaves) || (mode == 2 && wave >= 4);
  __syncthreads();
  if (do_mfma) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (lane + i));
      b[i] = (__bf16)(0.002f * (lane - i));
    }
    f32x16 acc[4] = {};
    t0 = __builtin_amdgcn_s_memtime();
    mfma_stream(acc, a, b);
    for (int j = 0; j < 4; ++j) res += acc[j][0];
    asm volatile("" ::"v"(res));
    t1 = __builtin_amdgcn_s_memtime();
  } else if (do_valu) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.5f + 0.001f * (lane + j);
    t0 = __builtin_amdgcn_s_memtime();
    valu_stream<OP>(x);
    for (int j = 0; j < 8; ++j) res += x[j];
    asm volatile("" ::"v"(res));
    t1 = __builtin_amdgcn_s_memtime();
  }
  if (lane == 0) out[blockIdx.x * 8 + wave] = t1 - t0;
  sink[blockIdx.x * 512 + threadIdx.x] = res;
}

template <int OP>
int run(const char* name, int mode, int nwaves, int nblk, uint64_t* d_out, float* d_sink, double* wave_cycles,
        double* ms) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int rep = 0; rep < 3; ++rep) {
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(cycles_kernel<OP>, dim3(nblk), dim3(512), kReserve, 0, mode, nwaves, d_out, d_sink);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
  }
  float t = 0.f;
  CHECK(hipEventElapsedTime(&t, e0, e1));
  std::vector<uint64_t> h((size_t)nblk * 8);
  CHECK(hipMemcpy(h.data(), d_out, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
  // mean over the waves that ran the measured stream (mode 2: the vector waves 4-7 and MFMA waves 0-3 separately)
  double s0 = 0, s1 = 0;
  int n0 = 0, n1 = 0;
  for (int b = 0; b < nblk; ++b)
    for (int w = 0; w < 8; ++w) {
      const double c = (double)h[b * 8 + w];
      if (c == 0) continue;
      if (w < 4) { s0 += c; ++n0; } else { s1 += c; ++n1; }
    }
  wave_cycles[0] = n0 ? s0 / n0 : 0;
  wave_cycles[1] = n1 ? s1 / n1 : 0;
  *ms = t;
  (void)name;
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return 0;
}

int main() {
  const int nblk = 256;   // one workgroup per compute unit
  CHECK(hipFuncSetAttribute((const void*)cycles_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, kReserve));
  CHECK(hipFuncSetAttribute((const void*)cycles_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, kReserve));
  CHECK(hipFuncSetAttribute((const void*)cycles_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, kReserve));
  CHECK(hipFuncSetAttribute((const void*)cycles_kernel<3>, hipFuncAttributeMaxDynamicSharedMemorySize, kReserve));
  CHECK(hipFuncSetAttribute((const void*)cycles_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize, kReserve));
  uint64_t* d_out;
  float* d_sink;
  CHECK(hipMalloc(&d_out, (size_t)nblk * 8 * sizeof(uint64_t)));
  CHECK(hipMalloc(&d_sink, (size_t)nblk * 512 * sizeof(float)));
  CHECK(hipMemset(d_out, 0, (size_t)nblk * 8 * sizeof(uint64_t)));
  double wc[2], ms;
  const double mfma_per_wave = 4.0 * kIters, flop_per_mfma = 2.0 * 32 * 32 * 16;

  // MFMA-only stream, one wave per SIMD (waves 0-3)
  if (run<0>("mfma", 0, 4, nblk, d_out, d_sink, wc, &ms)) return 1;
  const double tflops = nblk * 4 * mfma_per_wave * flop_per_mfma / (ms * 1e-3) / 1e12;
  printf("mfma_f32_32x32x16_bf16 register-fed: %.1f cycles per MFMA per SIMD; chip %.0f TFLOP/s (%.1f%% of 2,500); "
         "shader clock from s_memtime over the launch: %.2f GHz\n",
         wc[0] / mfma_per_wave, tflops, 100.0 * tflops / 2500.0, wc[0] / (ms * 1e6));
  const char* names[5] = {"v_fma_f32", "v_exp_f32", "v_max3_f32", "v_add_f32", "v_cvt_pk_bf16_f32"};
  double alone[5];
  for (int op = 0; op < 5; ++op) {
    int r = 0;
    if (op == 0) r = run<0>("", 1, 4, nblk, d_out, d_sink, wc, &ms);
    if (op == 1) r = run<1>("", 1, 4, nblk, d_out, d_sink, wc, &ms);
    if (op == 2) r = run<2>("", 1, 4, nblk, d_out, d_sink, wc, &ms);
    if (op == 3) r = run<3>("", 1, 4, nblk, d_out, d_sink, wc, &ms);
    if (op == 4) r = run<4>("", 1, 4, nblk, d_out, d_sink, wc, &ms);
    if (r) return 1;
    alone[op] = wc[0] / (8.0 * kIters);
    printf("%-18s one wave per SIMD: %.2f cycles per wave64 instruction\n", names[op], alone[op]);
  }
  // co-execution: one MFMA wave and one vector wave (v_fma_f32 or v_exp_f32) per SIMD
  for (int op = 0; op < 2; ++op) {
    const int r = op == 0 ? run<0>("", 2, 4, nblk, d_out, d_sink, wc, &ms) : run<1>("", 2, 4, nblk, d_out, d_sink, wc, &ms);
    if (r) return 1;
    printf("co-execution with %-10s: MFMA wave %.1f cycles per MFMA, vector wave %.2f cycles per instruction\n",
           names[op], wc[0] / mfma_per_wave, wc[1] / (8.0 * kIters));
  }
  CHECK(hipFree(d_out));
  CHECK(hipFree(d_sink));
  return 0;
}
