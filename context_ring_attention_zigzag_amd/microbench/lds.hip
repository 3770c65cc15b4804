// LDS costs on gfx950 that the kernel designs rest on: read and write
// throughput (16-byte row reads, ds_read_b64_tr_b16 transposed reads in two
// layouts, 16-byte writes) with 1-8 waves per workgroup; the issue cost of
// direct-to-LDS loads (buffer_load_dwordx4 ... lds); and whether an LDS read
// issued after such a load waits for it. Every LDS address stays inside the
// workgroup's array and every global offset inside its source buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                 \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));             \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = (int)(uint32_t)p;
  r.y = (int)((uint32_t)(p >> 32) & 0xffffu);
  r.z = (int)nbytes;
  r.w = 0x00020000;
  return r;
}

// ---- throughput: 16 operations per iteration, 8 KB per wave
constexpr int kIters = 1024;
// dynamic LDS added to the 64 KB arrays so that a compute unit holds one workgroup
constexpr size_t kReserve = 40 * 1024;

template <int MODE>
__global__ void __launch_bounds__(512) lds_rate(uint64_t* out, int* sink, int nwaves) {
  __shared__ __attribute__((aligned(16))) short lds[32768];   // 64 KB
  extern __shared__ char reserve[];
  if (threadIdx.x == 0) reserve[0] = 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 32768; i += blockDim.x) lds[i] = (short)i;
  __syncthreads();
  int acc = 0;
  uint64_t t0 = 0, t1 = 0;
  if (wave < nwaves) {
    const uint32_t base = (uint32_t)wave * 8192u;
    uint32_t off;
    if constexpr (MODE == 0 || MODE == 3) {   // 16 lanes per 256-byte sweep, 4 rows of 256 B
      off = base + (uint32_t)(lane & 15) * 16u + (uint32_t)(lane >> 4) * 256u;
    } else if constexpr (MODE == 1) {         // transposed: rows 256 B apart, 64 B of each (4 rows per 32 lanes)
      const int r = 4 * (lane >> 5) + ((lane & 15) >> 2);
      off = base + (uint32_t)r * 256u + (uint32_t)(((r & 3) * 4 + 2 * ((lane >> 4) & 1)) * 16) + (uint32_t)(lane & 3) * 8u;
    } else {                                  // transposed: 4 rows x 64 B contiguous per 32 lanes
      off = base + (uint32_t)(lane >> 5) * 256u + (uint32_t)((lane & 15) >> 2) * 64u + (uint32_t)((lane >> 4) & 1) * 32u +
            (uint32_t)(lane & 3) * 8u;
    }
    t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < kIters; ++it) {
      if constexpr (MODE == 0) {
        i32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          asm volatile("" ::: "memory");
          v[u] = *reinterpret_cast<const i32x4*>((const char*)lds + off + (uint32_t)(u & 7) * 1024u - ((u & 7) == 7 ? 1024u : 0u));
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc = acc * 31 + v[u].x + v[u].w;
      } else if constexpr (MODE == 3) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const i32x4 w = {acc + u, it, lane, wave};
          *reinterpret_cast<i32x4*>((char*)lds + off + (uint32_t)(u & 7) * 1024u - ((u & 7) == 7 ? 1024u : 0u)) = w;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        acc += lds[tid];
      } else {
        s16x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          asm volatile("" ::: "memory");
          v[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((const char*)lds + off + (uint32_t)(u & 3) * 2048u));
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc = acc * 31 + (int)v[u][0] + (int)v[u][3];
      }
    }
    t1 = __builtin_amdgcn_s_memtime();
  }
  __syncthreads();
  if (lane == 0 && wave < nwaves) out[blockIdx.x * 8 + wave] = t1 - t0;
  sink[blockIdx.x * 512 + tid] = acc;
}

// ---- the same reads with all 16 in flight before any is used: one asm statement consumes them, so the
// compiler waits once per group instead of in step with the reads
template <int MODE>
__global__ void __launch_bounds__(512) lds_rate16(uint64_t* out, int* sink, int nwaves) {
  __shared__ __attribute__((aligned(16))) short lds[32768];   // 64 KB
  extern __shared__ char reserve[];
  if (threadIdx.x == 0) reserve[0] = 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 32768; i += blockDim.x) lds[i] = (short)i;
  __syncthreads();
  int acc = 0;
  uint64_t t0 = 0, t1 = 0;
  if (wave < nwaves) {
    const uint32_t base = (uint32_t)wave * 8192u;
    uint32_t off;
    if constexpr (MODE == 0) {
      off = base + (uint32_t)(lane & 15) * 16u + (uint32_t)(lane >> 4) * 256u;
    } else {
      const int r = 4 * (lane >> 5) + ((lane & 15) >> 2);
      off = base + (uint32_t)r * 256u + (uint32_t)(((r & 3) * 4 + 2 * ((lane >> 4) & 1)) * 16) + (uint32_t)(lane & 3) * 8u;
    }
    t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < kIters; ++it) {
      if constexpr (MODE == 0) {
        i32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          asm volatile("" ::: "memory");
          v[u] = *reinterpret_cast<const i32x4*>((const char*)lds + off + (uint32_t)(u & 7) * 1024u - ((u & 7) == 7 ? 1024u : 0u));
        }
        asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
                     "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
        acc += v[0].x + it;
      } else {
        s16x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          asm volatile("" ::: "memory");
          v[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((const char*)lds + off + (uint32_t)(u & 3) * 2048u));
        }
        asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
                     "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
        acc += (int)v[0][0] + it;
      }
    }
    t1 = __builtin_amdgcn_s_memtime();
  }
  __syncthreads();
  if (lane == 0 && wave < nwaves) out[blockIdx.x * 8 + wave] = t1 - t0;
  sink[blockIdx.x * 512 + tid] = acc;
}

// ---- direct-to-LDS load issue cost: NL loads per wave, timed from the first issue to the last
template <int NL>
__global__ void __launch_bounds__(512) dma_issue(const char* src, uint64_t* out, int* sink, int nwaves) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  extern __shared__ char reserve[];
  if (threadIdx.x == 0) reserve[0] = 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const i32x4 rs = make_rsrc(src + (size_t)blockIdx.x * 65536, 65536u);
  uint64_t t0 = 0, t1 = 0;
  __syncthreads();
  if (wave < nwaves) {
    const uint32_t lbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)wave * 8192u));
    t0 = __builtin_amdgcn_s_memtime();
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const uint32_t m0 = lbase + (uint32_t)n * 1024u;
      const uint32_t voff = (uint32_t)(wave * 8192 + n * 1024 + lane * 16);
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(m0) : "memory");
    }
    t1 = __builtin_amdgcn_s_memtime();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (lane == 0 && wave < nwaves) out[blockIdx.x * 8 + wave] = t1 - t0;
  sink[blockIdx.x * 512 + tid] = lds[tid * 16];
}

// ---- an LDS read after a direct-to-LDS load into another region: cycles to the read's data
template <int MODE>
__global__ void __launch_bounds__(64) read_after_dma(const char* src, uint64_t* out, int* sink) {
  __shared__ __attribute__((aligned(16))) char lds[32768];
  const int lane = threadIdx.x;
  for (int i = lane; i < 32768 / 16; i += 64) reinterpret_cast<i32x4*>(lds)[i] = i32x4{i, i, i, i};
  __syncthreads();
  const i32x4 rs = make_rsrc(src + (size_t)blockIdx.x * 65536, 65536u);
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"((uint32_t)lane * 16u), "s"(rs), "{m0}"(16384u) : "memory");
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if constexpr (MODE == 1)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"((uint32_t)lane * 16u + 32768u), "s"(rs), "{m0}"(16384u) : "memory");
  const i32x4 v = *reinterpret_cast<const i32x4*>(lds + lane * 16);   // bytes 0 .. 1 KB, not the load's target
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const int x = v.x;
  asm volatile("" ::"v"(x));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0) out[blockIdx.x] = t1 - t0;
  sink[blockIdx.x * 64 + lane] = x;
}

static double mean_nonzero(const std::vector<uint64_t>& h, int nblk, int nw) {
  double s = 0;
  int n = 0;
  for (int b = 0; b < nblk; ++b)
    for (int w = 0; w < nw; ++w) { s += (double)h[b * 8 + w]; ++n; }
  return n ? s / n : 0;
}

int main() {
  const int nblk = 256;
  uint64_t* out;
  int* sink;
  char* src;
  CHECK(hipMalloc(&out, (size_t)nblk * 8 * sizeof(uint64_t)));
  CHECK(hipMalloc(&sink, (size_t)nblk * 512 * sizeof(int)));
  CHECK(hipMalloc(&src, (size_t)nblk * 65536));
  CHECK(hipMemset(src, 1, (size_t)nblk * 65536));
  std::vector<uint64_t> h((size_t)nblk * 8);
  const char* names[4] = {"ds_read_b128 rows", "ds_read_b64_tr_b16, rows 256 B apart", "ds_read_b64_tr_b16, 256 B contiguous",
                          "ds_write_b128 rows"};
  const double bytes_per_op[4] = {1024, 512, 512, 1024};
  for (int mode = 0; mode < 4; ++mode)
    for (int nw : {1, 2, 4, 8}) {
      for (int rep = 0; rep < 2; ++rep) {
        if (mode == 0) hipLaunchKernelGGL(lds_rate<0>, dim3(nblk), dim3(512), kReserve, 0, out, sink, nw);
        if (mode == 1) hipLaunchKernelGGL(lds_rate<1>, dim3(nblk), dim3(512), kReserve, 0, out, sink, nw);
        if (mode == 2) hipLaunchKernelGGL(lds_rate<2>, dim3(nblk), dim3(512), kReserve, 0, out, sink, nw);
        if (mode == 3) hipLaunchKernelGGL(lds_rate<3>, dim3(nblk), dim3(512), kReserve, 0, out, sink, nw);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
      }
      CHECK(hipMemcpy(h.data(), out, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
      const double cyc = mean_nonzero(h, nblk, nw);
      const double bytes = (double)kIters * 16 * bytes_per_op[mode];
      printf("%-38s waves %d: %5.1f cycles per instruction per wave, %6.1f B/cycle per wave, %6.1f per CU\n",
             names[mode], nw, cyc / (kIters * 16.0), bytes / cyc, nw * bytes / cyc);
    }
  const char* names16[2] = {"ds_read_b128 rows, 16 in flight", "ds_read_b64_tr_b16, 16 in flight"};
  for (int mode = 0; mode < 2; ++mode)
    for (int nw : {1, 4, 8}) {
      for (int rep = 0; rep < 2; ++rep) {
        if (mode == 0) hipLaunchKernelGGL(lds_rate16<0>, dim3(nblk), dim3(512), kReserve, 0, out, sink, nw);
        else hipLaunchKernelGGL(lds_rate16<1>, dim3(nblk), dim3(512), kReserve, 0, out, sink, nw);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
      }
      CHECK(hipMemcpy(h.data(), out, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
      const double cyc = mean_nonzero(h, nblk, nw);
      const double bytes = (double)kIters * 16 * (mode == 0 ? 1024 : 512);
      printf("%-38s waves %d: %5.1f cycles per instruction per wave, %6.1f B/cycle per wave, %6.1f per CU\n",
             names16[mode], nw, cyc / (kIters * 16.0), bytes / cyc, nw * bytes / cyc);
    }
  for (int nl : {1, 2, 4, 8})
    for (int nw : {1, 4, 8}) {
      for (int rep = 0; rep < 3; ++rep) {
        if (nl == 1) hipLaunchKernelGGL(dma_issue<1>, dim3(nblk), dim3(512), kReserve, 0, src, out, sink, nw);
        if (nl == 2) hipLaunchKernelGGL(dma_issue<2>, dim3(nblk), dim3(512), kReserve, 0, src, out, sink, nw);
        if (nl == 4) hipLaunchKernelGGL(dma_issue<4>, dim3(nblk), dim3(512), kReserve, 0, src, out, sink, nw);
        if (nl == 8) hipLaunchKernelGGL(dma_issue<8>, dim3(nblk), dim3(512), kReserve, 0, src, out, sink, nw);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
      }
      CHECK(hipMemcpy(h.data(), out, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
      printf("buffer_load_dwordx4 ... lds, %d per wave, %d waves: issue %.0f cycles per load\n", nl, nw,
             mean_nonzero(h, nblk, nw) / nl);
    }
  for (int mode = 0; mode < 2; ++mode) {
    for (int rep = 0; rep < 3; ++rep) {
      if (mode == 0) hipLaunchKernelGGL(read_after_dma<0>, dim3(nblk), dim3(64), 0, 0, src, out, sink);
      else hipLaunchKernelGGL(read_after_dma<1>, dim3(nblk), dim3(64), 0, 0, src, out, sink);
      CHECK(hipGetLastError());
      CHECK(hipDeviceSynchronize());
    }
    std::vector<uint64_t> h1(nblk);
    CHECK(hipMemcpy(h1.data(), out, nblk * sizeof(uint64_t), hipMemcpyDeviceToHost));
    double s = 0;
    for (auto x : h1) s += (double)x;
    printf("ds_read_b128 %s: %.0f cycles to its data\n", mode ? "after a direct-to-LDS load" : "alone", s / nblk);
  }
  CHECK(hipFree(out));
  CHECK(hipFree(sink));
  CHECK(hipFree(src));
  return 0;
}
