// Device helpers shared by the bf16 matrix-core kernels (gfx950): vector
// types, raw buffer descriptors, direct buffer->LDS loads with explicit waits,
// the K-tile swizzle, half-wave and wave reductions, the workgroup barrier and
// the ordered list of kept tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace cpring {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;        // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

// Fourth dword of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle, no format conversion).
constexpr int kBufWord3 = 0x00020000;

// Raw buffer descriptor (scalar registers): base, no stride, `nbytes` bytes
// addressable; offsets at or past nbytes read as zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = (int)(uint32_t)p;
  r.y = (int)((uint32_t)(p >> 32) & 0xffffu);
  r.z = (int)nbytes;
  r.w = kBufWord3;
  return r;
}

// LDS address (byte offset) of a __shared__ object
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) T*)p);
}

// Direct buffer -> LDS loads: lane i of the wave writes its 16 (4) bytes at
// LDS address m0 + 16*i (4*i). Issued as inline assembly on purpose: the
// compiler then neither counts them nor inserts waits for them before LDS
// reads of other tile buffers (it cannot tell the buffers apart), and the
// kernels wait for them explicitly with vm_wait<N>().
__device__ __forceinline__ void dma_b128(const i32x4& rsrc, uint32_t voff, uint32_t m0) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma_b32(const i32x4& rsrc, uint32_t voff, uint32_t m0) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0) : "memory");
}
// wait until at most N of this wave's vector-memory loads are outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// scheduling-group masks (AMDGPU sched_group_barrier)
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Row-major bf16 tile: physical 16-byte chunk = logical chunk XOR a function
// of the row, so the 16 consecutive rows one A-operand read touches per 16
// lanes hit 16 different bank groups. (An involution: also maps physical to
// logical.)
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
// waits for its own before a later barrier that precedes their first use).
// The memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
using ic = std::integral_constant<int, N>;

// Empty asm statement reading every fragment: the compiler must have the
// loaded values here, so it waits for their global loads at this point. Placed
// after loading a kernel's resident operands, before its tile loop; otherwise
// the wait lands at the first use inside the loop, where it would also wait for
// the direct-to-LDS loads of the next tile (the hardware counts both).
template <int N>
__device__ __forceinline__ void ready(const bf16x8 (&x)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(x[i]));
#endif
}

// Ordered list of kept tiles. flags8[t] (t < nseg) holds bit 0 = kept, bit 1 =
// needs the element mask; the list gets entry t | 0x8000 (masked) or t for
// every kept tile in increasing t, then kPad end markers equal to nseg.
// Thread tid covers tiles [8*tid, 8*tid + 8): count, workgroup scan, scatter.
// Must be called by every thread of the workgroup; returns the number kept
// (uniform). wcount holds NW ints of scratch.
template <int NW, int kPad>
__device__ __forceinline__ int build_tile_list(const uint8_t* flags8, int nseg, uint16_t* klist, int* wcount) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = 8 * tid;
  uint64_t fw = 0;
  if (t0 < nseg) {
    fw = *reinterpret_cast<const uint64_t*>(&flags8[t0]);
    if (nseg - t0 < 8) fw &= (1ull << (8 * (nseg - t0))) - 1ull;
  }
  const int cnt = __builtin_popcountll(fw & 0x0101010101010101ull);
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    incl += lane >= o ? y : 0;
  }
  if (lane == 63) wcount[wave] = incl;
  bar();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = wcount[w];
    before += w < wave ? c : 0;
    total += c;
  }
  int p = before + incl - cnt;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int f = (int)(fw >> (8 * e)) & 3;
    if (f & 1) klist[p++] = (uint16_t)((t0 + e) | ((f & 2) ? 0x8000 : 0));
  }
  if (tid < kPad) klist[total + tid] = (uint16_t)nseg;
  return __builtin_amdgcn_readfirstlane(total);
}

}  // namespace mfma
}  // namespace cpring
