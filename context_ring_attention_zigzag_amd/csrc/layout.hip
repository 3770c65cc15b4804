// Zigzag / contiguous layout builder and the row gather that applies it.
//
// Zigzag: "Context Parallelism v.s. Sequence Parallelism (Megatron-LM)",
// section "Implementation quirk: symmetric chunk assignment" - 2*cp equal
// chunks, rank r holds chunk r then chunk 2cp-1-r, positions stay global,
// the sequence is padded to a multiple of 2*cp.
// Contiguous: "Sequence Parallelism and Ring Attention", "Deep dive" - rank r
// holds one contiguous run of tokens.
// Striped: the same page, "The future of sequence parallelism and ring
// attention", names striped assignment beside zigzag as the way to even out
// causal work; the plain reading, taken here, deals token t to rank t mod cp,
// so rank r holds tokens r, r+cp, r+2cp, ... (the sequence padded to a
// multiple of cp).
#include "common.h"

namespace cpring {

// One thread per rank-major layout entry. All values fit int32 because
// S_pad <= 2^30 is checked by the caller.
__global__ void __launch_bounds__(256) partition_kernel(int32_t* __restrict__ token_idx,
                                                        int32_t* __restrict__ pos_ids, int32_t seq_len,
                                                        int32_t s_pad, int32_t cp, int32_t layout) {
  const int32_t k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= s_pad) return;
  const int32_t lr = s_pad / cp;         // tokens per rank
  const int32_t r = k / lr;              // owning rank
  const int32_t i = k - r * lr;          // local index
  int32_t tok;
  if (layout == CPR_ZIGZAG) {
    const int32_t c = lr >> 1;           // chunk length
    const bool front = i < c;
    const int32_t chunk = front ? r : 2 * cp - 1 - r;
    tok = chunk * c + (front ? i : i - c);
  } else if (layout == CPR_STRIPED) {
    tok = i * cp + r;
  } else {
    tok = k;
  }
  if (token_idx) token_idx[k] = tok;
  if (pos_ids) pos_ids[k] = tok < seq_len ? tok : -1;
}

hipError_t launch_partition(int64_t seq_len, int64_t s_pad, int32_t cp, int32_t layout,
                            int32_t* token_idx, int32_t* pos_ids, hipStream_t st) {
  const int threads = 256;
  const int64_t blocks = (s_pad + threads - 1) / threads;
  hipLaunchKernelGGL(partition_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, token_idx, pos_ids,
                     (int32_t)seq_len, (int32_t)s_pad, cp, layout);
  return hipGetLastError();
}

// Row gather, 16 bytes per thread. `vec_per_row` 16-byte vectors per row.
__global__ void __launch_bounds__(256) gather_kernel(const char* __restrict__ src, int64_t sb, int64_t sh,
                                                     int64_t sl, const int32_t* __restrict__ token_idx,
                                                     int64_t seq_len, int64_t n_out, int32_t H,
                                                     int32_t vec_per_row, int64_t total_vec,
                                                     char* __restrict__ dst) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= total_vec) return;
  const int64_t vr = g % vec_per_row;
  const int64_t row = g / vec_per_row;          // (b*H + h)*n_out + i
  const int64_t i = row % n_out;
  const int64_t bh = row / n_out;
  const int64_t b = bh / H, h = bh - b * H;
  const int32_t t = token_idx[i];
  uint4 val = make_uint4(0u, 0u, 0u, 0u);
  if (t >= 0 && t < seq_len) {
    // strides are byte strides here
    val = *reinterpret_cast<const uint4*>(src + b * sb + h * sh + (int64_t)t * sl + vr * 16);
  }
  reinterpret_cast<uint4*>(dst)[g] = val;
}

hipError_t launch_gather(int esize, int32_t B, int32_t H, int64_t seq_len, int32_t D, const cpr_view& src,
                         const int32_t* token_idx, int64_t n_out, void* dst, hipStream_t st) {
  const int32_t vec_per_row = D * esize / 16;
  const int64_t total = (int64_t)B * H * n_out * vec_per_row;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(threads), 0, st,
                     static_cast<const char*>(src.data), src.stride_b * esize, src.stride_h * esize,
                     src.stride_l * esize, token_idx, seq_len, n_out, H, vec_per_row, total,
                     static_cast<char*>(dst));
  return hipGetLastError();
}

}  // namespace cpring
