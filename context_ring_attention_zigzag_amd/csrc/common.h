// Internal declarations shared by the libcpring translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cpring.h"

namespace cpring {

// Kernel launchers; each returns hipSuccess or the launch error.
hipError_t launch_partition(int64_t seq_len, int64_t s_pad, int32_t cp, int32_t layout,
                            int32_t* token_idx, int32_t* pos_ids, hipStream_t st);
hipError_t launch_gather(int esize, int32_t B, int32_t H, int64_t seq_len, int32_t D, const cpr_view& src,
                         const int32_t* token_idx, int64_t n_out, void* dst, hipStream_t st);
hipError_t launch_state_init(int64_t rows, int32_t D, float* o, float* m, float* l, hipStream_t st);
hipError_t launch_merge(int64_t rows, int32_t D, float* o, float* m, float* l, const float* o2,
                        const float* m2, const float* l2, hipStream_t st);
hipError_t launch_finalize(int out_bf16, int64_t rows, int32_t D, const float* o, const float* m,
                           const float* l, void* out, float* lse, hipStream_t st);
// Merge of nsplit partial states (slice j at o + j * rows * D, m + j * rows,
// l + j * rows) followed by finalize into (out, lse).
hipError_t launch_merge_finalize(int out_bf16, int32_t nsplit, int64_t rows, int32_t D, const float* o,
                                 const float* m, const float* l, void* out, float* lse, hipStream_t st);

// Attention pass over `nblocks` KV blocks of Lk rows. Block t (t = 0..nblocks-1)
// is block (rank - t) mod cp of the K/V/kv_pos buffers. State handling:
// load_state reads (o_acc, m, l) first (else starts from O=0, m=-inf, l=0);
// finalize writes (o_out, lse) at the end (else writes (o_acc, m, l) back).
struct AttnArgs {
  const void* q; int64_t q_sb, q_sh, q_sl;
  const int32_t* q_pos;
  const void* k; int64_t k_sb, k_sh, k_sl;
  const void* v; int64_t v_sb, v_sh, v_sl;
  const int32_t* kv_pos;
  int32_t B, H, D, Lq, Lk;
  int32_t H_kv;                         // K/V heads; query head h reads K/V head h / (H / H_kv)
  const int32_t* kw_lo; const int32_t* kw_hi;   // per-query key-position window, or NULL
  int32_t nblocks, rank, cp;
  int32_t causal;
  float scale;
  float* o_acc; float* m; float* l;
  void* o_out; float* lse;
  int32_t load_state, finalize;
  // split over the keys (bf16 path only): kv_split > 1 launches kv_split
  // workgroups per query tile, slice j covering key tiles
  // [j * n / kv_split, (j + 1) * n / kv_split) of every block (n = key tiles per
  // block); each writes its partial state (o_acc, m, l) advanced by j slices of
  // state_rows rows, and finalize / load_state are ignored
  int32_t kv_split;
  int64_t state_rows;
};

// Key slices per query tile (AttnArgs::kv_split) for a bf16 pass over Lq
// queries of B*H heads and blocks of Lk keys: > 1 when the unsplit grid would
// leave most of the chip idle, else 1.
int32_t attn_bf16_kv_split(int32_t B, int32_t H, int32_t Lq, int32_t Lk);

// Backward pass. Preprocessing, per query row: lse2 = LSE in log2 units (+inf
// for a row that attends no key) and dvec = rowsum(dO * O); per query: qwin =
// {lo, hi}, the key positions it may attend (empty when lo > hi).
struct BwdPrepArgs {
  const void* o; int64_t o_sb, o_sh, o_sl;
  const void* dout; int64_t do_sb, do_sh, do_sl;
  const float* lse;                     // [B, H, Lq], natural log
  const int32_t* q_pos; const int32_t* kw_lo; const int32_t* kw_hi;
  int32_t causal;
  int32_t B, H, D, Lq;
  float* lse2;                          // [B, H, Lq]
  float* dvec;                          // [B, H, Lq]
  int2* qwin;                           // [Lq]
};

// Gradient kernels. The dQ kernel folds `nblocks` KV blocks of Lk rows in
// ring order (block t is block (rank - t) mod cp of k/v/kv_pos); the dK/dV
// kernel covers all nblocks * Lk rows of k/v at once. Outputs are fp32,
// contiguous: dq [B, H, Lq, D], dk and dv [B, H_kv, nblocks * Lk, D]; with
// accumulate set they are added to, else written.
struct BwdArgs {
  const void* q; int64_t q_sb, q_sh, q_sl;
  const void* dout; int64_t do_sb, do_sh, do_sl;
  const void* k; int64_t k_sb, k_sh, k_sl;
  const void* v; int64_t v_sb, v_sh, v_sl;
  const int32_t* kv_pos;
  const float* lse2;
  const float* dvec;
  const int2* qwin;
  int32_t B, H, H_kv, D, Lq, Lk;
  int32_t nblocks, rank, cp;
  float scale;
  float* dq; float* dk; float* dv;
  int32_t accumulate;
  // split for grids too small for the GPU (bf16 path): q_split > 1 gives each
  // dQ query tile q_split workgroups, slice j covering key tiles
  // [j * n / q_split, (j + 1) * n / q_split) of every block (n = key tiles per
  // block) and writing its partial dQ to dq_part + j * B*H*Lq*D; kv_split > 1
  // likewise splits the query tiles of each dK/dV key tile, partials at
  // dk_part / dv_part + j * B*H_kv*nblocks*Lk*D. launch_bwd_bf16 then sums the
  // partials in slice order into dq / dk / dv (added to them when accumulate).
  int32_t q_split, kv_split;
  float* dq_part; float* dk_part; float* dv_part;
};

// Slices of the backward split (BwdArgs::q_split, kv_split) for a bf16 pass:
// > 1 when the unsplit grid would leave most of the chip idle, else 1.
int32_t bwd_bf16_q_split(int32_t B, int32_t H, int32_t Lq);
int32_t bwd_bf16_kv_split(int32_t B, int32_t H_kv, int64_t Lk_total);

hipError_t launch_bwd_prep(int32_t dtype_bf16, const BwdPrepArgs& a, hipStream_t st);
hipError_t launch_bwd_bf16(const BwdArgs& a, int32_t do_dq, int32_t do_dkv, hipStream_t st);
hipError_t launch_bwd_f32(const BwdArgs& a, int32_t do_dq, int32_t do_dkv, hipStream_t st);

// Rotary embedding: out (contiguous [B, H, L, D]) = x rotated by pos [L].
struct RopeArgs {
  const void* x; int64_t x_sb, x_sh, x_sl;
  const int32_t* pos;
  int32_t B, H, L, D;
  float base;
  int32_t style;
  void* out;
};
hipError_t launch_rope(int32_t dtype_bf16, const RopeArgs& a, hipStream_t st);

// Tile census of the bf16 forward pass over nblocks blocks of Lk keys
// (kv_pos holds nblocks * Lk positions): kept[qt] and masked[qt] for every
// 256-query tile qt.
struct CensusArgs {
  const int32_t* q_pos; const int32_t* kv_pos;
  const int32_t* kw_lo; const int32_t* kw_hi;
  int32_t Lq, Lk, nblocks, causal;
  int32_t* kept; int32_t* masked;
};
hipError_t launch_tile_census(const CensusArgs& a, hipStream_t st);

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st);

}  // namespace cpring
