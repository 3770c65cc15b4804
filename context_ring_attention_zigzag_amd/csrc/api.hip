// C ABI of libcpring: argument validation and dispatch.
//
// Every entry point validates all arguments before it touches the HIP
// runtime, so a bad call returns an error without launching anything. The
// library holds no state besides the thread-local text of the last error and,
// for the allocation-free run, each device's address of its scratch array.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <string>

#include "common.h"

using namespace cpring;

namespace {

thread_local std::string g_last_error;

cpr_status fail(cpr_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

cpr_status ok() {
  g_last_error.clear();
  return CPR_OK;
}

cpr_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CPR_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// With CPRING_SYNC_CHECK=1 in the environment, every call that launches work
// waits for its stream before returning, so that a kernel failure (an illegal
// address, say) is reported as CPR_EHIP by the call that launched it instead
// of by a later call. A debugging aid: it makes every call synchronous.
bool sync_check() {
  const char* e = getenv("CPRING_SYNC_CHECK");
  return e && e[0] == '1' && e[1] == 0;
}

// Status of a call whose last launch returned `e` on stream `st`.
cpr_status launched(hipError_t e, hipStream_t st, const char* what) {
  if (e == hipSuccess && sync_check()) {
    e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
  }
  return hip_status(e, what);
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int esize_of(int32_t dtype) { return dtype == CPR_BF16 ? 2 : 4; }

// A [B, H, L, D] view with D contiguous. Rows must not overlap (stride_l >= D):
// the kernels address a block of rows as one byte range of rows * stride_l
// elements, which holds every row only when no two of them share memory.
cpr_status check_view(const char* name, const cpr_view* v, int32_t dtype, int32_t D) {
  if (!v) return fail(CPR_EINVAL, "%s: view pointer is NULL", name);
  if (!v->data) return fail(CPR_EINVAL, "%s: data pointer is NULL", name);
  if (v->stride_b < 0 || v->stride_h < 0 || v->stride_l < 0)
    return fail(CPR_EINVAL, "%s: negative stride", name);
  if (v->stride_l < D)
    return fail(CPR_EUNSUPPORTED, "%s: stride_l = %lld is below D = %d (overlapping rows)", name,
                (long long)v->stride_l, D);
  if (v->stride_l > ((int64_t)1 << 24)) return fail(CPR_EUNSUPPORTED, "%s: stride_l must be <= 2^24", name);
  const int64_t align_elems = dtype == CPR_BF16 ? 8 : 1;   // 16-byte rows for bf16
  if (dtype == CPR_BF16) {
    if (!aligned(v->data, 16)) return fail(CPR_EINVAL, "%s: bf16 data must be 16-byte aligned", name);
    if (v->stride_b % align_elems || v->stride_h % align_elems || v->stride_l % align_elems)
      return fail(CPR_EINVAL, "%s: bf16 strides must be multiples of 8 elements", name);
  } else if (!aligned(v->data, 4)) {
    return fail(CPR_EINVAL, "%s: f32 data must be 4-byte aligned", name);
  }
  return CPR_OK;
}

cpr_status check_dims(int32_t dtype, int32_t B, int32_t H, int32_t D) {
  if (dtype != CPR_F32 && dtype != CPR_BF16) return fail(CPR_EINVAL, "unknown dtype %d", dtype);
  if (B < 1 || H < 1) return fail(CPR_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (B > 65535 || H > 65535) return fail(CPR_EUNSUPPORTED, "B and H must be <= 65535");
  if (D != 64 && D != 128) return fail(CPR_EUNSUPPORTED, "head dim D must be 64 or 128 (got %d)", D);
  return CPR_OK;
}

cpr_status check_len(const char* name, int64_t L) {
  if (L < 1) return fail(CPR_EINVAL, "%s must be >= 1 (got %lld)", name, (long long)L);
  if (L > CPR_MAX_SEQ) return fail(CPR_EUNSUPPORTED, "%s must be <= 2^30", name);
  return CPR_OK;
}

cpr_status check_state(int64_t rows, const float* o, const float* m, const float* l) {
  if (!o || !m || !l) return fail(CPR_EINVAL, "state pointers o_acc, m, l must be non-NULL");
  if (!aligned(o, 16)) return fail(CPR_EINVAL, "o_acc must be 16-byte aligned");
  if (!aligned(m, 4) || !aligned(l, 4)) return fail(CPR_EINVAL, "m and l must be 4-byte aligned");
  (void)rows;
  return CPR_OK;
}

// Grid size of the attention kernels must stay below 2^31 workgroups.
cpr_status check_grid(int32_t B, int32_t H, int32_t Lq) {
  const int64_t tiles = (int64_t)B * H * ((Lq + 63) / 64);
  if (tiles >= ((int64_t)1 << 31)) return fail(CPR_EUNSUPPORTED, "B*H*Lq too large");
  return CPR_OK;
}

#define TRY(x)                        \
  do {                                \
    cpr_status s__ = (x);             \
    if (s__ != CPR_OK) return s__;    \
  } while (0)

}  // namespace

extern "C" {

int64_t cp_padded_len(int64_t seq_len, int32_t cp_size, int32_t layout) {
  if (seq_len < 1 || seq_len > CPR_MAX_SEQ || cp_size < 1) return -1;
  if (layout != CPR_ZIGZAG && layout != CPR_CONTIGUOUS && layout != CPR_STRIPED) return -1;
  const int64_t unit = layout == CPR_ZIGZAG ? 2 * (int64_t)cp_size : (int64_t)cp_size;
  const int64_t s_pad = (seq_len + unit - 1) / unit * unit;
  return s_pad > CPR_MAX_SEQ ? -1 : s_pad;
}

cpr_status cp_zigzag_partition(int64_t seq_len, int32_t cp_size, int32_t layout, int32_t* token_idx,
                               int32_t* pos_ids, void* stream) {
  if (cp_size < 1) return fail(CPR_EINVAL, "cp_size must be >= 1 (got %d)", cp_size);
  if (layout != CPR_ZIGZAG && layout != CPR_CONTIGUOUS && layout != CPR_STRIPED)
    return fail(CPR_EINVAL, "unknown layout %d", layout);
  TRY(check_len("seq_len", seq_len));
  const int64_t s_pad = cp_padded_len(seq_len, cp_size, layout);
  if (s_pad < 0) return fail(CPR_EUNSUPPORTED, "padded length exceeds 2^30");
  if (!token_idx && !pos_ids) return fail(CPR_EINVAL, "token_idx and pos_ids are both NULL");
  if ((token_idx && !aligned(token_idx, 4)) || (pos_ids && !aligned(pos_ids, 4)))
    return fail(CPR_EINVAL, "output arrays must be 4-byte aligned");
  return launched(launch_partition(seq_len, s_pad, cp_size, layout, token_idx, pos_ids,
                                     static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_zigzag_partition");
}

cpr_status cp_shard_gather(int32_t dtype, int32_t B, int32_t H, int64_t seq_len, int32_t D, const cpr_view* src,
                           const int32_t* token_idx, int64_t n_out, void* dst, void* stream) {
  TRY(check_dims(dtype, B, H, D));
  TRY(check_len("seq_len", seq_len));
  TRY(check_len("n_out", n_out));
  TRY(check_view("src", src, dtype, D));
  if (dtype == CPR_F32) {
    if (!aligned(src->data, 16) || src->stride_b % 4 || src->stride_h % 4 || src->stride_l % 4)
      return fail(CPR_EINVAL, "src: f32 gather needs 16-byte aligned rows");
  }
  if (!token_idx) return fail(CPR_EINVAL, "token_idx is NULL");
  if (!dst) return fail(CPR_EINVAL, "dst is NULL");
  if (!aligned(dst, 16)) return fail(CPR_EINVAL, "dst must be 16-byte aligned");
  return launched(launch_gather(esize_of(dtype), B, H, seq_len, D, *src, token_idx, n_out, dst,
                                  static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_shard_gather");
}

cpr_status cp_ring_attn_init(int32_t B, int32_t H, int32_t Lq, int32_t D, float* o_acc, float* m, float* l,
                             void* stream) {
  TRY(check_dims(CPR_F32, B, H, D));
  TRY(check_len("Lq", Lq));
  TRY(check_state(0, o_acc, m, l));
  const int64_t rows = (int64_t)B * H * Lq;
  return launched(launch_state_init(rows, D, o_acc, m, l, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_ring_attn_init");
}

// need_q_pos = 0 for calls that take no query positions (the backward step,
// whose windows come with the prepared workspace)
static cpr_status validate_attn(int32_t dtype, int32_t B, int32_t H, int32_t D, const cpr_view* q, int32_t Lq,
                                const int32_t* q_pos, const cpr_view* k, const cpr_view* v, int64_t Lk_total,
                                const int32_t* kv_pos, const cpr_attn_ext* ext, int need_q_pos = 1) {
  TRY(check_dims(dtype, B, H, D));
  if (ext) {
    if (ext->H_kv < 0 || (ext->H_kv > 0 && H % ext->H_kv != 0))
      return fail(CPR_EINVAL, "H_kv = %d must be 0 or divide H = %d", ext->H_kv, H);
    if ((ext->kw_lo && !aligned(ext->kw_lo, 4)) || (ext->kw_hi && !aligned(ext->kw_hi, 4)))
      return fail(CPR_EINVAL, "key-window arrays must be 4-byte aligned");
  }
  TRY(check_len("Lq", Lq));
  TRY(check_len("KV length", Lk_total));
  TRY(check_view("q", q, dtype, D));
  TRY(check_view("k", k, dtype, D));
  TRY(check_view("v", v, dtype, D));
  if ((need_q_pos && !q_pos) || !kv_pos) return fail(CPR_EINVAL, "position arrays must be non-NULL");
  TRY(check_grid(B, H, Lq));
  TRY(check_grid(B, ext && ext->H_kv > 0 ? ext->H_kv : H, (int32_t)Lk_total));   // Lk_total <= 2^30 here
  return CPR_OK;
}

static AttnArgs make_args(int32_t dtype, int32_t B, int32_t H, int32_t D, const cpr_view* q, int32_t Lq,
                          const int32_t* q_pos, const cpr_view* k, const cpr_view* v, int32_t Lk,
                          const int32_t* kv_pos, int32_t causal, float softmax_scale, const cpr_attn_ext* ext) {
  (void)dtype;
  AttnArgs a{};
  a.q = q->data; a.q_sb = q->stride_b; a.q_sh = q->stride_h; a.q_sl = q->stride_l;
  a.q_pos = q_pos;
  a.k = k->data; a.k_sb = k->stride_b; a.k_sh = k->stride_h; a.k_sl = k->stride_l;
  a.v = v->data; a.v_sb = v->stride_b; a.v_sh = v->stride_h; a.v_sl = v->stride_l;
  a.kv_pos = kv_pos;
  a.B = B; a.H = H; a.D = D; a.Lq = Lq; a.Lk = Lk;
  a.H_kv = (ext && ext->H_kv > 0) ? ext->H_kv : H;
  a.kw_lo = ext ? ext->kw_lo : nullptr;
  a.kw_hi = ext ? ext->kw_hi : nullptr;
  a.causal = causal ? 1 : 0;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  return a;
}

static hipError_t launch_attn(int32_t dtype, const AttnArgs& a, hipStream_t st) {
  return dtype == CPR_BF16 ? launch_attn_bf16(a, st) : launch_attn_f32(a, st);
}

cpr_status cp_ring_attn_step(int32_t dtype, int32_t B, int32_t H, int32_t D, const cpr_view* q, int32_t Lq,
                             const int32_t* q_pos, const cpr_view* k, const cpr_view* v, int32_t Lk,
                             const int32_t* kv_pos, int32_t causal, float softmax_scale, float* o_acc, float* m,
                             float* l, void* stream) {
  return cp_ring_attn_step_ex(dtype, B, H, D, q, Lq, q_pos, k, v, Lk, kv_pos, causal, softmax_scale, nullptr,
                              o_acc, m, l, stream);
}

cpr_status cp_ring_attn_step_ex(int32_t dtype, int32_t B, int32_t H, int32_t D, const cpr_view* q, int32_t Lq,
                                const int32_t* q_pos, const cpr_view* k, const cpr_view* v, int32_t Lk,
                                const int32_t* kv_pos, int32_t causal, float softmax_scale, const cpr_attn_ext* ext,
                                float* o_acc, float* m, float* l, void* stream) {
  TRY(validate_attn(dtype, B, H, D, q, Lq, q_pos, k, v, Lk, kv_pos, ext));
  const int32_t sf = ext ? ext->step_flags : 0;
  if (sf & ~(CPR_STEP_FIRST | CPR_STEP_LAST)) return fail(CPR_EINVAL, "unknown step_flags %d", sf);
  const bool first = (sf & CPR_STEP_FIRST) != 0, last = (sf & CPR_STEP_LAST) != 0;
  if (!(first && last)) TRY(check_state(0, o_acc, m, l));   // the state is read, written or both
  if (last) {
    if (!ext->o_out) return fail(CPR_EINVAL, "CPR_STEP_LAST needs o_out");
    if (!aligned(ext->o_out, 16)) return fail(CPR_EINVAL, "o_out must be 16-byte aligned");
    if (ext->lse_out && !aligned(ext->lse_out, 4)) return fail(CPR_EINVAL, "lse_out must be 4-byte aligned");
  }
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale))
    return fail(CPR_EINVAL, "softmax_scale must be finite");
  AttnArgs a = make_args(dtype, B, H, D, q, Lq, q_pos, k, v, Lk, kv_pos, causal, softmax_scale, ext);
  a.nblocks = 1; a.rank = 0; a.cp = 1;
  a.o_acc = o_acc; a.m = m; a.l = l;
  a.load_state = first ? 0 : 1;
  a.finalize = last ? 1 : 0;
  if (last) {
    a.o_out = ext->o_out;
    a.lse = ext->lse_out;
  }
  return launched(launch_attn(dtype, a, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_ring_attn_step");
}

cpr_status cp_ring_attn_merge(int32_t B, int32_t H, int32_t Lq, int32_t D, float* o_acc, float* m, float* l,
                              const float* o2, const float* m2, const float* l2, void* stream) {
  TRY(check_dims(CPR_F32, B, H, D));
  TRY(check_len("Lq", Lq));
  TRY(check_state(0, o_acc, m, l));
  if (!o2 || !m2 || !l2) return fail(CPR_EINVAL, "partial-state pointers must be non-NULL");
  if (!aligned(o2, 16) || !aligned(m2, 4) || !aligned(l2, 4)) return fail(CPR_EINVAL, "o2 must be 16-byte aligned");
  const int64_t rows = (int64_t)B * H * Lq;
  return launched(launch_merge(rows, D, o_acc, m, l, o2, m2, l2, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_ring_attn_merge");
}

cpr_status cp_ring_attn_finalize(int32_t out_dtype, int32_t B, int32_t H, int32_t Lq, int32_t D,
                                 const float* o_acc, const float* m, const float* l, void* o_out, float* lse_out,
                                 void* stream) {
  TRY(check_dims(out_dtype, B, H, D));
  TRY(check_len("Lq", Lq));
  TRY(check_state(0, o_acc, m, l));
  if (!o_out) return fail(CPR_EINVAL, "o_out is NULL");
  if (!aligned(o_out, 16)) return fail(CPR_EINVAL, "o_out must be 16-byte aligned");
  if (lse_out && !aligned(lse_out, 4)) return fail(CPR_EINVAL, "lse_out must be 4-byte aligned");
  const int64_t rows = (int64_t)B * H * Lq;
  return launched(launch_finalize(out_dtype == CPR_BF16, rows, D, o_acc, m, l, o_out, lse_out,
                                    static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_ring_attn_finalize");
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// float32 state of `n` partial passes: O [n][rows][D], m [n][rows], l [n][rows], each 256-byte aligned
static size_t state_bytes(size_t n, size_t rows, int32_t D) {
  return round256(n * rows * D * sizeof(float)) + 2 * round256(n * rows * sizeof(float));
}

size_t cp_ring_attn_workspace_size(int32_t B, int32_t H, int32_t Lq, int32_t D) {
  if (B < 1 || H < 1 || Lq < 1 || (D != 64 && D != 128)) return 0;
  const size_t rows = (size_t)B * H * Lq;
  // the stepwise state, or the partial states of a key-split fused run
  const size_t split = (size_t)attn_bf16_kv_split(B, H, Lq, Lq);
  return state_bytes(split > 1 ? split : 1, rows, D);
}

cpr_status cp_ring_attn_run(int32_t dtype, int32_t B, int32_t H, int32_t D, int32_t cp_size, int32_t rank,
                            const cpr_view* q_local, int32_t Lq, const int32_t* q_pos, const cpr_view* k_ring,
                            const cpr_view* v_ring, const int32_t* ring_pos, int32_t causal, float softmax_scale,
                            void* o_out, float* lse_out, void* workspace, size_t workspace_bytes, int32_t flags,
                            void* stream) {
  return cp_ring_attn_run_ex(dtype, B, H, D, cp_size, rank, q_local, Lq, q_pos, k_ring, v_ring, ring_pos, causal,
                             softmax_scale, nullptr, o_out, lse_out, workspace, workspace_bytes, flags, stream);
}

// Validation shared by the whole-ring entry points.
static cpr_status validate_run(int32_t dtype, int32_t B, int32_t H, int32_t D, int32_t cp_size, int32_t rank,
                               const cpr_view* q_local, int32_t Lq, const int32_t* q_pos, const cpr_view* k_ring,
                               const cpr_view* v_ring, const int32_t* ring_pos, float softmax_scale,
                               const cpr_attn_ext* ext, void* o_out, float* lse_out) {
  if (cp_size < 1) return fail(CPR_EINVAL, "cp_size must be >= 1 (got %d)", cp_size);
  if (rank < 0 || rank >= cp_size) return fail(CPR_EINVAL, "rank %d outside [0, %d)", rank, cp_size);
  TRY(validate_attn(dtype, B, H, D, q_local, Lq, q_pos, k_ring, v_ring, (int64_t)Lq * cp_size, ring_pos, ext));
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale))
    return fail(CPR_EINVAL, "softmax_scale must be finite");
  if (!o_out) return fail(CPR_EINVAL, "o_out is NULL");
  if (!aligned(o_out, 16)) return fail(CPR_EINVAL, "o_out must be 16-byte aligned");
  if (lse_out && !aligned(lse_out, 4)) return fail(CPR_EINVAL, "lse_out must be 4-byte aligned");
  return CPR_OK;
}

// Fused whole-ring launch. A grid too small for the chip is split over the
// keys when `ws` holds the ns partial states (ns = attn_bf16_kv_split);
// otherwise one launch does everything.
static cpr_status run_fused(int32_t dtype, AttnArgs a, int32_t cp_size, int32_t rank, void* o_out, float* lse_out,
                            void* ws, size_t ws_bytes, hipStream_t st) {
  const size_t rows = (size_t)a.B * a.H * a.Lq;
  a.nblocks = cp_size; a.rank = rank; a.cp = cp_size;
  const int32_t ns = dtype == CPR_BF16 ? attn_bf16_kv_split(a.B, a.H, a.Lq, a.Lq) : 1;
  if (ns > 1 && ws && ws_bytes >= state_bytes(ns, rows, a.D) && aligned(ws, 256)) {
    char* w = static_cast<char*>(ws);
    a.o_acc = reinterpret_cast<float*>(w);
    a.m = reinterpret_cast<float*>(w + round256(ns * rows * a.D * sizeof(float)));
    a.l = reinterpret_cast<float*>(w + round256(ns * rows * a.D * sizeof(float)) + round256(ns * rows * sizeof(float)));
    a.kv_split = ns; a.state_rows = (int64_t)rows;
    a.load_state = 0; a.finalize = 0;
    const hipError_t e = launch_attn(dtype, a, st);
    if (e != hipSuccess) return hip_status(e, "cp_ring_attn_run");
    return launched(launch_merge_finalize(1, ns, (int64_t)rows, a.D, a.o_acc, a.m, a.l, o_out, lse_out, st),
                    st, "cp_ring_attn_run(merge)");
  }
  a.o_out = o_out; a.lse = lse_out;
  a.load_state = 0; a.finalize = 1;
  return launched(launch_attn(dtype, a, st), st, "cp_ring_attn_run");
}

cpr_status cp_ring_attn_run_ex(int32_t dtype, int32_t B, int32_t H, int32_t D, int32_t cp_size, int32_t rank,
                               const cpr_view* q_local, int32_t Lq, const int32_t* q_pos, const cpr_view* k_ring,
                               const cpr_view* v_ring, const int32_t* ring_pos, int32_t causal, float softmax_scale,
                               const cpr_attn_ext* ext, void* o_out, float* lse_out, void* workspace,
                               size_t workspace_bytes, int32_t flags, void* stream) {
  TRY(validate_run(dtype, B, H, D, cp_size, rank, q_local, Lq, q_pos, k_ring, v_ring, ring_pos, softmax_scale, ext,
                   o_out, lse_out));
  if (flags != CPR_RUN_FUSED && flags != CPR_RUN_STEPWISE) return fail(CPR_EINVAL, "unknown flags %d", flags);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  AttnArgs a = make_args(dtype, B, H, D, q_local, Lq, q_pos, k_ring, v_ring, Lq, ring_pos, causal, softmax_scale,
                         ext);
  const size_t rows = (size_t)B * H * Lq;
  if (flags == CPR_RUN_FUSED) return run_fused(dtype, a, cp_size, rank, o_out, lse_out, workspace, workspace_bytes, st);
  const size_t need = state_bytes(1, rows, D);
  if (!workspace || workspace_bytes < need)
    return fail(CPR_EINVAL, "stepwise run needs a workspace of %zu bytes", need);
  if (!aligned(workspace, 256)) return fail(CPR_EINVAL, "workspace must be 256-byte aligned");
  char* w = static_cast<char*>(workspace);
  float* o_acc = reinterpret_cast<float*>(w);
  float* m = reinterpret_cast<float*>(w + round256(rows * D * sizeof(float)));
  float* l = reinterpret_cast<float*>(w + round256(rows * D * sizeof(float)) + round256(rows * sizeof(float)));
  // the per-hop calls: the first step starts from the empty state, the last
  // one writes the output (cp_ring_attn_step_ex with CPR_STEP_FIRST, CPR_STEP_LAST)
  a.o_acc = o_acc; a.m = m; a.l = l;
  a.o_out = o_out; a.lse = lse_out;
  a.nblocks = 1; a.cp = cp_size;
  for (int t = 0; t < cp_size; ++t) {
    a.rank = ((rank - t) % cp_size + cp_size) % cp_size;   // block held after t hops
    a.load_state = t > 0 ? 1 : 0;
    a.finalize = t == cp_size - 1 ? 1 : 0;
    const hipError_t e = launch_attn(dtype, a, st);
    if (e != hipSuccess) return hip_status(e, "cp_ring_attn_run(step)");
  }
  return launched(hipSuccess, st, "cp_ring_attn_run(stepwise)");
}

}  // extern "C"

// ------------------------------------------------ allocation-free fused run
//
// The partial states of a key-split fused run live in `scratch`, one copy per
// GPU, held from the library's load until the process ends. Size bound: the
// split happens only when the unsplit grid g = ceil(Lq / 256) * B * H has
// 2g <= 256 workgroups, into ns <= 256 / g slices, so the partial states cover
// ns * B * H * Lq <= ns * g * 256 <= 65,536 rows: at D = 128, 65,536 float32
// rows of O plus the m and l planes, each plane 256-byte aligned.
namespace {
constexpr size_t kScratchRows = 65536;
constexpr size_t kScratchBytes = CPR_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes == kScratchRows * 128 * sizeof(float) + 2 * kScratchRows * sizeof(float),
              "65,536 rows of the D = 128 state");
static_assert(kScratchBytes % 256 == 0 && (kScratchRows * 128 * sizeof(float)) % 256 == 0,
              "planes stay 256-byte aligned");
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch`: its address is looked up once per
// device with that device current; host code then uses only that address.
cpr_status current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CPR_EUNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(CPR_EHIP, "scratch address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CPR_OK;
}
}  // namespace

extern "C" {

cpr_status cp_ring_attn_run_noalloc(int32_t dtype, int32_t B, int32_t H, int32_t D, int32_t cp_size, int32_t rank,
                                    const cpr_view* q_local, int32_t Lq, const int32_t* q_pos,
                                    const cpr_view* k_ring, const cpr_view* v_ring, const int32_t* ring_pos,
                                    int32_t causal, float softmax_scale, const cpr_attn_ext* ext, void* o_out,
                                    float* lse_out, void* stream) {
  TRY(validate_run(dtype, B, H, D, cp_size, rank, q_local, Lq, q_pos, k_ring, v_ring, ring_pos, softmax_scale, ext,
                   o_out, lse_out));
  void* ws = nullptr;
  TRY(current_scratch(&ws));
  const size_t rows = (size_t)B * H * Lq;
  const int32_t ns = dtype == CPR_BF16 ? attn_bf16_kv_split(B, H, Lq, Lq) : 1;
  const size_t need = ns > 1 ? state_bytes(ns, rows, D) : 0;
  if (need > kScratchBytes)
    return fail(CPR_EUNSUPPORTED, "key-split partial states need %zu bytes, above the %zu-byte scratch", need,
                kScratchBytes);
  AttnArgs a = make_args(dtype, B, H, D, q_local, Lq, q_pos, k_ring, v_ring, Lq, ring_pos, causal, softmax_scale,
                         ext);
  return run_fused(dtype, a, cp_size, rank, o_out, lse_out, ns > 1 ? ws : nullptr, need,
                   static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------- backward

size_t cp_ring_attn_bwd_workspace_size(int32_t B, int32_t H, int32_t Lq) {
  if (B < 1 || H < 1 || Lq < 1 || Lq > CPR_MAX_SEQ) return 0;
  return 2 * round256((size_t)B * H * Lq * 4) + round256((size_t)Lq * 8);
}

// Bytes of the partial gradients a split backward launch keeps after the
// preprocessing planes (0 when neither kernel splits): dQ partials of
// q_split slices, then dK and dV partials of kv_split slices, each plane
// 256-byte aligned.
static size_t bwd_split_bytes(int32_t B, int32_t H, int32_t H_kv, int32_t D, int32_t Lq, int64_t Lk_total,
                              int32_t* q_split, int32_t* kv_split) {
  const int32_t nq = bwd_bf16_q_split(B, H, Lq);
  const int32_t nk = bwd_bf16_kv_split(B, H_kv, Lk_total);
  if (q_split) *q_split = nq;
  if (kv_split) *kv_split = nk;
  size_t bytes = 0;
  if (nq > 1) bytes += round256((size_t)nq * B * H * Lq * D * sizeof(float));
  if (nk > 1) bytes += 2 * round256((size_t)nk * B * H_kv * (size_t)Lk_total * D * sizeof(float));
  return bytes;
}

size_t cp_ring_attn_bwd_workspace_size_ex(int32_t B, int32_t H, int32_t H_kv, int32_t D, int32_t Lq, int64_t Lk) {
  const size_t base = cp_ring_attn_bwd_workspace_size(B, H, Lq);
  if (!base || (D != 64 && D != 128) || H_kv < 0 || (H_kv > 0 && H % H_kv) || Lk < 1 || Lk > CPR_MAX_SEQ) return 0;
  return base + bwd_split_bytes(B, H, H_kv > 0 ? H_kv : H, D, Lq, Lk, nullptr, nullptr);
}

// Engage the split of a bf16 backward launch when the workspace holds the
// partial gradients; otherwise leave it unsplit.
static void bwd_plan_split(int32_t dtype, BwdArgs& a, int64_t Lk_total, void* ws, size_t bytes) {
  a.q_split = a.kv_split = 1;
  if (dtype != CPR_BF16) return;
  int32_t nq, nk;
  const size_t extra = bwd_split_bytes(a.B, a.H, a.H_kv, a.D, a.Lq, Lk_total, &nq, &nk);
  const size_t base = cp_ring_attn_bwd_workspace_size(a.B, a.H, a.Lq);
  if (!extra || bytes < base + extra) return;
  char* w = static_cast<char*>(ws) + base;
  if (nq > 1) {
    a.q_split = nq;
    a.dq_part = reinterpret_cast<float*>(w);
    w += round256((size_t)nq * a.B * a.H * a.Lq * a.D * sizeof(float));
  }
  if (nk > 1) {
    const size_t plane = round256((size_t)nk * a.B * a.H_kv * (size_t)Lk_total * a.D * sizeof(float));
    a.kv_split = nk;
    a.dk_part = reinterpret_cast<float*>(w);
    a.dv_part = reinterpret_cast<float*>(w + plane);
  }
}

static cpr_status check_bwd_workspace(int32_t B, int32_t H, int32_t Lq, const void* ws, size_t bytes) {
  const size_t need = cp_ring_attn_bwd_workspace_size(B, H, Lq);
  if (!ws || bytes < need) return fail(CPR_EINVAL, "backward workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(CPR_EINVAL, "backward workspace must be 256-byte aligned");
  return CPR_OK;
}

// workspace: lse2 [B*H*Lq] float, dvec [B*H*Lq] float, qwin [Lq] int2, each 256-byte aligned
static void bwd_workspace(void* ws, int32_t B, int32_t H, int32_t Lq, float** lse2, float** dvec, int2** qwin) {
  char* w = static_cast<char*>(ws);
  const size_t plane = round256((size_t)B * H * Lq * 4);
  *lse2 = reinterpret_cast<float*>(w);
  *dvec = reinterpret_cast<float*>(w + plane);
  *qwin = reinterpret_cast<int2*>(w + 2 * plane);
}

static cpr_status check_grad(const char* name, const float* p) {
  if (!p) return fail(CPR_EINVAL, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(CPR_EINVAL, "%s must be 16-byte aligned", name);
  return CPR_OK;
}

// float32 views read 16 bytes at a time by the preprocessing pass
static cpr_status check_rows16(const char* name, const cpr_view* v, int32_t dtype) {
  if (dtype == CPR_F32 && (!aligned(v->data, 16) || v->stride_b % 4 || v->stride_h % 4 || v->stride_l % 4))
    return fail(CPR_EINVAL, "%s: float32 rows must be 16-byte aligned", name);
  return CPR_OK;
}

cpr_status cp_ring_attn_bwd_prep(int32_t dtype, int32_t B, int32_t H, int32_t D, int32_t Lq,
                                 const cpr_view* o_local, const cpr_view* do_local, const float* lse_local,
                                 const int32_t* q_pos, int32_t causal, const cpr_attn_ext* ext,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dims(dtype, B, H, D));
  TRY(check_len("Lq", Lq));
  TRY(check_view("o_local", o_local, dtype, D));
  TRY(check_view("do_local", do_local, dtype, D));
  TRY(check_rows16("o_local", o_local, dtype));
  TRY(check_rows16("do_local", do_local, dtype));
  if (!lse_local || !aligned(lse_local, 4)) return fail(CPR_EINVAL, "lse_local must be non-NULL and 4-byte aligned");
  if (!q_pos) return fail(CPR_EINVAL, "q_pos is NULL");
  if (ext && ((ext->kw_lo && !aligned(ext->kw_lo, 4)) || (ext->kw_hi && !aligned(ext->kw_hi, 4))))
    return fail(CPR_EINVAL, "key-window arrays must be 4-byte aligned");
  TRY(check_bwd_workspace(B, H, Lq, workspace, workspace_bytes));
  BwdPrepArgs a{};
  a.o = o_local->data; a.o_sb = o_local->stride_b; a.o_sh = o_local->stride_h; a.o_sl = o_local->stride_l;
  a.dout = do_local->data; a.do_sb = do_local->stride_b; a.do_sh = do_local->stride_h; a.do_sl = do_local->stride_l;
  a.lse = lse_local;
  a.q_pos = q_pos;
  a.kw_lo = ext ? ext->kw_lo : nullptr;
  a.kw_hi = ext ? ext->kw_hi : nullptr;
  a.causal = causal ? 1 : 0;
  a.B = B; a.H = H; a.D = D; a.Lq = Lq;
  bwd_workspace(workspace, B, H, Lq, &a.lse2, &a.dvec, &a.qwin);
  return launched(launch_bwd_prep(dtype == CPR_BF16, a, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_ring_attn_bwd_prep");
}

static BwdArgs make_bwd_args(int32_t B, int32_t H, int32_t D, int32_t H_kv, const cpr_view* q,
                             const cpr_view* dout, int32_t Lq, const cpr_view* k, const cpr_view* v, int32_t Lk,
                             const int32_t* kv_pos, float softmax_scale, void* workspace) {
  BwdArgs a{};
  a.q = q->data; a.q_sb = q->stride_b; a.q_sh = q->stride_h; a.q_sl = q->stride_l;
  a.dout = dout->data; a.do_sb = dout->stride_b; a.do_sh = dout->stride_h; a.do_sl = dout->stride_l;
  a.k = k->data; a.k_sb = k->stride_b; a.k_sh = k->stride_h; a.k_sl = k->stride_l;
  a.v = v->data; a.v_sb = v->stride_b; a.v_sh = v->stride_h; a.v_sl = v->stride_l;
  a.kv_pos = kv_pos;
  float *lse2, *dvec;
  int2* qwin;
  bwd_workspace(workspace, B, H, Lq, &lse2, &dvec, &qwin);
  a.lse2 = lse2;
  a.dvec = dvec;
  a.qwin = qwin;
  a.B = B; a.H = H; a.H_kv = H_kv > 0 ? H_kv : H; a.D = D; a.Lq = Lq; a.Lk = Lk;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  return a;
}

static hipError_t launch_bwd(int32_t dtype, const BwdArgs& a, hipStream_t st) {
  return dtype == CPR_BF16 ? launch_bwd_bf16(a, 1, 1, st) : launch_bwd_f32(a, 1, 1, st);
}

cpr_status cp_ring_attn_bwd_step(int32_t dtype, int32_t B, int32_t H, int32_t D, int32_t H_kv,
                                 const cpr_view* q, const cpr_view* dout, int32_t Lq,
                                 const cpr_view* k, const cpr_view* v, int32_t Lk, const int32_t* kv_pos,
                                 float softmax_scale, const void* workspace, size_t workspace_bytes,
                                 float* dq_acc, float* dk_acc, float* dv_acc, void* stream) {
  cpr_attn_ext ext{H_kv, nullptr, nullptr};
  TRY(validate_attn(dtype, B, H, D, q, Lq, nullptr, k, v, Lk, kv_pos, &ext, /*need_q_pos=*/0));
  TRY(check_view("dout", dout, dtype, D));
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale))
    return fail(CPR_EINVAL, "softmax_scale must be finite");
  TRY(check_bwd_workspace(B, H, Lq, workspace, workspace_bytes));
  TRY(check_grad("dq_acc", dq_acc));
  TRY(check_grad("dk_acc", dk_acc));
  TRY(check_grad("dv_acc", dv_acc));
  BwdArgs a = make_bwd_args(B, H, D, H_kv, q, dout, Lq, k, v, Lk, kv_pos, softmax_scale,
                            const_cast<void*>(workspace));
  a.nblocks = 1; a.rank = 0; a.cp = 1;
  a.dq = dq_acc; a.dk = dk_acc; a.dv = dv_acc;
  a.accumulate = 1;
  bwd_plan_split(dtype, a, Lk, const_cast<void*>(workspace), workspace_bytes);
  return launched(launch_bwd(dtype, a, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_ring_attn_bwd_step");
}

cpr_status cp_ring_attn_bwd_run(int32_t dtype, int32_t B, int32_t H, int32_t D,
                                int32_t cp_size, int32_t rank,
                                const cpr_view* q_local, int32_t Lq, const int32_t* q_pos,
                                const cpr_view* k_ring, const cpr_view* v_ring, const int32_t* ring_pos,
                                const cpr_view* o_local, const cpr_view* do_local, const float* lse_local,
                                int32_t causal, float softmax_scale, const cpr_attn_ext* ext,
                                float* dq_local, float* dk_ring, float* dv_ring,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (cp_size < 1) return fail(CPR_EINVAL, "cp_size must be >= 1 (got %d)", cp_size);
  if (rank < 0 || rank >= cp_size) return fail(CPR_EINVAL, "rank %d outside [0, %d)", rank, cp_size);
  TRY(validate_attn(dtype, B, H, D, q_local, Lq, q_pos, k_ring, v_ring, (int64_t)Lq * cp_size, ring_pos, ext));
  if ((int64_t)Lq * cp_size > CPR_MAX_SEQ) return fail(CPR_EUNSUPPORTED, "cp_size * Lq must be <= 2^30");
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale))
    return fail(CPR_EINVAL, "softmax_scale must be finite");
  TRY(check_grad("dq_local", dq_local));
  TRY(check_grad("dk_ring", dk_ring));
  TRY(check_grad("dv_ring", dv_ring));
  // the preprocessing validates o_local, do_local, lse_local and the workspace
  TRY(cp_ring_attn_bwd_prep(dtype, B, H, D, Lq, o_local, do_local, lse_local, q_pos, causal, ext, workspace,
                            workspace_bytes, stream));
  const int32_t h_kv = ext ? ext->H_kv : 0;
  BwdArgs a = make_bwd_args(B, H, D, h_kv, q_local, do_local, Lq, k_ring, v_ring, Lq, ring_pos, softmax_scale,
                            workspace);
  a.nblocks = cp_size; a.rank = rank; a.cp = cp_size;
  a.dq = dq_local; a.dk = dk_ring; a.dv = dv_ring;
  a.accumulate = 0;
  bwd_plan_split(dtype, a, (int64_t)Lq * cp_size, workspace, workspace_bytes);
  return launched(launch_bwd(dtype, a, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_ring_attn_bwd_run");
}

cpr_status cp_rope_apply(int32_t dtype, int32_t B, int32_t H, int32_t L, int32_t D, const cpr_view* x,
                         const int32_t* pos, float base, int32_t style, void* out, void* stream) {
  TRY(check_dims(dtype, B, H, D));
  TRY(check_len("L", L));
  TRY(check_view("x", x, dtype, D));
  TRY(check_rows16("x", x, dtype));
  if (!pos) return fail(CPR_EINVAL, "pos is NULL");
  if (!(base > 0.f) || isinf(base)) return fail(CPR_EINVAL, "base must be positive and finite");
  if (style != CPR_ROPE_INTERLEAVED && style != CPR_ROPE_HALF) return fail(CPR_EINVAL, "unknown rotary style %d", style);
  if (!out) return fail(CPR_EINVAL, "out is NULL");
  if (!aligned(out, 16)) return fail(CPR_EINVAL, "out must be 16-byte aligned");
  RopeArgs a{};
  a.x = x->data; a.x_sb = x->stride_b; a.x_sh = x->stride_h; a.x_sl = x->stride_l;
  a.pos = pos;
  a.B = B; a.H = H; a.L = L; a.D = D;
  a.base = base;
  a.style = style;
  a.out = out;
  return launched(launch_rope(dtype == CPR_BF16, a, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "cp_rope_apply");
}

cpr_status cp_ring_attn_tile_census(int32_t cp_size, int32_t Lq, const int32_t* q_pos, const int32_t* ring_pos,
                                    int32_t causal, const cpr_attn_ext* ext, int32_t* kept, int32_t* masked,
                                    void* stream) {
  if (cp_size < 1) return fail(CPR_EINVAL, "cp_size must be >= 1 (got %d)", cp_size);
  TRY(check_len("Lq", Lq));
  if ((int64_t)Lq * cp_size > CPR_MAX_SEQ) return fail(CPR_EUNSUPPORTED, "cp_size * Lq must be <= 2^30");
  if (!q_pos || !ring_pos) return fail(CPR_EINVAL, "position arrays must be non-NULL");
  if (!kept || !masked) return fail(CPR_EINVAL, "kept and masked must be non-NULL");
  if (!aligned(kept, 4) || !aligned(masked, 4)) return fail(CPR_EINVAL, "kept and masked must be 4-byte aligned");
  if (ext && ((ext->kw_lo && !aligned(ext->kw_lo, 4)) || (ext->kw_hi && !aligned(ext->kw_hi, 4))))
    return fail(CPR_EINVAL, "key-window arrays must be 4-byte aligned");
  CensusArgs a{};
  a.q_pos = q_pos;
  a.kv_pos = ring_pos;
  a.kw_lo = ext ? ext->kw_lo : nullptr;
  a.kw_hi = ext ? ext->kw_hi : nullptr;
  a.Lq = Lq; a.Lk = Lq; a.nblocks = cp_size;
  a.causal = causal ? 1 : 0;
  a.kept = kept; a.masked = masked;
  return launched(launch_tile_census(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream),
                  "cp_ring_attn_tile_census");
}

const char* cp_status_string(int32_t status) {
  switch (status) {
    case CPR_OK: return "ok";
    case CPR_EINVAL: return "invalid argument";
    case CPR_EUNSUPPORTED: return "unsupported configuration";
    case CPR_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* cp_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
