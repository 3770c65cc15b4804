/*
 * cpring.h - C ABI of libcpring: one context-parallel rank's ring-attention
 * forward and backward passes, for AMD Instinct MI355X (gfx950).
 *
 * Method (pages cited by title and section):
 *  - "Context Parallelism" (Ultralytics glossary), "How context parallelism
 *    works": each device computes partial attention on its local data, hands
 *    its KV block to the next device, and repeats until the whole sequence is
 *    seen; the result equals full-sequence attention up to rounding.
 *  - "Sequence Parallelism and Ring Attention" (aiunderstanding.org), "Deep
 *    dive" and "Technical insight": local queries stay put while KV blocks
 *    travel the ring; each arriving block is folded in with the online-softmax
 *    running max / running sum, rescaling earlier partial sums when a larger
 *    score appears.
 *  - "Context Parallelism v.s. Sequence Parallelism (Megatron-LM)",
 *    "Implementation quirk: symmetric chunk assignment": the sequence is cut
 *    into 2*cp chunks and rank r holds chunks r and 2*cp-1-r, so every rank
 *    does the same causal work; positions and masks must use global token
 *    positions; the sequence is padded to a multiple of 2*cp.
 *
 * Conventions shared by every call:
 *  - Tensors are [B, H, L, D] (sequence on dim 2, as in the SDPA call on the
 *    glossary page, "Practical use and trade-offs"). A cpr_view gives element
 *    strides for B, H and L; the D dimension must be contiguous and rows may
 *    not overlap (stride_l >= D, else CPR_EUNSUPPORTED; B and H strides may
 *    be 0 for a broadcast input). Views of bf16 tensors need every stride and
 *    the base address 16-byte aligned.
 *  - Every pointer argument named as device memory must point to memory of
 *    the current HIP device; position arrays are int32 device arrays.
 *  - The caller owns every buffer. The library never allocates or frees
 *    device memory and keeps no state between calls, apart from the static
 *    scratch array of cp_ring_attn_run_noalloc (loaded with the library).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and does not synchronise. Results are valid once the stream has
 *    reached the call. Debugging aid: with CPRING_SYNC_CHECK=1 in the
 *    environment, every call that launches work waits for its stream before
 *    it returns, so that a failure of its kernels is reported as CPR_EHIP by
 *    that call rather than by a later one.
 *  - Arguments are validated before anything is launched. On failure the call
 *    returns a non-zero cpr_status, launches nothing, and cp_last_error()
 *    describes the problem. A launch failure returns CPR_EHIP. No C++
 *    exception crosses this boundary. Results are deterministic: no atomics
 *    are used, so the same inputs give bit-identical outputs.
 *  - The state of a rank between ring steps is (O, m, l), all float32 and
 *    contiguous: O [B, H, Lq, D] is the unnormalised output
 *    sum_j exp(s_j - m) v_j, m [B, H, Lq] the running max of the allowed
 *    scaled scores s (natural-log units, -inf when nothing was allowed yet),
 *    l [B, H, Lq] the running sum_j exp(s_j - m).
 *  - A key j is allowed for query i iff pos_j >= 0, pos_i >= 0 and, when
 *    causal, pos_j <= pos_i (global positions; -1 marks a pad token). A query
 *    with no allowed key finalises to O = 0, LSE = -inf.
 *  - softmax_scale <= 0 selects 1/sqrt(D), the SDPA default.
 *  - Values in pad rows of K and V must be finite (zero-filled rows, as
 *    cp_shard_gather writes, are fine): they are multiplied by zero weights.
 */
#ifndef CPRING_H
#define CPRING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CPR_OK = 0,
  CPR_EINVAL = 1,       /* an argument is out of range, null or misaligned */
  CPR_EUNSUPPORTED = 2, /* valid request outside what the kernels implement */
  CPR_EHIP = 3          /* the HIP runtime reported an error at launch */
} cpr_status;

typedef enum { CPR_F32 = 0, CPR_BF16 = 1 } cpr_dtype;

typedef enum {
  CPR_ZIGZAG = 0,     /* rank r: chunks r and 2cp-1-r of 2cp chunks */
  CPR_CONTIGUOUS = 1, /* rank r: tokens [r*L/cp, (r+1)*L/cp) */
  CPR_STRIPED = 2     /* rank r: tokens r, r+cp, r+2cp, ... */
} cpr_layout;

/* Flags for cp_ring_attn_run. */
enum {
  CPR_RUN_FUSED = 0,    /* one launch walks every ring block; optional workspace */
  CPR_RUN_STEPWISE = 1  /* cp calls of the step kernel, the first from the empty state and the last
                           writing the output (CPR_STEP_FIRST, CPR_STEP_LAST); needs the workspace */
};

/* Strided [B, H, L, D] view; strides in elements, D contiguous. */
typedef struct cpr_view {
  const void* data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_l;
} cpr_view;

/* Largest supported values. */
#define CPR_MAX_SEQ ((int64_t)1 << 30)

/*
 * Padded sequence length for `seq_len` tokens over `cp_size` ranks: the next
 * multiple of 2*cp_size for CPR_ZIGZAG (Megatron page, symmetric chunk
 * assignment: the sequence must split into 2*cp equal chunks), of cp_size for
 * CPR_CONTIGUOUS ("Sequence Parallelism and Ring Attention", "Deep dive") and
 * CPR_STRIPED (the same page, "The future of sequence parallelism and ring
 * attention": striped assignment, the other way to even out causal work).
 * Returns -1 for seq_len < 1 or > CPR_MAX_SEQ, cp_size < 1, or an unknown layout.
 */
int64_t cp_padded_len(int64_t seq_len, int32_t cp_size, int32_t layout);

/*
 * Token and position-id layout of all ranks, rank-major: entry r*Lr + i
 * (Lr = S_pad/cp_size) describes the i-th local token of rank r.
 *   token_idx[k]  index of that token in the padded natural order
 *                 (zigzag: chunk r then chunk 2cp-1-r, each in order;
 *                 contiguous: r*Lr + i; striped: i*cp_size + r);
 *   pos_ids[k]    its global position, or -1 for a pad token (>= seq_len).
 * Both are int32 device arrays of cp_padded_len(...) entries; either may be
 * NULL (not both). Cited: Megatron page, symmetric chunk assignment (chunk
 * pairing, global positions for position ids and masks, padding).
 */
cpr_status cp_zigzag_partition(int64_t seq_len, int32_t cp_size, int32_t layout,
                               int32_t* token_idx, int32_t* pos_ids, void* stream);

/*
 * Gather rows into layout order: dst[b,h,i,:] = src[b,h,token_idx[i],:] when
 * 0 <= token_idx[i] < seq_len, else zeros (pad rows). dst is a contiguous
 * [B, H, n_out, D] device buffer of `dtype`; src a view of [B, H, seq_len, D].
 * This materialises a rank's local Q (token_idx of that rank) or the
 * ring-ordered K and V of all ranks (the whole token_idx), the inputs that the
 * Megatron page says must follow the chunk pairing.
 */
cpr_status cp_shard_gather(int32_t dtype, int32_t B, int32_t H, int64_t seq_len, int32_t D,
                           const cpr_view* src, const int32_t* token_idx, int64_t n_out,
                           void* dst, void* stream);

/*
 * Reset the running state before the first ring step: O = 0, m = -inf, l = 0
 * ("Sequence Parallelism and Ring Attention", "Technical insight").
 * o_acc [B,H,Lq,D], m and l [B,H,Lq]: contiguous float32 device buffers.
 */
cpr_status cp_ring_attn_init(int32_t B, int32_t H, int32_t Lq, int32_t D,
                             float* o_acc, float* m, float* l, void* stream);

/*
 * One ring step: fold the KV block that has just arrived into the running
 * state of the local queries ("Sequence Parallelism and Ring Attention",
 * "Deep dive": blockwise attention with the running max/sum trick).
 *   q        [B,H,Lq,D] local queries, with global positions q_pos [Lq];
 *   k, v     [B,H,Lk,D] one KV block, with global positions kv_pos [Lk];
 *   causal   non-zero: key allowed only if kv_pos <= q_pos;
 *   o_acc, m, l  the state (see above), read and updated in place.
 * dtype CPR_BF16 runs on bf16 MFMA with float32 accumulation (the
 * probabilities are rounded to bf16 before the P*V product); CPR_F32 runs in
 * float32. D must be 64 or 128. q/k/v must not alias the state.
 */
cpr_status cp_ring_attn_step(int32_t dtype, int32_t B, int32_t H, int32_t D,
                             const cpr_view* q, int32_t Lq, const int32_t* q_pos,
                             const cpr_view* k, const cpr_view* v, int32_t Lk, const int32_t* kv_pos,
                             int32_t causal, float softmax_scale,
                             float* o_acc, float* m, float* l, void* stream);

/*
 * Fold a second partial state (o2, m2, l2), built over a disjoint set of keys,
 * into (o_acc, m, l) in place: m' = max(m, m2), each side scaled by
 * exp(m_side - m') (the same rescaling rule, "Technical insight").
 * All buffers contiguous float32, shapes as for the state.
 */
cpr_status cp_ring_attn_merge(int32_t B, int32_t H, int32_t Lq, int32_t D,
                              float* o_acc, float* m, float* l,
                              const float* o2, const float* m2, const float* l2, void* stream);

/*
 * Normalise the state after the last step: o_out = O / l, rounded to nearest
 * even in out_dtype (CPR_BF16 or CPR_F32), and lse_out = m + ln l (float32).
 * The running normaliser l and max m are those of "Sequence Parallelism and
 * Ring Attention", "Technical insight": dividing the unnormalised sum by l
 * once every block is folded in gives the softmax-weighted output, which
 * "Context Parallelism", "How context parallelism works", states equals
 * full-sequence attention.
 * Rows with l = 0 give O = 0, LSE = -inf. o_out is a contiguous [B,H,Lq,D]
 * device buffer, lse_out a contiguous [B,H,Lq] float32 buffer (may be NULL).
 */
cpr_status cp_ring_attn_finalize(int32_t out_dtype, int32_t B, int32_t H, int32_t Lq, int32_t D,
                                 const float* o_acc, const float* m, const float* l,
                                 void* o_out, float* lse_out, void* stream);

/* Workspace bytes for cp_ring_attn_run in either mode: the float32 state
 * ([B,H,Lq,D] O, [B,H,Lq] m and l) that CPR_RUN_STEPWISE needs, or, for a bf16
 * pass whose grid is too small to fill the GPU, the n partial states of a
 * key-split CPR_RUN_FUSED run (n = 1 for large shapes, so the two coincide).
 * Returns 0 for invalid sizes. */
size_t cp_ring_attn_workspace_size(int32_t B, int32_t H, int32_t Lq, int32_t D);

/*
 * One rank's whole ring pass: Lq = Lk local tokens per rank, cp_size blocks.
 *   q_local  [B,H,Lq,D] the rank's queries, positions q_pos [Lq];
 *   k_ring, v_ring  [B,H,cp_size*Lq,D] every rank's KV block, rank-major
 *            (block s = rows [s*Lq, (s+1)*Lq)), positions ring_pos [cp_size*Lq];
 *   rank     0 <= rank < cp_size.
 * Step t folds the block of rank (rank - t) mod cp_size: after t hops of a
 * ring in which every device passes its block to the next, that is the block
 * rank `rank` holds ("Context Parallelism", "How context parallelism works").
 * Writes o_out [B,H,Lq,D] (dtype, contiguous) and lse_out [B,H,Lq] (float32,
 * may be NULL). flags: CPR_RUN_FUSED or CPR_RUN_STEPWISE; the latter needs
 * `workspace` of at least the float32 state's bytes (256-byte aligned; size it
 * with cp_ring_attn_workspace_size()), else CPR_EINVAL. CPR_RUN_FUSED takes the
 * workspace as an option: for a bf16 pass with too few query tiles to fill the
 * GPU, a 256-byte-aligned workspace of cp_ring_attn_workspace_size() bytes lets
 * it split every block's keys over several workgroups per query tile and
 * merge their partial states (the running-max rescale rule of "Sequence
 * Parallelism and Ring Attention", "Technical insight", over disjoint key
 * sets); with no workspace, or a smaller one, it runs unsplit. The split
 * changes only the float32 summation order. In either mode the workspace is
 * scratch that the call overwrites: calls in flight at the same time must not
 * share one.
 */
cpr_status cp_ring_attn_run(int32_t dtype, int32_t B, int32_t H, int32_t D,
                            int32_t cp_size, int32_t rank,
                            const cpr_view* q_local, int32_t Lq, const int32_t* q_pos,
                            const cpr_view* k_ring, const cpr_view* v_ring, const int32_t* ring_pos,
                            int32_t causal, float softmax_scale,
                            void* o_out, float* lse_out,
                            void* workspace, size_t workspace_bytes, int32_t flags, void* stream);

/*
 * Extensions of the ring pass for real workloads (all optional: a NULL
 * extension, or H_kv = 0 and NULL windows, is the plain pass above).
 *   H_kv   heads of K and V (grouped-query attention): 0 means H; otherwise
 *          1 <= H_kv and H % H_kv == 0, and query head h reads K/V head
 *          h / (H / H_kv). The k/v views are then [B, H_kv, L, D]. The
 *          Megatron page ("Context Parallelism (CP)", communication) counts
 *          the ring traffic in K/V heads, H_kv.
 *   kw_lo, kw_hi  int32 device arrays of Lq entries, each may be NULL: query
 *          i may only attend keys whose position p satisfies
 *          kw_lo[i] <= p <= kw_hi[i] (in addition to causal masking). This is
 *          how packed sequences are attended: with the bounds of each query's
 *          own document, attention never crosses a document boundary. The
 *          Megatron page ("Implementation quirk: symmetric chunk assignment")
 *          requires the attention mask and the packed-sequence metadata to
 *          follow the chunk pairing: the bounds are global positions, given
 *          per local query in the same order as q_pos.
 */
typedef struct cpr_attn_ext {
  int32_t H_kv;
  const int32_t* kw_lo;
  const int32_t* kw_hi;
  /* Read by cp_ring_attn_step_ex only (ignored by every other entry point):
   * step_flags, a combination of CPR_STEP_FIRST and CPR_STEP_LAST (0: an
   * ordinary step), and the outputs o_out, lse_out of a CPR_STEP_LAST step. */
  int32_t step_flags;
  void* o_out;
  float* lse_out;
} cpr_attn_ext;

/*
 * The first and the last hop of a ring, for cp_ring_attn_step_ex. The running
 * state starts empty and is normalised once after the last block
 * ("Sequence Parallelism and Ring Attention", "Technical insight"); these
 * flags fold those two ends into the steps themselves:
 *   CPR_STEP_FIRST  o_acc, m, l are not read on entry: the step starts from
 *                   O = 0, m = -inf, l = 0, so no cp_ring_attn_init is needed.
 *   CPR_STEP_LAST   o_acc, m, l are not written: the step writes
 *                   o_out = O / l [B,H,Lq,D] in the dtype of q (16-byte
 *                   aligned, contiguous) and, when lse_out is not NULL,
 *                   lse_out = m + ln l [B,H,Lq] float32, as
 *                   cp_ring_attn_finalize would after an ordinary step.
 * With both flags the state pointers may be NULL (one block is the whole
 * ring). o_out and lse_out must not alias q, k, v or the state. Unknown bits,
 * or CPR_STEP_LAST with o_out NULL, return CPR_EINVAL.
 */
#define CPR_STEP_FIRST 1
#define CPR_STEP_LAST 2

/* cp_ring_attn_step with the extensions above; k and v are [B, H_kv, Lk, D]. */
cpr_status cp_ring_attn_step_ex(int32_t dtype, int32_t B, int32_t H, int32_t D,
                                const cpr_view* q, int32_t Lq, const int32_t* q_pos,
                                const cpr_view* k, const cpr_view* v, int32_t Lk, const int32_t* kv_pos,
                                int32_t causal, float softmax_scale, const cpr_attn_ext* ext,
                                float* o_acc, float* m, float* l, void* stream);

/* cp_ring_attn_run with the extensions above; k_ring and v_ring are
 * [B, H_kv, cp_size*Lq, D]. */
cpr_status cp_ring_attn_run_ex(int32_t dtype, int32_t B, int32_t H, int32_t D,
                               int32_t cp_size, int32_t rank,
                               const cpr_view* q_local, int32_t Lq, const int32_t* q_pos,
                               const cpr_view* k_ring, const cpr_view* v_ring, const int32_t* ring_pos,
                               int32_t causal, float softmax_scale, const cpr_attn_ext* ext,
                               void* o_out, float* lse_out,
                               void* workspace, size_t workspace_bytes, int32_t flags, void* stream);

/*
 * cp_ring_attn_run_ex in CPR_RUN_FUSED mode, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Arguments, results and
 * errors are those of cp_ring_attn_run_ex with flags = CPR_RUN_FUSED; there is
 * no workspace argument. When the grid is too small for the GPU, the per-slice
 * partial states of the key split go to a scratch array inside the library
 * (CPR_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load until the
 * process ends) instead of a caller's workspace; the split, and so the result,
 * is the same as cp_ring_attn_run's with a workspace of
 * cp_ring_attn_workspace_size() bytes. A split whose partial states would not
 * fit returns CPR_EUNSUPPORTED (the split rule keeps them within 65,536 rows,
 * so this does not happen for any valid shape). The call allocates nothing:
 * the scratch address is looked up on the call's first use of a device.
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * behind: calls that overlap in time on one GPU (two streams, two threads)
 * race and must be ordered by the caller. Each split launch writes every
 * partial row it later reads, so no clearing is needed between calls.
 */
#define CPR_NOALLOC_SCRATCH_BYTES ((size_t)34078720) /* 65,536 rows x (128 + 2) floats */

cpr_status cp_ring_attn_run_noalloc(int32_t dtype, int32_t B, int32_t H, int32_t D,
                                    int32_t cp_size, int32_t rank,
                                    const cpr_view* q_local, int32_t Lq, const int32_t* q_pos,
                                    const cpr_view* k_ring, const cpr_view* v_ring, const int32_t* ring_pos,
                                    int32_t causal, float softmax_scale, const cpr_attn_ext* ext,
                                    void* o_out, float* lse_out, void* stream);

/*
 * Backward pass: the gradients of one rank's attention output (the glossary
 * page, "Context Parallelism", "Practical use and trade-offs", differentiates
 * the context-parallel output). With O and LSE saved by the forward pass and
 * dO the gradient of the loss with respect to O, for every block the rank sees:
 *   P    = exp(scale * q k^T - LSE), the final probabilities, recomputed
 *          (masked entries 0; a query with LSE = -inf has P = 0);
 *   Dvec = rowsum(dO * O), dP = dO v^T, dS = P * (dP - Dvec);
 *   dQ   = scale * dS k, summed over every block: it stays on the rank;
 *   dK   = scale * dS^T q and dV = P^T dO: this rank's share of the block's
 *          gradient. In a ring these travel with their block and reach its
 *          owner after a full circle, summed over the ranks ("Sequence
 *          Parallelism and Ring Attention", "Deep dive": blocks move to the
 *          next device each hop).
 * dtype CPR_BF16 runs on bf16 MFMA with float32 accumulation: P and dS are
 * rounded to bf16 (nearest even) before the products that use them. CPR_F32
 * runs in float32. Gradients are float32, contiguous. The masking rules, the
 * extensions (cpr_attn_ext) and the softmax_scale default are the forward's.
 */

/* Workspace bytes of the backward pass for B*H*Lq query rows: a float
 * LSE * log2(e) per row, a float Dvec per row, then an int2 {lo, hi} allowed
 * key-position window per query. Returns 0 for invalid sizes. */
size_t cp_ring_attn_bwd_workspace_size(int32_t B, int32_t H, int32_t Lq);

/* Workspace bytes that also let a bf16 backward call on a grid too small for
 * the GPU split its work: the dQ kernel over the keys of each block, the
 * dK/dV kernel over the queries, each slice writing float32 partial
 * gradients that a reduction pass then sums in slice order (deterministic:
 * no atomics). This is the partial-sum counterpart of the forward's key split
 * (the running-max rule of "Sequence Parallelism and Ring Attention",
 * "Technical insight", is not needed here: gradients simply add up over
 * disjoint key or query sets), sized for the glossary page's small example
 * ("Context Parallelism", "Practical use and trade-offs": 1 x 4 x 4096 x 64
 * on two ranks, differentiated). H_kv = 0 means H; Lk is the number of K/V
 * rows the call covers: cp_size * Lq for cp_ring_attn_bwd_run, the block's
 * Lk for cp_ring_attn_bwd_step. Equals cp_ring_attn_bwd_workspace_size(B, H,
 * Lq) when the grids are large enough not to split. Returns 0 for invalid
 * sizes. A call given at least this many bytes splits; given fewer (but at
 * least the base size) it runs unsplit. Only the float32 summation order
 * changes. */
size_t cp_ring_attn_bwd_workspace_size_ex(int32_t B, int32_t H, int32_t H_kv, int32_t D, int32_t Lq, int64_t Lk);

/*
 * Backward preprocessing of one rank's queries, once per backward pass. Fills
 * `workspace` (cp_ring_attn_bwd_workspace_size(B, H, Lq) bytes, 256-byte
 * aligned) from:
 *   o_local, do_local  [B,H,Lq,D] views of dtype: the forward output and dO
 *                      (float32 views need 16-byte aligned rows);
 *   lse_local          [B,H,Lq] contiguous float32: the forward's LSE;
 *   q_pos, causal, ext the forward's positions, causal flag and windows
 *                      (only the windows of ext are used here).
 */
cpr_status cp_ring_attn_bwd_prep(int32_t dtype, int32_t B, int32_t H, int32_t D, int32_t Lq,
                                 const cpr_view* o_local, const cpr_view* do_local, const float* lse_local,
                                 const int32_t* q_pos, int32_t causal, const cpr_attn_ext* ext,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * One backward ring step: add the contributions of one KV block.
 *   q, dout    [B,H,Lq,D] views of dtype: local queries and dO;
 *   k, v       [B,H_kv,Lk,D] views of dtype: the block (H_kv = 0 means H),
 *              positions kv_pos [Lk];
 *   workspace  filled by cp_ring_attn_bwd_prep for these queries; with
 *              cp_ring_attn_bwd_workspace_size_ex(B, H, H_kv, D, Lq, Lk)
 *              bytes a small grid splits, using the bytes past the
 *              preprocessing planes as scratch;
 *   dq_acc     [B,H,Lq,D] float32: dq_acc += scale * dS k;
 *   dk_acc, dv_acc  [B,H_kv,Lk,D] float32: += the rank's share of the
 *              block's dK and dV (the buffers that travel with the block).
 * The accumulators must not overlap the inputs or each other.
 */
cpr_status cp_ring_attn_bwd_step(int32_t dtype, int32_t B, int32_t H, int32_t D, int32_t H_kv,
                                 const cpr_view* q, const cpr_view* dout, int32_t Lq,
                                 const cpr_view* k, const cpr_view* v, int32_t Lk, const int32_t* kv_pos,
                                 float softmax_scale, const void* workspace, size_t workspace_bytes,
                                 float* dq_acc, float* dk_acc, float* dv_acc, void* stream);

/*
 * One rank's whole backward ring pass, the counterpart of cp_ring_attn_run_ex
 * (q_local, q_pos, k_ring, v_ring, ring_pos, causal, softmax_scale and ext as
 * there): preprocessing, dQ over every block in ring order, and the rank's
 * share of dK and dV of every block.
 *   o_local, do_local  [B,H,Lq,D] views of dtype; lse_local [B,H,Lq] float32;
 *   dq_local   [B,H,Lq,D] float32, written;
 *   dk_ring, dv_ring  [B,H_kv,cp_size*Lq,D] float32, written, in ring order
 *              like k_ring: summed over all ranks they are the full
 *              gradients of K and V;
 *   workspace  cp_ring_attn_bwd_workspace_size(B, H, Lq) bytes, 256-byte
 *              aligned, or cp_ring_attn_bwd_workspace_size_ex(B, H, H_kv, D,
 *              Lq, cp_size * Lq) bytes to let a small grid split.
 * The workspace is scratch that the call overwrites: calls in flight at the
 * same time must not share one.
 */
cpr_status cp_ring_attn_bwd_run(int32_t dtype, int32_t B, int32_t H, int32_t D,
                                int32_t cp_size, int32_t rank,
                                const cpr_view* q_local, int32_t Lq, const int32_t* q_pos,
                                const cpr_view* k_ring, const cpr_view* v_ring, const int32_t* ring_pos,
                                const cpr_view* o_local, const cpr_view* do_local, const float* lse_local,
                                int32_t causal, float softmax_scale, const cpr_attn_ext* ext,
                                float* dq_local, float* dk_ring, float* dv_ring,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Pairing of the dimensions a rotary embedding rotates together. */
typedef enum {
  CPR_ROPE_INTERLEAVED = 0, /* pairs (2j, 2j+1) */
  CPR_ROPE_HALF = 1         /* pairs (j, j + D/2) */
} cpr_rope_style;

/*
 * Rotary position embedding by global position. The Megatron page
 * ("Implementation quirk: symmetric chunk assignment") requires rotary
 * embeddings to use each token's global position under the chunk pairing:
 * a rank holding chunks r and 2cp-1-r rotates its tokens by those chunks'
 * global positions, as cp_zigzag_partition's pos_ids give them, never by a
 * local renumbering. The rotation is the standard one: pair (a_j, b_j),
 * j = 0 .. D/2-1, becomes (a cos t - b sin t, a sin t + b cos t) with
 * t = pos * base^(-2j/D).
 *   x      [B,H,L,D] view of dtype (rows 16-byte aligned for float32);
 *   pos    int32 device array [L]: the rows' global positions, -1 = pad (the
 *          row is copied unchanged);
 *   base   > 0 (10000 is the usual value);
 *   style  CPR_ROPE_INTERLEAVED or CPR_ROPE_HALF;
 *   out    contiguous [B,H,L,D] device buffer of dtype; may be x's own
 *          memory when x is contiguous (in place).
 * Angles are reduced modulo 2*pi in double precision; sin and cos are then
 * taken in float32. D must be 64 or 128.
 */
cpr_status cp_rope_apply(int32_t dtype, int32_t B, int32_t H, int32_t L, int32_t D, const cpr_view* x,
                         const int32_t* pos, float base, int32_t style, void* out, void* stream);

/*
 * Tile census of the bf16 forward pass of cp_ring_attn_run_ex over the same
 * positions (q_pos [Lq], ring_pos [cp_size * Lq], causal, and the windows of
 * ext; H_kv is ignored): the pass takes its queries in tiles of 256 and the
 * keys of every block in tiles of 64, and classifies every (query tile, key
 * tile) pair from position ranges as skipped (no query of the tile may attend
 * any of its keys: neither loaded nor computed), full (computed without the
 * element mask) or masked (computed with the element mask). For every query
 * tile qt (ceil(Lq / 256) of them) this writes to the int32 device arrays
 *   kept[qt]    the key tiles computed, over all cp_size blocks,
 *   masked[qt]  those of them that need the element mask,
 * with the forward kernel's own classification code. The Megatron page
 * ("Implementation quirk: symmetric chunk assignment") pairs chunks r and
 * 2cp-1-r so that every rank does the same causal work; the census shows it
 * at tile granularity (the same sum on every rank). B, H and D do not enter.
 */
cpr_status cp_ring_attn_tile_census(int32_t cp_size, int32_t Lq, const int32_t* q_pos, const int32_t* ring_pos,
                                    int32_t causal, const cpr_attn_ext* ext, int32_t* kept, int32_t* masked,
                                    void* stream);

/* Static description of a status code. */
const char* cp_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* cp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CPRING_H */
