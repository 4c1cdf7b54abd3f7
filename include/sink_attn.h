/*
 * sink_attn.h -- C ABI of the gfx950 (MI355X) sink-aware grouped-query attention
 * library (libsinkattn.so).
 *
 * The operation ("GPT-OSS on day 0", section "Kernels for GPT-OSS" > "Sink attention"):
 * for every query row and query head h,
 *
 *     out = softmax( [ q.K^T * sm_scale , sinks[h] ] ) . [ V ; 0 ]
 *
 * i.e. the head's sink is one extra logit in the softmax denominator that has no value
 * row.  The softmax is evaluated online with the running maximum subtracted; the
 * running state starts at (max = sink, sum = 1); when the key axis is split into
 * chunks the sink joins the first chunk only and the chunks are combined by a
 * log-sum-exp merge.  Attention is grouped-query: query head h reads KV head
 * h / (num_q_heads / num_kv_heads) (same page, "model deltas").  K and V are stored
 * head-major ("HND": [kv_head][token][head_dim], tokens contiguous per head), the KV
 * cache layout of "Hosting Qwen on Blackwell" (introduction).
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer; the caller owns all memory.  The
 *    library never allocates, frees or synchronises: work is enqueued on `stream`
 *    (a hipStream_t; NULL = the legacy default stream) and the call returns at once.
 *  - bf16 is IEEE bfloat16 (1-8-7); outputs are rounded to nearest even.
 *  - Causal alignment is bottom-right: query i of a sequence with Lq queries and Lk
 *    keys sees key j iff j <= i + Lk - Lq.
 *  - lse is the natural-log partition function of the row INCLUDING the sink term
 *    (ln(e^sink + sum_j e^(s_j))); -inf for a row with no key and no sink.
 *  - A NULL `sinks` means no sink (every sink = -inf).  A sink may be -inf per head.
 *  - Return value: a sink_attn_status.  Every precondition that the host can check is
 *    checked before any kernel launch (the only HIP calls before then read the device's
 *    compute-unit count); device-side preconditions (monotone index arrays,
 *    offsets within the totals) are documented, not checked, because checking them
 *    would need a synchronisation -- but every device read of K, V and Q goes through
 *    bounded buffer loads, so a violation yields wrong numbers, never a fault.
 *  - Thread-safe; no global mutable state beyond a per-thread last-HIP-error slot and
 *    the compute-unit count of each device, read once per device (std::call_once) the
 *    first time a plan is made with it current.
 */
#ifndef SINK_ATTN_H
#define SINK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SINK_ATTN_OK = 0,
  SINK_ATTN_ERR_INVALID_ARG = 1,   /* null pointer, bad size, non-finite scale, ...   */
  SINK_ATTN_ERR_UNSUPPORTED = 2,   /* valid but not instantiated (head_dim, q_len...) */
  SINK_ATTN_ERR_WORKSPACE = 3,     /* workspace missing or too small                  */
  SINK_ATTN_ERR_HIP = 4,           /* a HIP call failed; see sink_attn_last_hip_error */
  SINK_ATTN_ERR_INTERNAL = 5,      /* unexpected internal failure                     */
  SINK_ATTN_ERR_SCRATCH_LIMIT = 6  /* larger than the no-allocation entry point holds */
} sink_attn_status;

/*
 * YaRN rotary position encoding ("GPT-OSS on day 0", model deltas: YaRN position
 * encoding as in DeepSeek-V3; the published YaRN method).  Pairs are half-split
 * (dimension i rotates with i + D/2) by angle pos * f_i, f_i = theta^(-2i/D); with
 * factor s > 1 frequencies with at least beta_fast turns over original_max_pos keep f_i,
 * those with at most beta_slow turns become f_i / s, linear in between, and rotated
 * vectors are scaled by 0.1 ln s + 1.  Angles are formed and reduced in double precision.
 * Passing NULL where an entry point takes a `const sink_attn_rope*` means no rotation;
 * invalid parameters (theta <= 1, factor <= 0, non-finite, or for s > 1
 * original_max_pos < 1 or beta_fast <= beta_slow or beta_slow < 0) give
 * SINK_ATTN_ERR_INVALID_ARG.
 */
typedef struct {
  float theta;
  float factor;
  int32_t original_max_pos;
  float beta_fast;
  float beta_slow;
} sink_attn_rope;

/*
 * Variable-length prefill ("Sink attention": the same sink rule serves prefill).
 *
 *  q             bf16 [total_q, num_q_heads, head_dim], token-major, contiguous.
 *  k, v          bf16 [num_kv_heads, total_kv, head_dim], head-major, contiguous.
 *  sinks         fp32 [num_q_heads] or NULL.
 *  cu_seqlens_q  int32 [batch+1], cu_seqlens_q[0] = 0, nondecreasing, last = total_q.
 *  cu_seqlens_kv int32 [batch+1], likewise over the token axis of k and v.
 *  max_seqlen_q  host upper bound of cu_seqlens_q[b+1]-cu_seqlens_q[b] (sizes the grid;
 *                rows beyond it are not computed).
 *  head_dim      64 or 128.  num_q_heads % num_kv_heads == 0.
 *  sm_scale      finite, > 0; multiplies q.k (not the sink).
 *  causal        0 or 1.  When 1, each sequence must have Lk >= Lq (documented).
 *  out           bf16 [total_q, num_q_heads, head_dim].
 *  lse           fp32 [total_q, num_q_heads] or NULL.
 *  rope          NULL, or YaRN parameters: query i of a sequence is rotated at position
 *                Lk - Lq + i while it is loaded (keys are used as given: rotate them when
 *                they are written, see sink_attn_kv_append / sink_attn_rope_apply).
 */
int sink_attn_prefill(const void* q, const void* k, const void* v, const float* sinks,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                      int32_t batch, int32_t max_seqlen_q, int64_t total_q,
                      int64_t total_kv, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, float sm_scale, int32_t causal, void* out,
                      float* lse, const sink_attn_rope* rope, void* stream);

/*
 * Prefill with the key axis split across workgroups ("Sink attention": attention is
 * parallelised over heads and KV length; the sink enters the first block only; blocks
 * merge by log-sum-exp).  For chunked prefill over a cached prefix (Lk >> Lq) and other
 * inputs whose (head group, sequence, query tile) grid leaves the GPU under-filled.
 * Arguments as for sink_attn_prefill, plus:
 *  max_seqlen_kv  host upper bound of cu_seqlens_kv[b+1] - cu_seqlens_kv[b].
 *  num_splits     0 = planner (sink_attn_prefill_num_splits); k in 1..64 = k splits of
 *                 ceil(ceil(max_seqlen_kv/64)/k) 64-key units each.  One split is
 *                 exactly sink_attn_prefill.
 *  workspace      256-byte aligned, at least sink_attn_prefill_workspace_bytes(total_q,
 *                 num_q_heads, head_dim, S) bytes for the resolved split count S (none when
 *                 S = 1): fp32 partial outputs [total_q*Hq, S, D] and lse [total_q*Hq, S],
 *                 merged by the merge kernel into out/lse.  No initialisation needed.
 */
int sink_attn_prefill_split(const void* q, const void* k, const void* v, const float* sinks,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                            int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                            int64_t total_q, int64_t total_kv, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                            int32_t causal, int32_t num_splits, void* workspace,
                            size_t workspace_bytes, void* out, float* lse,
                            const sink_attn_rope* rope, void* stream);

/* Resolved split count of sink_attn_prefill_split (0 if the arguments are invalid): with
 * num_splits = 0, enough splits for about four workgroups per compute unit, at most 16,
 * each of at least 512 keys.  num_cus: compute units to plan for; 0 = those of the
 * current device (what sink_attn_prefill_split uses), or 256 when no device is current. */
int32_t sink_attn_prefill_num_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t num_splits, int32_t num_cus);

/* Workspace bytes of sink_attn_prefill_split for S resolved splits (0 when S = 1 or the
 * arguments are invalid). */
size_t sink_attn_prefill_workspace_bytes(int64_t total_q, int32_t num_q_heads, int32_t head_dim,
                                         int32_t num_splits);

/*
 * Decode with 1..4 query tokens per sequence (multi-token / speculative decode), split
 * along the key axis ("Sink attention": attention parallelised over heads and KV
 * length; the sink enters the first block only) and merged by log-sum-exp.
 *
 *  q          bf16 [batch, q_len, num_q_heads, head_dim].
 *  k, v       bf16 [num_kv_heads, total_kv, head_dim] (HND).
 *  kv_indptr  int32 [batch+1]: sequence b owns tokens [kv_indptr[b], kv_indptr[b+1]) of
 *             the token axis.  The KV already contains the q_len new tokens, so query t
 *             sits at position Lk - q_len + t; with causal=1 it sees keys <= that
 *             position (causal within the draft).
 *  max_kv_len host upper bound of kv_indptr[b+1]-kv_indptr[b].
 *  num_splits 0 = planner: n = ceil(Lk/256) rounded up to a multiple of C and clamped
 *             to [4, 16] chunks for each sequence, where C =
 *             sink_attn_decode_chunks_per_slot(...) is the number of chunks one
 *             workgroup takes together; k in 1..64 = exactly k chunks per sequence.  A
 *             chunk holds ceil(ceil(Lk/n)/32)*32 keys; trailing chunks may be empty
 *             (sink_attn_decode_chunk_bounds).  Every chunk keeps its own online softmax,
 *             chunk 0 starting from (sink, 1) and every other chunk from (-inf, 0), and the
 *             chunks are merged by log-sum-exp: first the C chunks one workgroup takes
 *             (in parallel, or in turn as one run of consecutive chunks), then the slots.
 *             With num_splits = 0, q_len * num_q_heads/num_kv_heads <= 64, total_kv <
 *             2^31 and more than one partial slot (see sink_attn_decode_num_slots), the
 *             stream plan is used instead: each KV head's token axis (all sequences back
 *             to back) is cut into equal ranges of R tokens, each streamed by one
 *             wavefront (<= 16 rows) or by one workgroup of 2 or 4 wavefronts that
 *             share the staged keys (<= 32 / <= 64 rows), whose partials are merged
 *             with the sinks (sink_attn_decode_stream_plan).  Before either, with
 *             num_splits = 0 and more than 16 rows per KV head: when the batch alone
 *             gives at least two workgroups per compute unit (batch * num_kv_heads *
 *             row_groups >= 2 * CUs) and the sequences are of nearly equal length
 *             (8 * total_kv >= 7 * batch * max_kv_len), one workgroup per (sequence,
 *             KV head, row group) takes every chunk of its sequence in turn, as one
 *             run, and writes the result (no partials, no merge).  Which of the three
 *             a call uses: sink_attn_decode_plan_kind.
 *  workspace  device scratch of at least sink_attn_decode_workspace_bytes(...) bytes,
 *             256-byte aligned; contents need no initialisation.  Calls that share one
 *             workspace must be stream-ordered.
 *  out        bf16 [batch, q_len, num_q_heads, head_dim];  lse fp32 [batch, q_len,
 *             num_q_heads] or NULL.
 *  rope       NULL, or YaRN parameters: query t is rotated at position Lk - q_len + t
 *             while it is loaded (keys as given).
 */
int sink_attn_decode(const void* q, const void* k, const void* v, const float* sinks,
                     const int32_t* kv_indptr, int32_t batch, int32_t q_len,
                     int64_t total_kv, int32_t max_kv_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                     int32_t causal, int32_t num_splits, void* workspace,
                     size_t workspace_bytes, void* out, float* lse,
                     const sink_attn_rope* rope, void* stream);

/*
 * sink_attn_decode without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Arguments, plan, kernels and results are those of sink_attn_decode; the
 * partials live in a file-scope device array of the library instead of a caller's
 * workspace.  Nothing is allocated or freed by the call.
 *  - Limit: inputs whose sink_attn_decode_workspace_bytes(...) exceeds
 *    sink_attn_decode_noalloc_scratch_bytes() (32 MiB) are rejected with
 *    SINK_ATTN_ERR_SCRATCH_LIMIT before any kernel launch, unless sink_attn_decode_plan_kind
 *    reports whole-sequence runs, which write no partials.  (The gpt-oss-like batch of 64
 *    sequences up to 8192 keys, 64 query heads over 8, fits; so does the 256-sequence
 *    speculative-decode batch of equal lengths, through whole-sequence runs on a 256-CU
 *    MI355X; a multi-token batch of unequal lengths with that many rows does not: use
 *    sink_attn_decode with a workspace.)
 *  - Each GPU holds its own copy of the array from the library's load until the process
 *    ends; its device address is looked up on the first call with that GPU current.
 *  - Every call on one GPU shares that GPU's array and it keeps the last call's
 *    contents: calls that may overlap on one GPU (different streams, or different host
 *    threads) race and must be serialised by the caller.  No content needs clearing
 *    between calls.
 */
int sink_attn_decode_noalloc(const void* q, const void* k, const void* v, const float* sinks,
                             const int32_t* kv_indptr, int32_t batch, int32_t q_len,
                             int64_t total_kv, int32_t max_kv_len, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                             int32_t causal, int32_t num_splits, void* out, float* lse,
                             const sink_attn_rope* rope, void* stream);

/* Bytes of the no-allocation entry point's scratch array on each GPU (its size limit). */
size_t sink_attn_decode_noalloc_scratch_bytes(void);

/* Which plan sink_attn_decode uses for these sizes, with num_cus the compute units to plan
 * for (0 = the current device's, what sink_attn_decode uses, or 256 when no device is
 * current); -1 if the arguments are invalid.  sink_attn_decode_paged makes the same choice
 * between whole-sequence runs and the chunk plan with total_kv taken as
 * (num_page_entries - batch) * page_size, a lower bound of the tokens its page list
 * holds (it has no stream plan above 16 rows per KV head). */
typedef enum {
  SINK_ATTN_PLAN_CHUNKS = 0,     /* chunk plan: sink_attn_decode_num_slots slots, merged
                                    by log-sum-exp when there is more than one          */
  SINK_ATTN_PLAN_STREAM = 1,     /* stream plan (sink_attn_decode_stream_plan)          */
  SINK_ATTN_PLAN_WHOLE_RUNS = 2  /* every chunk of a sequence in one workgroup, which
                                    writes the result                                  */
} sink_attn_plan_kind;
int32_t sink_attn_decode_plan_kind(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int64_t total_kv,
                                   int32_t max_kv_len, int32_t num_splits, int32_t num_cus);

/* Workspace bytes sink_attn_decode needs for these sizes (0 if the arguments are
 * invalid).  Holds fp32 partial outputs and partial lse for every (row, slot): S slots of
 * the chunk plan, or 17 where the stream plan may be used. */
size_t sink_attn_decode_workspace_bytes(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_kv_len, int32_t num_splits);

/* Chunks per partial slot, C (0 if the arguments are invalid).  With
 * q_len * (num_q_heads/num_kv_heads) <= 16 rows per KV head one workgroup streams C
 * consecutive chunks in parallel (one wavefront each, C = 4 for head_dim 64 and 2 for
 * 128) and merges them before writing.  Otherwise one workgroup streams a run of C
 * consecutive chunks in turn, each chunk with its own online softmax, merging each
 * finished chunk into the run's state: C = 1 in planner mode, and with a forced chunk
 * count k the longest run that still gives about four workgroups per compute unit,
 * C = clamp(floor(k * batch * num_kv_heads * row_groups / (4 * num_cus)), 1, k), with
 * row_groups = ceil(rows / 64) (1 for rows <= 64).  num_cus: compute units to plan for,
 * 0 = the current device's (what sink_attn_decode uses), or 256 when no device is
 * current. */
int32_t sink_attn_decode_chunks_per_slot(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_kv_len, int32_t num_splits,
                                         int32_t num_cus);

/* Chunk plan of one sequence with kv_len keys ("Sink attention": blocks along the key
 * axis; the pages fix no size): the number of chunks n (0 if the arguments are invalid)
 * and, in bounds[0..min(n+1, capacity)), their boundaries: chunk c covers keys
 * [bounds[c], bounds[c+1]), bounds[0] = 0, bounds[n] = kv_len.  The kernels derive the
 * same plan on the device from each sequence's length (no plan is passed to them). */
int32_t sink_attn_decode_chunk_bounds(int32_t kv_len, int32_t q_len, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t num_splits,
                                      int32_t* bounds, int32_t capacity);

/* Partial slots per row the chunk kernels use (the S of the partial layout):
 * ceil(n_max / C) with n_max the chunk count at max_kv_len and C as above; num_cus as
 * above.  0 if the arguments are invalid. */
int32_t sink_attn_decode_num_slots(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_kv_len,
                                   int32_t num_splits, int32_t num_cus);

/*
 * First stage of sink_attn_decode on its own: for every row
 * r = (b*q_len + t)*num_q_heads + h and slot j < S, the normalised output
 * part_o[r][j][0..head_dim) (fp32) and natural-log partition function part_lse[r][j]
 * (fp32; -inf when empty) of the keys of plan chunks [j*C, j*C + C) together (chunk 0
 * includes the sink).  S = sink_attn_decode_num_slots(..., 0), C =
 * sink_attn_decode_chunks_per_slot(..., 0) (planned for the current device).  Exported
 * so the partials can be checked and timed; sink_attn_decode = this + merge (with S = 1
 * the kernel writes the result).
 */
int sink_attn_decode_partial(const void* q, const void* k, const void* v,
                             const float* sinks, const int32_t* kv_indptr, int32_t batch,
                             int32_t q_len, int64_t total_kv, int32_t max_kv_len,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             float sm_scale, int32_t causal, int32_t num_splits,
                             float* part_o, float* part_lse, const sink_attn_rope* rope,
                             void* stream);

/*
 * Stream plan of sink_attn_decode (contiguous K/V).  "Sink attention": the key axis is
 * split into blocks merged by their log-sum-exp and the sink is counted once.  Here the
 * blocks are ranges of R tokens of one KV head's token axis, all sequences back to back:
 * range i of head g covers tokens [i*R, (i+1)*R) and one wavefront (or a workgroup of 2
 * or 4 for more than 16 query rows per KV head, each owning 16 rows) streams it, closing a
 * partial wherever a sequence ends inside it.  Partial j of row r (sequence b) covers the
 * keys of b inside range floor(kv_indptr[b]/R) + j and carries no sink; the merge adds
 * the sink of head h once, as a log-sum-exp term of value zero.
 *
 * sink_attn_decode_stream_plan: 1 if the stream plan applies to these sizes (then R, the
 *   ranges per head and the slots S per row are written where the pointers are not
 *   NULL), else 0.  sink_attn_decode uses it unless whole-sequence runs are chosen
 *   first (sink_attn_decode_plan_kind); the two step entry points below accept every
 *   size it applies to.  R is a multiple of 32, at least ceil(max_kv_len/16), so S <= 17.
 *   The plan gives about 4 wavefronts (<= 16 rows) or 2 workgroups per compute unit:
 *   num_cus is the count to plan for, 0 = the current device's (what sink_attn_decode
 *   uses), or 256 when no device is current.
 * sink_attn_decode_stream_partial: the first step on its own, into `workspace` (size and
 *   alignment as for sink_attn_decode): part_o fp32 [rows, S, head_dim] at offset 0,
 *   part_lse fp32 [rows, S] at the next 256-byte boundary, rows = batch*q_len*num_q_heads.
 *   Slots past a row's last range are not written.  Returns SINK_ATTN_ERR_UNSUPPORTED
 *   where the plan does not apply.
 * sink_attn_decode_stream_merge: the second step on its own: out / lse from the partials
 *   in `workspace` and the sinks (NULL = no sink).  A sequence with no keys gets out = 0
 *   and lse = sink (or -inf).
 * Both are exported so each step can be checked and timed; sink_attn_decode runs them
 * back to back wherever it uses the stream plan.
 */
int32_t sink_attn_decode_stream_plan(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int64_t total_kv,
                                     int32_t max_kv_len, int32_t num_cus, int32_t* range_tokens,
                                     int32_t* ranges_per_head, int32_t* slots);
int sink_attn_decode_stream_partial(const void* q, const void* k, const void* v,
                                    const int32_t* kv_indptr, int32_t batch, int32_t q_len,
                                    int64_t total_kv, int32_t max_kv_len, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                    int32_t causal, void* workspace, size_t workspace_bytes,
                                    const sink_attn_rope* rope, void* stream);
int sink_attn_decode_stream_merge(const float* sinks, const int32_t* kv_indptr, int32_t batch,
                                  int32_t q_len, int64_t total_kv, int32_t max_kv_len,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  const void* workspace, size_t workspace_bytes, void* out,
                                  float* lse, void* stream);

/*
 * Log-sum-exp merge of chunk partials ("Sink attention": blocks along the key axis are
 * combined; the sink is already inside chunk 0's partial).  For each row:
 *   m* = max_c part_lse[r][c],  w_c = e^(part_lse[r][c] - m*),
 *   out[r] = sum_c w_c part_o[r][c] / sum_c w_c   (bf16),  lse[r] = m* + ln sum_c w_c.
 * Slots with part_lse = -inf carry no weight (their part_o is not read); a row with
 * every slot -inf gets out = 0 and lse = -inf.
 *  part_o fp32 [rows, num_slots, head_dim], part_lse fp32 [rows, num_slots],
 *  splits_per_row int32 [rows] or NULL: row r merges only its first splits_per_row[r]
 *  slots (clamped to [0, num_slots]; 0 gives out = 0, lse = -inf), whose lse and part_o
 *  alone are read; NULL = every row merges all num_slots,
 *  num_slots 1..256 (the row stride of part_o and part_lse), head_dim 64 or 128,
 *  out bf16 [rows, head_dim], lse fp32 [rows] or NULL.
 */
int sink_attn_merge(const float* part_o, const float* part_lse, const int32_t* splits_per_row,
                    int64_t rows, int32_t num_slots, int32_t head_dim, void* out, float* lse,
                    void* stream);

/*
 * Paged KV cache.  "Hosting Qwen on Blackwell" (introduction) keeps KV caches head-major
 * so they can be split or joined by head; "GPT-OSS on day 0" ("Kernels for GPT-OSS")
 * puts the sink into the attention templates of a paged-KV library.  The page table
 * follows that library's convention:
 *
 *  k_cache, v_cache  bf16 [num_pages, num_kv_heads, page_size, head_dim]: inside a page
 *                    heads lead and each head's tokens are contiguous (HND per page).
 *  kv_page_indptr    int32 [batch+1]: sequence b owns entries [indptr[b], indptr[b+1])
 *                    of kv_page_indices, in token order.
 *  kv_page_indices   int32 [num_page_entries]: page ids in [0, num_pages).
 *  kv_last_page_len  int32 [batch]: tokens in the sequence's last page (1..page_size);
 *                    length L_b = (n_b - 1) * page_size + last_page_len[b], 0 if n_b = 0.
 *  page_size         a multiple of 16, at most 4096 (a 32-key tile then spans at most
 *                    two pages).
 * Device-side values are clamped (page ids to the cache, list offsets to the list), so
 * a malformed table gives wrong numbers, never a fault.
 */

/* Decode over a paged cache; every other argument and the workspace are as for
 * sink_attn_decode (workspace size from sink_attn_decode_workspace_bytes).  max_kv_len
 * is a host upper bound of L_b.  Plans: in planner mode at most 16 rows per KV head take
 * the stream plan along the page list laid end to end; more rows take whole-sequence
 * runs when sink_attn_decode_plan_kind's rule holds with total_kv =
 * (num_page_entries - batch) * page_size, else the chunk plan. */
int sink_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                           const float* sinks, const int32_t* kv_page_indptr,
                           const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
                           int32_t batch, int32_t q_len, int64_t num_page_entries,
                           int64_t num_pages, int32_t page_size, int32_t max_kv_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           float sm_scale, int32_t causal, int32_t num_splits, void* workspace,
                           size_t workspace_bytes, void* out, float* lse,
                           const sink_attn_rope* rope, void* stream);

/*
 * Append new keys and values to a paged cache (the step before attention reads them).
 *  k_new, v_new   bf16 [total_new, num_kv_heads, head_dim], token-major as a projection
 *                 writes them; sequence b owns rows [append_indptr[b], append_indptr[b+1]).
 *  The page table already describes the sequences WITH the new tokens: new token i of
 *  sequence b (of n_b) is written at position L_b - n_b + i.  Rows whose position would
 *  be negative are skipped.  max_append_len: host upper bound of n_b.
 *  rope: NULL, or YaRN parameters: each new key is rotated at its position as it is
 *  written (values are copied unchanged).
 *  k_new, v_new, k_cache and v_cache must be 16-byte aligned (the copies are 16-byte
 *  vector accesses), else SINK_ATTN_ERR_INVALID_ARG.
 */
int sink_attn_kv_append(const void* k_new, const void* v_new, const int32_t* append_indptr,
                        const int32_t* kv_page_indptr, const int32_t* kv_page_indices,
                        const int32_t* kv_last_page_len, int32_t batch, int32_t max_append_len,
                        int64_t total_new, int64_t num_page_entries, int64_t num_pages,
                        int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                        void* k_cache, void* v_cache, const sink_attn_rope* rope,
                        void* stream);

/* In-place YaRN rotation of bf16 vectors: element (t, h, d), t < num_tokens,
 * h < num_heads, d < head_dim, at x + t*token_stride + h*head_stride + d (strides in
 * elements, multiples of 8; x 16-byte aligned), token t at positions[t] (int32, device).
 * For example contiguous HND keys [Hkv, total, D] have token_stride D and head_stride
 * total*D.  rope must not be NULL.  The rows must not overlap (they are rewritten in
 * place): the smaller stride of an axis with more than one index must be at least
 * head_dim and the larger at least the smaller axis's extent, as in [T, H, D] and
 * [H, T, D] layouts; anything else is SINK_ATTN_ERR_INVALID_ARG. */
int sink_attn_rope_apply(void* x, int64_t num_tokens, int32_t num_heads, int32_t head_dim,
                         int64_t token_stride, int64_t head_stride, const int32_t* positions,
                         const sink_attn_rope* rope, void* stream);

/* Static text for a status code. */
const char* sink_attn_status_str(int status);

/* The hipError_t of the last SINK_ATTN_ERR_HIP returned on the calling thread. */
int sink_attn_last_hip_error(void);

/* Library version, "major.minor.patch". */
const char* sink_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_H */
