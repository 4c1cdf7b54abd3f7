// C ABI of libsinkattn: argument validation, planning and launch.  Every
// host-checkable precondition is checked before the first HIP call; no C++ exception
// crosses the boundary.  Plain host C++: the kernels are reached only through the
// launch layer (sa_launch.h), so this file also builds with a host compiler against a
// stub of that layer (the sanitizer build).
#include <math.h>
#include <stdint.h>

#include <new>

#include "../../include/sink_attn.h"
#include "sa_launch.h"
#include "sa_plan.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxSplits = 64;
constexpr int kMaxSlots = 256;
constexpr int64_t kMaxSpanBytes = 0x7fffffffLL;  // bounded-load window of one sequence

inline int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return SINK_ATTN_ERR_HIP;
}

inline bool dim_ok(int d) { return d == 64 || d == 128; }

inline bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

// Decode slot plan.  The kernels derive each sequence's chunk plan themselves
// (sa::plan_chunks); the host fixes how chunks group into partial slots:
//  - at most 16 rows per KV head: the chunk-wave kernel streams cw = 4 (head_dim 64) or
//    2 (128) consecutive chunks in parallel, one per wavefront, and merges them;
//  - otherwise the split kernel streams a run of consecutive chunks in turn.  With a
//    forced chunk count the run is as long as keeps about four workgroups per compute
//    unit (two rounds of the two that fit), so long runs stream unbroken and few
//    partials are written; in planner mode the run is one chunk (sink_attn_decode may
//    instead give one workgroup every chunk of its sequence: whole_runs below).
// slots = ceil(n_max / chunks per slot), n_max the chunk count at max_kv_len (the plan
// is nondecreasing in the length).
constexpr int kRunWgsPerCu = 4;
struct SlotPlan {
  int cw;     // chunks per workgroup in parallel (chunk-wave kernel) or 1
  int run;    // chunks per workgroup in turn (split kernel) or 1
  int slots;  // partial slots per row
};
SlotPlan slot_plan(int32_t batch, int32_t q_len, int32_t hq, int32_t hkv, int32_t d,
                   int32_t max_kv_len, int32_t num_splits, int cus) {
  const int rows = q_len * (hq / hkv);
  SlotPlan p{};
  p.cw = sa::decode_chunk_waves(rows, d);
  const int n = sa::plan_chunks(max_kv_len, num_splits, p.cw);
  p.run = 1;
  if (p.cw == 1 && num_splits > 0) {
    const int w = sa::decode_waves(rows);
    const int64_t row_groups = (rows + 16 * w - 1) / (16 * w);
    const int64_t wgs = (int64_t)n * batch * hkv * row_groups;  // workgroups at runs of one
    const int64_t r = wgs / ((int64_t)kRunWgsPerCu * cus);
    p.run = (int)(r < 1 ? 1 : (r > n ? n : r));
  }
  const int per_slot = p.cw > 1 ? p.cw : p.run;
  p.slots = (n + per_slot - 1) / per_slot;
  return p;
}

// Compute units the planners size grids for: the caller's count if positive, else the
// current device's (read once per device), else 256 (MI355X) when no device is current.
inline int resolve_cus(int32_t num_cus) {
  if (num_cus > 0) return num_cus;
  const int c = sa::device_cu_count();
  return c > 0 ? c : 256;
}

// Stream decode plan (contiguous K/V, at most 64 query rows per KV head, planner mode,
// more than one partial per row).  Up to 16 rows: about 4 wavefronts per CU, each taking
// R tokens of one KV head's token axis; up to 64 rows: about 2 workgroups per CU of 2 or 4
// wavefronts (16 rows each) sharing each range.  R is at least max_kv/16 (so a sequence
// overlaps at most 17 ranges, the slots a row needs) and a multiple of 32.
using sa::kStreamMaxSlots;
constexpr int kStreamWavesPerCu = 4;
constexpr int kStreamGroupsPerCu = 2;
inline bool stream_eligible(int32_t q_len, int32_t hq, int32_t hkv, int32_t d,
                            int32_t max_kv_len, int32_t num_splits) {
  if (num_splits != 0 || q_len * (hq / hkv) > 64) return false;
  // planner mode, whenever the chunk plan would need more than one slot (the batch and
  // compute units do not matter in planner mode)
  return slot_plan(1, q_len, hq, hkv, d, max_kv_len, 0, 256).slots > 1;
}
inline int64_t round32(int64_t x) { return (x + 31) / 32 * 32; }
sa::StreamPlan stream_plan(int32_t batch, int32_t q_len, int32_t hq, int32_t hkv,
                           int64_t total_kv, int32_t max_kv_len, int cus) {
  sa::StreamPlan p{};
  const int rows = q_len * (hq / hkv);
  p.waves = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  const int total = cus * (p.waves == 1 ? kStreamWavesPerCu : kStreamGroupsPerCu);
  p.nph = total / hkv > 0 ? total / hkv : 1;
  int64_t r = round32((total_kv + p.nph - 1) / p.nph);
  const int64_t r_floor = round32((max_kv_len + kStreamMaxSlots - 2) / (kStreamMaxSlots - 1));
  if (r < r_floor) r = r_floor;
  if (r < 32) r = 32;
  p.R = (int32_t)r;
  const int64_t sm = (max_kv_len + r - 1) / r + 1;
  p.smax = (int32_t)(sm < kStreamMaxSlots ? sm : kStreamMaxSlots);
  p.batch = batch;
  p.num_kv_heads = hkv;
  return p;
}
// Whole-sequence runs (planner mode, more than 16 rows per KV head): when
// the batch alone gives at least kWholeRunWgsPerCu workgroups per compute unit and the
// sequences are of nearly equal length (total_kv >= 7/8 of batch * max_kv_len), one
// workgroup per (sequence, KV head, row group) streams every chunk of its sequence in
// turn and writes the result: the work is already balanced, so the stream plan's equal
// ranges, its partials and its merge buy nothing.
constexpr int kWholeRunWgsPerCu = 2;
inline bool whole_runs(int32_t batch, int32_t q_len, int32_t hq, int32_t hkv, int64_t total_kv,
                       int32_t max_kv_len, int32_t num_splits, int cus) {
  const int rows = q_len * (hq / hkv);
  if (num_splits != 0 || rows <= 16 || max_kv_len < 1) return false;
  const int w = sa::decode_waves(rows);
  const int64_t row_groups = (rows + 16 * w - 1) / (16 * w);
  const int64_t wgs = (int64_t)batch * hkv * row_groups;
  return wgs >= (int64_t)kWholeRunWgsPerCu * cus && 8 * total_kv >= 7 * (int64_t)batch * max_kv_len;
}
inline size_t partial_bytes(int64_t rows, int64_t slots, int d) {
  int64_t bytes = rows * slots * d * 4;   // partial outputs
  bytes = (bytes + 255) & ~(int64_t)255;
  bytes += rows * slots * 4;              // partial lse
  return (size_t)((bytes + 255) & ~(int64_t)255);
}

// Key-axis splits of a prefill: num_splits > 0 forces them; 0 splits only when the
// (head group, sequence, query tile) grid would leave the GPU under-filled (fewer than
// four 8-wavefront workgroups per CU), keeping at least 8 key units (512 keys) per split.
constexpr int kPrefillWgsPerCu = 4;
int heads_per_wg(int group);
int prefill_splits(int32_t batch, int32_t max_q, int32_t max_kv, int32_t hq, int32_t hkv,
                   int32_t num_splits, int cus) {
  if (num_splits > 0) return num_splits;
  const int64_t target = (int64_t)kPrefillWgsPerCu * cus;
  const int group = hq / hkv;
  const int hg = heads_per_wg(group);
  const int64_t qtiles = (max_q + 32 * (8 / hg) - 1) / (32 * (8 / hg));
  const int64_t base = (int64_t)hkv * (group / hg) * batch * (qtiles > 0 ? qtiles : 1);
  int64_t s = (target + base - 1) / base;
  const int64_t units = (max_kv + 63) / 64;
  if (s > units / 8) s = units / 8;
  if (s > 16) s = 16;
  return s < 1 ? 1 : (int)s;
}

// Query heads per prefill workgroup: the largest divisor of the GQA group size <= 4.
int heads_per_wg(int group) {
  for (int hg = 4; hg >= 1; --hg)
    if (group % hg == 0) return hg;
  return 1;
}

int check_decode_args(const void* q, const void* k, const void* v, const int32_t* kv_indptr,
                      int32_t batch, int32_t q_len, int64_t total_kv, int32_t max_kv_len,
                      int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t causal,
                      int32_t num_splits) {
  if (!q || !k || !v || !kv_indptr) return SINK_ATTN_ERR_INVALID_ARG;
  if (batch < 1 || hq < 1 || hkv < 1 || total_kv < 0 || max_kv_len < 0)
    return SINK_ATTN_ERR_INVALID_ARG;
  if (hq % hkv != 0) return SINK_ATTN_ERR_INVALID_ARG;
  if (!scale_ok(sm_scale)) return SINK_ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SINK_ATTN_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > kMaxSplits) return SINK_ATTN_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > 4) return SINK_ATTN_ERR_UNSUPPORTED;
  if (!dim_ok(d)) return SINK_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)max_kv_len * d * 2 > kMaxSpanBytes) return SINK_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)q_len * hq * d * 2 > kMaxSpanBytes) return SINK_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)batch * q_len * hq > ((int64_t)1 << 40)) return SINK_ATTN_ERR_UNSUPPORTED;
  return SINK_ATTN_OK;
}

sa::DecodeArgs decode_args(const void* q, const void* k, const void* v, const float* sinks,
                           const int32_t* kv_indptr, int32_t batch, int32_t q_len,
                           int64_t total_kv, int32_t max_kv_len, int32_t hq, int32_t hkv,
                           int32_t d, float sm_scale, int32_t causal, int32_t num_splits) {
  sa::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.sinks = sinks;
  a.kv_indptr = kv_indptr;
  a.total_kv = total_kv;
  a.q_len = q_len;
  a.num_q_heads = hq;
  a.group = hq / hkv;
  const int rows = q_len * a.group;
  const int w = sa::decode_waves(rows);
  a.row_groups = (rows + 16 * w - 1) / (16 * w);
  a.num_splits = num_splits;
  a.num_kv_heads = hkv;
  const SlotPlan sp = slot_plan(batch, q_len, hq, hkv, d, max_kv_len, num_splits, resolve_cus(0));
  a.chunk_waves = sp.cw;
  a.chunk_run = sp.run;
  a.num_slots = sp.slots;
  a.causal = causal;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  return a;
}

// YaRN rotary frequencies for the device, in double precision: f_i = theta^(-2i/D); with
// factor s > 1 the published YaRN interpolation keeps frequencies with at least
// beta_fast turns over the original context L, divides those with at most beta_slow
// turns by s, mixes linearly in between, and scales q and k by 0.1 ln s + 1.
int make_rope(const sink_attn_rope* r, int d, sa::RopeArgs* out) {
  *out = sa::RopeArgs{};
  if (r == nullptr) return SINK_ATTN_OK;
  const bool finite = isfinite(r->theta) && isfinite(r->factor) && isfinite(r->beta_fast) &&
                      isfinite(r->beta_slow);
  if (!finite || r->theta <= 1.0f || r->factor <= 0.0f) return SINK_ATTN_ERR_INVALID_ARG;
  const bool yarn = r->factor > 1.0f;
  if (yarn && (r->original_max_pos < 1 || !(r->beta_fast > r->beta_slow) || r->beta_slow < 0.f))
    return SINK_ATTN_ERR_INVALID_ARG;
  const double two_pi = 6.283185307179586476925;
  for (int i = 0; i < d / 2; ++i) {
    double f = pow((double)r->theta, -2.0 * i / d);
    if (yarn) {
      const double turns = (double)r->original_max_pos * f / two_pi;
      double g = (turns - r->beta_slow) / ((double)r->beta_fast - r->beta_slow);
      g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
      f = (1.0 - g) * (f / r->factor) + g * f;
    }
    out->freq[i] = f;
  }
  out->mscale = yarn ? (float)(0.1 * log((double)r->factor) + 1.0) : 1.0f;
  out->enabled = 1;
  return SINK_ATTN_OK;
}

// Split kernel (+ merge when there is more than one slot) for contiguous or paged KV.
int run_decode(sa::DecodeArgs& a, int32_t batch, int32_t q_len, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_dim, int32_t max_kv_len, int32_t num_splits,
               const int32_t* page_ids, const sa::RopeArgs& rope, void* workspace,
               size_t workspace_bytes, void* out, float* lse, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  // A paged cache streams along its page list laid end to end (single-wavefront plans).
  const bool paged = page_ids != nullptr;
  // tokens on the key axis: a paged cache's list of n pages holds more than
  // (n - batch) * page_size of them
  const int64_t tokens = paged ? (a.num_page_entries - batch) * (int64_t)a.page_size : a.total_kv;
  if (whole_runs(batch, q_len, num_q_heads, num_kv_heads, tokens, max_kv_len, num_splits,
                 resolve_cus(0))) {
    // one slot holding every chunk of the plan at max_kv_len (a sequence's own plan has
    // no more chunks): the split kernel writes the result
    a.chunk_run = sa::plan_chunks(max_kv_len, 0, 1);
    a.num_slots = 1;
    a.out = out;
    a.lse = lse;
    hipError_t e = sa::launch_decode_split(a, head_dim, batch, num_kv_heads, true, page_ids, rope, st);
    if (e != hipSuccess) return hip_fail(e);
    return SINK_ATTN_OK;
  }
  const int64_t axis = paged ? a.num_page_entries * (int64_t)a.page_size : a.total_kv;
  if (axis <= INT32_MAX && (!paged || q_len * (num_q_heads / num_kv_heads) <= 16) &&
      stream_eligible(q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, num_splits)) {
    const size_t need = sink_attn_decode_workspace_bytes(batch, q_len, num_q_heads, num_kv_heads,
                                                         head_dim, max_kv_len, num_splits);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
      return SINK_ATTN_ERR_WORKSPACE;
    const sa::StreamPlan sp =
        stream_plan(batch, q_len, num_q_heads, num_kv_heads, axis, max_kv_len, resolve_cus(0));
    a.total_kv = axis;
    const int64_t rows = (int64_t)batch * q_len * num_q_heads;
    a.part_o = (float*)workspace;
    a.part_lse = (float*)((char*)workspace + ((rows * sp.smax * head_dim * 4 + 255) & ~(int64_t)255));
    a.out = out;
    a.lse = lse;
    hipError_t e = sa::launch_decode_stream(a, head_dim, sp, rope, page_ids, st);
    if (e != hipSuccess) return hip_fail(e);
    e = sa::launch_merge_stream(a, head_dim, sp, rows, paged, st);
    if (e != hipSuccess) return hip_fail(e);
    return SINK_ATTN_OK;
  }
  if (a.num_slots == 1) {  // one slot per row: the split kernel writes the result
    a.out = out;
    a.lse = lse;
    hipError_t e = sa::launch_decode_split(a, head_dim, batch, num_kv_heads, true, page_ids, rope, st);
    if (e != hipSuccess) return hip_fail(e);
    return SINK_ATTN_OK;
  }
  const size_t need = sink_attn_decode_workspace_bytes(batch, q_len, num_q_heads, num_kv_heads,
                                                       head_dim, max_kv_len, num_splits);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return SINK_ATTN_ERR_WORKSPACE;
  const int64_t rows = (int64_t)batch * q_len * num_q_heads;
  int64_t obytes = rows * a.num_slots * head_dim * 4;
  obytes = (obytes + 255) & ~(int64_t)255;
  a.part_o = (float*)workspace;
  a.part_lse = (float*)((char*)workspace + obytes);
  hipError_t e = sa::launch_decode_split(a, head_dim, batch, num_kv_heads, false, page_ids, rope, st);
  if (e != hipSuccess) return hip_fail(e);
  e = sa::launch_merge(a.part_o, a.part_lse, nullptr, rows, a.num_slots, head_dim, out, lse, st);
  if (e != hipSuccess) return hip_fail(e);
  return SINK_ATTN_OK;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Rows of d elements at t*ts + h*hs (t < nt, h < nh) are pairwise disjoint when the
// layout nests: the smaller stride (of an axis with more than one index) is at least d
// and the larger is at least the smaller's extent.  Covers token-major [T, H, D] and
// head-major [H, T, D]; other overlapping-free layouts are rejected too (conservative).
inline bool rows_disjoint(int64_t nt, int64_t ts, int64_t nh, int64_t hs, int64_t d) {
  int64_t n1 = nt, s1 = ts, n2 = nh, s2 = hs;
  if (n1 <= 1) { n1 = 1; s1 = 0; }
  if (n2 <= 1) { n2 = 1; s2 = 0; }
  if (n1 == 1 && n2 == 1) return true;
  if (n1 == 1) return s2 >= d;
  if (n2 == 1) return s1 >= d;
  if (s1 > s2) { const int64_t tn = n1, tsd = s1; n1 = n2; s1 = s2; n2 = tn; s2 = tsd; }
  return s1 >= d && s2 / n1 >= s1;
}

// Paged caches: page_size a multiple of 16 (a 32-key stage then spans at most two pages
// and no copy instruction straddles a page boundary).
constexpr int kMaxPageSize = 4096;
inline bool page_size_ok(int32_t ps) { return ps >= 16 && ps <= kMaxPageSize && ps % 16 == 0; }

}  // namespace

extern "C" {

const char* sink_attn_status_str(int status) {
  switch (status) {
    case SINK_ATTN_OK: return "SINK_ATTN_OK";
    case SINK_ATTN_ERR_INVALID_ARG: return "SINK_ATTN_ERR_INVALID_ARG: invalid argument";
    case SINK_ATTN_ERR_UNSUPPORTED: return "SINK_ATTN_ERR_UNSUPPORTED: unsupported size or head_dim";
    case SINK_ATTN_ERR_WORKSPACE: return "SINK_ATTN_ERR_WORKSPACE: workspace missing or too small";
    case SINK_ATTN_ERR_HIP: return "SINK_ATTN_ERR_HIP: a HIP call failed";
    case SINK_ATTN_ERR_INTERNAL: return "SINK_ATTN_ERR_INTERNAL: internal error";
    case SINK_ATTN_ERR_SCRATCH_LIMIT:
      return "SINK_ATTN_ERR_SCRATCH_LIMIT: the input needs more scratch than the no-allocation "
             "entry point holds (sink_attn_decode_noalloc_scratch_bytes)";
    default: return "unknown sink_attn status";
  }
}

int sink_attn_last_hip_error(void) { return g_last_hip_error; }

const char* sink_attn_version(void) { return "0.1.0"; }

static int prefill_common(const void* q, const void* k, const void* v, const float* sinks,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                          int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                          int64_t total_q, int64_t total_kv, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                          int32_t causal, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, void* out, float* lse,
                          const sink_attn_rope* rope, void* stream) {
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_kv || !out) return SINK_ATTN_ERR_INVALID_ARG;
  if (batch < 1 || num_q_heads < 1 || num_kv_heads < 1 || max_seqlen_q < 0 || total_q < 0 ||
      total_kv < 0 || max_seqlen_kv < 0)
    return SINK_ATTN_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return SINK_ATTN_ERR_INVALID_ARG;
  if (!scale_ok(sm_scale)) return SINK_ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SINK_ATTN_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > kMaxSplits) return SINK_ATTN_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SINK_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)64 * num_q_heads * head_dim * 2 > kMaxSpanBytes) return SINK_ATTN_ERR_UNSUPPORTED;
  if (total_kv * head_dim * 2 > kMaxSpanBytes) return SINK_ATTN_ERR_UNSUPPORTED;
  if (batch > 65535) return SINK_ATTN_ERR_UNSUPPORTED;
  sa::RopeArgs ra;
  if (make_rope(rope, head_dim, &ra) != SINK_ATTN_OK) return SINK_ATTN_ERR_INVALID_ARG;
  if (max_seqlen_q == 0 || total_q == 0) return SINK_ATTN_OK;  // nothing to compute

  sa::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.sinks = sinks;
  a.cu_q = cu_seqlens_q;
  a.cu_kv = cu_seqlens_kv;
  a.total_q = total_q;
  a.total_kv = total_kv;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.group = num_q_heads / num_kv_heads;
  a.hg = heads_per_wg(a.group);
  a.pw = 8 / a.hg;
  a.n_hgroups = a.group / a.hg;
  a.n_qtiles = (max_seqlen_q + 32 * a.pw - 1) / (32 * a.pw);
  a.causal = causal;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  const int S = prefill_splits(batch, max_seqlen_q, max_seqlen_kv, num_q_heads, num_kv_heads,
                               num_splits, resolve_cus(0));
  const int units = (max_seqlen_kv + 63) / 64;
  a.num_splits = S;
  a.split_units = S > 1 ? (units + S - 1) / S : 0x7fffffff / 64;
  if ((int64_t)a.n_qtiles * S > 65535) return SINK_ATTN_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (S == 1) {
    hipError_t e = sa::launch_prefill(a, head_dim, num_kv_heads, ra, st);
    if (e != hipSuccess) return hip_fail(e);
    return SINK_ATTN_OK;
  }
  const int64_t rows = total_q * num_q_heads;
  const size_t need = sink_attn_prefill_workspace_bytes(total_q, num_q_heads, head_dim, S);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return SINK_ATTN_ERR_WORKSPACE;
  int64_t obytes = rows * S * head_dim * 4;
  obytes = (obytes + 255) & ~(int64_t)255;
  a.part_o = (float*)workspace;
  a.part_lse = (float*)((char*)workspace + obytes);
  hipError_t e = sa::launch_prefill(a, head_dim, num_kv_heads, ra, st);
  if (e != hipSuccess) return hip_fail(e);
  e = sa::launch_merge(a.part_o, a.part_lse, nullptr, rows, S, head_dim, out, lse, st);
  if (e != hipSuccess) return hip_fail(e);
  return SINK_ATTN_OK;
}

int sink_attn_prefill(const void* q, const void* k, const void* v, const float* sinks,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t batch,
                      int32_t max_seqlen_q, int64_t total_q, int64_t total_kv,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      float sm_scale, int32_t causal, void* out, float* lse,
                      const sink_attn_rope* rope, void* stream) {
  try {
    return prefill_common(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, batch, max_seqlen_q, 0,
                          total_q, total_kv, num_q_heads, num_kv_heads, head_dim, sm_scale,
                          causal, 1, nullptr, 0, out, lse, rope, stream);
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

int32_t sink_attn_prefill_num_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t num_splits, int32_t num_cus) {
  if (batch < 1 || max_seqlen_q < 0 || max_seqlen_kv < 0 || num_q_heads < 1 ||
      num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 || num_splits < 0 ||
      num_splits > kMaxSplits || num_cus < 0)
    return 0;
  return prefill_splits(batch, max_seqlen_q, max_seqlen_kv, num_q_heads, num_kv_heads, num_splits,
                        resolve_cus(num_cus));
}

size_t sink_attn_prefill_workspace_bytes(int64_t total_q, int32_t num_q_heads, int32_t head_dim,
                                         int32_t num_splits) {
  if (total_q < 0 || num_q_heads < 1 || !dim_ok(head_dim) || num_splits < 1 ||
      num_splits > kMaxSplits)
    return 0;
  if (num_splits == 1) return 0;
  const int64_t rows = total_q * num_q_heads;
  int64_t bytes = rows * num_splits * head_dim * 4;
  bytes = (bytes + 255) & ~(int64_t)255;
  bytes += rows * num_splits * 4;
  return (size_t)((bytes + 255) & ~(int64_t)255);
}

int sink_attn_prefill_split(const void* q, const void* k, const void* v, const float* sinks,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                            int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                            int64_t total_q, int64_t total_kv, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                            int32_t causal, int32_t num_splits, void* workspace,
                            size_t workspace_bytes, void* out, float* lse,
                            const sink_attn_rope* rope, void* stream) {
  try {
    return prefill_common(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, batch, max_seqlen_q,
                          max_seqlen_kv, total_q, total_kv, num_q_heads, num_kv_heads, head_dim,
                          sm_scale, causal, num_splits, workspace, workspace_bytes, out, lse,
                          rope, stream);
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

static bool slot_args_ok(int32_t q_len, int32_t hq, int32_t hkv, int32_t d) {
  return q_len >= 1 && q_len <= 4 && hq >= 1 && hkv >= 1 && hq % hkv == 0 && dim_ok(d);
}

static bool plan_args_ok(int32_t batch, int32_t q_len, int32_t hq, int32_t hkv, int32_t d,
                         int32_t max_kv_len, int32_t num_splits, int32_t num_cus) {
  return batch >= 1 && slot_args_ok(q_len, hq, hkv, d) && max_kv_len >= 0 && num_splits >= 0 &&
         num_splits <= kMaxSplits && num_cus >= 0;
}

int32_t sink_attn_decode_chunks_per_slot(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_kv_len, int32_t num_splits,
                                         int32_t num_cus) {
  if (!plan_args_ok(batch, q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, num_splits,
                    num_cus))
    return 0;
  const SlotPlan sp = slot_plan(batch, q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len,
                                num_splits, resolve_cus(num_cus));
  return sp.cw > 1 ? sp.cw : sp.run;
}

int32_t sink_attn_decode_chunk_bounds(int32_t kv_len, int32_t q_len, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t num_splits,
                                      int32_t* bounds, int32_t capacity) {
  if (!slot_args_ok(q_len, num_q_heads, num_kv_heads, head_dim) || kv_len < 0 ||
      num_splits < 0 || num_splits > kMaxSplits || capacity < 0 || (capacity > 0 && !bounds))
    return 0;
  const int cw = sa::decode_chunk_waves(q_len * (num_q_heads / num_kv_heads), head_dim);
  const int n = sa::plan_chunks(kv_len, num_splits, cw);
  const int cl = sa::chunk_len(kv_len, n);
  for (int c = 0; c <= n && c < capacity; ++c) {
    const int64_t a = (int64_t)c * cl;
    bounds[c] = (c == n || a > kv_len) ? kv_len : (int32_t)a;
  }
  return n;
}

int32_t sink_attn_decode_num_slots(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_kv_len,
                                   int32_t num_splits, int32_t num_cus) {
  if (!plan_args_ok(batch, q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, num_splits,
                    num_cus))
    return 0;
  return slot_plan(batch, q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, num_splits,
                   resolve_cus(num_cus)).slots;
}

size_t sink_attn_decode_workspace_bytes(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_kv_len, int32_t num_splits) {
  const int64_t S = sink_attn_decode_num_slots(batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                               max_kv_len, num_splits, 0);
  if (S == 0) return 0;
  const int64_t rows = (int64_t)batch * q_len * num_q_heads;
  // the stream plan (contiguous caches) needs up to kStreamMaxSlots slots per row
  const int64_t slots =
      stream_eligible(q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, num_splits) &&
              S < kStreamMaxSlots
          ? kStreamMaxSlots
          : S;
  return partial_bytes(rows, slots, head_dim);
}

int sink_attn_decode_partial(const void* q, const void* k, const void* v, const float* sinks,
                             const int32_t* kv_indptr, int32_t batch, int32_t q_len,
                             int64_t total_kv, int32_t max_kv_len, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                             int32_t causal, int32_t num_splits, float* part_o,
                             float* part_lse, const sink_attn_rope* rope, void* stream) {
  try {
    int rc = check_decode_args(q, k, v, kv_indptr, batch, q_len, total_kv, max_kv_len,
                               num_q_heads, num_kv_heads, head_dim, sm_scale, causal, num_splits);
    if (rc != SINK_ATTN_OK) return rc;
    if (!part_o || !part_lse) return SINK_ATTN_ERR_INVALID_ARG;
    if (batch > 65535) return SINK_ATTN_ERR_UNSUPPORTED;
    sa::DecodeArgs a = decode_args(q, k, v, sinks, kv_indptr, batch, q_len, total_kv, max_kv_len,
                                   num_q_heads, num_kv_heads, head_dim, sm_scale, causal,
                                   num_splits);
    a.part_o = part_o;
    a.part_lse = part_lse;
    sa::RopeArgs ra;
    if (make_rope(rope, head_dim, &ra) != SINK_ATTN_OK) return SINK_ATTN_ERR_INVALID_ARG;
    hipError_t e = sa::launch_decode_split(a, head_dim, batch, num_kv_heads, false, nullptr, ra,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SINK_ATTN_OK;
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

int32_t sink_attn_decode_plan_kind(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int64_t total_kv,
                                   int32_t max_kv_len, int32_t num_splits, int32_t num_cus) {
  if (batch < 1 || !slot_args_ok(q_len, num_q_heads, num_kv_heads, head_dim) || total_kv < 0 ||
      max_kv_len < 0 || num_splits < 0 || num_splits > kMaxSplits || num_cus < 0)
    return -1;
  const int cus = resolve_cus(num_cus);
  if (whole_runs(batch, q_len, num_q_heads, num_kv_heads, total_kv, max_kv_len, num_splits, cus))
    return SINK_ATTN_PLAN_WHOLE_RUNS;
  if (total_kv <= INT32_MAX &&
      stream_eligible(q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, num_splits))
    return SINK_ATTN_PLAN_STREAM;
  return SINK_ATTN_PLAN_CHUNKS;
}

int32_t sink_attn_decode_stream_plan(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int64_t total_kv,
                                     int32_t max_kv_len, int32_t num_cus, int32_t* range_tokens,
                                     int32_t* ranges_per_head, int32_t* slots) {
  if (batch < 1 || !slot_args_ok(q_len, num_q_heads, num_kv_heads, head_dim) || total_kv < 0 ||
      total_kv > INT32_MAX || max_kv_len < 0 || num_cus < 0 ||
      !stream_eligible(q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, 0))
    return 0;
  const sa::StreamPlan sp = stream_plan(batch, q_len, num_q_heads, num_kv_heads, total_kv,
                                        max_kv_len, resolve_cus(num_cus));
  if (range_tokens) *range_tokens = sp.R;
  if (ranges_per_head) *ranges_per_head = sp.nph;
  if (slots) *slots = sp.smax;
  return 1;
}

// The two steps of the stream plan on their own (sink_attn_decode runs both).
static int stream_step(bool partial, const void* q, const void* k, const void* v,
                       const float* sinks, const int32_t* kv_indptr, int32_t batch,
                       int32_t q_len, int64_t total_kv, int32_t max_kv_len, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, float sm_scale, int32_t causal,
                       void* workspace, size_t workspace_bytes, void* out, float* lse,
                       const sink_attn_rope* rope, void* stream) {
  int rc = check_decode_args(q, k, v, kv_indptr, batch, q_len, total_kv, max_kv_len, num_q_heads,
                             num_kv_heads, head_dim, sm_scale, causal, 0);
  if (rc != SINK_ATTN_OK) return rc;
  if (total_kv > INT32_MAX ||
      !stream_eligible(q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, 0))
    return SINK_ATTN_ERR_UNSUPPORTED;
  if (!partial && !out) return SINK_ATTN_ERR_INVALID_ARG;
  const size_t need = sink_attn_decode_workspace_bytes(batch, q_len, num_q_heads, num_kv_heads,
                                                       head_dim, max_kv_len, 0);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return SINK_ATTN_ERR_WORKSPACE;
  sa::DecodeArgs a = decode_args(q, k, v, sinks, kv_indptr, batch, q_len, total_kv, max_kv_len,
                                 num_q_heads, num_kv_heads, head_dim, sm_scale, causal, 0);
  sa::RopeArgs ra;
  if (make_rope(rope, head_dim, &ra) != SINK_ATTN_OK) return SINK_ATTN_ERR_INVALID_ARG;
  const sa::StreamPlan sp = stream_plan(batch, q_len, num_q_heads, num_kv_heads, total_kv,
                                        max_kv_len, resolve_cus(0));
  const int64_t rows = (int64_t)batch * q_len * num_q_heads;
  a.part_o = (float*)workspace;
  a.part_lse = (float*)((char*)workspace + ((rows * sp.smax * head_dim * 4 + 255) & ~(int64_t)255));
  a.out = out;
  a.lse = lse;
  hipError_t e = partial ? sa::launch_decode_stream(a, head_dim, sp, ra, nullptr, (hipStream_t)stream)
                         : sa::launch_merge_stream(a, head_dim, sp, rows, false, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return SINK_ATTN_OK;
}

int sink_attn_decode_stream_partial(const void* q, const void* k, const void* v,
                                    const int32_t* kv_indptr, int32_t batch, int32_t q_len,
                                    int64_t total_kv, int32_t max_kv_len, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                    int32_t causal, void* workspace, size_t workspace_bytes,
                                    const sink_attn_rope* rope, void* stream) {
  try {
    return stream_step(true, q, k, v, nullptr, kv_indptr, batch, q_len, total_kv, max_kv_len,
                       num_q_heads, num_kv_heads, head_dim, sm_scale, causal, workspace,
                       workspace_bytes, nullptr, nullptr, rope, stream);
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

int sink_attn_decode_stream_merge(const float* sinks, const int32_t* kv_indptr, int32_t batch,
                                  int32_t q_len, int64_t total_kv, int32_t max_kv_len,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  const void* workspace, size_t workspace_bytes, void* out,
                                  float* lse, void* stream) {
  try {
    // q, k and v are not read by the merge; the workspace stands in for the checks
    return stream_step(false, workspace, workspace, workspace, sinks, kv_indptr, batch, q_len,
                       total_kv, max_kv_len, num_q_heads, num_kv_heads, head_dim, 1.0f, 1,
                       (void*)workspace, workspace_bytes, out, lse, nullptr, stream);
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

int sink_attn_decode(const void* q, const void* k, const void* v, const float* sinks,
                     const int32_t* kv_indptr, int32_t batch, int32_t q_len, int64_t total_kv,
                     int32_t max_kv_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, float sm_scale, int32_t causal, int32_t num_splits,
                     void* workspace, size_t workspace_bytes, void* out, float* lse,
                     const sink_attn_rope* rope, void* stream) {
  try {
    int rc = check_decode_args(q, k, v, kv_indptr, batch, q_len, total_kv, max_kv_len,
                               num_q_heads, num_kv_heads, head_dim, sm_scale, causal, num_splits);
    if (rc != SINK_ATTN_OK) return rc;
    if (!out) return SINK_ATTN_ERR_INVALID_ARG;
    if (batch > 65535) return SINK_ATTN_ERR_UNSUPPORTED;
    sa::DecodeArgs a = decode_args(q, k, v, sinks, kv_indptr, batch, q_len, total_kv, max_kv_len,
                                   num_q_heads, num_kv_heads, head_dim, sm_scale, causal,
                                   num_splits);
    sa::RopeArgs ra;
    if (make_rope(rope, head_dim, &ra) != SINK_ATTN_OK) return SINK_ATTN_ERR_INVALID_ARG;
    return run_decode(a, batch, q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len,
                      num_splits, nullptr, ra, workspace, workspace_bytes, out, lse, stream);
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

int sink_attn_decode_noalloc(const void* q, const void* k, const void* v, const float* sinks,
                             const int32_t* kv_indptr, int32_t batch, int32_t q_len,
                             int64_t total_kv, int32_t max_kv_len, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                             int32_t causal, int32_t num_splits, void* out, float* lse,
                             const sink_attn_rope* rope, void* stream) {
  try {
    int rc = check_decode_args(q, k, v, kv_indptr, batch, q_len, total_kv, max_kv_len,
                               num_q_heads, num_kv_heads, head_dim, sm_scale, causal, num_splits);
    if (rc != SINK_ATTN_OK) return rc;
    if (!out) return SINK_ATTN_ERR_INVALID_ARG;
    if (batch > 65535) return SINK_ATTN_ERR_UNSUPPORTED;
    sa::RopeArgs ra;
    if (make_rope(rope, head_dim, &ra) != SINK_ATTN_OK) return SINK_ATTN_ERR_INVALID_ARG;
    // the workspace sink_attn_decode would need must fit the scratch array, unless the
    // call takes whole-sequence runs, which write no partials
    if (!whole_runs(batch, q_len, num_q_heads, num_kv_heads, total_kv, max_kv_len, num_splits,
                    resolve_cus(0)) &&
        sink_attn_decode_workspace_bytes(batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                         max_kv_len, num_splits) > sa::kNoAllocScratchBytes)
      return SINK_ATTN_ERR_SCRATCH_LIMIT;
    void* scratch = nullptr;
    const hipError_t e = sa::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e);
    sa::DecodeArgs a = decode_args(q, k, v, sinks, kv_indptr, batch, q_len, total_kv, max_kv_len,
                                   num_q_heads, num_kv_heads, head_dim, sm_scale, causal,
                                   num_splits);
    return run_decode(a, batch, q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len,
                      num_splits, nullptr, ra, scratch, sa::kNoAllocScratchBytes, out, lse,
                      stream);
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

size_t sink_attn_decode_noalloc_scratch_bytes(void) { return sa::kNoAllocScratchBytes; }

int sink_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                           const float* sinks, const int32_t* kv_page_indptr,
                           const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
                           int32_t batch, int32_t q_len, int64_t num_page_entries,
                           int64_t num_pages, int32_t page_size, int32_t max_kv_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           float sm_scale, int32_t causal, int32_t num_splits, void* workspace,
                           size_t workspace_bytes, void* out, float* lse,
                           const sink_attn_rope* rope, void* stream) {
  try {
    if (!kv_page_indices || !kv_last_page_len) return SINK_ATTN_ERR_INVALID_ARG;
    if (num_page_entries < 0 || num_pages < 1) return SINK_ATTN_ERR_INVALID_ARG;
    if (!page_size_ok(page_size)) return SINK_ATTN_ERR_UNSUPPORTED;
    int rc = check_decode_args(q, k_cache, v_cache, kv_page_indptr, batch, q_len, 0, max_kv_len,
                               num_q_heads, num_kv_heads, head_dim, sm_scale, causal, num_splits);
    if (rc != SINK_ATTN_OK) return rc;
    if (!out) return SINK_ATTN_ERR_INVALID_ARG;
    if (batch > 65535) return SINK_ATTN_ERR_UNSUPPORTED;
    sa::DecodeArgs a = decode_args(q, k_cache, v_cache, sinks, nullptr, batch, q_len, 0, max_kv_len,
                                   num_q_heads, num_kv_heads, head_dim, sm_scale, causal,
                                   num_splits);
    a.kv_page_indptr = kv_page_indptr;
    a.kv_last_page_len = kv_last_page_len;
    a.num_page_entries = num_page_entries;
    a.num_pages = num_pages;
    a.page_size = page_size;
    sa::RopeArgs ra;
    if (make_rope(rope, head_dim, &ra) != SINK_ATTN_OK) return SINK_ATTN_ERR_INVALID_ARG;
    return run_decode(a, batch, q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len,
                      num_splits, kv_page_indices, ra, workspace, workspace_bytes, out, lse,
                      stream);
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

int sink_attn_kv_append(const void* k_new, const void* v_new, const int32_t* append_indptr,
                        const int32_t* kv_page_indptr, const int32_t* kv_page_indices,
                        const int32_t* kv_last_page_len, int32_t batch, int32_t max_append_len,
                        int64_t total_new, int64_t num_page_entries, int64_t num_pages,
                        int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                        void* k_cache, void* v_cache, const sink_attn_rope* rope,
                        void* stream) {
  try {
    if (!k_new || !v_new || !append_indptr || !kv_page_indptr || !kv_page_indices ||
        !kv_last_page_len || !k_cache || !v_cache)
      return SINK_ATTN_ERR_INVALID_ARG;
    if (batch < 1 || max_append_len < 0 || total_new < 0 || num_page_entries < 0 ||
        num_pages < 1 || num_kv_heads < 1)
      return SINK_ATTN_ERR_INVALID_ARG;
    if (!page_size_ok(page_size) || !dim_ok(head_dim)) return SINK_ATTN_ERR_UNSUPPORTED;
    if (batch > 65535) return SINK_ATTN_ERR_UNSUPPORTED;
    // the copies are 16-byte vector accesses
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
      return SINK_ATTN_ERR_INVALID_ARG;
    sa::RopeArgs ra;
    if (make_rope(rope, head_dim, &ra) != SINK_ATTN_OK) return SINK_ATTN_ERR_INVALID_ARG;
    if (max_append_len == 0 || total_new == 0) return SINK_ATTN_OK;
    sa::AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.append_indptr = append_indptr;
    a.kv_page_indptr = kv_page_indptr;
    a.kv_last_page_len = kv_last_page_len;
    a.total_new = total_new;
    a.num_page_entries = num_page_entries;
    a.num_pages = num_pages;
    a.page_size = page_size;
    a.num_kv_heads = num_kv_heads;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    hipError_t e = sa::launch_kv_append(a, head_dim, batch, max_append_len, kv_page_indices,
                                        ra, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SINK_ATTN_OK;
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

int sink_attn_rope_apply(void* x, int64_t num_tokens, int32_t num_heads, int32_t head_dim,
                         int64_t token_stride, int64_t head_stride, const int32_t* positions,
                         const sink_attn_rope* rope, void* stream) {
  try {
    if (!x || !positions || !rope || num_tokens < 0 || num_heads < 1) return SINK_ATTN_ERR_INVALID_ARG;
    if (!dim_ok(head_dim)) return SINK_ATTN_ERR_UNSUPPORTED;
    if (token_stride < 0 || head_stride < 0 || (token_stride % 8) != 0 || (head_stride % 8) != 0 ||
        !aligned16(x))
      return SINK_ATTN_ERR_INVALID_ARG;  // 16-byte vector access
    // in place: two (token, head) rows that overlap would be rotated by racing lanes
    if (!rows_disjoint(num_tokens, token_stride, num_heads, head_stride, head_dim))
      return SINK_ATTN_ERR_INVALID_ARG;
    if (num_tokens * num_heads * (head_dim / 16) > ((int64_t)1 << 38)) return SINK_ATTN_ERR_UNSUPPORTED;
    sa::RopeArgs ra;
    if (make_rope(rope, head_dim, &ra) != SINK_ATTN_OK) return SINK_ATTN_ERR_INVALID_ARG;
    if (num_tokens == 0) return SINK_ATTN_OK;
    hipError_t e = sa::launch_rope_apply(x, num_tokens, num_heads, head_dim, token_stride,
                                         head_stride, positions, ra, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SINK_ATTN_OK;
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

int sink_attn_merge(const float* part_o, const float* part_lse, const int32_t* splits_per_row,
                    int64_t rows, int32_t num_slots, int32_t head_dim, void* out, float* lse,
                    void* stream) {
  try {
    if (!part_o || !part_lse || !out || rows < 0) return SINK_ATTN_ERR_INVALID_ARG;
    if (num_slots < 1 || num_slots > kMaxSlots) return SINK_ATTN_ERR_INVALID_ARG;
    if (!dim_ok(head_dim)) return SINK_ATTN_ERR_UNSUPPORTED;
    if ((rows + 3) / 4 > 0x7fffffffLL) return SINK_ATTN_ERR_UNSUPPORTED;
    if (rows == 0) return SINK_ATTN_OK;
    hipError_t e = sa::launch_merge(part_o, part_lse, splits_per_row, rows, num_slots, head_dim,
                                    out, lse, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return SINK_ATTN_OK;
  } catch (...) {
    return SINK_ATTN_ERR_INTERNAL;
  }
}

}  // extern "C"
