// Launch interface between the C ABI (api.cpp, plain host C++) and the kernel files.
// Host-only: the argument structs, the launch functions the kernel files define, and
// the per-device runtime queries.  Nothing here needs the device compiler, so the host
// validation and planning code also builds with a plain C++ compiler (for the
// sanitizer build, with a stub of the launch layer).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

constexpr int kMaxRopePairs = 64;  // head_dim <= 128

// YaRN rotation table, filled on the host in double precision.
struct RopeArgs {
  double freq[kMaxRopePairs];  // radians per position of pair i (after YaRN interpolation)
  float mscale;                // attention temperature factor, applied to q and to k
  int32_t enabled;             // 0: no rotation
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  int64_t total_q;
  int64_t total_kv;
  int32_t batch;
  int32_t num_q_heads;
  int32_t group;      // query heads per KV head
  int32_t hg;         // query heads per workgroup (divides group, <= 4)
  int32_t pw;         // 32-position blocks per workgroup (= 8 / hg)
  int32_t n_hgroups;  // group / hg
  int32_t n_qtiles;   // ceil(max_seqlen_q / (32 * pw))
  int32_t causal;
  float scale_log2;   // sm_scale * log2(e)
  void* out;
  float* lse;
  // Split along the key axis (num_splits > 1): split s takes key units
  // [s*split_units, (s+1)*split_units) and writes a partial into part_o/part_lse
  // ([total_q*Hq, num_splits, D] and [total_q*Hq, num_splits], fp32) for the merge.
  int32_t num_splits;
  int32_t split_units;
  float* part_o;
  float* part_lse;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  const int32_t* kv_indptr;
  int64_t total_kv;
  int32_t q_len;
  int32_t num_q_heads;
  int32_t group;       // query heads per KV head
  int32_t row_groups;  // ceil(q_len * group / (16 * decode_waves(q_len * group)))
  int32_t num_splits;  // 0 = planner
  int32_t num_slots;   // partial slots per row (chunk groups of chunk_waves chunks)
  int32_t chunk_waves; // chunks one workgroup takes in parallel (4 or 2: chunk-wave kernel; 1: split kernel)
  int32_t chunk_run;   // split kernel: consecutive chunks one workgroup takes in turn (a slot)
  int32_t causal;
  float scale_log2;
  float* part_o;       // [rows, num_slots, D]   (split mode)
  float* part_lse;     // [rows, num_slots]
  void* out;           // [rows, D] bf16         (direct mode: one chunk per sequence)
  float* lse;          // [rows]
  // Paged KV (paged kernels only): k and v are caches [num_pages, Hkv, page_size, D];
  // sequence b owns page-list entries [kv_page_indptr[b], kv_page_indptr[b+1]) of the
  // page ids (passed to the kernels separately) and fills its last page up to
  // kv_last_page_len[b].
  const int32_t* kv_page_indptr;
  const int32_t* kv_last_page_len;
  int64_t num_page_entries;
  int64_t num_pages;
  int32_t page_size;   // a multiple of 16
  int32_t num_kv_heads;
};

// KV append into a paged cache [num_pages, Hkv, page_size, D] (bf16).
struct AppendArgs {
  const void* k_new;             // [total_new, Hkv, D]
  const void* v_new;
  const int32_t* append_indptr;  // [B+1] rows of k_new/v_new per sequence
  const int32_t* kv_page_indptr; // [B+1] (after the append)
  const int32_t* kv_last_page_len;
  int64_t total_new;
  int64_t num_page_entries;
  int64_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  void* k_cache;
  void* v_cache;
};

// Stream decode plan: the token axis of each KV head is cut into ranges of R tokens (a
// multiple of 32), nph ranges per head, one wavefront (or one workgroup) each; a row's
// partials occupy smax slots ([rows, smax, D] outputs then [rows, smax] lse).
constexpr int kStreamMaxSlots = 17;  // partial slots a row can need under the stream plan
struct StreamPlan {
  int32_t R;
  int32_t nph;
  int32_t smax;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t waves;  // 1: independent wavefronts, one range each (<= 16 rows); 2 or 4:
                  // one workgroup of that many wavefronts per range (<= 32 / <= 64 rows)
};

// Wavefronts per decode workgroup (16 query rows each) for M rows sharing a KV head.
inline int decode_waves(int rows) { return rows <= 16 ? 1 : (rows <= 32 ? 2 : 4); }

// Chunks per decode workgroup: with at most 16 rows per KV head the chunk-wave kernel
// takes 4 (head_dim 64) or 2 (head_dim 128) chunks per workgroup, one per wavefront.
inline int decode_chunk_waves(int rows, int head_dim) {
  return rows <= 16 ? (head_dim == 64 ? 4 : 2) : 1;
}

// Compute units of the current device, read once per device (0 if no device is
// current or the query fails).
int device_cu_count();

// The scratch array of the no-allocation decode entry point on the current device: its
// device address, looked up once per device (the first call with that device current).
// Returns the HIP error of reading the current device or of that lookup.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

// rope: YaRN rotation of Q (and of new K in the append) at each row's position;
// rope.enabled == 0 leaves them unrotated.
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int num_kv_heads,
                          const RopeArgs& rope, hipStream_t stream);
// page_ids: the page list of a paged cache (nullptr for contiguous HND K/V).
hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int batch,
                               int num_kv_heads, bool direct, const int32_t* page_ids,
                               const RopeArgs& rope, hipStream_t stream);
hipError_t launch_kv_append(const AppendArgs& a, int head_dim, int batch, int max_new,
                            const int32_t* page_ids, const RopeArgs& rope, hipStream_t stream);
// In-place rotation of x: element (t, h, d) at x + t*token_stride + h*head_stride + d.
hipError_t launch_rope_apply(void* x, int64_t tokens, int heads, int head_dim,
                             int64_t token_stride, int64_t head_stride,
                             const int32_t* positions, const RopeArgs& rope, hipStream_t stream);
// Stream decode (contiguous K/V, q_len * G <= 64): partials into a.part_o / a.part_lse,
// then their merge with the sinks into a.out / a.lse.
// page_ids: NULL for the contiguous cache, else the page list of a paged cache (the plan
// must then be a single-wavefront plan over the page-list axis).
hipError_t launch_decode_stream(const DecodeArgs& a, int head_dim, const StreamPlan& sp,
                                const RopeArgs& rope, const int32_t* page_ids, hipStream_t stream);
hipError_t launch_merge_stream(const DecodeArgs& a, int head_dim, const StreamPlan& sp,
                               int64_t rows, bool paged, hipStream_t stream);
// counts: valid slots per row (nullptr = all num_slots)
hipError_t launch_merge(const float* part_o, const float* part_lse, const int32_t* counts,
                        int64_t rows, int num_slots, int head_dim, void* out, float* lse,
                        hipStream_t stream);

}  // namespace sa
