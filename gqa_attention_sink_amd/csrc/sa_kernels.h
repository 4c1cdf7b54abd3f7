// Internal launch interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  const int32_t* cu_q;
  const int32_t* cu_kv;
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
  int32_t chunk_waves; // chunks one workgroup takes together (1: split kernel; 4 or 2: chunk-wave kernel)
  int32_t causal;
  float scale_log2;
  float* part_o;       // [rows, num_slots, D]   (split mode)
  float* part_lse;     // [rows, num_slots]
  void* out;           // [rows, D] bf16         (direct mode: one chunk per sequence)
  float* lse;          // [rows]
};

// Wavefronts per decode workgroup (16 query rows each) for M rows sharing a KV head.
inline int decode_waves(int rows) { return rows <= 16 ? 1 : (rows <= 32 ? 2 : 4); }

// Chunks per decode workgroup: with at most 16 rows per KV head the chunk-wave kernel
// takes 4 (head_dim 64) or 2 (head_dim 128) chunks per workgroup, one per wavefront.
inline int decode_chunk_waves(int rows, int head_dim) {
  return rows <= 16 ? (head_dim == 64 ? 4 : 2) : 1;
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int num_kv_heads,
                          hipStream_t stream);
hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int batch,
                               int num_kv_heads, bool direct, hipStream_t stream);
hipError_t launch_merge(const float* part_o, const float* part_lse, int64_t rows,
                        int num_slots, int head_dim, void* out, float* lse,
                        hipStream_t stream);

}  // namespace sa
