// Device helpers shared by the decode kernels (split, chunk-wave and stream).
#pragma once

#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// Sequence b's token range, clamped to the token axis so that no copy can leave K or V
// even when the index array is malformed.
__device__ __forceinline__ int seq_begin(const DecodeArgs& a, int b) {
  return (int)min<int64_t>(max(a.kv_indptr[b], 0), a.total_kv);
}
__device__ __forceinline__ int seq_end(const DecodeArgs& a, int b) {
  return (int)min<int64_t>(max(a.kv_indptr[b + 1], seq_begin(a, b)), a.total_kv);
}
// Paged sequence b: its first page-list entry and its length, clamped so that every
// page-list read stays inside the list.
__device__ __forceinline__ int page_begin(const DecodeArgs& a, int b) {
  return (int)min<int64_t>(max(a.kv_page_indptr[b], 0), a.num_page_entries);
}
__device__ __forceinline__ int paged_len(const DecodeArgs& a, int b, int e0) {
  const int np = (int)min<int64_t>(max(a.kv_page_indptr[b + 1], e0), a.num_page_entries) - e0;
  if (np == 0) return 0;
  const int last = min(max(a.kv_last_page_len[b], 1), a.page_size);
  return (int)min<int64_t>((int64_t)(np - 1) * a.page_size + last, 1 << 24);
}

// Key of slot i (0..7) in the 32-key step for k-group cg: the S^T accumulator of key
// tile kt holds keys kt*16 + 4*cg + j (j = 0..3) for the lane's row.
__device__ __forceinline__ int slot_key(int cg, int i) {
  return (i < 4) ? (4 * cg + i) : (16 + 4 * cg + (i - 4));
}

// XOR swizzle of 16-byte chunks inside a K row in LDS: the 16 rows read by one MFMA
// operand load land in distinct banks.
template <int D>
__device__ __forceinline__ int dswz(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}

}  // namespace sa
