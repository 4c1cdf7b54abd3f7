// Decode chunk plan, shared by the host (plan queries, workspace sizing) and the
// kernels (each workgroup derives its chunk from its sequence's length, so no plan is
// copied to the device and nothing synchronises).
//
// "GPT-OSS on day 0", "Kernels for GPT-OSS" > "Sink attention": attention is spread
// over heads and over the key axis in blocks; the pages fix no block size.  The plan
// here: num_splits > 0 forces that many chunks per sequence; 0 picks ceil(Lk/256)
// rounded up to a multiple of cw (the chunks one workgroup takes together) and clamped
// to [4, 16].  Every chunk spans the same 32-key-aligned length, so trailing chunks may
// be empty.
#pragma once

#if defined(__HIPCC__)
#define SA_HD __host__ __device__
#else
#define SA_HD
#endif

namespace sa {

SA_HD inline int plan_chunks(int lk, int num_splits, int cw) {
  if (num_splits > 0) return num_splits;
  const int n = (((lk + 255) >> 8) + cw - 1) / cw * cw;
  return n < 4 ? 4 : (n > 16 ? 16 : n);
}

// Keys per chunk of a sequence with lk keys in n chunks: ceil(lk/n) rounded up to 32.
SA_HD inline int chunk_len(int lk, int n) {
  const int cl = lk > 0 ? (lk + n - 1) / n : 0;
  return (cl + 31) & ~31;
}

}  // namespace sa
