// KV append into a paged HND cache for gfx950.
//
// Every decode or prefill step writes its new keys and values into the cache before
// attention reads them.  The cache is head-major inside each page ("Hosting Qwen on
// Blackwell", introduction: KV caches are kept HND so they can be split or joined by
// head), [num_pages, Hkv, page_size, D]; the new tokens arrive token-major
// [total_new, Hkv, D] as a projection writes them.  The step is a pure copy, bound by
// HBM: each 16-byte piece is read once and written once.  One workgroup takes up to
// kTok new tokens of one sequence; consecutive lanes take consecutive 16-byte pieces of
// a token, so both the read (a token's Hkv*D values are contiguous) and the write (a
// head's D values are contiguous inside a page) are whole-vector accesses.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

constexpr int kAppendThreads = 256;
constexpr int kAppendTok = 16;  // new tokens per workgroup

template <int D>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendArgs a,
                                                                   const int32_t* __restrict__ page_ids) {
  constexpr int CPR = D / 8;  // 16-byte pieces per head row
  const int b = blockIdx.y;
  const int hkv = a.num_kv_heads;
  const int ps = a.page_size;
  // new rows [r0, r1) of k_new / v_new belong to sequence b (clamped to the tensor)
  const int64_t r0 = min<int64_t>(max<int64_t>(a.append_indptr[b], 0), a.total_new);
  const int64_t r1 = min<int64_t>(max<int64_t>(a.append_indptr[b + 1], r0), a.total_new);
  const int n_new = (int)(r1 - r0);
  // the sequence's length after the append, from its page list (clamped to the list)
  const int64_t e0 = min<int64_t>(max<int64_t>(a.kv_page_indptr[b], 0), a.num_page_entries);
  const int64_t e1 = min<int64_t>(max<int64_t>(a.kv_page_indptr[b + 1], e0), a.num_page_entries);
  const int np = (int)(e1 - e0);
  const int64_t len = np > 0 ? (int64_t)(np - 1) * ps + min(max(a.kv_last_page_len[b], 1), ps) : 0;

  const int tok_begin = blockIdx.x * kAppendTok;
  const int pieces = kAppendTok * hkv * CPR;
  for (int p = threadIdx.x; p < pieces; p += kAppendThreads) {
    const int tl = p / (hkv * CPR);
    const int rem = p - tl * hkv * CPR;
    const int h = rem / CPR;
    const int cc = rem - h * CPR;
    const int i = tok_begin + tl;                 // new token i of the sequence
    if (i >= n_new) break;                        // tl grows with p
    const int64_t t = len - n_new + i;            // its position in the sequence
    if (t < 0) continue;                          // page list shorter than the append
    const int64_t slot = t / ps;                  // < np because t < len
    int64_t pid = page_ids[e0 + slot];
    pid = min<int64_t>(max<int64_t>(pid, 0), a.num_pages - 1);
    const size_t src = ((size_t)(r0 + i) * hkv + h) * D + cc * 8;
    const size_t dst = (((size_t)pid * hkv + h) * ps + (t - slot * ps)) * D + cc * 8;
    const u32x4 kx = *(const u32x4*)((const __bf16*)a.k_new + src);
    const u32x4 vx = *(const u32x4*)((const __bf16*)a.v_new + src);
    *(u32x4*)((__bf16*)a.k_cache + dst) = kx;
    *(u32x4*)((__bf16*)a.v_cache + dst) = vx;
  }
}

hipError_t launch_kv_append(const AppendArgs& a, int head_dim, int batch, int max_new,
                            const int32_t* page_ids, hipStream_t stream) {
  dim3 grid((unsigned)((max_new + kAppendTok - 1) / kAppendTok), (unsigned)batch);
  if (head_dim == 64)
    hipLaunchKernelGGL(kv_append_kernel<64>, grid, dim3(kAppendThreads), 0, stream, a, page_ids);
  else
    hipLaunchKernelGGL(kv_append_kernel<128>, grid, dim3(kAppendThreads), 0, stream, a, page_ids);
  return hipGetLastError();
}

}  // namespace sa
