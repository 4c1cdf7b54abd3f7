// KV append into a paged HND cache, with optional YaRN rotation of the keys, and the
// standalone in-place rotation, for gfx950.
//
// Every decode or prefill step writes its new keys and values into the cache before
// attention reads them.  The cache is head-major inside each page ("Hosting Qwen on
// Blackwell", introduction: KV caches are kept HND so they can be split or joined by
// head), [num_pages, Hkv, page_size, D]; the new tokens arrive token-major
// [total_new, Hkv, D] as a projection writes them.  Rotating the keys here ("GPT-OSS on
// day 0", model deltas: YaRN position encoding) costs no extra pass over them.  The step
// is a copy bound by HBM: each byte is read once and written once.  One workgroup
// takes up to kTok new tokens of one sequence; a lane takes the 16-byte piece of
// dims [8c, 8c+8) and its rotation partner [D/2 + 8c, ...) of one (token, head), so
// reads (a token's Hkv*D values are contiguous) and writes (a head's D values are
// contiguous inside a page) are whole 16-byte vectors.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

constexpr int kAppendThreads = 256;
constexpr int kAppendTok = 4;  // new tokens per workgroup

template <int D>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendArgs a,
                                                                   const int32_t* __restrict__ page_ids,
                                                                   RopeArgs rope) {
  constexpr int HP = D / 16;  // 16-byte piece pairs (dims c and c + D/2) per head row
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
  // (cos, sin) of every (token, pair) of this workgroup, shared by all KV heads
  __shared__ float2 cs[kAppendTok][D / 2];
  if (rope.enabled) {
    for (int q = threadIdx.x; q < kAppendTok * (D / 2); q += kAppendThreads) {
      const int tl = q / (D / 2);
      const int pi = q - tl * (D / 2);
      const int64_t t = len - n_new + tok_begin + tl;
      float c = 1.f, sn = 0.f;
      if (tok_begin + tl < n_new && t >= 0) rope_cos_sin(rope.freq[pi], t, c, sn);
      cs[tl][pi] = make_float2(c, sn);
    }
    __syncthreads();
  }
  const int pairs = kAppendTok * hkv * HP;
  for (int p = threadIdx.x; p < pairs; p += kAppendThreads) {
    const int tl = p / (hkv * HP);
    const int rem = p - tl * hkv * HP;
    const int h = rem / HP;
    const int c = rem - h * HP;
    const int i = tok_begin + tl;                 // new token i of the sequence
    if (i >= n_new) break;                        // tl grows with p
    const int64_t t = len - n_new + i;            // its position in the sequence
    if (t < 0) continue;                          // page list shorter than the append
    const int64_t slot = t / ps;                  // < np because t < len
    int64_t pid = page_ids[e0 + slot];
    pid = min<int64_t>(max<int64_t>(pid, 0), a.num_pages - 1);
    const size_t src = ((size_t)(r0 + i) * hkv + h) * D + c * 8;
    const size_t dst = (((size_t)pid * hkv + h) * ps + (t - slot * ps)) * D + c * 8;
    u32x4 k_lo = *(const u32x4*)((const __bf16*)a.k_new + src);
    u32x4 k_hi = *(const u32x4*)((const __bf16*)a.k_new + src + D / 2);
    const u32x4 v_lo = *(const u32x4*)((const __bf16*)a.v_new + src);
    const u32x4 v_hi = *(const u32x4*)((const __bf16*)a.v_new + src + D / 2);
    if (rope.enabled) {
      bf16x8 lo = as_bf16x8(k_lo), hi = as_bf16x8(k_hi);
      rope_rotate8_cs(lo, hi, &cs[tl][c * 8], rope.mscale);
      k_lo = __builtin_bit_cast(u32x4, lo);
      k_hi = __builtin_bit_cast(u32x4, hi);
    }
    *(u32x4*)((__bf16*)a.k_cache + dst) = k_lo;
    *(u32x4*)((__bf16*)a.k_cache + dst + D / 2) = k_hi;
    *(u32x4*)((__bf16*)a.v_cache + dst) = v_lo;
    *(u32x4*)((__bf16*)a.v_cache + dst + D / 2) = v_hi;
  }
}

hipError_t launch_kv_append(const AppendArgs& a, int head_dim, int batch, int max_new,
                            const int32_t* page_ids, const RopeArgs& rope, hipStream_t stream) {
  dim3 grid((unsigned)((max_new + kAppendTok - 1) / kAppendTok), (unsigned)batch);
  if (head_dim == 64)
    hipLaunchKernelGGL(kv_append_kernel<64>, grid, dim3(kAppendThreads), 0, stream, a, page_ids, rope);
  else
    hipLaunchKernelGGL(kv_append_kernel<128>, grid, dim3(kAppendThreads), 0, stream, a, page_ids, rope);
  return hipGetLastError();
}

// In-place YaRN rotation of x (element (t, h, d) at t*token_stride + h*head_stride + d),
// token t at positions[t]: one lane per (token, head, pair of 16-byte pieces).
template <int D>
__global__ __launch_bounds__(256) void rope_apply_kernel(__bf16* x, int64_t tokens, int heads,
                                                         int64_t token_stride, int64_t head_stride,
                                                         const int32_t* __restrict__ positions,
                                                         RopeArgs rope) {
  constexpr int HP = D / 16;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= tokens * heads * HP) return;
  const int64_t t = p / (heads * HP);
  const int rem = (int)(p - t * heads * HP);
  const int h = rem / HP;
  const int c = rem - h * HP;
  __bf16* row = x + t * token_stride + h * head_stride + c * 8;
  bf16x8 lo = as_bf16x8(*(const u32x4*)row);
  bf16x8 hi = as_bf16x8(*(const u32x4*)(row + D / 2));
  rope_rotate8(lo, hi, c * 8, positions[t], rope);
  *(u32x4*)row = __builtin_bit_cast(u32x4, lo);
  *(u32x4*)(row + D / 2) = __builtin_bit_cast(u32x4, hi);
}

hipError_t launch_rope_apply(void* x, int64_t tokens, int heads, int head_dim,
                             int64_t token_stride, int64_t head_stride,
                             const int32_t* positions, const RopeArgs& rope, hipStream_t stream) {
  const int64_t n = tokens * heads * (head_dim / 16);
  dim3 grid((unsigned)((n + 255) / 256));
  if (head_dim == 64)
    hipLaunchKernelGGL(rope_apply_kernel<64>, grid, dim3(256), 0, stream, (__bf16*)x, tokens, heads,
                       token_stride, head_stride, positions, rope);
  else
    hipLaunchKernelGGL(rope_apply_kernel<128>, grid, dim3(256), 0, stream, (__bf16*)x, tokens,
                       heads, token_stride, head_stride, positions, rope);
  return hipGetLastError();
}

}  // namespace sa
