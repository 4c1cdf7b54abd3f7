// Split-KV decode and log-sum-exp merge kernels for gfx950.
//
// "GPT-OSS on day 0", "Kernels for GPT-OSS" > "Sink attention": attention is spread
// over heads and over the key axis; the online softmax keeps a running maximum m and
// sum d, starting from (m, d) = (sink, 1) so the sink is counted; when the key axis is
// split into blocks the sink enters only the first block.  Here chunk 0 starts from
// (sink, 1) and every other chunk from (-inf, 0); the merge then combines the chunks
// by their log-sum-exp.
//
// One wavefront owns one (sequence, KV head, row group, chunk).  The q_len * G query
// rows that share the KV head (GQA) are the N dimension of the MFMAs, so each K/V byte
// is read from HBM once per KV head.  Scores are computed transposed, S^T = K . Q^T,
// with v_mfma_f32_16x16x32_bf16: the accumulator of S^T leaves every lane holding
// scores of ONE query row, which is exactly the B-operand layout of the next product
// O^T = V^T . P^T, so probabilities never leave registers and the per-row softmax
// state (m, d, rescale) is lane-local.  K and V stream straight from HBM into
// registers with bounded 16-byte buffer loads; V is transposed in registers.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// Split planner: chunk count of a sequence with lk keys and the chunk's key range.
// num_splits > 0 forces that many chunks; 0 picks clamp(ceil(lk/512), 4, 16).  Every
// chunk spans the same 32-key-aligned length, so trailing chunks may be empty.
__device__ __forceinline__ int plan_chunks(int lk, int num_splits) {
  return num_splits > 0 ? num_splits : min(16, max(4, (lk + 511) >> 9));
}
__device__ __forceinline__ int chunk_len(int lk, int n) {
  int cl = lk > 0 ? (lk + n - 1) / n : 0;
  return (cl + 31) & ~31;
}

// Key of slot i (0..7) in the 32-key step for k-group cg: the S^T accumulator of key
// tile kt holds keys kt*16 + 4*cg + j (j = 0..3) for the lane's row.
__device__ __forceinline__ int slot_key(int cg, int i) {
  return (i < 4) ? (4 * cg + i) : (16 + 4 * cg + (i - 4));
}

template <int D, int NT, bool DIRECT>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;   // k-steps (32 head dims each) of S^T
  constexpr int DPL = D / 16;  // head dims per lane in a V row load = d-tiles of O^T
  constexpr int ROW_BYTES = D * 2;

  const int lane = threadIdx.x;
  const int l16 = lane & 15;
  const int cg = lane >> 4;
  const int c = blockIdx.x;
  const int g = blockIdx.y / a.row_groups;
  const int rg = blockIdx.y - g * a.row_groups;
  const int b = blockIdx.z;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int M = a.q_len * G;

  const int kv0 = a.kv_indptr[b];
  const int lk = a.kv_indptr[b + 1] - kv0;
  const int n = plan_chunks(lk, a.num_splits);
  const int cl = chunk_len(lk, n);
  const int S = a.num_slots;

  // Rows owned by this lane, one per n-tile.
  int row_t[NT], row_h[NT];
  bool row_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int R = rg * 64 + nt * 16 + l16;
    row_t[nt] = R / G;
    row_h[nt] = blockIdx.y / a.row_groups * G + (R - row_t[nt] * G);
    row_ok[nt] = R < M;
  }

  if (c >= n) {  // unused slot: no mass
    if (!DIRECT && cg == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if (row_ok[nt]) {
          const int64_t qrow = ((int64_t)b * a.q_len + row_t[nt]) * Hq + row_h[nt];
          a.part_lse[qrow * S + c] = kNegInf;
        }
    }
    return;
  }
  const int kb = min(lk, c * cl);
  const int ke = min(lk, kb + cl);

  // Q^T operands (B of S^T): lane holds Q[row][ks*32 + cg*8 .. +8].
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(
      (const __bf16*)a.q + (size_t)b * a.q_len * Hq * D, (uint32_t)(a.q_len * Hq * ROW_BYTES));
  bf16x8 qop[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // rows past M have row_t >= q_len (or a padded head): zero via the bound, or
      // explicitly for padded heads of the last token.
      const uint32_t off = (uint32_t)((row_t[nt] * Hq + row_h[nt]) * ROW_BYTES + (ks * 32 + cg * 8) * 2);
      u32x4 v = load16(qr, row_ok[nt] ? off : 0xFFFFFFF0u);
      qop[nt][ks] = as_bf16x8(v);
    }

  // Online-softmax state in log2 units; the sink joins chunk 0 only.
  float m[NT], dsum[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float sig = kNegInf;
    if (c == 0 && a.sinks != nullptr && row_ok[nt]) sig = a.sinks[row_h[nt]] * kLog2e;
    m[nt] = sig;
    dsum[nt] = (sig != kNegInf && cg == 0) ? 1.0f : 0.0f;  // counted once per row
  }
  f32x4 o[DPL][NT];
#pragma unroll
  for (int t = 0; t < DPL; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t head_base = ((size_t)g * a.total_kv + kv0) * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + head_base, (uint32_t)lk * ROW_BYTES);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + head_base, (uint32_t)lk * ROW_BYTES);
  const float sl2 = a.scale_log2;
  const int causal_first_masked = a.causal ? (lk - a.q_len + 1) : 0x7fffffff;

  for (int kbase = kb; kbase < ke; kbase += 32) {
    // ---- K operands (A of S^T): K[key = kbase + kt*16 + l16][ks*32 + cg*8 .. +8]
    u32x4 kop[2][KS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kop[kt][ks] = load16(kr, (uint32_t)(kbase + kt * 16 + l16) * ROW_BYTES + (ks * 32 + cg * 8) * 2);
    // ---- V rows: lane reads DPL head dims [DPL*l16, +DPL) of the 8 keys of its slots
    uint32_t vw[8][DPL / 2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = (uint32_t)(kbase + slot_key(cg, i)) * ROW_BYTES + l16 * DPL * 2;
      if constexpr (DPL == 8) {
        u32x4 t4 = load16(vr, off);
        vw[i][0] = t4.x; vw[i][1] = t4.y; vw[i][2] = t4.z; vw[i][3] = t4.w;
      } else {
        u32x2 t2 = load8(vr, off);
        vw[i][0] = t2.x; vw[i][1] = t2.y;
      }
    }

    // ---- S^T = K . Q^T
    f32x4 s[2][NT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16(as_bf16x8(kop[kt][ks]), qop[nt][ks], acc);
        s[kt][nt] = acc;
      }

    // ---- mask: keys past the chunk end, and (causal) keys after the row's position.
    if (kbase + 32 > ke || kbase + 32 > causal_first_masked) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int lim = a.causal ? min(ke - 1, lk - a.q_len + row_t[nt]) : ke - 1;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kbase + kt * 16 + 4 * cg + j;
            s[kt][nt][j] = (key <= lim) ? s[kt][nt][j] : kNegInf;
          }
      }
    }

    // ---- online softmax (exp2 domain) and P^T operands
    bf16x8 pop[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = fmaxf(fmaxf(fmaxf(s[0][nt][0], s[0][nt][1]), fmaxf(s[0][nt][2], s[0][nt][3])),
                       fmaxf(fmaxf(s[1][nt][0], s[1][nt][1]), fmaxf(s[1][nt][2], s[1][nt][3])));
      mx = wave_xor_max(mx, 16);
      mx = wave_xor_max(mx, 32);
      const float mnew = fmaxf(m[nt], mx * sl2);
      const bool dead = (mnew == kNegInf);
      const float alpha = dead ? 1.0f : fast_exp2(m[nt] - mnew);
      const float msub = dead ? 0.0f : mnew;
      float p[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = fast_exp2(__builtin_fmaf(s[0][nt][j], sl2, -msub));
        p[4 + j] = fast_exp2(__builtin_fmaf(s[1][nt][j], sl2, -msub));
      }
      float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      dsum[nt] = __builtin_fmaf(dsum[nt], alpha, ps);
      m[nt] = mnew;
#pragma unroll
      for (int t = 0; t < DPL; ++t) o[t][nt] *= alpha;
      u32x4 pk;
      pk.x = pack_bf16x2(p[0], p[1]);
      pk.y = pack_bf16x2(p[2], p[3]);
      pk.z = pack_bf16x2(p[4], p[5]);
      pk.w = pack_bf16x2(p[6], p[7]);
      pop[nt] = as_bf16x8(pk);
    }

    // ---- O^T += V^T . P^T ; V^T operand of d-tile t holds V[slot key i][DPL*l16 + t]
#pragma unroll
    for (int t = 0; t < DPL; ++t) {
      u32x4 va;
      const int w = t >> 1;
      if ((t & 1) == 0) {
        va.x = lo_lo(vw[0][w], vw[1][w]);
        va.y = lo_lo(vw[2][w], vw[3][w]);
        va.z = lo_lo(vw[4][w], vw[5][w]);
        va.w = lo_lo(vw[6][w], vw[7][w]);
      } else {
        va.x = hi_hi(vw[0][w], vw[1][w]);
        va.y = hi_hi(vw[2][w], vw[3][w]);
        va.z = hi_hi(vw[4][w], vw[5][w]);
        va.w = hi_hi(vw[6][w], vw[7][w]);
      }
      const bf16x8 vop = as_bf16x8(va);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[t][nt] = mfma16(vop, pop[nt], o[t][nt]);
    }
  }

  // ---- epilogue: lane holds head dims [4*cg*DPL, 4*cg*DPL + 4*DPL) of its row;
  // O^T accumulator element (t, j) is head dim DPL*(4*cg + j) + t.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float dr = wave_xor_sum(dsum[nt], 16);
    dr = wave_xor_sum(dr, 32);
    const float inv = dr > 0.f ? 1.0f / dr : 0.f;
    const float lse_nat = dr > 0.f ? (m[nt] + __builtin_log2f(dr)) * kLn2 : kNegInf;
    if (!row_ok[nt]) continue;
    const int64_t qrow = ((int64_t)b * a.q_len + row_t[nt]) * Hq + row_h[nt];
    float vals[4 * DPL];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < DPL; ++t) vals[j * DPL + t] = o[t][nt][j] * inv;
    const int d0 = 4 * cg * DPL;
    if constexpr (DIRECT) {
      uint32_t* dst = (uint32_t*)((__bf16*)a.out + qrow * D + d0);
#pragma unroll
      for (int e = 0; e < 4 * DPL; e += 8) {
        u32x4 w4;
        w4.x = pack_bf16x2(vals[e + 0], vals[e + 1]);
        w4.y = pack_bf16x2(vals[e + 2], vals[e + 3]);
        w4.z = pack_bf16x2(vals[e + 4], vals[e + 5]);
        w4.w = pack_bf16x2(vals[e + 6], vals[e + 7]);
        *(u32x4*)(dst + e / 2) = w4;
      }
      if (cg == 0 && a.lse != nullptr) a.lse[qrow] = lse_nat;
    } else {
      float* dst = a.part_o + (qrow * S + c) * D + d0;
#pragma unroll
      for (int e = 0; e < 4 * DPL; e += 4)
        *(f32x4*)(dst + e) = f32x4{vals[e], vals[e + 1], vals[e + 2], vals[e + 3]};
      if (cg == 0) a.part_lse[qrow * S + c] = lse_nat;
    }
  }
}

// One wavefront per row: weights from the partial lse, then the weighted sum of the
// partial outputs.  Slots with lse = -inf are skipped (their output is not read).
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    int64_t rows, int S, __bf16* out,
                                                    float* lse) {
  constexpr int E = D / 64;  // head dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const float* pl = part_lse + row * S;
  float mx = kNegInf;
  for (int c = lane; c < S; c += 64) mx = fmaxf(mx, pl[c]);
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) mx = wave_xor_max(mx, msk);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (mx != kNegInf) {
    const float* po = part_o + row * S * D + lane * E;
    for (int c = 0; c < S; ++c) {
      const float w = __expf(pl[c] - mx);
      if (w == 0.f) continue;
      wsum += w;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(w, po[(size_t)c * D + e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  __bf16* dst = out + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = (__bf16)(acc[e] * inv);
  if (lane == 0 && lse != nullptr) lse[row] = wsum > 0.f ? mx + __logf(wsum) : kNegInf;
}

template <int D, bool DIRECT>
static hipError_t launch_decode_d(const DecodeArgs& a, int nt, dim3 grid, hipStream_t st) {
  switch (nt) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, DIRECT>), grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, DIRECT>), grid, dim3(64), 0, st, a); break;
    case 3: hipLaunchKernelGGL((decode_split_kernel<D, 3, DIRECT>), grid, dim3(64), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_split_kernel<D, 4, DIRECT>), grid, dim3(64), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int batch, int num_kv_heads,
                               bool direct, hipStream_t stream) {
  const int M = a.q_len * a.group;
  const int nt = a.row_groups > 1 ? 4 : (M + 15) / 16;
  dim3 grid(a.num_slots, num_kv_heads * a.row_groups, batch);
  if (head_dim == 64)
    return direct ? launch_decode_d<64, true>(a, nt, grid, stream)
                  : launch_decode_d<64, false>(a, nt, grid, stream);
  return direct ? launch_decode_d<128, true>(a, nt, grid, stream)
                : launch_decode_d<128, false>(a, nt, grid, stream);
}

hipError_t launch_merge(const float* part_o, const float* part_lse, int64_t rows, int num_slots,
                        int head_dim, void* out, float* lse, hipStream_t stream) {
  dim3 grid((unsigned)((rows + 3) / 4));
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, stream, part_o, part_lse, rows,
                       num_slots, (__bf16*)out, lse);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, part_o, part_lse, rows,
                       num_slots, (__bf16*)out, lse);
  return hipGetLastError();
}

}  // namespace sa
