// Causal variable-length prefill kernel for gfx950.
//
// "GPT-OSS on day 0", "Kernels for GPT-OSS" > "Sink attention": softmax(q.K^T*scale
// + sink).V with the online (max-subtracted) softmax started from (m, d) = (sink, 1);
// the whole key range of a row is handled by one wavefront (or, when the key axis is
// split for parallelism, by one wavefront per split, the sink entering split 0 only and
// the splits merged by log-sum-exp afterwards), so the sink is counted exactly once.
//
// Work unit (one workgroup of 8 wavefronts, two per SIMD): one sequence, 32*pw query
// positions and hg query heads that share one KV head (GQA), hg*pw = 8.  Each
// wavefront owns 32 query rows of one head (one 32-row MFMA column tile); the two
// wavefronts of a SIMD overlap one's exponentials with the other's MFMAs.
//
// Scores are computed transposed, S^T = K . Q^T (v_mfma_f32_32x32x16_bf16), so each
// lane holds scores of one query row: the P^T accumulator is directly the B operand
// of O^T = V^T . P^T and the per-row softmax state is lane-local (one swap of the
// wavefront's 32-lane halves per row max).
//
// Keys are processed in units of 64.  K/V units stream through a 4-slot LDS ring with
// asynchronous buffer->LDS copies issued 3 units ahead (prefill_kernel, head_dim 64; the
// head_dim 128 kernel, prefill_pp_kernel below, alternates the two wavefronts of each
// SIMD between MFMA and exponential phases).  The running maximum is
// raised only when a row's maximum grows by more than 2^8 (exact: numerator and
// denominator share the stale maximum), so O is rarely rescaled.  Workgroups are
// dispatched heaviest causal tile first.
#include <type_traits>

#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

template <int D>
struct PrefillCfg {
  static constexpr int UNIT = 64;              // keys per pipeline unit
  static constexpr int KS = D / 16;            // k-steps of S^T (16 head dims each)
  static constexpr int DT = D / 32;            // d-tiles of O^T (32 head dims each)
  static constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
  static constexpr int ROW = D * 2;            // bytes per K/V row
  static constexpr int UB = UNIT * ROW;        // bytes of K (or V) per unit
  static constexpr int NS = 4;                 // LDS ring slots
  static constexpr int PD = NS - 1;            // units issued ahead of use
  static constexpr int NT = 512;               // threads per workgroup (8 wavefronts)
  static constexpr int NDMA = UB / (NT * 16);  // copies per thread per tensor per unit
  static_assert(NDMA * NT * 16 == UB, "unit must split evenly over the workgroup");
};

// XOR swizzle of 16-byte chunks inside a K row so that the 32 rows read by one MFMA
// operand load fall into distinct LDS banks.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}

// XOR swizzle of 16-byte chunks inside a V row for the transposing reads.  The LDS
// serves 256 bytes (64 banks) per cycle, i.e. 32 lanes of an 8-byte read; those 32 lanes
// read four consecutive rows (4*cg .. +3, plus a multiple of 8) at four consecutive
// 16-byte chunks 4t .. 4t+3.  D=128 (one row per 256 bytes): XOR by 4*(row%4) spreads
// the four rows over disjoint chunk quads.  D=64 (two rows per 256 bytes, rows of equal
// parity sharing banks): XOR by 4 on rows 2 and 3 separates row 0 from 2 and 1 from 3.
// (A swizzle by row%8 left 2-way (D=64) and 4-way (D=128) bank conflicts.)
template <int D>
__device__ __forceinline__ int vswz(int row) {
  if constexpr (D == 128) return (row & 3) << 2;
  else return (row & 2) << 1;
}

template <int D>
__global__ __launch_bounds__(512, 1) void prefill_kernel(PrefillArgs a, RopeArgs rope) {
  using C = PrefillCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char ring[C::NS][2][C::UB];

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int cg = lane >> 5;
  const int Hq = a.num_q_heads;

  // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2); when the
  // head-group axis is a multiple of 8, give each XCD a contiguous range of head groups
  // so the K/V of a KV head stays in few L2s.
  int hgi = blockIdx.x;
  if ((gridDim.x & 7) == 0) hgi = (hgi & 7) * (int)(gridDim.x >> 3) + (hgi >> 3);
  const int g = hgi / a.n_hgroups;
  const int hgrp = hgi - g * a.n_hgroups;
  const int b = blockIdx.y;
  const int S = a.num_splits;
  const int qt = a.n_qtiles - 1 - (int)blockIdx.z / S;  // heaviest tiles dispatched first
  const int split = (int)blockIdx.z % S;

  // sequence bounds, clamped to the token axes so that no access leaves the tensors
  const int q0 = (int)min<int64_t>(max(a.cu_q[b], 0), a.total_q);
  const int lq = (int)min<int64_t>(max(a.cu_q[b + 1], q0), a.total_q) - q0;
  const int kv0 = (int)min<int64_t>(max(a.cu_kv[b], 0), a.total_kv);
  const int lk = (int)min<int64_t>(max(a.cu_kv[b + 1], kv0), a.total_kv) - kv0;
  const int wg_p0 = qt * 32 * a.pw;
  if (wg_p0 >= lq) return;
  const int off = lk - lq;  // bottom-right causal alignment

  // wavefront -> (query head, block of 32 query positions)
  const bool active = (wave / a.hg) < a.pw;
  const int h = g * a.group + hgrp * a.hg + (wave % a.hg);
  const int p0 = wg_p0 + (wave / a.hg) * 32;
  const bool has_rows = active && p0 < lq;

  int kend_wg = a.causal ? min(lk, wg_p0 + 32 * a.pw + off) : lk;
  kend_wg = max(kend_wg, 0);
  // this split's key units [u0, u1) of the workgroup's causal range (one split: all)
  const int u0 = split * a.split_units;
  const int n_wg = min((kend_wg + C::UNIT - 1) / C::UNIT, u0 + a.split_units);
  int kend_w = a.causal ? min(lk, p0 + 32 + off) : lk;
  kend_w = has_rows ? max(kend_w, 0) : 0;
  const int n_w = min((kend_w + C::UNIT - 1) / C::UNIT, n_wg);
  const int pos = p0 + l32;
  const bool split_out = S > 1;
  if (u0 >= n_wg && split > 0) {  // nothing of this split is visible: an empty partial
    if (has_rows && pos < lq && cg == 0)
      a.part_lse[((size_t)(q0 + pos) * Hq + h) * S + split] = kNegInf;
    return;
  }

  // ---- K/V of this (KV head, sequence) through bounded descriptors: units past the
  // sequence end read zeros and cost no memory traffic.
  const size_t head_base = ((size_t)g * a.total_kv + kv0) * D;
  const uint32_t kvbytes = (uint32_t)max(lk, 0) * C::ROW;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + head_base, kvbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + head_base, kvbytes);
  auto issue = [&](int u) {
    unsigned char* kbuf = ring[u % C::NS][0];
    unsigned char* vbuf = ring[u % C::NS][1];
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) {
      const int blk = i * (C::NT / 64) + wave;
      const int p = blk * 64 + lane;
      const int row = p / C::CPR;
      const int cc = p - row * C::CPR;
      const uint32_t rb = (uint32_t)(u * C::UNIT + row) * C::ROW;
      dma16(kr, rb + (uint32_t)((cc ^ kswz<D>(row)) * 16), kbuf + blk * 1024);
      dma16(vr, rb + (uint32_t)((cc ^ vswz<D>(row)) * 16), vbuf + blk * 1024);
    }
  };

  // ---- Q^T operands: lane holds Q[p0 + l32][h][ks*16 + cg*8 .. +8]
  bf16x8 qop[C::KS];
  {
    const int nrows = max(0, min(32, lq - p0));
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc((const __bf16*)a.q + ((size_t)(q0 + max(p0, 0)) * Hq) * D,
                  has_rows ? (uint32_t)(nrows * Hq * C::ROW) : 0u);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const uint32_t o = (uint32_t)((l32 * Hq + h) * C::ROW + (ks * 16 + cg * 8) * 2);
      qop[ks] = as_bf16x8(load16(qr, o));
    }
  }
  // YaRN rotation of query position p0 + l32 at its key-axis position (bottom-right
  // alignment): pair (i, i + D/2) sits in qop[ks] and qop[ks + KS/2] of the same lane.
  if (rope.enabled) {
    const int64_t pos = (int64_t)off + p0 + l32;
#pragma unroll
    for (int ks = 0; ks < C::KS / 2; ++ks)
      rope_rotate8(qop[ks], qop[ks + C::KS / 2], ks * 16 + cg * 8, pos, rope);
  }

  // ---- online-softmax state (log2 units), started from the head's sink
  // the sink enters the first split only ("Sink attention": first block only)
  const float sig = (a.sinks != nullptr && has_rows && split == 0) ? a.sinks[h] * kLog2e : kNegInf;
  float m = sig;
  float dsum = (sig != kNegInf && cg == 0) ? 1.0f : 0.0f;  // counted once per row
  f32x16 o[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[t][j] = 0.f;
  const float sl2 = a.scale_log2;
  const int lim = a.causal ? min(lk - 1, pos + off) : lk - 1;

  // Per-lane part of the transposing V reads: lane p of each 16-lane group supplies
  // row 4*cg + p/4 (+ a multiple of 8, which leaves the swizzle unchanged) at head dims
  // 32*t + 16*((lane/16)%2) + 4*(p%4).
  uint32_t v_lane_off[C::DT];
  {
    const int p16 = lane & 15;
    const int lrow = 4 * cg + (p16 >> 2);
    const int dsub = 16 * ((lane >> 4) & 1) + 4 * (p16 & 3);
#pragma unroll
    for (int t = 0; t < C::DT; ++t) {
      const int d = 32 * t + dsub;
      v_lane_off[t] = (uint32_t)(lrow * C::ROW + (((d >> 3) ^ vswz<D>(lrow)) * 16) + (d & 7) * 2);
    }
  }

#pragma unroll
  for (int i = 0; i < C::PD; ++i) issue(u0 + i);

  for (int u = u0; u < n_wg; ++u) {
    // unit u has landed once only the PD-1 units issued after it are pending
    wait_vmcnt<(C::PD - 1) * 2 * C::NDMA>();
    stage_barrier();
    issue(u + C::PD);  // refills the slot of unit u-1, which every wavefront finished
    if (u < n_w) {
      const unsigned char* kbuf = ring[u % C::NS][0];
      const unsigned char* vbuf = ring[u % C::NS][1];
      const int kbase = u * C::UNIT;
      // ---- S^T: element j of key tile kt is key kbase + kt*32 + 8*(j/4) + 4*cg + j%4
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kt][j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int cc = ks * 2 + cg;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int row = kt * 32 + l32;
          const bf16x8 ka =
              as_bf16x8(*(const u32x4*)(kbuf + row * C::ROW + ((cc ^ kswz<D>(row)) * 16)));
          s[kt] = mfma32(ka, qop[ks], s[kt]);
        }
      }
      // ---- mask only where the unit crosses the diagonal or the sequence end
      if (kbase + C::UNIT > lk || (a.causal && kbase + C::UNIT - 1 > p0 + off)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = kbase + kt * 32 + 8 * (j >> 2) + 4 * cg + (j & 3);
            s[kt][j] = (key <= lim) ? s[kt][j] : kNegInf;
          }
      }
      // ---- probabilities as bf16 B operands against the running max, with fp32 sums of
      // each group of 8.  The running max is raised only when the row max exceeds it by
      // more than 2^8; if no group sum exceeds 128 no probability does, so the row max is
      // only computed when some sum is larger (or overflowed), or while the running max
      // is still -inf (a -inf sink before the row's first finite score).
      bf16x8 pk[2][2];  // [kt][kk]
      float gs[2][2];
      auto probs = [&]() __attribute__((always_inline)) {
        const float msub = (m == kNegInf) ? 0.0f : m;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            float p[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) p[i] = fast_exp2(__builtin_fmaf(s[kt][kk * 8 + i], sl2, -msub));
            u32x4 w4;
            w4.x = pack_bf16x2(p[0], p[1]);
            w4.y = pack_bf16x2(p[2], p[3]);
            w4.z = pack_bf16x2(p[4], p[5]);
            w4.w = pack_bf16x2(p[6], p[7]);
            gs[kt][kk] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            pk[kt][kk] = as_bf16x8(w4);
          }
      };
      probs();
      const float gmax = fmaxf(fmaxf(gs[0][0], gs[0][1]), fmaxf(gs[1][0], gs[1][1]));
      if (__any(!(gmax <= 128.0f) || m == kNegInf)) {
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int j = 2; j < 16; j += 2) mx = fmaxf(fmaxf(mx, s[0][j]), s[0][j + 1]);
#pragma unroll
        for (int j = 0; j < 16; j += 2) mx = fmaxf(fmaxf(mx, s[1][j]), s[1][j + 1]);
        const float mxs = half_swap_max(mx) * sl2;
        if (__any(mxs > m + 8.0f)) {
          const float mnew = fmaxf(m, mxs);
          const float alpha = (mnew == kNegInf) ? 1.0f : fast_exp2(m - mnew);
          dsum *= alpha;
#pragma unroll
          for (int t = 0; t < C::DT; ++t) o[t] *= alpha;
          m = mnew;
          probs();
        }
      }
      dsum += gs[0][0];
      dsum += gs[0][1];
      dsum += gs[1][0];
      dsum += gs[1][1];
      // ---- O^T += V^T . P^T.  Slot i of 16-key step (kt, kk) for k-group cg is key
      // kt*32 + 16*kk + 8*(i/4) + 4*cg + i%4, read transposed from LDS: for half h of
      // the slots, lane p of each 16-lane group supplies key row
      // kt*32 + 16*kk + 8*h + 4*cg + p/4 at head dims 32*t + 16*((lane/16)%2) + 4*(p%4),
      // so lane l receives V[slot keys][32*t + l%32] (d-tile t, MFMA row l%32).
      uint32_t vaddr[C::DT];
#pragma unroll
      for (int t = 0; t < C::DT; ++t) vaddr[t] = lds_addr(vbuf) + v_lane_off[t];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        u32x2 vr2[2][C::DT][2];  // [kk][t][h]
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int t = 0; t < C::DT; ++t)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              vr2[kk][t][hh] = ds_read_tr16(vaddr[t], (kt * 32 + 16 * kk + 8 * hh) * C::ROW);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if constexpr (C::DT == 4) {
            lds_wait(vr2[kk][0][0], vr2[kk][0][1], vr2[kk][1][0], vr2[kk][1][1]);
            lds_wait(vr2[kk][2][0], vr2[kk][2][1], vr2[kk][3][0], vr2[kk][3][1]);
          } else {
            lds_wait(vr2[kk][0][0], vr2[kk][0][1], vr2[kk][1][0], vr2[kk][1][1]);
          }
#pragma unroll
          for (int t = 0; t < C::DT; ++t) {
            const u32x4 va = {vr2[kk][t][0].x, vr2[kk][t][0].y, vr2[kk][t][1].x, vr2[kk][t][1].y};
            o[t] = mfma32(as_bf16x8(va), pk[kt][kk], o[t]);
          }
        }
      }
    }
  }
  wait_vmcnt<0>();  // no copy may land after the workgroup's LDS is released

  if (!has_rows || pos >= lq) return;
  // ---- epilogue.  O^T element (t, j) is head dim 32*t + 8*(j/4) + 4*cg + j%4 of
  // query position pos: four runs of 4 consecutive head dims per d-tile.
  const float dr = half_swap_sum(dsum);
  const float inv = dr > 0.f ? 1.0f / dr : 0.f;
  const size_t orow = (size_t)(q0 + pos) * Hq + h;
  if (split_out) {  // fp32 partial of this split for the log-sum-exp merge
    float* pdst = a.part_o + (orow * S + split) * D;
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4*)(pdst + 32 * t + 8 * q4 + 4 * cg) =
            f32x4{o[t][q4 * 4 + 0] * inv, o[t][q4 * 4 + 1] * inv, o[t][q4 * 4 + 2] * inv,
                  o[t][q4 * 4 + 3] * inv};
    if (cg == 0) a.part_lse[orow * S + split] = dr > 0.f ? (m + __builtin_log2f(dr)) * kLn2 : kNegInf;
    return;
  }
  __bf16* dst = (__bf16*)a.out + orow * D;
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 w2;
      w2.x = pack_bf16x2(o[t][q4 * 4 + 0] * inv, o[t][q4 * 4 + 1] * inv);
      w2.y = pack_bf16x2(o[t][q4 * 4 + 2] * inv, o[t][q4 * 4 + 3] * inv);
      *(u32x2*)(dst + 32 * t + 8 * q4 + 4 * cg) = w2;
    }
  if (cg == 0 && a.lse != nullptr)
    a.lse[orow] = dr > 0.f ? (m + __builtin_log2f(dr)) * kLn2 : kNegInf;
}

// Scheduling hints for a matrix phase: after the first LA operand reads, one MFMA and
// the reads LA MFMAs ahead of it alternate (K reads: one per MFMA for the first NQ;
// transposing V reads: two per MFMA after them).
template <int NQ, int LA>
constexpr int operand_reads(int i) { return i < NQ ? 1 : 2; }
template <int I, int N, int NQ, int LA>
__device__ __forceinline__ void matrix_sched() {
  if constexpr (I < N) {
    if constexpr (I + LA < N)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, operand_reads<NQ, LA>(I + LA), 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    matrix_sched<I + 1, N, NQ, LA>();
  }
}

// Workgroup barrier that also fences the instruction scheduler, so that no
// instruction of one phase is moved into the neighbouring phase.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Ping-pong variant of the prefill kernel (used for head_dim 128).  The two wavefronts
// that share a SIMD (wave w and w+4) alternate between a matrix phase and a vector phase,
// offset by one phase, so one wavefront's MFMAs run while the other computes its
// exponentials:
//   matrix phase of unit j: S^T(j) = K(j).Q^T, then O^T += V^T(j-1).P^T(j-1);
//   vector phase of unit j: mask, row max, rescale, P(j) = exp2(S - m), row sums.
// Every phase ends at a workgroup barrier.  K and V have separate 4-slot rings; the copies
// are issued between the MFMAs of the matrix phases, each group copying half of a unit.
// Operand reads run six MFMAs ahead of their use.  The copies are written as assembly
// (the compiler does not see them), so the compiler waits for LDS reads only with
// lgkmcnt; the kernel orders reads after copies with its own vmcnt waits and barriers.
template <int D>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(PrefillArgs a, RopeArgs rope) {
  using C = PrefillCfg<D>;
  struct Smem {
    unsigned char k[4][C::UB];
    unsigned char v[4][C::UB];
  };
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int cg = lane >> 5;
  const int Hq = a.num_q_heads;
  const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)

  int hgi = blockIdx.x;
  if ((gridDim.x & 7) == 0) hgi = (hgi & 7) * (int)(gridDim.x >> 3) + (hgi >> 3);
  const int g = hgi / a.n_hgroups;
  const int hgrp = hgi - g * a.n_hgroups;
  const int b = blockIdx.y;
  const int S = a.num_splits;
  const int qt = a.n_qtiles - 1 - (int)blockIdx.z / S;
  const int split = (int)blockIdx.z % S;

  const int q0 = (int)min<int64_t>(max(a.cu_q[b], 0), a.total_q);
  const int lq = (int)min<int64_t>(max(a.cu_q[b + 1], q0), a.total_q) - q0;
  const int kv0 = (int)min<int64_t>(max(a.cu_kv[b], 0), a.total_kv);
  const int lk = (int)min<int64_t>(max(a.cu_kv[b + 1], kv0), a.total_kv) - kv0;
  const int wg_p0 = qt * 32 * a.pw;
  if (wg_p0 >= lq) return;
  const int off = lk - lq;

  const bool active = (wave / a.hg) < a.pw;
  const int h = g * a.group + hgrp * a.hg + (wave % a.hg);
  const int p0 = wg_p0 + (wave / a.hg) * 32;
  const bool has_rows = active && p0 < lq;

  int kend_wg = a.causal ? min(lk, wg_p0 + 32 * a.pw + off) : lk;
  kend_wg = max(kend_wg, 0);
  const int u0 = split * a.split_units;
  const int n_wg = min((kend_wg + C::UNIT - 1) / C::UNIT, u0 + a.split_units);
  int kend_w = a.causal ? min(lk, p0 + 32 + off) : lk;
  kend_w = has_rows ? max(kend_w, 0) : 0;
  const int n_w = min((kend_w + C::UNIT - 1) / C::UNIT, n_wg);
  const int pos = p0 + l32;
  const bool split_out = S > 1;
  if (u0 >= n_wg && split > 0) {
    if (has_rows && pos < lq && cg == 0)
      a.part_lse[((size_t)(q0 + pos) * Hq + h) * S + split] = kNegInf;
    return;
  }
  const int n = n_wg - u0;  // units of the workgroup
  const int nw = n_w - u0;  // units of this wavefront

  const size_t head_base = ((size_t)g * a.total_kv + kv0) * D;
  const uint32_t kvbytes = (uint32_t)max(lk, 0) * C::ROW;
  const u32x4 kr = make_rsrc_words((const __bf16*)a.k + head_base, kvbytes);
  const u32x4 vr = make_rsrc_words((const __bf16*)a.v + head_base, kvbytes);
  // Copies of one 64-key unit of K or V: the two groups copy alternate halves (group g:
  // 1 KiB blocks g*4*NDMA .. +4*NDMA), each wavefront NDMA blocks per tensor.
  auto copy_block = [&](int u, bool is_v, int i) __attribute__((always_inline)) {
    const int blk = grp * 4 * C::NDMA + i * 4 + (wave & 3);
    const int p = blk * 64 + lane;
    const int row = p / C::CPR;
    const int cc = p - row * C::CPR;
    const uint32_t rb = (uint32_t)(u * C::UNIT + row) * C::ROW;
    if (is_v)
      dma16_asm(vr, rb + (uint32_t)((cc ^ vswz<D>(row)) * 16), lds_addr(sm.v[u & 3] + blk * 1024));
    else
      dma16_asm(kr, rb + (uint32_t)((cc ^ kswz<D>(row)) * 16), lds_addr(sm.k[u & 3] + blk * 1024));
  };
  auto issue_k = [&](int u) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) copy_block(u, false, i);
  };
  auto issue_v = [&](int u) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) copy_block(u, true, i);
  };

  // The first copies go out before the Q loads; one wait for everything then leaves no
  // register load pending inside the loop.
  issue_k(u0);
  issue_k(u0 + 1);
  issue_v(u0);
  issue_k(u0 + 2);
  issue_v(u0 + 1);

  bf16x8 qop[C::KS];
  {
    const int nrows = max(0, min(32, lq - p0));
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc((const __bf16*)a.q + ((size_t)(q0 + max(p0, 0)) * Hq) * D,
                  has_rows ? (uint32_t)(nrows * Hq * C::ROW) : 0u);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const uint32_t o = (uint32_t)((l32 * Hq + h) * C::ROW + (ks * 16 + cg * 8) * 2);
      qop[ks] = as_bf16x8(load16(qr, o));
    }
  }
  if (rope.enabled) {
    const int64_t rpos = (int64_t)off + p0 + l32;
#pragma unroll
    for (int ks = 0; ks < C::KS / 2; ++ks)
      rope_rotate8(qop[ks], qop[ks + C::KS / 2], ks * 16 + cg * 8, rpos, rope);
  }

  const float sig = (a.sinks != nullptr && has_rows && split == 0) ? a.sinks[h] * kLog2e : kNegInf;
  wait_vmcnt<0>();  // Q, the sink and the first copies
  float m = sig;
  float dsum = (sig != kNegInf && cg == 0) ? 1.0f : 0.0f;
  f32x16 o[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[t][j] = 0.f;
  const float sl2 = a.scale_log2;
  const int lim = a.causal ? min(lk - 1, pos + off) : lk - 1;

  uint32_t v_lane_off[C::DT];
  {
    const int p16 = lane & 15;
    const int lrow = 4 * cg + (p16 >> 2);
    const int dsub = 16 * ((lane >> 4) & 1) + 4 * (p16 & 3);
#pragma unroll
    for (int t = 0; t < C::DT; ++t) {
      const int d = 32 * t + dsub;
      v_lane_off[t] = (uint32_t)(lrow * C::ROW + (((d >> 3) ^ vswz<D>(lrow)) * 16) + (d & 7) * 2);
    }
  }

  f32x16 sc[2];     // S^T of the unit between its matrix and vector phases
  bf16x8 pk[2][2];  // P^T of the unit between its vector phase and the next matrix phase
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) pk[kt][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});

  // K operand offsets (loop-invariant): lane reads key row kt*32 + l32, chunk
  // (2*ks + cg) ^ kswz(row); kswz(row) does not depend on kt.
  uint32_t koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    koff[ks] = (uint32_t)(l32 * C::ROW + (((ks * 2 + cg) ^ kswz<D>(l32)) * 16));

  // Matrix phase of relative unit j: S^T(j) = K(j).Q^T (NQ MFMAs, one 16-byte K read
  // each), then O^T += V^T(j-1).P^T(j-1) (NP MFMAs, two transposing V reads each).
  // Operand reads run LA MFMAs ahead of their use, through explicit LDS waits.
  constexpr int NQ = 2 * C::KS;
  constexpr int NP = 4 * C::DT;
  constexpr int LA = 6;
  // K operands 0 .. LA-1 of the next matrix phase, read during the vector phase before it
  u32x4 kpre[LA];
  auto preload_k = [&](int jk) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)((u0 + jk) & 3) * C::UB;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      kpre[i] = *(const u32x4*)(sm.k[0] + (kb + koff[i >> 1] + (i & 1) * 32 * C::ROW));
  };
  auto matrix_ops = [&](int jk, int jv, int jc, auto qk_tag, auto pv_tag) __attribute__((always_inline)) {
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    const uint32_t kb = (uint32_t)((u0 + jk) & 3) * C::UB;  // slot of K(jk)
    const uint32_t vb = (uint32_t)((u0 + jv) & 3) * C::UB;  // slot of V(jv)
    u32x4 kop[NQ];
    u32x2 vlo[NP], vhi[NP];
    auto reads = [&](int i) __attribute__((always_inline)) {
      if (i < NQ) {
        if (QK) kop[i] = i < LA ? kpre[i] : *(const u32x4*)(sm.k[0] + (kb + koff[i >> 1] + (i & 1) * 32 * C::ROW));
      } else if (PV) {
        const int q = (i - NQ) / C::DT, t = (i - NQ) % C::DT;
        const int ro = ((q >> 1) * 32 + 16 * (q & 1)) * C::ROW;
        vlo[i - NQ] = ds_read_tr16_c(sm.v[0] + (vb + v_lane_off[t] + ro));
        vhi[i - NQ] = ds_read_tr16_c(sm.v[0] + (vb + v_lane_off[t] + ro + 8 * C::ROW));
      }
    };
    if (QK) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kt][i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < LA; ++i) reads(i);
#pragma unroll
    for (int i = 0; i < NQ + NP; ++i) {
      if (i + LA < NQ + NP) reads(i + LA);
      if (i < NQ) {
        if (QK) {
          sc[i & 1] = mfma32(as_bf16x8(kop[i]), qop[i >> 1], sc[i & 1]);
        }
      } else if (PV) {
        const int q = (i - NQ) / C::DT, t = (i - NQ) % C::DT;
        const u32x4 va = {vlo[i - NQ].x, vlo[i - NQ].y, vhi[i - NQ].x, vhi[i - NQ].y};
        o[t] = mfma32(as_bf16x8(va), pk[q >> 1][q & 1], o[t]);
      }
      // this wavefront's copies of K(jc+3) and V(jc+2), one every 8 MFMAs
      if (i % 8 == 3 && i / 8 < 2 * C::NDMA) {
        const int c = i / 8;
        if (c < C::NDMA) copy_block(u0 + jc + 3, false, c);
        else copy_block(u0 + jc + 2, true, c - C::NDMA);
      }
    }
    matrix_sched<0, NQ + NP, NQ, LA>();
  };
  // One code path for every step (the MFMA accumulators then keep their registers):
  // S^T of a unit the wavefront does not need is computed and ignored, and the
  // probabilities of a unit it skips are zero, so that unit's V^T.P^T adds nothing.
  // The first step reads the V slot of unit 0 (landed, finite) with zero probabilities.
  // The wavefront in its matrix phase runs at the higher issue priority, so its MFMAs
  // are not held back behind the other wavefront's vector work (measured +2.4 %).
  auto matrix_phase = [&](int j) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(3);
    matrix_ops(j, j > 0 ? j - 1 : 0, j, std::true_type{}, std::true_type{});
    __builtin_amdgcn_s_setprio(0);
  };

  // vector phase of relative unit j
  auto vector_phase = [&](int j) __attribute__((always_inline)) {
    if (j >= nw) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) pk[kt][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      return;
    }
    const int kbase = (u0 + j) * C::UNIT;
    if (kbase + C::UNIT > lk || (a.causal && kbase + C::UNIT - 1 > p0 + off)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + kt * 32 + 8 * (i >> 2) + 4 * cg + (i & 3);
          sc[kt][i] = (key <= lim) ? sc[kt][i] : kNegInf;
        }
    }
    // Probabilities against the running max, in groups of 8 (bf16 operands and fp32 group
    // sums).  The running max is raised when a row's max exceeds it by more than 2^8; if
    // no group sum exceeds 128, no probability does, so that test would fail and these
    // probabilities stand: the row max is only computed when some group sum is larger
    // (or overflowed), or while the running max is still -inf (a -inf sink before the
    // row's first finite score), where the test always raises it.
    float gs[2][2];
    auto probs = [&]() __attribute__((always_inline)) {
      const float msub = (m == kNegInf) ? 0.0f : m;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) p[i] = fast_exp2(__builtin_fmaf(sc[kt][kk * 8 + i], sl2, -msub));
          u32x4 w4;
          w4.x = pack_bf16x2(p[0], p[1]);
          w4.y = pack_bf16x2(p[2], p[3]);
          w4.z = pack_bf16x2(p[4], p[5]);
          w4.w = pack_bf16x2(p[6], p[7]);
          gs[kt][kk] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
          pk[kt][kk] = as_bf16x8(w4);
        }
    };
    probs();
    const float gmax = fmaxf(fmaxf(gs[0][0], gs[0][1]), fmaxf(gs[1][0], gs[1][1]));
    if (__any(!(gmax <= 128.0f) || m == kNegInf)) {
      float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) mx = fmaxf(fmaxf(mx, sc[0][i]), sc[0][i + 1]);
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, sc[1][i]), sc[1][i + 1]);
      const float mxs = half_swap_max(mx) * sl2;
      if (__any(mxs > m + 8.0f)) {
        const float mnew = fmaxf(m, mxs);
        const float alpha = (mnew == kNegInf) ? 1.0f : fast_exp2(m - mnew);
        dsum *= alpha;
#pragma unroll
        for (int t = 0; t < C::DT; ++t) o[t] *= alpha;
        m = mnew;
        probs();
      }
    }
    dsum += gs[0][0];
    dsum += gs[0][1];
    dsum += gs[1][0];
    dsum += gs[1][1];
  };

  // Half-phase h: group 0 runs the matrix phase of unit j at h = 2j and its vector phase
  // at h = 2j+1; group 1 runs both one half-phase later (an extra barrier before its
  // loop; group 0 balances it after the loop), so both groups execute the same loop body.
  // The matrix phase of step j also copies this wavefront's half of K(j+3) and V(j+2)
  // into the slots of K(j-1) and V(j-2), whose last readers finished before h = 2j.
  // Each vector phase first reads the leading K operands of the wavefront's next matrix
  // phase, so that phase's MFMAs start without waiting on the LDS.  Hence K(j) and V(j-1)
  // must be complete before the barrier that starts h = 2j, and K(j+1) before the one
  // that starts h = 2j+1; the waits before each barrier leave in flight only the copy
  // groups (one tensor of one unit each) issued after those: group 0 issues at h = 2c,
  // so 5 after a matrix phase and 4 after a vector phase, group 1 at h = 2c+1, so 4 and 3.
  phase_barrier();
  if (grp == 1) phase_barrier();
  preload_k(0);
  for (int j = 0; j <= n; ++j) {
    matrix_phase(j);
    if (grp == 0) wait_vmcnt<5 * C::NDMA>();
    else wait_vmcnt<4 * C::NDMA>();
    phase_barrier();
    preload_k(j + 1);
    vector_phase(j);
    if (grp == 0) wait_vmcnt<4 * C::NDMA>();
    else wait_vmcnt<3 * C::NDMA>();
    phase_barrier();
  }
  if (grp == 0) phase_barrier();
  wait_vmcnt<0>();

  if (!has_rows || pos >= lq) return;
  const float dr = half_swap_sum(dsum);
  const float inv = dr > 0.f ? 1.0f / dr : 0.f;
  const size_t orow = (size_t)(q0 + pos) * Hq + h;
  if (split_out) {
    float* pdst = a.part_o + (orow * S + split) * D;
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4*)(pdst + 32 * t + 8 * q4 + 4 * cg) =
            f32x4{o[t][q4 * 4 + 0] * inv, o[t][q4 * 4 + 1] * inv, o[t][q4 * 4 + 2] * inv,
                  o[t][q4 * 4 + 3] * inv};
    if (cg == 0) a.part_lse[orow * S + split] = dr > 0.f ? (m + __builtin_log2f(dr)) * kLn2 : kNegInf;
    return;
  }
  __bf16* dst = (__bf16*)a.out + orow * D;
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 w2;
      w2.x = pack_bf16x2(o[t][q4 * 4 + 0] * inv, o[t][q4 * 4 + 1] * inv);
      w2.y = pack_bf16x2(o[t][q4 * 4 + 2] * inv, o[t][q4 * 4 + 3] * inv);
      *(u32x2*)(dst + 32 * t + 8 * q4 + 4 * cg) = w2;
    }
  if (cg == 0 && a.lse != nullptr)
    a.lse[orow] = dr > 0.f ? (m + __builtin_log2f(dr)) * kLn2 : kNegInf;
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int num_kv_heads,
                          const RopeArgs& rope, hipStream_t stream) {
  dim3 grid((unsigned)(num_kv_heads * a.n_hgroups), (unsigned)a.batch,
            (unsigned)(a.n_qtiles * a.num_splits));
  // head_dim 64 keeps the lock-step kernel: there the exponentials outweigh the MFMAs,
  // and two of its workgroups share a CU (it needs fewer registers), which the
  // ping-pong kernel cannot.
  if (head_dim == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(512), 0, stream, a, rope);
  else
    hipLaunchKernelGGL(prefill_pp_kernel<128>, grid, dim3(512), 0, stream, a, rope);
  return hipGetLastError();
}

}  // namespace sa
