// Stream decode for q_len * G <= 64 query rows per KV head on contiguous HND K/V.
//
// "GPT-OSS on day 0", "Kernels for GPT-OSS" > "Sink attention": attention is spread over
// heads and over the key axis; blocks of the key axis merge by their log-sum-exp and the
// sink is counted once.  Here the token axis of each KV head (all sequences back to back,
// contiguous in the HND layout) is cut into equal ranges of R tokens, one per wavefront,
// regardless of where sequences begin and end.  A wavefront streams its range of K and V
// through its own LDS ring without a break; wherever a sequence begins or ends inside
// the range it closes the current partial (the online-softmax state of that sequence's
// keys in the range) and starts the next sequence's with that sequence's queries.  Every
// wavefront reads the same number of bytes (no tail of short chunks; what remains is
// HBM serving the XCDs at uneven rates), and each wavefront's reads are one contiguous
// stream of K and one of V, copied with the non-temporal cache policy.
//
// Partials carry no sink: the sink of head h enters once, in the merge, as one more
// log-sum-exp term with value zero (equivalent to counting it in the first block, and it
// also covers sequences with no keys).  Partial p of a sequence is the p-th range that
// overlaps it: slot = range index - first range index of the sequence.
//
// Per stage of 32 keys the math is that of the chunk kernels: S^T = K . Q^T with
// v_mfma_f32_16x16x32_bf16 (the query rows are the N dimension), lane-local online
// softmax in the exp2 domain, O^T += V^T . P^T with V transposed in registers.
#include "sa_decode.h"

namespace sa {

// A wave-uniform int32 read through the scalar unit.  The paged bounds are read while
// copies are in flight; as vector loads they would first wait for every copy.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
// Two such reads under one wait.
__device__ __forceinline__ void sload2_i32(const int32_t* p0, const int32_t* p1, int& v0, int& v1) {
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(v0), "=&s"(v1)
               : "s"(p0), "s"(p1)
               : "memory");
}

constexpr int kStreamWaves = 4;  // wavefronts per workgroup (independent, no barriers)

// The sequence bounds are a separate __restrict__ argument so that the compiler reads
// them with scalar loads, which wait for no copy in flight (a struct field is read with
// vector loads, and every such read would wait for all copies).
// PAGED: the token axis is the page list laid end to end (entry e holds tokens
// [e*page_size, (e+1)*page_size)), so sequence b spans [first entry * page_size, + L_b);
// kv_indptr is then the page-list indptr and last_len the last-page lengths.
template <int D, bool PAGED>
__global__ __launch_bounds__(64 * kStreamWaves) void decode_stream_kernel(
    DecodeArgs a, const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ page_ids,
    const int32_t* __restrict__ last_len, StreamPlan sp, RopeArgs rope) {
  constexpr int KS = D / 32;
  constexpr int DPL = D / 16;
  constexpr int ROW = D * 2;
  constexpr int CPR = D / 8;
  constexpr int STEP = 32;
  constexpr int NST = 2;                  // ring stages per wavefront
  constexpr int SB = STEP * ROW;
  constexpr int NDMA = SB / (64 * 16);    // copies per lane per tensor per stage
  constexpr int QB = 16 * ROW;            // one Q tile (16 rows)
  constexpr int NQD = QB / (64 * 16);     // copies per lane per Q tile
  // One LDS object for the rings and the Q tiles (so the compiler attaches no wait for
  // the copies in flight to the ring and Q reads).
  struct Smem {
    unsigned char ring[kStreamWaves][NST][2][SB];
    unsigned char q[kStreamWaves][2][QB];
  };
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int l16 = lane & 15;
  const int cg = lane >> 4;
  const int gw = (int)blockIdx.x * kStreamWaves + w;
  const int g = gw / sp.nph;
  const int piece = gw - g * sp.nph;
  if (g >= sp.num_kv_heads) return;
  const int t0 = (int)min<int64_t>((int64_t)piece * sp.R, a.total_kv);
  const int t1 = (int)min<int64_t>((int64_t)t0 + sp.R, a.total_kv);
  if (t0 >= t1) return;

  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int M = a.q_len * G;
  const int B = sp.batch;
  const int S = sp.smax;
  // sequence bounds clamped to the token axis (as seq_begin / seq_end, or page_begin /
  // paged_len on the page-list axis)
  auto sbeg = [&](int bb) {
    if constexpr (PAGED)
      return (int)(min<int64_t>(max(sload_i32(kv_indptr + bb), 0), a.num_page_entries) * a.page_size);
    else
      return (int)min<int64_t>(max(kv_indptr[bb], 0), a.total_kv);
  };
  auto send = [&](int bb) {
    if constexpr (PAGED) {
      const int64_t e0 = min<int64_t>(max(sload_i32(kv_indptr + bb), 0), a.num_page_entries);
      const int64_t np =
          min<int64_t>(max<int64_t>(sload_i32(kv_indptr + bb + 1), e0), a.num_page_entries) - e0;
      const int last = min(max(sload_i32(last_len + bb), 1), a.page_size);
      const int64_t len = np > 0 ? min<int64_t>((np - 1) * a.page_size + last, 1 << 24) : 0;
      return (int)(e0 * a.page_size + len);
    } else {
      return (int)min<int64_t>(max(kv_indptr[bb + 1], sbeg(bb)), a.total_kv);
    }
  };
  const int row_t = l16 / G;
  const int row_h = g * G + (l16 - row_t * G);
  const bool row_ok = l16 < M;

  // K and V of this range that belong to some sequence, [c0, c1) (sequences are back to
  // back, so only tokens before the first or after the last lie outside): one bounded
  // view each; copies of tokens outside it read zeros, so no value outside every
  // sequence (possibly not finite) reaches a product with a zero probability.
  const int c0 = max(t0, sbeg(0));
  const int c1 = max(c0, min(t1, send(B - 1)));
  const size_t head_base = ((size_t)g * a.total_kv + c0) * D;
  const uint32_t range_bytes = (uint32_t)(c1 - c0) * ROW;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + head_base, range_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + head_base, range_bytes);
  const int lead = c0 - t0;  // tokens of the range before the view
  unsigned char (*my)[2][SB] = sm.ring[w];
  // PAGED: first sequence not ending before the half-stage being issued (monotone, since
  // stages are issued in order), with its bounds kept in registers
  int ib = 0, ib_s = 0, ib_e = 0;
  auto issue = [&](int st) {
    unsigned char* kbuf = my[st % NST][0];
    unsigned char* vbuf = my[st % NST][1];
    if constexpr (PAGED) {
      // Each 16-row half of the stage lies in one page (the range starts on a multiple of
      // 32 and the page size is a multiple of 16): one bounded view per half, holding the
      // rows before its sequence's end, so unused page slots and gaps read zeros.
      const int ps = a.page_size;
      int rows[2], ent[2], pid[2] = {0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int vt = __builtin_amdgcn_readfirstlane(t0 + st * STEP + 16 * h);
        int bi = __builtin_amdgcn_readfirstlane(ib);
        while (bi < B && ib_e <= vt) {  // next sequence (rare: once per sequence end)
          ++bi;
          if (bi < B) {
            ib_s = sbeg(bi);
            ib_e = send(bi);
          }
        }
        ib = __builtin_amdgcn_readfirstlane(bi);
        const int r = (ib < B && vt >= ib_s) ? min(ib_e - vt, 16) : 0;
        rows[h] = __builtin_amdgcn_readfirstlane(r);
        ent[h] = vt / ps;  // rows > 0: vt < ib_e <= num_page_entries * ps, in the list
      }
      if (rows[0] > 0 && rows[1] > 0) sload2_i32(page_ids + ent[0], page_ids + ent[1], pid[0], pid[1]);
      else if (rows[0] > 0) pid[0] = sload_i32(page_ids + ent[0]);
      else if (rows[1] > 0) pid[1] = sload_i32(page_ids + ent[1]);
      __amdgpu_buffer_rsrc_t kh[2], vh[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (rows[h] > 0) {
          const int64_t pc = min<int64_t>(max<int64_t>(pid[h], 0), a.num_pages - 1);
          const int vt = t0 + st * STEP + 16 * h;
          const size_t base = (((size_t)pc * a.num_kv_heads + g) * ps + (vt - ent[h] * ps)) * D;
          kh[h] = make_rsrc((const __bf16*)a.k + base, (uint32_t)rows[h] * ROW);
          vh[h] = make_rsrc((const __bf16*)a.v + base, (uint32_t)rows[h] * ROW);
        } else {
          kh[h] = make_rsrc(a.k, 0u);
          vh[h] = make_rsrc(a.v, 0u);
        }
      }
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int p = i * 64 + lane;
        const int row = p / CPR;
        const int cc = p - row * CPR;
        const int h = (i * (64 / CPR)) / 16;  // every row of copy i lies in half h
        const uint32_t rb = (uint32_t)(row - 16 * h) * ROW;
        dma16_nt(kh[h], rb + (uint32_t)((cc ^ dswz<D>(row)) * 16), kbuf + i * 1024);
        dma16_nt(vh[h], rb + (uint32_t)(cc * 16), vbuf + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int p = i * 64 + lane;
        const int row = p / CPR;
        const int cc = p - row * CPR;
        const int tok = st * STEP + row - lead;  // token relative to the view
        const uint32_t rbase = tok >= 0 ? (uint32_t)tok * ROW : kNoRead;
        dma16_nt(kr, rbase + (uint32_t)((cc ^ dswz<D>(row)) * 16), kbuf + i * 1024);
        dma16_nt(vr, rbase + (uint32_t)(cc * 16), vbuf + i * 1024);
      }
    }
  };
  // Q tile of sequence bb (rows past M, or bb < 0, read nothing and land as zeros).
  auto issue_q = [&](int bb, int buf) {
    const uint32_t qbytes = (uint32_t)(a.q_len * Hq * ROW);
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc((const __bf16*)a.q + (size_t)max(bb, 0) * a.q_len * Hq * D, bb >= 0 ? qbytes : 0u);
#pragma unroll
    for (int i = 0; i < NQD; ++i) {
      const int p = i * 64 + lane;
      const int r = p / CPR;
      const int rt = r / G;
      const int rh = g * G + (r - rt * G);
      const uint32_t off = (r < M) ? (uint32_t)((rt * Hq + rh) * ROW + (p - r * CPR) * 16) : kNoRead;
      dma16(qr, off, &sm.q[w][buf][i * 1024]);
    }
  };
  // first sequence b >= bb with keys, or B (wave-uniform, so its bounds come through
  // scalar loads that wait for no copy)
  auto next_seq = [&](int bb) {
    bb = __builtin_amdgcn_readfirstlane(bb);
    while (bb < B && send(bb) <= sbeg(bb)) ++bb;
    return (int)__builtin_amdgcn_readfirstlane(bb);
  };

  // ---- the first two sequences of the range: the one holding token t0 (binary search
  // over the nondecreasing clamped bounds), then the next one with keys.
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (send(mid) <= t0) lo = mid + 1;
    else hi = mid;
  }
  ib = lo;
  if constexpr (PAGED) {
    if (lo < B) {
      ib_s = sbeg(lo);
      ib_e = send(lo);
    }
  }
  int b = next_seq(lo);
  bool have = b < B && sbeg(b) < t1;
  int bn = have ? next_seq(b + 1) : B;
  bool have_n = bn < B && sbeg(bn) < t1;
  int kseg = 0;  // index of the current segment (its Q tile sits in buffer kseg & 1)
  // D=64: the YaRN frequencies of the lane's dims, read once before any copy goes out
  // (read at each segment start they would wait for every copy in flight)
  double rfreq[8];
  if constexpr (D == 64) {
    if (rope.enabled) {
#pragma unroll
      for (int j = 0; j < 8; ++j) rfreq[j] = rope.freq[cg * 8 + j];
    }
  }
  issue_q(have ? b : -1, 0);
  issue_q(have_n ? bn : -1, 1);
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue(st);
  wait_vmcnt<(NST - 1) * 2 * NDMA>();  // both Q tiles (issued first) have landed
  int q_st = -NST;  // stage during which the next segment's Q tile was issued

  // ---- per-segment state
  bf16x8 qop[KS];
  float m = kNegInf, dsum = 0.f;
  f32x4 o[DPL];
  int sb = 0, se = 0, lim = 0, causal_first = 0;
  auto start_segment = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = *(const bf16x8*)&sm.q[w][kseg & 1][l16 * ROW + (ks * 32 + cg * 8) * 2];
    const int s0 = sbeg(b), e0 = send(b);
    if (rope.enabled) {  // YaRN rotation of the query row at position Lk - q_len + t
      const int64_t pos = (int64_t)(e0 - s0) - a.q_len + row_t;
      if constexpr (D == 64) {
        rope_rotate8_f(qop[0], qop[1], rfreq, pos, rope.mscale);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) rope_rotate8(qop[ks], qop[ks + KS / 2], ks * 32 + cg * 8, pos, rope);
      }
    }
    sb = max(t0, s0);
    se = min(t1, e0);
    // last visible key of the lane's row (causal within the draft), global coordinates
    lim = min(se - 1, a.causal ? e0 - a.q_len + row_t : 0x7fffffff);
    causal_first = a.causal ? e0 - a.q_len + 1 : 0x7fffffff;
    m = kNegInf;
    dsum = 0.f;
#pragma unroll
    for (int t = 0; t < DPL; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto flush_segment = [&]() {
    float dr = wave_xor_sum(dsum, 16);
    dr = wave_xor_sum(dr, 32);
    const int slot = piece - sbeg(b) / sp.R;
    if (!row_ok || slot < 0 || slot >= S) return;
    const float inv = dr > 0.f ? 1.0f / dr : 0.f;
    const int64_t qrow = ((int64_t)b * a.q_len + row_t) * Hq + row_h;
    float* dst = a.part_o + (qrow * S + slot) * D + 4 * cg * DPL;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < DPL; t += 4)
        *(f32x4*)(dst + j * DPL + t) = f32x4{o[t][j] * inv, o[t + 1][j] * inv, o[t + 2][j] * inv,
                                             o[t + 3][j] * inv};
    if (cg == 0) a.part_lse[qrow * S + slot] = dr > 0.f ? (m + __builtin_log2f(dr)) * kLn2 : kNegInf;
  };
  if (have) start_segment();

  const float sl2 = a.scale_log2;
  const int nsteps = (t1 - t0 + STEP - 1) / STEP;
  for (int st = 0; st < nsteps; ++st) {
    issue(st + NST - 1);
    wait_vmcnt<(NST - 1) * 2 * NDMA>();
    const unsigned char* kbuf = my[st % NST][0];
    const unsigned char* vbuf = my[st % NST][1];
    const int kbase = t0 + st * STEP;

    while (have && sb < kbase + STEP) {
      f32x4 s2[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int row = kt * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kv = *(const u32x4*)(kbuf + row * ROW + (((ks * 4 + cg) ^ dswz<D>(row)) * 16));
          acc = mfma16(as_bf16x8(kv), qop[ks], acc);
        }
        s2[kt] = acc;
      }
      // keys outside the segment or past the row's causal limit (the last q_len - 1
      // keys of the sequence are causal-masked for some rows)
      if (kbase < sb || kbase + STEP > se || kbase + STEP > causal_first) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kbase + kt * 16 + 4 * cg + j;
            s2[kt][j] = (key >= sb && key <= lim) ? s2[kt][j] : kNegInf;
          }
      }
      float mx = fmaxf(fmaxf(fmaxf(s2[0][0], s2[0][1]), fmaxf(s2[0][2], s2[0][3])),
                       fmaxf(fmaxf(s2[1][0], s2[1][1]), fmaxf(s2[1][2], s2[1][3])));
      mx = max_over_16_32(mx);
      const float mxs = mx * sl2;
      if (__any(mxs > m + 8.0f)) {
        const float mnew = fmaxf(m, mxs);
        const float alpha = (mnew == kNegInf) ? 1.0f : fast_exp2(m - mnew);
        dsum *= alpha;
#pragma unroll
        for (int t = 0; t < DPL; ++t) o[t] *= alpha;
        m = mnew;
      }
      const float msub = (m == kNegInf) ? 0.0f : m;
      float p[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = fast_exp2(__builtin_fmaf(s2[0][j], sl2, -msub));
        p[4 + j] = fast_exp2(__builtin_fmaf(s2[1][j], sl2, -msub));
      }
      dsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      u32x4 pk;
      pk.x = pack_bf16x2(p[0], p[1]);
      pk.y = pack_bf16x2(p[2], p[3]);
      pk.z = pack_bf16x2(p[4], p[5]);
      pk.w = pack_bf16x2(p[6], p[7]);
      const bf16x8 pop = as_bf16x8(pk);
      uint32_t vw[8][DPL / 2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned char* src = vbuf + slot_key(cg, i) * ROW + l16 * DPL * 2;
        if constexpr (DPL == 8) {
          const u32x4 t4 = *(const u32x4*)src;
          vw[i][0] = t4.x; vw[i][1] = t4.y; vw[i][2] = t4.z; vw[i][3] = t4.w;
        } else {
          const u32x2 t2 = *(const u32x2*)src;
          vw[i][0] = t2.x; vw[i][1] = t2.y;
        }
      }
#pragma unroll
      for (int t = 0; t < DPL; ++t) {
        u32x4 va;
        const int wd = t >> 1;
        if ((t & 1) == 0) {
          va.x = lo_lo(vw[0][wd], vw[1][wd]);
          va.y = lo_lo(vw[2][wd], vw[3][wd]);
          va.z = lo_lo(vw[4][wd], vw[5][wd]);
          va.w = lo_lo(vw[6][wd], vw[7][wd]);
        } else {
          va.x = hi_hi(vw[0][wd], vw[1][wd]);
          va.y = hi_hi(vw[2][wd], vw[3][wd]);
          va.z = hi_hi(vw[4][wd], vw[5][wd]);
          va.w = hi_hi(vw[6][wd], vw[7][wd]);
        }
        o[t] = mfma16(as_bf16x8(va), pop, o[t]);
      }
      if (se > kbase + STEP) break;  // the segment continues in the next stage
      // ---- the segment ends in this stage: write its partial, move to the next one
      flush_segment();
      b = bn;
      have = have_n;
      if (!have) break;
      ++kseg;
      // Its Q tile has landed if it was issued before the stage group whose arrival the
      // wait at the top of this iteration ensured (copies complete in order): that is,
      // unless it was issued during this iteration's or one of the NST - 2 previous
      // iterations' segment switches; then wait for everything.
      if (st < q_st + NST - 1) wait_vmcnt<0>();
      start_segment();
      bn = next_seq(b + 1);
      have_n = bn < B && sbeg(bn) < t1;
      issue_q(have_n ? bn : -1, (kseg + 1) & 1);  // into the buffer of segment kseg - 1
      q_st = st;
    }
  }
  wait_vmcnt<0>();  // no copy may land after the wavefront's LDS is released
}

// The stream plan for 16 < q_len * G <= 64 query rows per KV head: one workgroup of W
// wavefronts per range (wavefront w owns rows 16w .. 16w+15), all reading every stage of
// one shared LDS ring (one barrier per stage), so each K/V byte still leaves HBM once per
// KV head.  Segments, masks, the Q prefetch and the partials are those of
// decode_stream_kernel; the sequence boundaries are the same for every wavefront.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void decode_stream_wg_kernel(
    DecodeArgs a, const int32_t* __restrict__ kv_indptr, StreamPlan sp, RopeArgs rope) {
  constexpr int KS = D / 32;
  constexpr int DPL = D / 16;
  constexpr int ROW = D * 2;
  constexpr int CPR = D / 8;
  constexpr int STEP = 32;
  constexpr int NST = 3;                     // shared ring stages
  constexpr int SB = STEP * ROW;
  constexpr int NDMA = SB / (64 * W * 16);   // copies per lane per tensor per stage
  static_assert(NDMA * 64 * W * 16 == SB, "stage must split evenly over the workgroup");
  constexpr int QB = 16 * ROW;
  constexpr int NQD = QB / (64 * 16);
  struct Smem {
    unsigned char ring[NST][2][SB];
    unsigned char q[W][2][QB];
  };
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int l16 = lane & 15;
  const int cg = lane >> 4;
  const int g = (int)blockIdx.x / sp.nph;
  const int piece = (int)blockIdx.x - g * sp.nph;
  if (g >= sp.num_kv_heads) return;
  const int t0 = (int)min<int64_t>((int64_t)piece * sp.R, a.total_kv);
  const int t1 = (int)min<int64_t>((int64_t)t0 + sp.R, a.total_kv);
  if (t0 >= t1) return;  // workgroup-uniform: no wavefront reaches a barrier

  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int M = a.q_len * G;
  const int B = sp.batch;
  const int S = sp.smax;
  auto sbeg = [&](int bb) { return (int)min<int64_t>(max(kv_indptr[bb], 0), a.total_kv); };
  auto send = [&](int bb) {
    return (int)min<int64_t>(max(kv_indptr[bb + 1], sbeg(bb)), a.total_kv);
  };
  const int R = w * 16 + l16;  // the lane's query row
  const int row_t = R / G;
  const int row_h = g * G + (R - row_t * G);
  const bool row_ok = R < M;

  const int c0 = max(t0, sbeg(0));
  const int c1 = max(c0, min(t1, send(B - 1)));
  const size_t head_base = ((size_t)g * a.total_kv + c0) * D;
  const uint32_t range_bytes = (uint32_t)(c1 - c0) * ROW;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + head_base, range_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + head_base, range_bytes);
  const int lead = c0 - t0;
  auto issue = [&](int st) {
    unsigned char* kbuf = sm.ring[st % NST][0];
    unsigned char* vbuf = sm.ring[st % NST][1];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int blk = i * W + w;  // 1 KiB block of the stage this wavefront fills
      const int p = blk * 64 + lane;
      const int row = p / CPR;
      const int cc = p - row * CPR;
      const int tok = st * STEP + row - lead;
      const uint32_t rbase = tok >= 0 ? (uint32_t)tok * ROW : kNoRead;
      dma16_nt(kr, rbase + (uint32_t)((cc ^ dswz<D>(row)) * 16), kbuf + blk * 1024);
      dma16_nt(vr, rbase + (uint32_t)(cc * 16), vbuf + blk * 1024);
    }
  };
  // this wavefront's 16 query rows of sequence bb (bb < 0: zeros)
  auto issue_q = [&](int bb, int buf) {
    const uint32_t qbytes = (uint32_t)(a.q_len * Hq * ROW);
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc((const __bf16*)a.q + (size_t)max(bb, 0) * a.q_len * Hq * D, bb >= 0 ? qbytes : 0u);
#pragma unroll
    for (int i = 0; i < NQD; ++i) {
      const int p = i * 64 + lane;
      const int r = w * 16 + p / CPR;
      const int rt = r / G;
      const int rh = g * G + (r - rt * G);
      const uint32_t off =
          (r < M) ? (uint32_t)((rt * Hq + rh) * ROW + (p - (p / CPR) * CPR) * 16) : kNoRead;
      dma16(qr, off, &sm.q[w][buf][i * 1024]);
    }
  };
  auto next_seq = [&](int bb) {
    bb = __builtin_amdgcn_readfirstlane(bb);
    while (bb < B && send(bb) <= sbeg(bb)) ++bb;
    return (int)__builtin_amdgcn_readfirstlane(bb);
  };

  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (send(mid) <= t0) lo = mid + 1;
    else hi = mid;
  }
  int b = next_seq(lo);
  bool have = b < B && sbeg(b) < t1;
  int bn = have ? next_seq(b + 1) : B;
  bool have_n = bn < B && sbeg(bn) < t1;
  int kseg = 0;
  issue_q(have ? b : -1, 0);
  issue_q(have_n ? bn : -1, 1);
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue(st);
  wait_vmcnt<(NST - 1) * 2 * NDMA>();  // this wavefront's Q tiles (issued first) have landed
  int q_st = -NST;

  bf16x8 qop[KS];
  float m = kNegInf, dsum = 0.f;
  f32x4 o[DPL];
  int sb = 0, se = 0, lim = 0, causal_first = 0;
  auto start_segment = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = *(const bf16x8*)&sm.q[w][kseg & 1][l16 * ROW + (ks * 32 + cg * 8) * 2];
    const int s0 = sbeg(b), e0 = send(b);
    if (rope.enabled) {
      const int64_t pos = (int64_t)(e0 - s0) - a.q_len + row_t;
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks) rope_rotate8(qop[ks], qop[ks + KS / 2], ks * 32 + cg * 8, pos, rope);
    }
    sb = max(t0, s0);
    se = min(t1, e0);
    lim = min(se - 1, a.causal ? e0 - a.q_len + row_t : 0x7fffffff);
    causal_first = a.causal ? e0 - a.q_len + 1 : 0x7fffffff;
    m = kNegInf;
    dsum = 0.f;
#pragma unroll
    for (int t = 0; t < DPL; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto flush_segment = [&]() {
    float dr = wave_xor_sum(dsum, 16);
    dr = wave_xor_sum(dr, 32);
    const int slot = piece - sbeg(b) / sp.R;
    if (!row_ok || slot < 0 || slot >= S) return;
    const float inv = dr > 0.f ? 1.0f / dr : 0.f;
    const int64_t qrow = ((int64_t)b * a.q_len + row_t) * Hq + row_h;
    float* dst = a.part_o + (qrow * S + slot) * D + 4 * cg * DPL;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < DPL; t += 4)
        *(f32x4*)(dst + j * DPL + t) = f32x4{o[t][j] * inv, o[t + 1][j] * inv, o[t + 2][j] * inv,
                                             o[t + 3][j] * inv};
    if (cg == 0) a.part_lse[qrow * S + slot] = dr > 0.f ? (m + __builtin_log2f(dr)) * kLn2 : kNegInf;
  };
  if (have) start_segment();

  const float sl2 = a.scale_log2;
  const int nsteps = (t1 - t0 + STEP - 1) / STEP;
  for (int st = 0; st < nsteps; ++st) {
    // stage st has landed (this wavefront's copies) once only the NST-2 stages issued
    // after it are pending; after the barrier every wavefront's copies have, and every
    // wavefront has finished stage st-1, whose slot is refilled
    wait_vmcnt<(NST - 2) * 2 * NDMA>();
    stage_barrier();
    issue(st + NST - 1);
    const unsigned char* kbuf = sm.ring[st % NST][0];
    const unsigned char* vbuf = sm.ring[st % NST][1];
    const int kbase = t0 + st * STEP;

    while (have && sb < kbase + STEP) {
      f32x4 s2[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int row = kt * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kv = *(const u32x4*)(kbuf + row * ROW + (((ks * 4 + cg) ^ dswz<D>(row)) * 16));
          acc = mfma16(as_bf16x8(kv), qop[ks], acc);
        }
        s2[kt] = acc;
      }
      if (kbase < sb || kbase + STEP > se || kbase + STEP > causal_first) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kbase + kt * 16 + 4 * cg + j;
            s2[kt][j] = (key >= sb && key <= lim) ? s2[kt][j] : kNegInf;
          }
      }
      float mx = fmaxf(fmaxf(fmaxf(s2[0][0], s2[0][1]), fmaxf(s2[0][2], s2[0][3])),
                       fmaxf(fmaxf(s2[1][0], s2[1][1]), fmaxf(s2[1][2], s2[1][3])));
      mx = max_over_16_32(mx);
      const float mxs = mx * sl2;
      if (__any(mxs > m + 8.0f)) {
        const float mnew = fmaxf(m, mxs);
        const float alpha = (mnew == kNegInf) ? 1.0f : fast_exp2(m - mnew);
        dsum *= alpha;
#pragma unroll
        for (int t = 0; t < DPL; ++t) o[t] *= alpha;
        m = mnew;
      }
      const float msub = (m == kNegInf) ? 0.0f : m;
      float p[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = fast_exp2(__builtin_fmaf(s2[0][j], sl2, -msub));
        p[4 + j] = fast_exp2(__builtin_fmaf(s2[1][j], sl2, -msub));
      }
      dsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      u32x4 pk;
      pk.x = pack_bf16x2(p[0], p[1]);
      pk.y = pack_bf16x2(p[2], p[3]);
      pk.z = pack_bf16x2(p[4], p[5]);
      pk.w = pack_bf16x2(p[6], p[7]);
      const bf16x8 pop = as_bf16x8(pk);
      uint32_t vw[8][DPL / 2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned char* src = vbuf + slot_key(cg, i) * ROW + l16 * DPL * 2;
        if constexpr (DPL == 8) {
          const u32x4 t4 = *(const u32x4*)src;
          vw[i][0] = t4.x; vw[i][1] = t4.y; vw[i][2] = t4.z; vw[i][3] = t4.w;
        } else {
          const u32x2 t2 = *(const u32x2*)src;
          vw[i][0] = t2.x; vw[i][1] = t2.y;
        }
      }
#pragma unroll
      for (int t = 0; t < DPL; ++t) {
        u32x4 va;
        const int wd = t >> 1;
        if ((t & 1) == 0) {
          va.x = lo_lo(vw[0][wd], vw[1][wd]);
          va.y = lo_lo(vw[2][wd], vw[3][wd]);
          va.z = lo_lo(vw[4][wd], vw[5][wd]);
          va.w = lo_lo(vw[6][wd], vw[7][wd]);
        } else {
          va.x = hi_hi(vw[0][wd], vw[1][wd]);
          va.y = hi_hi(vw[2][wd], vw[3][wd]);
          va.z = hi_hi(vw[4][wd], vw[5][wd]);
          va.w = hi_hi(vw[6][wd], vw[7][wd]);
        }
        o[t] = mfma16(as_bf16x8(va), pop, o[t]);
      }
      if (se > kbase + STEP) break;
      flush_segment();
      b = bn;
      have = have_n;
      if (!have) break;
      ++kseg;
      if (st < q_st + NST - 1) wait_vmcnt<0>();
      start_segment();
      bn = next_seq(b + 1);
      have_n = bn < B && sbeg(bn) < t1;
      issue_q(have_n ? bn : -1, (kseg + 1) & 1);
      q_st = st;
    }
  }
  wait_vmcnt<0>();
}

// Merge of the stream partials: row (b, t, h) combines the partials of the ranges that
// overlap sequence b with the sink of head h, a term of value zero and log-sum-exp
// sink[h].  D/4 lanes per row, four consecutive head dims each.  The sequence bounds and
// the row's log-sum-exps (4 bytes a slot) are loaded together; then only the partial
// outputs of the n slots this call wrote (read once: non-temporal) are loaded, all
// together, so a row waits for two memory latencies and reads n, not kStreamMaxSlots,
// partial outputs.
template <int D, bool PAGED>
__global__ __launch_bounds__(128) void merge_stream_kernel(DecodeArgs a, StreamPlan sp,
                                                           int64_t rows) {
  constexpr int LPR = D / 4;
  constexpr int RPB = 128 / LPR;
  const int q = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  if (row >= rows) return;
  const int Hq = a.num_q_heads;
  const int b = (int)(row / ((int64_t)a.q_len * Hq));
  const int h = (int)(row % Hq);
  const int S = sp.smax;
  const float* pl = a.part_lse + row * S;
  const f32x4* po = (const f32x4*)(a.part_o + row * S * D) + q;
  float lc[kStreamMaxSlots];
  f32x4 x[kStreamMaxSlots];
#pragma unroll
  for (int c = 0; c < kStreamMaxSlots; ++c) lc[c] = (c < S) ? __builtin_nontemporal_load(pl + c) : kNegInf;
  const float sink = (a.sinks != nullptr) ? a.sinks[h] : kNegInf;
  int s0, e0;
  if constexpr (PAGED) {  // the sequence's extent on the page-list axis
    const int ep = page_begin(a, b);
    s0 = ep * a.page_size;
    e0 = s0 + paged_len(a, b, ep);
  } else {
    s0 = seq_begin(a, b);
    e0 = seq_end(a, b);
  }
  const int n = (e0 > s0) ? min(S, (e0 - 1) / sp.R - s0 / sp.R + 1) : 0;
#pragma unroll
  for (int c = 0; c < kStreamMaxSlots; ++c)
    x[c] = (c < n) ? __builtin_nontemporal_load(po + (size_t)c * (D / 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kStreamMaxSlots; ++c)
    if (c >= n) lc[c] = kNegInf;  // not written by this call: no weight
  float mx = sink;
#pragma unroll
  for (int c = 0; c < kStreamMaxSlots; ++c) mx = fmaxf(mx, lc[c]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != kNegInf) {
    wsum = (sink != kNegInf) ? __expf(sink - mx) : 0.f;
#pragma unroll
    for (int c = 0; c < kStreamMaxSlots; ++c) {
      // an empty slot (lse -inf) has weight 0 and its output is selected away
      const float wc = (lc[c] != kNegInf) ? __expf(lc[c] - mx) : 0.f;
      wsum += wc;
      if (wc > 0.f) {
        acc[0] = __builtin_fmaf(wc, x[c][0], acc[0]);
        acc[1] = __builtin_fmaf(wc, x[c][1], acc[1]);
        acc[2] = __builtin_fmaf(wc, x[c][2], acc[2]);
        acc[3] = __builtin_fmaf(wc, x[c][3], acc[3]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  u32x2 pk2;
  pk2.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk2.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(u32x2*)((__bf16*)a.out + row * D + 4 * q) = pk2;
  if (q == 0 && a.lse != nullptr) a.lse[row] = wsum > 0.f ? mx + __logf(wsum) : kNegInf;
}

hipError_t launch_decode_stream(const DecodeArgs& a, int head_dim, const StreamPlan& sp,
                                const RopeArgs& rope, const int32_t* page_ids, hipStream_t stream) {
  if (page_ids != nullptr && sp.waves > 1) return hipErrorInvalidValue;  // single-wavefront plan only
  if (sp.waves > 1) {  // one workgroup of sp.waves wavefronts per range
    const dim3 grid((unsigned)(sp.num_kv_heads * sp.nph));
    if (head_dim == 64) {
      if (sp.waves == 2)
        hipLaunchKernelGGL((decode_stream_wg_kernel<64, 2>), grid, dim3(128), 0, stream, a, a.kv_indptr, sp, rope);
      else
        hipLaunchKernelGGL((decode_stream_wg_kernel<64, 4>), grid, dim3(256), 0, stream, a, a.kv_indptr, sp, rope);
    } else {
      if (sp.waves == 2)
        hipLaunchKernelGGL((decode_stream_wg_kernel<128, 2>), grid, dim3(128), 0, stream, a, a.kv_indptr, sp, rope);
      else
        hipLaunchKernelGGL((decode_stream_wg_kernel<128, 4>), grid, dim3(256), 0, stream, a, a.kv_indptr, sp, rope);
    }
    return hipGetLastError();
  }
  const int waves = sp.num_kv_heads * sp.nph;
  const dim3 grid((unsigned)((waves + kStreamWaves - 1) / kStreamWaves));
  const dim3 block(64 * kStreamWaves);
  if (page_ids != nullptr) {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_stream_kernel<64, true>), grid, block, 0, stream, a,
                         a.kv_page_indptr, page_ids, a.kv_last_page_len, sp, rope);
    else
      hipLaunchKernelGGL((decode_stream_kernel<128, true>), grid, block, 0, stream, a,
                         a.kv_page_indptr, page_ids, a.kv_last_page_len, sp, rope);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL((decode_stream_kernel<64, false>), grid, block, 0, stream, a, a.kv_indptr,
                       nullptr, nullptr, sp, rope);
  } else {
    hipLaunchKernelGGL((decode_stream_kernel<128, false>), grid, block, 0, stream, a, a.kv_indptr,
                       nullptr, nullptr, sp, rope);
  }
  return hipGetLastError();
}

hipError_t launch_merge_stream(const DecodeArgs& a, int head_dim, const StreamPlan& sp,
                               int64_t rows, bool paged, hipStream_t stream) {
  const dim3 g64((unsigned)((rows + 7) / 8)), g128((unsigned)((rows + 3) / 4));
  if (head_dim == 64) {
    if (paged) hipLaunchKernelGGL((merge_stream_kernel<64, true>), g64, dim3(128), 0, stream, a, sp, rows);
    else hipLaunchKernelGGL((merge_stream_kernel<64, false>), g64, dim3(128), 0, stream, a, sp, rows);
  } else {
    if (paged) hipLaunchKernelGGL((merge_stream_kernel<128, true>), g128, dim3(128), 0, stream, a, sp, rows);
    else hipLaunchKernelGGL((merge_stream_kernel<128, false>), g128, dim3(128), 0, stream, a, sp, rows);
  }
  return hipGetLastError();
}

}  // namespace sa
