// Split-KV decode and log-sum-exp merge kernels for gfx950.
//
// "GPT-OSS on day 0", "Kernels for GPT-OSS" > "Sink attention": attention is spread
// over heads and over the key axis; the online softmax keeps a running maximum m and
// sum d, starting from (m, d) = (sink, 1) so the sink is counted; when the key axis is
// split into blocks the sink enters only the first block.  Here chunk 0 starts from
// (sink, 1) and every other chunk from (-inf, 0); the merge then combines the chunks
// by their log-sum-exp.
//
// One workgroup owns one (sequence, KV head, row group, chunk).  The q_len * G query
// rows that share the KV head (GQA) are the N dimension of the MFMAs, so each K/V byte
// is read from HBM once per KV head.  Scores are computed transposed, S^T = K . Q^T,
// with v_mfma_f32_16x16x32_bf16: the accumulator of S^T leaves every lane holding
// scores of ONE query row, which is exactly the B-operand layout of the next product
// O^T = V^T . P^T, so probabilities never leave registers and the per-row softmax
// state (m, d, rescale) is lane-local.  K and V stream from HBM through
// an LDS ring with asynchronous buffer->LDS copies; V is transposed in registers.
#include "sa_decode.h"


namespace sa {

// Bounded views of K and V for the rows of page-list slot `ps_slot` of a paged sequence
// that lie before key `ke` (<= the sequence length): page ids are read with scalar
// loads and clamped to the cache, rows at or past ke read zeros.
template <int D>
__device__ __forceinline__ void page_views(const DecodeArgs& a, const int32_t* __restrict__ page_ids,
                                           int e0, int g, int ps_slot, int ke,
                                           __amdgpu_buffer_rsrc_t& kr, __amdgpu_buffer_rsrc_t& vr) {
  const int ps = a.page_size;
  const int rows = min(max(ke - ps_slot * ps, 0), ps);
  if (rows == 0) {  // nothing of this page is read (also covers empty sequences)
    kr = make_rsrc(a.k, 0u);
    vr = make_rsrc(a.v, 0u);
    return;
  }
  // rows > 0 implies ps_slot * ps < ke <= lk, so the entry lies inside the sequence's list
  int64_t pid = page_ids[e0 + ps_slot];
  pid = min<int64_t>(max<int64_t>(pid, 0), a.num_pages - 1);
  const size_t base = ((size_t)pid * a.num_kv_heads + g) * ps * D;
  kr = make_rsrc((const __bf16*)a.k + base, (uint32_t)rows * D * 2);
  vr = make_rsrc((const __bf16*)a.v + base, (uint32_t)rows * D * 2);
}

// Decode split kernel.  Workgroup = W wavefronts = one (sequence, KV head, row group,
// slot); wavefront w owns 16 query rows.  A slot holds a run of a.chunk_run consecutive
// chunks of the plan: their keys are one contiguous span, which streams from HBM into an
// NST-stage LDS ring with asynchronous 16-byte buffer->LDS copies (no registers), NST-1
// stages ahead of the compute, every wavefront reading each stage from LDS.  Each chunk
// keeps its own online softmax ("Sink attention": blocks of the key axis; the sink in
// the first block only): chunk 0 starts from (sink, 1), every other chunk from
// (-inf, 0), and at the end of each chunk its state is merged by log-sum-exp into the
// run's state, which the slot writes.  A chunk is a whole number of 32-key stages, and
// stages are counted from the run's first key, so the result for a sequence does not
// depend on where it sits in the batch.
template <int D, int W, bool DIRECT, bool PAGED>
__global__ __launch_bounds__(64 * W, 2) void decode_split_kernel(DecodeArgs a,
                                                                 const int32_t* __restrict__ page_ids,
                                                                 RopeArgs rope) {
  constexpr int KS = D / 32;              // k-steps (32 head dims) of S^T
  constexpr int DPL = D / 16;             // head dims per lane per V row read = O^T d-tiles
  constexpr int ROW = D * 2;              // bytes per K/V row
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int STEP = 32;                // keys per stage
  // LDS ring stages: deeper rings cost workgroups per CU (fewer wavefronts to issue
  // copies), which measured slower; 3 stages for head_dim 64, 4 for 128.
  constexpr int NST = (D == 64) ? 3 : 4;
  constexpr int SB = STEP * ROW;          // bytes of K (or V) per stage
  constexpr int NDMA = SB / (64 * W * 16);  // copies per thread per tensor per stage
  static_assert(NDMA * 64 * W * 16 == SB, "stage must split evenly over the workgroup");
  __shared__ __attribute__((aligned(16))) unsigned char ring[NST][2][SB];

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int cg = lane >> 4;
  const int slot = blockIdx.x;
  const int g = blockIdx.y / a.row_groups;
  const int rg = blockIdx.y - g * a.row_groups;
  const int b = blockIdx.z;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int M = a.q_len * G;

  int kv0 = 0, e0 = 0, lk;
  if constexpr (PAGED) {
    e0 = page_begin(a, b);
    lk = paged_len(a, b, e0);
  } else {
    kv0 = seq_begin(a, b);
    lk = seq_end(a, b) - kv0;
  }
  const int n = plan_chunks(lk, a.num_splits, 1);
  const int cl = chunk_len(lk, n);
  const int S = a.num_slots;
  const int run = a.chunk_run;

  // The lane's query row: R -> (draft token t, query head h).
  const int R = rg * 16 * W + wave * 16 + l16;
  const int row_t = R / G;
  const int row_h = g * G + (R - row_t * G);
  const bool row_ok = R < M;
  const int64_t qrow = ((int64_t)b * a.q_len + row_t) * Hq + row_h;

  const int c_first = slot * run;  // first chunk of this slot's run
  if (c_first >= n) {  // unused slot: no mass
    if (!DIRECT && cg == 0 && row_ok) a.part_lse[qrow * S + slot] = kNegInf;
    return;
  }
  const int kb = (int)min<int64_t>(lk, (int64_t)c_first * cl);
  const int ke = (int)min<int64_t>(lk, (int64_t)min(c_first + run, n) * cl);
  const int nsteps = (ke - kb + STEP - 1) / STEP;
  const int chunk_steps = max(cl / STEP, 1);  // stages per chunk

  // K/V of this run: loads past its end return zero.  Contiguous HND: one view of the
  // run.  Paged: a 32-key stage spans at most two pages (page_size is a multiple of 16),
  // and each copy instruction's rows lie inside one of them.
  const size_t head_base = PAGED ? 0 : ((size_t)g * a.total_kv + kv0 + kb) * D;
  const uint32_t run_bytes = PAGED ? 0u : (uint32_t)(ke - kb) * ROW;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + head_base, run_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + head_base, run_bytes);
  auto issue = [&](int st) {
    unsigned char* kbuf = ring[st % NST][0];
    unsigned char* vbuf = ring[st % NST][1];
    if constexpr (PAGED) {
      const int t0 = kb + st * STEP;          // the stage's first key
      const int ps = a.page_size;
      const int pa = t0 / ps;
      __amdgpu_buffer_rsrc_t ka, va, kb2, vb2;
      page_views<D>(a, page_ids, e0, g, pa, ke, ka, va);
      page_views<D>(a, page_ids, e0, g, pa + 1, ke, kb2, vb2);
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int blk = i * W + wave;
        const int p = blk * 64 + lane;
        const int row = p / CPR;
        const int cc = p - row * CPR;
        const int tok0 = t0 + blk * (64 / CPR);  // first row of this copy instruction
        const bool second = tok0 / ps != pa;
        const uint32_t rbase = (uint32_t)(t0 + row - (pa + (second ? 1 : 0)) * ps) * ROW;
        dma16_nt(second ? kb2 : ka, rbase + (uint32_t)((cc ^ dswz<D>(row)) * 16), kbuf + blk * 1024);
        dma16_nt(second ? vb2 : va, rbase + (uint32_t)(cc * 16), vbuf + blk * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int blk = i * W + wave;           // 1 KiB block of the stage this wave fills
        const int p = blk * 64 + lane;          // 16-byte chunk index inside the stage
        const int row = p / CPR;
        const int cc = p - row * CPR;
        const uint32_t rbase = (uint32_t)(st * STEP + row) * ROW;
        dma16_nt(kr, rbase + (uint32_t)((cc ^ dswz<D>(row)) * 16), kbuf + blk * 1024);
        dma16_nt(vr, rbase + (uint32_t)(cc * 16), vbuf + blk * 1024);
      }
    }
  };

  // Q^T operands (B of S^T): lane holds Q[row][ks*32 + cg*8 .. +8]; zero for padding.
  const uint32_t qbytes = (uint32_t)(a.q_len * Hq * ROW);
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc((const __bf16*)a.q + (size_t)b * a.q_len * Hq * D, qbytes);
  bf16x8 qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)((row_t * Hq + row_h) * ROW + (ks * 32 + cg * 8) * 2);
    qop[ks] = as_bf16x8(load16(qr, row_ok ? off : qbytes));
  }
  // YaRN rotation of the query row at its position Lk - q_len + t: pair (i, i + D/2)
  // sits in qop[ks] and qop[ks + KS/2] of the same lane.
  if (rope.enabled) {
    const int64_t pos = (int64_t)lk - a.q_len + row_t;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) rope_rotate8(qop[ks], qop[ks + KS / 2], ks * 32 + cg * 8, pos, rope);
  }
  // Online-softmax state of the current chunk in log2 units (the sink joins chunk 0
  // only and is counted by one lane of the four that share a row), and the merged state
  // of the run's finished chunks.
  float sig = kNegInf;
  if (c_first == 0 && a.sinks != nullptr && row_ok) sig = a.sinks[row_h] * kLog2e;
  float m = sig;
  float dsum = (sig != kNegInf && cg == 0) ? 1.0f : 0.0f;
  f32x4 o[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float am = kNegInf, ad = 0.f;
  f32x4 ao[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) ao[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto fold_chunk = [&]() {
    const float mn = fmaxf(am, m);
    const float ca = (am == kNegInf) ? 0.f : fast_exp2(am - mn);
    const float cm = (m == kNegInf) ? 0.f : fast_exp2(m - mn);
    ad = __builtin_fmaf(dsum, cm, ad * ca);
#pragma unroll
    for (int t = 0; t < DPL; ++t) ao[t] = o[t] * cm + ao[t] * ca;
    am = mn;
  };

  const float sl2 = a.scale_log2;
  const int causal_first_masked = a.causal ? (lk - a.q_len + 1) : 0x7fffffff;
  const int lim = min(ke - 1, a.causal ? lk - a.q_len + row_t : 0x7fffffff);

  // Stages are issued unconditionally: a stage past the run end reads zeros through
  // the bounded descriptor (no memory traffic), which keeps the copy count per stage
  // constant so one fixed wait suffices.
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue(st);

  int in_chunk = 0;  // stages of the current chunk done
  for (int st = 0; st < nsteps; ++st) {
    // stage st has landed once only the NST-2 stages issued after it are pending
    wait_vmcnt<((NST - 2) * 2 * NDMA < 63 ? (NST - 2) * 2 * NDMA : 63)>();
    stage_barrier();
    issue(st + NST - 1);  // refills the slot every wavefront finished with (st-1)

    const unsigned char* kbuf = ring[st % NST][0];
    const unsigned char* vbuf = ring[st % NST][1];
    const int kbase = kb + st * STEP;

    // ---- S^T = K . Q^T for two 16-key tiles
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
    // ---- mask: keys past the run end, and (causal) keys after the row's position
    if (kbase + STEP > ke || kbase + STEP > causal_first_masked) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kbase + kt * 16 + 4 * cg + j;
          s2[kt][j] = (key <= lim) ? s2[kt][j] : kNegInf;
        }
    }
    // ---- online softmax; the running max is raised only when a row's max grows by
    // more than 2^8 (exact: numerator and denominator share the stale max)
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

    // ---- O^T += V^T . P^T.  V row of slot key i, head dims [DPL*l16, +DPL); d-tile t
    // of the MFMA holds head dim DPL*m + t in row m.
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
      o[t] = mfma16(as_bf16x8(va), pop, o[t]);
    }
    // ---- chunk end: merge its state into the run's and start the next chunk
    if (++in_chunk == chunk_steps && st + 1 < nsteps) {
      fold_chunk();
      in_chunk = 0;
      m = kNegInf;
      dsum = 0.f;
#pragma unroll
      for (int t = 0; t < DPL; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  fold_chunk();

  wait_vmcnt<0>();  // no copy may land after the workgroup's LDS is released

  // ---- epilogue: lane holds head dims [4*cg*DPL, +4*DPL) of its row; O^T element
  // (t, j) is head dim DPL*(4*cg + j) + t.
  float dr = wave_xor_sum(ad, 16);
  dr = wave_xor_sum(dr, 32);
  if (!row_ok) return;
  const float inv = dr > 0.f ? 1.0f / dr : 0.f;
  const float lse_nat = dr > 0.f ? (am + __builtin_log2f(dr)) * kLn2 : kNegInf;
  float vals[4 * DPL];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int t = 0; t < DPL; ++t) vals[j * DPL + t] = ao[t][j] * inv;
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
    float* dst = a.part_o + (qrow * S + slot) * D + d0;
#pragma unroll
    for (int e = 0; e < 4 * DPL; e += 4)
      *(f32x4*)(dst + e) = f32x4{vals[e], vals[e + 1], vals[e + 2], vals[e + 3]};
    if (cg == 0) a.part_lse[qrow * S + slot] = lse_nat;
  }
}

// Chunk-wave decode kernel, for at most 16 query rows per KV head (q_len * G <= 16,
// e.g. single-token decode with G = 8).  Workgroup = CW wavefronts = one (sequence,
// KV head) and CW consecutive chunks of its plan, c = CW * blockIdx.x + w; each
// wavefront streams its own chunk through its own NST-stage LDS ring (asynchronous
// buffer->LDS copies, no barriers) exactly like a one-wavefront split kernel, and the
// CW online-softmax states are then combined in LDS ("Sink attention": blocks along the
// key axis merge by their log-sum-exp; the sink sits in chunk 0).  One partial (or,
// with a single slot, the final output) leaves the workgroup instead of CW of them,
// which cuts the partial traffic written during the KV stream and read by the merge.
template <int D, int CW, bool DIRECT, bool PAGED>
__global__ __launch_bounds__(64 * CW) void decode_cw_kernel(DecodeArgs a,
                                                            const int32_t* __restrict__ page_ids,
                                                            RopeArgs rope) {
  constexpr int KS = D / 32;
  constexpr int DPL = D / 16;
  constexpr int ROW = D * 2;
  constexpr int CPR = D / 8;
  constexpr int STEP = 32;
  // Per-wavefront ring depth: 2 stages keep the workgroup under half the LDS, so two
  // workgroups share a CU and one's start-up and drain overlap the other's stream
  // (measured faster than 4 stages at one workgroup per CU).
  constexpr int NST = 2;
  constexpr int SB = STEP * ROW;
  constexpr int NDMA = SB / (64 * 16);    // copies per lane per tensor per stage
  static_assert(CW * NST * 2 * SB <= 160 * 1024, "LDS");
  static_assert(CW * 16 * (D + 2) * 4 <= CW * NST * 2 * SB, "combine scratch fits the rings");
  // One LDS object holds the rings, the Q tiles and the sinks (with separate objects
  // the compiler cannot tell the ring reads from the copies in flight and waits for all
  // of them before every stage).
  struct Smem {
    unsigned char ring[CW][NST][2][SB];
    unsigned char q[CW][16 * ROW];
    float sink[CW][64];
  };
  __shared__ __attribute__((aligned(16))) Smem sm;
  auto& ring = sm.ring;
  auto& q_lds = sm.q;
  auto& sink_lds = sm.sink;

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int l16 = lane & 15;
  const int cg = lane >> 4;
  const int slot = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int M = a.q_len * G;
  const int S = a.num_slots;

  int kv0 = 0, e0 = 0, lk;
  if constexpr (PAGED) {
    e0 = page_begin(a, b);
    lk = paged_len(a, b, e0);
  } else {
    kv0 = seq_begin(a, b);
    lk = seq_end(a, b) - kv0;
  }
  const int n = plan_chunks(lk, a.num_splits, CW);
  const int cl = chunk_len(lk, n);

  // The lane's query row R = l16 -> (draft token t, query head h).
  const int row_t = l16 / G;
  const int row_h = g * G + (l16 - row_t * G);
  const bool row_ok = l16 < M;
  const int64_t qrow = ((int64_t)b * a.q_len + row_t) * Hq + row_h;

  if (slot * CW >= n) {  // unused slot: no mass
    if (!DIRECT && w == 0 && cg == 0 && row_ok) a.part_lse[qrow * S + slot] = kNegInf;
    return;
  }
  const int c = slot * CW + w;
  const int kb = min(lk, c * cl);
  const int ke = (c < n) ? min(lk, kb + cl) : kb;
  const int nsteps = (ke - kb + STEP - 1) / STEP;

  // K/V views as in the split kernel (one chunk view, or per-page views when paged).
  const size_t head_base = PAGED ? 0 : ((size_t)g * a.total_kv + kv0 + kb) * D;
  const uint32_t chunk_bytes = PAGED ? 0u : (uint32_t)(ke - kb) * ROW;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + head_base, chunk_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + head_base, chunk_bytes);
  unsigned char (*my)[2][SB] = ring[w];
  auto issue = [&](int st) {
    unsigned char* kbuf = my[st % NST][0];
    unsigned char* vbuf = my[st % NST][1];
    if constexpr (PAGED) {
      const int t0 = kb + st * STEP;
      const int ps = a.page_size;
      const int pa = t0 / ps;
      __amdgpu_buffer_rsrc_t ka, va, kb2, vb2;
      page_views<D>(a, page_ids, e0, g, pa, ke, ka, va);
      page_views<D>(a, page_ids, e0, g, pa + 1, ke, kb2, vb2);
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int p = i * 64 + lane;
        const int row = p / CPR;
        const int cc = p - row * CPR;
        const int tok0 = t0 + i * (64 / CPR);
        const bool second = tok0 / ps != pa;
        const uint32_t rbase = (uint32_t)(t0 + row - (pa + (second ? 1 : 0)) * ps) * ROW;
        dma16_nt(second ? kb2 : ka, rbase + (uint32_t)((cc ^ dswz<D>(row)) * 16), kbuf + i * 1024);
        dma16_nt(second ? vb2 : va, rbase + (uint32_t)(cc * 16), vbuf + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int p = i * 64 + lane;            // 16-byte chunk index inside the stage
        const int row = p / CPR;
        const int cc = p - row * CPR;
        const uint32_t rbase = (uint32_t)(st * STEP + row) * ROW;
        dma16_nt(kr, rbase + (uint32_t)((cc ^ dswz<D>(row)) * 16), kbuf + i * 1024);
        dma16_nt(vr, rbase + (uint32_t)(cc * 16), vbuf + i * 1024);
      }
    }
  };

  // The 16 Q rows and the sinks arrive through asynchronous copies into LDS issued
  // ahead of the ring prologue, so no register load is pending when the stage loop
  // starts (a pending one would make the loop wait for the whole prologue).
  {
    const uint32_t qbytes = (uint32_t)(a.q_len * Hq * ROW);
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc((const __bf16*)a.q + (size_t)b * a.q_len * Hq * D, qbytes);
#pragma unroll
    for (int i = 0; i < 16 * CPR / 64; ++i) {
      const int p = i * 64 + lane;            // 16-byte piece of the [16][D] Q tile
      const int r = p / CPR;
      const int rt = r / G;
      const int rh = g * G + (r - rt * G);
      const uint32_t off = (r < M) ? (uint32_t)((rt * Hq + rh) * ROW + (p - r * CPR) * 16) : qbytes;
      dma16(qr, off, &q_lds[w][i * 1024]);
    }
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.sinks, a.sinks != nullptr ? (uint32_t)Hq * 4 : 0u);
    dma4(sr, (c == 0 && row_ok) ? (uint32_t)row_h * 4 : kNoRead, &sink_lds[w][0]);
  }

#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue(st);
  wait_vmcnt<(NST - 1) * 2 * NDMA>();  // the Q rows and sinks (issued first) have landed

  // Q^T operands (B of S^T): lane holds Q[row][ks*32 + cg*8 .. +8]; zero for padding.
  bf16x8 qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qop[ks] = *(const bf16x8*)&q_lds[w][l16 * ROW + (ks * 32 + cg * 8) * 2];
  if (rope.enabled) {  // YaRN rotation of the query row at position Lk - q_len + t
    const int64_t pos = (int64_t)lk - a.q_len + row_t;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) rope_rotate8(qop[ks], qop[ks + KS / 2], ks * 32 + cg * 8, pos, rope);
  }
  const float sig = (c == 0 && a.sinks != nullptr && row_ok) ? sink_lds[w][lane] * kLog2e : kNegInf;
  float m = sig;
  float dsum = (sig != kNegInf && cg == 0) ? 1.0f : 0.0f;
  f32x4 o[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const float sl2 = a.scale_log2;
  const int causal_first_masked = a.causal ? (lk - a.q_len + 1) : 0x7fffffff;
  const int lim = min(ke - 1, a.causal ? lk - a.q_len + row_t : 0x7fffffff);

  for (int st = 0; st < nsteps; ++st) {
    // The ring is this wavefront's own and its reads of slot (st-1) completed in the
    // previous iteration, so that slot is refilled before waiting: NST stages are in
    // flight during the wait.  Stage st has landed once only the NST-1 stages issued
    // after it are pending.
    issue(st + NST - 1);
    wait_vmcnt<(NST - 1) * 2 * NDMA>();

    const unsigned char* kbuf = my[st % NST][0];
    const unsigned char* vbuf = my[st % NST][1];
    const int kbase = kb + st * STEP;

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
    if (kbase + STEP > ke || kbase + STEP > causal_first_masked) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kbase + kt * 16 + 4 * cg + j;
          s2[kt][j] = (key <= lim) ? s2[kt][j] : kNegInf;
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
  }

  // ---- combine the CW chunk states.  Wavefront w leaves, per row, its max (log2
  // units), its sum and its unnormalised output (head dim DPL*(4*cg + j) + t of O^T
  // element (t, j)) in LDS, over its own ring.
  wait_vmcnt<0>();
  __syncthreads();
  float dr = wave_xor_sum(dsum, 16);
  dr = wave_xor_sum(dr, 32);
  float* red = (float*)&ring[0][0][0][0];          // [CW][16][D] outputs, then m, d
  float* red_m = red + CW * 16 * D;                // [CW][16]
  float* red_d = red_m + CW * 16;                  // [CW][16]
  {
    float* dst = red + (w * 16 + l16) * D + 4 * cg * DPL;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < DPL; t += 4)
        *(f32x4*)(dst + j * DPL + t) = f32x4{o[t][j], o[t + 1][j], o[t + 2][j], o[t + 3][j]};
    if (cg == 0) {
      red_m[w * 16 + l16] = m;
      red_d[w * 16 + l16] = dr;
    }
  }
  __syncthreads();
  // Wavefront w writes rows [16/CW * w, +16/CW); LPR lanes per row, four dims each.
  constexpr int LPR = D / 4;
  constexpr int RPP = 64 / LPR;                    // rows per pass
  constexpr int RPW = 16 / CW;                     // rows per wavefront
#pragma unroll
  for (int r0 = 0; r0 < RPW; r0 += RPP) {
    const int r = w * RPW + r0 + lane / LPR;
    const int q4 = lane % LPR;
    if (r0 + lane / LPR >= RPW || r >= M) continue;
    float mstar = kNegInf;
#pragma unroll
    for (int x = 0; x < CW; ++x) mstar = fmaxf(mstar, red_m[x * 16 + r]);
    const float msub = (mstar == kNegInf) ? 0.0f : mstar;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll
    for (int x = 0; x < CW; ++x) {
      const float dx = red_d[x * 16 + r];
      const float sc = (dx > 0.f) ? fast_exp2(red_m[x * 16 + r] - msub) : 0.f;
      den = __builtin_fmaf(sc, dx, den);
      const f32x4 ox = *(const f32x4*)(red + (x * 16 + r) * D + 4 * q4);
      acc[0] = __builtin_fmaf(sc, ox[0], acc[0]);
      acc[1] = __builtin_fmaf(sc, ox[1], acc[1]);
      acc[2] = __builtin_fmaf(sc, ox[2], acc[2]);
      acc[3] = __builtin_fmaf(sc, ox[3], acc[3]);
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    const float lse_nat = den > 0.f ? (msub + __builtin_log2f(den)) * kLn2 : kNegInf;
    const int rt = r / G;
    const int64_t orow = ((int64_t)b * a.q_len + rt) * Hq + g * G + (r - rt * G);
    if constexpr (DIRECT) {
      u32x2 pk2;
      pk2.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      pk2.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
      *(u32x2*)((__bf16*)a.out + orow * D + 4 * q4) = pk2;
      if (q4 == 0 && a.lse != nullptr) a.lse[orow] = lse_nat;
    } else {
      *(f32x4*)(a.part_o + (orow * S + slot) * D + 4 * q4) =
          f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
      if (q4 == 0) a.part_lse[orow * S + slot] = lse_nat;
    }
  }
}

// Merge: D/4 lanes per row, each owning four consecutive head dims, so a row's
// partial outputs are read as whole 16-byte vectors and a wavefront covers 256/D rows.
// Slots are taken eight at a time, their loads issued together (eight in flight per
// lane measured 11 % faster than four on 32 slots).  A slot with lse = -inf has weight 0
// and its partial output (possibly never written) is selected away, never multiplied.
// The partials are read once, with the non-temporal cache policy.  counts (optional): row r
// merges only its first counts[r] slots (clamped to [0, S]); the rest are not read.
constexpr int kMergeThreads = 128;
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_lse,
                                                              const int32_t* __restrict__ counts,
                                                              int64_t rows, int S, __bf16* out,
                                                              float* lse) {
  constexpr int LPR = D / 4;
  constexpr int RPB = kMergeThreads / LPR;
  const int q = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  if (row >= rows) return;
  const float* pl = part_lse + row * S;
  const f32x4* po = (const f32x4*)(part_o + row * S * D) + q;
  const int n = counts != nullptr ? min(max(counts[row], 0), S) : S;
  float mx = kNegInf;
  for (int c = 0; c < n; c += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = (c + u < n) ? __builtin_nontemporal_load(pl + c + u) : kNegInf;
#pragma unroll
    for (int u = 0; u < 8; ++u) mx = fmaxf(mx, t[u]);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != kNegInf) {  // then n >= 1
    for (int c = 0; c < n; c += 8) {
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = (c + u < n) ? __expf(__builtin_nontemporal_load(pl + c + u) - mx) : 0.f;
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(po + (size_t)min(c + u, n - 1) * (D / 4));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        wsum += w[u];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[e] = (w[u] != 0.f) ? __builtin_fmaf(w[u], x[u][e], acc[e]) : acc[e];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  u32x2 pk;
  pk.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(u32x2*)(out + row * D + 4 * q) = pk;
  if (q == 0 && lse != nullptr) lse[row] = wsum > 0.f ? mx + __logf(wsum) : kNegInf;
}

template <int D, bool DIRECT, bool PAGED>
static void launch_split_d(const DecodeArgs& a, int w, dim3 grid, const int32_t* ids,
                           const RopeArgs& r, hipStream_t st) {
  switch (w) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, DIRECT, PAGED>), grid, dim3(64), 0, st, a, ids, r); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, DIRECT, PAGED>), grid, dim3(128), 0, st, a, ids, r); break;
    default: hipLaunchKernelGGL((decode_split_kernel<D, 4, DIRECT, PAGED>), grid, dim3(256), 0, st, a, ids, r); break;
  }
}

template <bool DIRECT, bool PAGED>
static void launch_decode_mode(const DecodeArgs& a, int head_dim, int batch, int num_kv_heads,
                               const int32_t* ids, const RopeArgs& r, hipStream_t stream) {
  if (a.chunk_waves > 1) {  // q_len * G <= 16: chunk-wave kernel, one row group
    dim3 grid(a.num_slots, num_kv_heads, batch);
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_cw_kernel<64, 4, DIRECT, PAGED>), grid, dim3(256), 0, stream, a, ids, r);
    else
      hipLaunchKernelGGL((decode_cw_kernel<128, 2, DIRECT, PAGED>), grid, dim3(128), 0, stream, a, ids, r);
    return;
  }
  const int w = decode_waves(a.q_len * a.group);
  dim3 grid(a.num_slots, num_kv_heads * a.row_groups, batch);
  if (head_dim == 64) launch_split_d<64, DIRECT, PAGED>(a, w, grid, ids, r, stream);
  else launch_split_d<128, DIRECT, PAGED>(a, w, grid, ids, r, stream);
}

hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int batch, int num_kv_heads,
                               bool direct, const int32_t* page_ids, const RopeArgs& rope,
                               hipStream_t stream) {
  if (page_ids != nullptr) {
    if (direct) launch_decode_mode<true, true>(a, head_dim, batch, num_kv_heads, page_ids, rope, stream);
    else launch_decode_mode<false, true>(a, head_dim, batch, num_kv_heads, page_ids, rope, stream);
  } else {
    if (direct) launch_decode_mode<true, false>(a, head_dim, batch, num_kv_heads, nullptr, rope, stream);
    else launch_decode_mode<false, false>(a, head_dim, batch, num_kv_heads, nullptr, rope, stream);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const float* part_o, const float* part_lse, const int32_t* counts,
                        int64_t rows, int num_slots, int head_dim, void* out, float* lse,
                        hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)((rows + 7) / 8)), dim3(kMergeThreads),
                       0, stream, part_o, part_lse, counts, rows, num_slots, (__bf16*)out, lse);
  else
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)((rows + 3) / 4)), dim3(kMergeThreads),
                       0, stream, part_o, part_lse, counts, rows, num_slots, (__bf16*)out, lse);
  return hipGetLastError();
}

}  // namespace sa
