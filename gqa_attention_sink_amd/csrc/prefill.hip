// Causal variable-length prefill kernel for gfx950.
//
// "GPT-OSS on day 0", "Kernels for GPT-OSS" > "Sink attention": softmax(q.K^T*scale
// + sink).V with the online (max-subtracted) softmax started from (m, d) = (sink, 1);
// the whole key range of a row is handled by one wavefront, so the sink is counted
// exactly once.
//
// Work unit (one workgroup of 4 wavefronts): one sequence, 64*pw query positions and
// hg query heads that share one KV head (GQA), hg*pw = 4.  Each wavefront owns 64
// query rows of one head (two 32-row MFMA column tiles).  K/V tiles of 64 keys are
// staged in LDS once per workgroup and read by all four wavefronts; the next tile's
// global loads are issued before the current tile is computed.
//
// Scores are computed transposed, S^T = K . Q^T (v_mfma_f32_32x32x16_bf16), so each
// lane holds scores of one query row: the P^T accumulator is directly the B operand
// of O^T = V^T . P^T and the per-row softmax state is lane-local (one cross-lane max
// per tile between the two lanes of a row).  V^T operands are assembled from 8-byte
// LDS reads of 8 key rows and a register transpose.  Workgroups are dispatched
// heaviest causal tile first.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

template <int D>
struct PrefillCfg {
  static constexpr int BC = 64;          // keys per tile
  static constexpr int KS = D / 16;      // k-steps of S^T (16 head dims each)
  static constexpr int DT = D / 32;      // d-tiles of O^T (32 head dims each)
  static constexpr int CPR = D / 8;      // 16-byte chunks per K/V row
  static constexpr int ROW = D * 2;      // bytes per K/V row
  static constexpr int TILE = BC * ROW;  // bytes per K (or V) tile
  static constexpr int NLD = BC * CPR / 256;  // 16-byte loads per thread per tensor
};

// XOR swizzle of 16-byte chunks inside a K row so that the 32 rows read by one MFMA
// operand load fall into distinct LDS banks.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}

template <int D>
__global__ __launch_bounds__(256, 1) void prefill_kernel(PrefillArgs a) {
  using C = PrefillCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[C::TILE];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v[C::TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int cg = lane >> 5;
  const int Hq = a.num_q_heads;

  const int hgi = blockIdx.x;
  const int g = hgi / a.n_hgroups;
  const int hgrp = hgi - g * a.n_hgroups;
  const int b = blockIdx.y;
  const int qt = a.n_qtiles - 1 - (int)blockIdx.z;  // heaviest tiles dispatched first

  const int q0 = a.cu_q[b];
  const int lq = a.cu_q[b + 1] - q0;
  const int kv0 = a.cu_kv[b];
  const int lk = a.cu_kv[b + 1] - kv0;
  const int wg_p0 = qt * 64 * a.pw;
  if (wg_p0 >= lq) return;
  const int off = lk - lq;  // bottom-right causal alignment

  const bool active = (wave / a.hg) < a.pw;
  const int h = g * a.group + hgrp * a.hg + (wave % a.hg);
  const int p0 = wg_p0 + (wave / a.hg) * 64;

  int kend_wg = a.causal ? min(lk, wg_p0 + 64 * a.pw + off) : lk;
  kend_wg = max(kend_wg, 0);
  const int ntiles = (kend_wg + C::BC - 1) / C::BC;
  int kend_w = a.causal ? min(lk, p0 + 64 + off) : lk;
  kend_w = max(kend_w, 0);
  const bool has_rows = active && p0 < lq;

  // ---- Q^T operands: lane holds Q[p0 + nt*32 + l32][h][ks*16 + cg*8 .. +8]
  bf16x8 qop[2][C::KS];
  {
    const int nrows = max(0, min(64, lq - p0));
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc((const __bf16*)a.q + ((size_t)(q0 + max(p0, 0)) * Hq) * D,
                  has_rows ? (uint32_t)(nrows * Hq * C::ROW) : 0u);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const uint32_t o = (uint32_t)(((nt * 32 + l32) * Hq + h) * C::ROW + (ks * 16 + cg * 8) * 2);
        qop[nt][ks] = as_bf16x8(load16(qr, o));
      }
  }

  // ---- online-softmax state (log2 units), started from the head's sink
  const float sig = (a.sinks != nullptr && active) ? a.sinks[h] * kLog2e : kNegInf;
  float m[2] = {sig, sig};
  const float d_init = (sig != kNegInf && cg == 0) ? 1.0f : 0.0f;  // counted once per row
  float dsum[2] = {d_init, d_init};
  f32x16 o[C::DT][2];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[t][nt][j] = 0.f;

  const size_t head_base = ((size_t)g * a.total_kv + kv0) * D;
  const float sl2 = a.scale_log2;

  // ---- global -> register -> LDS staging of one K/V tile
  u32x4 kreg[C::NLD], vreg[C::NLD];
  auto gload = [&](int kb) {
    const uint32_t bytes = (uint32_t)max(0, min(C::BC, lk - kb)) * C::ROW;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + head_base + (size_t)kb * D, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + head_base + (size_t)kb * D, bytes);
#pragma unroll
    for (int i = 0; i < C::NLD; ++i) {
      const int id = tid + 256 * i;
      kreg[i] = load16(kr, (uint32_t)id * 16);
      vreg[i] = load16(vr, (uint32_t)id * 16);
    }
  };
  auto lwrite = [&]() {
#pragma unroll
    for (int i = 0; i < C::NLD; ++i) {
      const int id = tid + 256 * i;
      const int row = id / C::CPR;
      const int cc = id - row * C::CPR;
      *(u32x4*)(lds_k + row * C::ROW + ((cc ^ kswz<D>(row)) * 16)) = kreg[i];
      *(u32x4*)(lds_v + id * 16) = vreg[i];
    }
  };

  if (ntiles > 0) {
    gload(0);
    lwrite();
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int kb = it * C::BC;
    if (it + 1 < ntiles) gload(kb + C::BC);

    if (has_rows && kb < kend_w) {
      // ---- S^T[key][row] for two 32-key tiles x two 32-row tiles
      f32x16 s[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int j = 0; j < 16; ++j) s[kt][nt][j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int row = kt * 32 + l32;
          const int cc = ks * 2 + cg;
          const bf16x8 ka = as_bf16x8(*(const u32x4*)(lds_k + row * C::ROW + ((cc ^ kswz<D>(row)) * 16)));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) s[kt][nt] = mfma32(ka, qop[nt][ks], s[kt][nt]);
        }
      }

      // ---- mask (only tiles that cross the causal diagonal or the sequence end).
      // Accumulator element j of key tile kt is key kb + kt*32 + 8*(j/4) + 4*cg + j%4.
      const bool need_mask = (kb + C::BC > lk) || (a.causal && kb + C::BC - 1 > p0 + off);
      if (need_mask) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int pos = p0 + nt * 32 + l32;
          const int lim = a.causal ? min(lk - 1, pos + off) : lk - 1;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int key = kb + kt * 32 + 8 * (j >> 2) + 4 * cg + (j & 3);
              s[kt][nt][j] = (key <= lim) ? s[kt][nt][j] : kNegInf;
            }
        }
      }

      // ---- online softmax; P^T packed as the B operands of the four 16-key PV steps
      bf16x8 pop[2][2][2];  // [kt][kk][nt]
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kt][nt][j]);
        mx = wave_xor_max(mx, 32);
        const float mnew = fmaxf(m[nt], mx * sl2);
        const bool dead = (mnew == kNegInf);
        const float alpha = dead ? 1.0f : fast_exp2(m[nt] - mnew);
        const float msub = dead ? 0.0f : mnew;
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          float p[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            p[j] = fast_exp2(__builtin_fmaf(s[kt][nt][j], sl2, -msub));
            ps += p[j];
          }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            u32x4 pk;
            pk.x = pack_bf16x2(p[kk * 8 + 0], p[kk * 8 + 1]);
            pk.y = pack_bf16x2(p[kk * 8 + 2], p[kk * 8 + 3]);
            pk.z = pack_bf16x2(p[kk * 8 + 4], p[kk * 8 + 5]);
            pk.w = pack_bf16x2(p[kk * 8 + 6], p[kk * 8 + 7]);
            pop[kt][kk][nt] = as_bf16x8(pk);
          }
        }
        dsum[nt] = __builtin_fmaf(dsum[nt], alpha, ps);
        m[nt] = mnew;
#pragma unroll
        for (int t = 0; t < C::DT; ++t) o[t][nt] *= alpha;
      }

      // ---- O^T += V^T . P^T.  Slot i of 16-key step (kt, kk) for k-group cg is key
      // kt*32 + 16*kk + 8*(i/4) + 4*cg + i%4; the lane reads DT head dims
      // [DT*l32, DT*l32 + DT) of those 8 rows and transposes them in registers, so
      // d-tile t holds head dim DT*m + t in MFMA row m.
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          uint32_t vw[8][C::DT / 2];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = kt * 32 + 16 * kk + 8 * (i >> 2) + 4 * cg + (i & 3);
            const unsigned char* src = lds_v + row * C::ROW + l32 * C::DT * 2;
            if constexpr (C::DT == 4) {
              const u32x2 t2 = *(const u32x2*)src;
              vw[i][0] = t2.x;
              vw[i][1] = t2.y;
            } else {
              vw[i][0] = *(const uint32_t*)src;
            }
          }
#pragma unroll
          for (int t = 0; t < C::DT; ++t) {
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
            for (int nt = 0; nt < 2; ++nt) o[t][nt] = mfma32(vop, pop[kt][kk][nt], o[t][nt]);
          }
        }
    }

    __syncthreads();
    if (it + 1 < ntiles) lwrite();
    __syncthreads();
  }

  if (!has_rows) return;
  // ---- epilogue.  O^T element (t, j) of column tile nt is head dim
  // DT*(8*(j/4) + 4*cg + j%4) + t of query position p0 + nt*32 + l32.
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float dr = wave_xor_sum(dsum[nt], 32);
    const int pos = p0 + nt * 32 + l32;
    if (pos >= lq) continue;
    const float inv = dr > 0.f ? 1.0f / dr : 0.f;
    const size_t orow = (size_t)(q0 + pos) * Hq + h;
    __bf16* dst = (__bf16*)a.out + orow * D;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float vals[4 * C::DT];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int t = 0; t < C::DT; ++t) vals[jj * C::DT + t] = o[t][nt][q4 * 4 + jj] * inv;
      const int d0 = C::DT * (8 * q4 + 4 * cg);
#pragma unroll
      for (int e = 0; e < 4 * C::DT; e += 8) {
        u32x4 w4;
        w4.x = pack_bf16x2(vals[e + 0], vals[e + 1]);
        w4.y = pack_bf16x2(vals[e + 2], vals[e + 3]);
        w4.z = pack_bf16x2(vals[e + 4], vals[e + 5]);
        w4.w = pack_bf16x2(vals[e + 6], vals[e + 7]);
        *(u32x4*)(dst + d0 + e) = w4;
      }
    }
    if (cg == 0 && a.lse != nullptr)
      a.lse[orow] = dr > 0.f ? (m[nt] + __builtin_log2f(dr)) * kLn2 : kNegInf;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int num_kv_heads, hipStream_t stream) {
  dim3 grid((unsigned)(num_kv_heads * a.n_hgroups), (unsigned)a.batch, (unsigned)a.n_qtiles);
  if (head_dim == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
