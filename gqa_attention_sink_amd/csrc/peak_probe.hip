// Achievable-peak probes for the measurement harness (not part of the attention path):
// how fast this chip streams HBM with the read pattern the decode kernels use, how many
// bf16 MFMA flops it sustains when nothing else runs, how many when softmax-like vector
// work shares the SIMD (issued by the same wavefront or by its neighbour), and the issue
// rate of the softmax's vector instructions.  The attention kernels'
// roofline fractions are quoted against the spec-sheet peaks; these give the measured
// ceilings beside them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sink_attn_peak.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane

// Every 16-byte piece of [p, p + n16*16) is read once, with the non-temporal policy the
// decode kernels use.  Like them, each workgroup streams one contiguous span (its share
// of the buffer, in order); lane i of a wavefront reads piece i of a contiguous KiB, so
// every load instruction is one coalesced KiB, and kUnroll loads per lane are in flight.
// Indices stay inside [begin, end) by construction.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                               int64_t n16, uint32_t* out) {
  const int64_t span = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * span;
  const int64_t end = begin + span < n16 ? begin + span : n16;
  int64_t i = begin + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(p + i + k * kThreads);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < end; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the loads must not be removed: the result is stored in the rare case it matches
  if (acc == 0x9e3779b9u) out[0] = acc;
}

// Eight independent chains of v_mfma_f32_32x32x16_bf16 per wavefront, no memory traffic
// inside the loop; each lane stores one sum at the end (out has grid * 256 floats).
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((lane + j) & 7));
    b[j] = (__bf16)(0.002f * (float)((lane * 3 + j) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][15];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// MFMA issue beside softmax-like vector work: per v_mfma_f32_32x32x16_bf16 of a chain,
// E pairs of one FMA and one exp2 (the arithmetic of one score of an online softmax), on
// independent registers.
//   SPLIT false: workgroups of 4 wavefronts (one per SIMD); each issues MFMA i and then
//     its E pairs, in that order (fenced from the scheduler), as a wavefront that
//     software-pipelines its own exponentials against its own MFMAs would.
//   SPLIT true: workgroups of 8 wavefronts (two per SIMD); wavefronts 0-3 issue only the
//     MFMAs, 4-7 only the pairs, E per MFMA of the neighbour, as in a ping-pong schedule.
// Either way the MFMA chains are those of mfma_loop_kernel's first four wavefronts.
template <int E, bool SPLIT>
__global__ __launch_bounds__(512) void coissue_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  float s = 0.f;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.01f * (float)((lane + j) & 15);
  if (!SPLIT || w < 4) {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = (__bf16)(0.001f * (float)((lane + j) & 7));
      b[j] = (__bf16)(0.002f * (float)((lane * 3 + j) & 7));
    }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        if (!SPLIT) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            x[(c * E + e) & 7] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[(c * E + e) & 7], 0.999f, -0.001f));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][15];
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int e = 0; e < 8 * E; ++e) x[e & 7] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e & 7], 0.999f, -0.001f));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = s;
}

// Vector issue rate: each wavefront runs iters x 8 independent chains of one instruction
// (OP 0: v_exp_f32 of the negated value, OP 1: v_fma_f32), W wavefronts per SIMD, no
// memory traffic inside the loop.  out has grid * 256 * W floats: lane 0 of each
// wavefront stores the shader-clock cycles its loop took (so the rate does not depend on
// the clock the GPU runs at), the other lanes their sums.
template <int OP, int W>
__global__ __launch_bounds__(256 * W) void valu_rate_kernel(int iters, float a, float b, float* out) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.25f + 0.01f * (float)(threadIdx.x & 7) + 0.001f * (float)i;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (OP == 0) x[i] = __builtin_amdgcn_exp2f(-x[i]);
      else x[i] = __builtin_fmaf(x[i], a, b);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  out[(int64_t)blockIdx.x * 256 * W + threadIdx.x] = (threadIdx.x & 63) == 0 ? (float)(t1 - t0) : s;
}

template <int OP>
void launch_valu(int waves, int iters, int blocks, float* out, hipStream_t st) {
  const dim3 g((unsigned)blocks);
  switch (waves) {
    case 1: hipLaunchKernelGGL((valu_rate_kernel<OP, 1>), g, dim3(256), 0, st, iters, 0.999f, 0.001f, out); break;
    case 2: hipLaunchKernelGGL((valu_rate_kernel<OP, 2>), g, dim3(512), 0, st, iters, 0.999f, 0.001f, out); break;
    default: hipLaunchKernelGGL((valu_rate_kernel<OP, 4>), g, dim3(1024), 0, st, iters, 0.999f, 0.001f, out); break;
  }
}

template <int E>
void launch_coissue(bool split, int iters, int blocks, float* out, hipStream_t st) {
  if (split)
    hipLaunchKernelGGL((coissue_kernel<E, true>), dim3((unsigned)blocks), dim3(512), 0, st, iters, out);
  else
    hipLaunchKernelGGL((coissue_kernel<E, false>), dim3((unsigned)blocks), dim3(256), 0, st, iters, out);
}

}  // namespace

extern "C" {

int sink_attn_peak_stream_read(const void* buf, size_t bytes, int32_t num_blocks, void* out4,
                               void* stream) {
  if (!buf || !out4 || bytes == 0 || (bytes & 15u) != 0 || ((uintptr_t)buf & 15u) != 0 ||
      num_blocks < 1)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)num_blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (const u32x4*)buf, (int64_t)(bytes / 16),
                     (uint32_t*)out4);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int sink_attn_peak_mfma_bf16(int32_t iters, int32_t num_blocks, float* out, void* stream) {
  if (!out || iters < 1 || num_blocks < 1) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)num_blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (int)iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int sink_attn_peak_coissue(int32_t pairs_per_mfma, int32_t split, int32_t iters,
                           int32_t num_blocks, float* out, void* stream) {
  if (!out || iters < 1 || num_blocks < 1 || pairs_per_mfma < 0 || pairs_per_mfma > 4) return 1;
  const hipStream_t st = (hipStream_t)stream;
  switch (pairs_per_mfma) {
    case 0: launch_coissue<0>(split != 0, iters, num_blocks, out, st); break;
    case 1: launch_coissue<1>(split != 0, iters, num_blocks, out, st); break;
    case 2: launch_coissue<2>(split != 0, iters, num_blocks, out, st); break;
    case 3: launch_coissue<3>(split != 0, iters, num_blocks, out, st); break;
    default: launch_coissue<4>(split != 0, iters, num_blocks, out, st); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int sink_attn_peak_valu(int32_t op, int32_t waves_per_simd, int32_t iters, int32_t num_blocks,
                        float* out, void* stream) {
  if (!out || iters < 1 || num_blocks < 1 || (op != 0 && op != 1) ||
      (waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4))
    return 1;
  const hipStream_t st = (hipStream_t)stream;
  if (op == 0) launch_valu<0>(waves_per_simd, iters, num_blocks, out, st);
  else launch_valu<1>(waves_per_simd, iters, num_blocks, out, st);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
