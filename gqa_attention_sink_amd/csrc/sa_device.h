// Device helpers for the gfx950 sink-attention kernels: MFMA wrappers, bounded
// buffer loads, bf16 packing and the exp2-domain online-softmax constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Raw buffer descriptor word 3 for gfx9-family raw (untyped) buffers.
constexpr int kBufferWord3 = 0x00020000;

// A bounded view of `bytes` bytes at `base`: loads at offsets >= bytes return zero
// instead of touching memory, which is how every tail (keys past a sequence's end,
// queries past a tile) is handled without branches or faults.
// Both arguments must be wave-uniform; they are pinned to scalar registers so the
// descriptor never needs a per-lane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* up = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(up, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           kBufferWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Asynchronous 16-byte copy global -> LDS (no registers): lane i of the wavefront
// writes its 16 bytes at lds_wave_base + 16*i.  lds_wave_base must be wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, off, 0, 0, 0);
}
// The same copy with the non-temporal cache policy (nt), for data read once per launch:
// streamed this way HBM delivers ~6.7-6.8 TB/s to 1024 wavefronts against ~5.9 TB/s with
// the default policy (measured with plain register loads and with LDS rings alike).
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, off, 0, 0, kCachePolicyNT);
}

// The same bounded view as four descriptor words in scalar registers (base address,
// stride 0, size in bytes, raw-buffer word 3), for the assembly copy below.
__device__ __forceinline__ u32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xffffu;
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = (uint32_t)kBufferWord3;
  return r;
}

// dma16 written as assembly: the compiler does not see that the copy writes LDS, so it
// attaches no wait for it to later LDS reads.  Callers order every LDS read of the
// copied bytes after their own wait_vmcnt and a workgroup barrier.  lds_base must be
// wave-uniform.
__device__ __forceinline__ void dma16_asm(u32x4 rsrc, uint32_t off, uint32_t lds_base) {
  // the LDS destination goes through M0, which the compiler loads for the statement
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// An offset no bounded view reaches (views are < 2^31 bytes): the copy reads nothing
// and writes zeros.
constexpr uint32_t kNoRead = 0x80000000u;

// Asynchronous 4-byte copy global -> LDS: lane i writes its 4 bytes at base + 4*i.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_wave_base, 4, off, 0, 0, 0);
}

// Workgroup barrier for the streaming loops, without the memory-model fences that
// __syncthreads() adds: the release fence would wait for every outstanding vector-memory
// operation, including the asynchronous LDS copies issued stages ahead, and so drain
// the ring at every stage.  Callers wait for the copies they need (wait_vmcnt) and their
// LDS reads are consumed before the barrier; the memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most N vector-memory operations of this wavefront are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | 0x0F70);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, fp32) += A(16x32) * B(32x16), bf16 inputs.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// D(32x32, fp32) += A(32x16) * B(16x32), bf16 inputs.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 values -> a packed bf16 pair (lo in bits 0-15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// max / sum over the two lanes l and l^32 (the two halves of the wavefront).
__device__ __forceinline__ float half_swap_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }
__device__ __forceinline__ float half_swap_sum(float v) { return v + __shfl_xor(v, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max over the four lanes l, l^16, l^32, l^48 with the lane-swap instructions (VALU, no
// LDS round trip): with both operands holding v, v_permlane16_swap leaves the values of
// the even and of the odd 16-lane rows in the two registers (each in both rows of a
// pair), and v_permlane32_swap does the same for the two halves.  The s_nop covers the
// wait a swap needs after a VALU write of its operands.
__device__ __forceinline__ float max_over_16_32(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  float m = fmaxf(a, b);
  float c = m, e = m;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(c), "+v"(e));
  return fmaxf(c, e);
}

__device__ __forceinline__ float wave_xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

// Halves of two packed bf16 pairs: (lo16(x), lo16(y)) and (hi16(x), hi16(y)).
// (v_perm_b32 selects bytes from {y:x}, x being bytes 0-3.)
__device__ __forceinline__ uint32_t lo_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// Transposing LDS read of 16-bit data (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j supplies the address of an 8-byte piece (4 elements); lane i receives
// element i%4 of the pieces of lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.  With lane j
// pointing at row j/4, columns 4*(j%4)..+3 of a 4-row x 16-column block, lane i gets
// column i of the 4 rows.  Written as inline assembly so that no wait for pending
// buffer->LDS copies is attached to it: the caller orders it after its own waits and
// barrier, and must call lds_wait() before using the result.
// `off` must fold to a constant in [0, 65535] (the instruction's immediate offset).
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t lds_addr, const int off) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(off) : "memory");
  return r;
}
// The same read through the compiler builtin, from a pointer into a __shared__ object
// (so that the compiler knows which object it reads): the compiler sees the load and
// places the wait before the first use itself.
__device__ __forceinline__ u32x2 ds_read_tr16_c(const void* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(void*)p);
  return __builtin_bit_cast(u32x2, r);
}
// Wait for all outstanding LDS reads; ties the given registers to the wait.
__device__ __forceinline__ void lds_wait(u32x2& a, u32x2& b, u32x2& c, u32x2& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : : "memory");
}
// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Index of the calling wavefront inside its workgroup, as a wave-uniform value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Scheduling-group hints (instruction classes of sched_group_barrier).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedValu = 0x002;
constexpr int kSchedDsRead = 0x100;

}  // namespace sa
