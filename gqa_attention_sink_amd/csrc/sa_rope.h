// YaRN rotary position encoding on the device ("GPT-OSS on day 0", model deltas: YaRN
// position encoding as in DeepSeek-V3; the published YaRN method: rotary embedding with
// NTK-by-parts frequency interpolation and an attention temperature).  The host fills
// the per-pair frequencies in double precision; the device forms each angle
// position * frequency and reduces it modulo 2*pi in double precision, so large
// positions keep their accuracy, then takes cos/sin in float.  Pairs are half-split:
// dimension i rotates with dimension i + D/2.
#pragma once

#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

__device__ __forceinline__ void rope_cos_sin(double f, int64_t pos, float& c, float& s) {
  const double a = (double)pos * f;
  const double k = __builtin_rint(a * 0.15915494309189533577);  // turns, rounded
  const double r = __builtin_fma(-k, 6.283185307179586232, a);   // |r| <= pi (+ rounding)
  sincosf((float)r, &s, &c);
}

// Rotate eight half-split pairs with precomputed (cos, sin) of their angles.
__device__ __forceinline__ void rope_rotate8_cs(bf16x8& lo, bf16x8& hi, const float2* cs,
                                                float mscale) {
  float x[8], y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float c = cs[j].x, s = cs[j].y;
    const float a = (float)lo[j], b = (float)hi[j];
    x[j] = mscale * (a * c - b * s);
    y[j] = mscale * (b * c + a * s);
  }
  u32x4 xl, yl;
  xl.x = pack_bf16x2(x[0], x[1]); xl.y = pack_bf16x2(x[2], x[3]);
  xl.z = pack_bf16x2(x[4], x[5]); xl.w = pack_bf16x2(x[6], x[7]);
  yl.x = pack_bf16x2(y[0], y[1]); yl.y = pack_bf16x2(y[2], y[3]);
  yl.z = pack_bf16x2(y[4], y[5]); yl.w = pack_bf16x2(y[6], y[7]);
  lo = as_bf16x8(xl);
  hi = as_bf16x8(yl);
}

// Rotate eight half-split pairs held as two bf16 vectors: lo = dims [i0, i0+8),
// hi = dims [i0 + D/2, i0 + D/2 + 8), whose frequencies are f[0..8), at one position;
// results rounded to bf16 (RNE).
__device__ __forceinline__ void rope_rotate8_f(bf16x8& lo, bf16x8& hi, const double* f,
                                               int64_t pos, float mscale) {
  float x[8], y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float c, s;
    rope_cos_sin(f[j], pos, c, s);
    const float a = (float)lo[j], b = (float)hi[j];
    x[j] = mscale * (a * c - b * s);
    y[j] = mscale * (b * c + a * s);
  }
  u32x4 xl, yl;
  xl.x = pack_bf16x2(x[0], x[1]); xl.y = pack_bf16x2(x[2], x[3]);
  xl.z = pack_bf16x2(x[4], x[5]); xl.w = pack_bf16x2(x[6], x[7]);
  yl.x = pack_bf16x2(y[0], y[1]); yl.y = pack_bf16x2(y[2], y[3]);
  yl.z = pack_bf16x2(y[4], y[5]); yl.w = pack_bf16x2(y[6], y[7]);
  lo = as_bf16x8(xl);
  hi = as_bf16x8(yl);
}
// The same with the frequencies read from the table of `r`.
__device__ __forceinline__ void rope_rotate8(bf16x8& lo, bf16x8& hi, int i0, int64_t pos,
                                             const RopeArgs& r) {
  double f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = r.freq[i0 + j];
  rope_rotate8_f(lo, hi, f, pos, r.mscale);
}

}  // namespace sa
