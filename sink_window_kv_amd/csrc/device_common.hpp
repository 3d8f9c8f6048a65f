// Device helpers shared by the gfx950 kernels: bf16 rounding, 16-byte
// vectors and the RoPE rotation.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"

namespace sa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 -> packed bf16x2 (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Unpack 8 bf16 (one 16-byte vector) into fp32.
__device__ __forceinline__ void unpack_bf16x8(const u32x4 v, float out[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);
    out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float in[8]) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
  return v;
}

// e4m3 (OCP) bytes of 8 values x * inv, clamped to +-448 first (the
// converter rounds to nearest even and does not saturate).
__device__ __forceinline__ uint2 to_e4m3x8(const float x[8], float inv) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(x[i] * inv, -448.f), 448.f);
  uint2 r;
  r.x = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0u, false);
  r.x = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r.x, true);
  r.y = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0u, false);
  r.y = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], r.y, true);
  return r;
}

// Position of channel pair p for a token at (t, row, col).
__device__ __forceinline__ double rope_pair_pos(const RopeArgs& r, int p, int64_t t, int row,
                                                int col) {
  return p < r.pairs_t ? static_cast<double>(t)
                       : (p < r.pairs_th ? static_cast<double>(row) : static_cast<double>(col));
}

// sin and cos of pos * w.  The angle is formed and reduced to [-pi, pi] in
// fp64 (Cody-Waite with a two-part 2*pi), so large time positions keep full
// fp32 accuracy; the reduced angle is evaluated in fp32.
__device__ __forceinline__ void rope_sincos(double pos, double w, float* s, float* c) {
  const double a = pos * w;
  const double k = rint(a * 0.15915494309189535);  // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, a);         // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);           // 2 pi, low part
  sincosf(static_cast<float>(r), s, c);
}

// sin and cos of channel pair p's angle for head h at (t, row, col): the
// time axis is evaluated here (the angle depends on the frame); the grid
// axes come from the precomputed table when there is one.
__device__ __forceinline__ void rope_cs(const RopeArgs& r, int h, int p, int64_t t, int row, int col,
                                        float* s, float* c) {
  if (p < r.pairs_t || r.grid_cs == nullptr) {
    rope_sincos(rope_pair_pos(r, p, t, row, col), r.freq[static_cast<size_t>(h) * r.pairs_all + p], s, c);
    return;
  }
  const int ph = r.pairs_th - r.pairs_t;
  const int idx = p < r.pairs_th ? row * ph + (p - r.pairs_t)
                                 : r.grid_h * ph + col * (r.pairs_all - r.pairs_th) + (p - r.pairs_th);
  const float2 v = reinterpret_cast<const float2*>(r.grid_cs)[(r.grid_per_head ? h * r.grid_stride : 0) + idx];
  *c = v.x;
  *s = v.y;
}

// Rotate 4 adjacent pairs (8 channels starting at channel 8*chunk) of head h
// in place: (x0, x1) -> (x0 c - x1 s, x0 s + x1 c).
__device__ __forceinline__ void rope_rotate8(const RopeArgs& r, int h, int chunk, int64_t t, int row, int col,
                                             float x[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = chunk * 4 + i;
    float s, c;
    rope_cs(r, h, p, t, row, col, &s, &c);
    const float x0 = x[2 * i], x1 = x[2 * i + 1];
    x[2 * i] = x0 * c - x1 * s;
    x[2 * i + 1] = x0 * s + x1 * c;
  }
}

// Map the hardware workgroup id to a logical one so that each XCD (workgroups
// are dealt round-robin to the 8 XCDs) gets a contiguous range of logical
// ids: neighbouring logical workgroups, which a kernel arranges to share
// operand tiles, then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int n) {
  constexpr int X = 8;
  const int xcd = pid % X;
  const int local = pid / X;
  const int per = (n + X - 1) / X;
  const int tall = n % X == 0 ? X : n % X;
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

}  // namespace sa
