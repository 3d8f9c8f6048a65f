// Device helpers shared by the attention kernels (bf16 and e4m3 caches):
// operand types, the exp2-domain row statistics, half-wave exchanges,
// direct-to-LDS buffer loads and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace sa {
namespace {

typedef float mfma_f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kQW = 32;                 // query rows per wave
constexpr int kKTile = 64;              // keys per LDS stage
constexpr float kNegInf = -__builtin_huge_valf();

// Per-row statistic from a row's final (m, l) in the exp2 domain: the
// log2-sum-exp2 of its scaled scores is m + log2(l).
__device__ __forceinline__ void write_stat(int mode, float* dst, float m, float l) {
  const float lse = m + log2f(l);
  if (mode == kStatLse) *dst = lse;
  else if (mode == kStatMass) *dst = exp2f(lse - *dst);
  else *dst = 0.f;
}

// Two fp32 -> packed bf16x2 with the hardware converter (round to nearest even).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}


// max(x, x of the lane 32 apart): the two half-waves swap their copies with
// v_permlane32_swap (a VALU op, no LDS round trip).  The s_nop covers the
// VALU-write -> permlane-read hazard on the operands.
__device__ __forceinline__ float max_halves(float x) {
  float lo = x, hi = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
  return fmaxf(lo, hi);
}

// Max of the 32 scores a lane holds for one 64-key tile, as a shallow tree
// of three-input maxima (a dependent chain would be 16 deep).
__device__ __forceinline__ float tile_max(const mfma_f32x16 (&s)[2]) {
  float a[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int j = 3 * i;
    const float x0 = s[j >> 4][j & 15], x1 = s[(j + 1) >> 4][(j + 1) & 15], x2 = s[(j + 2) >> 4][(j + 2) & 15];
    a[i] = fmaxf(fmaxf(x0, x1), x2);
  }
  a[10] = fmaxf(s[1][14], s[1][15]);
  const float b0 = fmaxf(fmaxf(a[0], a[1]), a[2]), b1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  const float b2 = fmaxf(fmaxf(a[6], a[7]), a[8]), b3 = fmaxf(a[9], a[10]);
  return fmaxf(fmaxf(b0, b1), fmaxf(b2, b3));
}

// Raw buffer descriptor (gfx9 layout) over [base, base + bytes), in SGPRs.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32) & 0xffffu);  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes);  // num_records: loads past the end return 0
  r[3] = 0x00020000u;
  return r;
}

// One 16-byte-per-lane global -> LDS transfer (buffer_load_dwordx4 ... lds):
// lane L's chunk lands at lds_base + 16 L.  Written as inline asm so that the
// compiler does not serialise it against reads of the other LDS stage (it
// cannot prove they do not alias and would wait for every load in flight);
// completion is tracked with explicit vmcnt waits instead.  The asm has no
// output registers; M0 (the LDS base) is set inside the same block.
__device__ __forceinline__ void dma16(const u32x4 rsrc, uint32_t voff, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_base)));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// The same transfer without a memory clobber: LDS reads of other stages may be
// scheduled across it (the stage it fills is read only after a later wait and
// barrier, both of which do clobber memory).
__device__ __forceinline__ void dma16_nomem(const u32x4 rsrc, uint32_t voff, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_base)));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
               : "m0");
}

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Plain s_barrier: a __syncthreads() fence would also wait for every load in
// flight.  The "memory" clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace
}  // namespace sa
