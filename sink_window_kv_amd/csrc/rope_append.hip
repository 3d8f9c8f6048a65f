// RoPE, cache-append and cache-read kernels (HBM-bound elementwise work).
//
// sa_rope3d_apply: 3D RoPE with per-head frequencies (LoL paper review,
//   background "Rotary Position Embedding" and "method steps" (5)-(7)).
// sa_cache_append: a latent frame's keys are rotated at the frame's time and
//   written to its slot; values are written transposed ([D][T] per slot,
//   stream and head) so the attention kernel can feed them to the matrix
//   cores without an LDS transpose (LongLive paper review, section 3
//   "Frame Sink": sink frames keep their slots, local frames rotate through
//   the ring).
#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace sa {
namespace {

__device__ __forceinline__ void load8(const uint16_t* p, float x[8]) {
  unpack_bf16x8(*reinterpret_cast<const u32x4*>(p), x);
}
__device__ __forceinline__ void load8(const float* p, float x[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float x[8]) {
  *reinterpret_cast<u32x4*>(p) = pack_bf16x8(x);
}
__device__ __forceinline__ void store8(float* p, const float x[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = x[i];
    b[i] = x[4 + i];
  }
  reinterpret_cast<f32x4*>(p)[0] = a;
  reinterpret_cast<f32x4*>(p)[1] = b;
}

// One thread rotates 8 channels (4 pairs) of one (stream, token, head).  It
// reads its 8 channels before writing the same 8 positions of y, so y may be
// x itself (no __restrict__: the two may alias).
template <typename E>
__global__ void __launch_bounds__(256) rope3d_kernel(RopeArgs rope, const E* x, E* y, int B, int H, int D,
                                                      int T, int n_frames, int64_t t0) {
  const int chunks = D / 8;
  const int64_t total = static_cast<int64_t>(B) * n_frames * T * H * chunks;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int c = static_cast<int>(idx % chunks);
    int64_t rest = idx / chunks;
    const int h = static_cast<int>(rest % H);
    rest /= H;
    const int64_t i = rest % (static_cast<int64_t>(n_frames) * T);
    const int j = static_cast<int>(i / T);
    const int tok = static_cast<int>(i - static_cast<int64_t>(j) * T);
    float v[8];
    load8(x + idx * 8, v);
    rope_rotate8(rope, h, c, t0 + j, tok / rope.grid_w,
                 tok % rope.grid_w, v);
    store8(y + idx * 8, v);
  }
}

// Keys of a chunk: rotate at the frame's time, scatter to [slot][b][h][tok][d].
template <typename E>
__global__ void __launch_bounds__(256) append_k_kernel(RopeArgs rope, CacheGeom g,
                                                        const E* __restrict__ k,
                                                        FrameTable chunk) {
  const int chunks = g.D / 8;
  const int64_t total = static_cast<int64_t>(g.B) * chunk.n * g.T * g.H * chunks;
  E* kst = static_cast<E*>(g.k_store);
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int c = static_cast<int>(idx % chunks);
    int64_t rest = idx / chunks;
    const int h = static_cast<int>(rest % g.H);
    rest /= g.H;
    const int64_t nt = static_cast<int64_t>(chunk.n) * g.T;
    const int64_t i = rest % nt;
    const int b = static_cast<int>(rest / nt);
    const int j = static_cast<int>(i / g.T);
    const int tok = static_cast<int>(i - static_cast<int64_t>(j) * g.T);
    float v[8];
    load8(k + idx * 8, v);
    rope_rotate8(rope, h, c, chunk.t[j],
                 tok / rope.grid_w, tok % rope.grid_w, v);
    const int64_t dst =
        ((((static_cast<int64_t>(chunk.store_slot[j]) * g.B + b) * g.H + h) * g.T + tok) * g.D) +
        c * 8;
    store8(kst + dst, v);
  }
}

constexpr int kVTileTok = 64;

// Values of a chunk: tile of 64 tokens x D of one (frame, stream, head),
// transposed through LDS into [slot][b][h][d][tok].
template <typename E, int D>
__global__ void __launch_bounds__(256) append_v_kernel(CacheGeom g, const E* __restrict__ v,
                                                        FrameTable chunk) {
  constexpr int VE = 16 / sizeof(E);  // elements per 16-byte vector
  constexpr int PAD = VE;             // row padding (elements) against bank conflicts
  __shared__ E tile[kVTileTok][D + PAD];
  const int tok0 = blockIdx.x * kVTileTok;
  const int h = blockIdx.y;
  const int j = blockIdx.z % chunk.n;
  const int b = blockIdx.z / chunk.n;
  const int64_t src_row0 =
      (static_cast<int64_t>(b) * chunk.n * g.T + static_cast<int64_t>(j) * g.T) * g.H + h;
  // load: rows of D elements, 16-byte vectors
  constexpr int VPR = D / VE;  // vectors per row
  for (int e = threadIdx.x; e < kVTileTok * VPR; e += 256) {
    const int r = e / VPR, cv = e % VPR;
    const int tok = tok0 + r;
    if (tok < g.T) {
      const u32x4 val =
          *reinterpret_cast<const u32x4*>(v + (src_row0 + static_cast<int64_t>(tok) * g.H) * D +
                                          cv * VE);
      *reinterpret_cast<u32x4*>(&tile[r][cv * VE]) = val;
    }
  }
  __syncthreads();
  // store: D rows of 64 tokens, VE tokens per vector
  E* vst = static_cast<E*>(g.v_store);
  const int64_t dst0 =
      ((static_cast<int64_t>(chunk.store_slot[j]) * g.B + b) * g.H + h) * static_cast<int64_t>(D) *
      g.T;
  constexpr int VPC = kVTileTok / VE;  // vectors per output row segment
  for (int e = threadIdx.x; e < D * VPC; e += 256) {
    const int d = e / VPC, cv = e % VPC;
    const int tok = tok0 + cv * VE;
    if (tok < g.T) {
      E vals[VE];
#pragma unroll
      for (int i = 0; i < VE; ++i) vals[i] = tile[cv * VE + i][d];
      *reinterpret_cast<u32x4*>(vst + dst0 + static_cast<int64_t>(d) * g.T + tok) =
          *reinterpret_cast<const u32x4*>(vals);
    }
  }
}

// bf16 keys and values of a chunk in one pass: a workgroup owns 64 tokens
// x 64 channels of one (frame, stream, head), so even one frame of one
// stream spreads over a few hundred workgroups.  Every load is issued first
// (16-byte vectors, 128-byte row pieces), then K is rotated and written into
// [slot][b][h][tok][d] and V goes through LDS into [slot][b][h][d][tok]
// (128-byte row pieces).  Store offsets are 32-bit (a store is below 4 GiB).
template <int D>
__global__ void __launch_bounds__(256) append_kv_bf16_kernel(RopeArgs rope, CacheGeom g,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              FrameTable chunk) {
  constexpr int VE = 8;                      // bf16 per 16-byte vector
  constexpr int DW = 64;                     // channels per workgroup
  constexpr int VPR = DW / VE;               // vectors per token row piece
  constexpr int NV = kVTileTok * VPR / 256;  // vectors per thread (K and V each)
  static_assert(NV * 256 == kVTileTok * VPR, "whole tile per workgroup");
  __shared__ uint16_t tile[kVTileTok][DW + VE];
  constexpr int parts = D / DW;
  const int tok0 = (blockIdx.x / parts) * kVTileTok;
  const int d0 = (blockIdx.x % parts) * DW;
  const int h = blockIdx.y;
  const int j = blockIdx.z % chunk.n;
  const int b = blockIdx.z / chunk.n;
  const int T = g.T;
  const int64_t src0 = ((static_cast<int64_t>(b) * chunk.n + j) * T * g.H + h) * D + d0;
  const uint64_t src_tok_stride = static_cast<uint64_t>(g.H) * D;
  u32x4 kv[NV], vv[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int r = e / VPR, cv = e % VPR;
    const int tok = min(tok0 + r, T - 1);
    const uint64_t off = static_cast<uint64_t>(tok) * src_tok_stride + cv * VE;
    kv[u] = *reinterpret_cast<const u32x4*>(k + src0 + off);
    vv[u] = *reinterpret_cast<const u32x4*>(v + src0 + off);
  }
  const int slot = chunk.store_slot[j];
  const uint32_t blk = ((static_cast<uint32_t>(slot) * g.B + b) * g.H + h) * static_cast<uint32_t>(T) * D;
  uint16_t* kst = static_cast<uint16_t*>(g.k_store);
  uint16_t* vst = static_cast<uint16_t*>(g.v_store);
  const int64_t t = chunk.t[j];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int r = e / VPR, cv = e % VPR;
    const int tok = tok0 + r;
    *reinterpret_cast<u32x4*>(&tile[r][cv * VE]) = vv[u];
    if (tok < T) {
      float x[8];
      unpack_bf16x8(kv[u], x);
      rope_rotate8(rope, h, d0 / 8 + cv, t, tok / rope.grid_w, tok % rope.grid_w, x);
      *reinterpret_cast<u32x4*>(kst + blk + static_cast<uint32_t>(tok) * D + d0 + cv * VE) = pack_bf16x8(x);
    }
  }
  __syncthreads();
  constexpr int VPC = kVTileTok / VE;  // vectors per output row piece
#pragma unroll
  for (int u = 0; u < DW * VPC / 256; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int d = e / VPC, cv = e % VPC;
    const int tok = tok0 + cv * VE;
    if (tok < T) {
      uint16_t vals[VE];
#pragma unroll
      for (int i = 0; i < VE; ++i) vals[i] = tile[cv * VE + i][d];
      *reinterpret_cast<u32x4*>(vst + blk + static_cast<uint32_t>(d0 + d) * T + tok) =
          *reinterpret_cast<const u32x4*>(vals);
    }
  }
}

// The same append into an e4m3 cache: bf16 k and v in, K rotated in fp32,
// divided by k_scale, V divided by v_scale, both rounded to e4m3; 8-byte
// stores (V^T rows are T bytes, T % 8 == 0).
template <int D>
__global__ void __launch_bounds__(256) append_kv_fp8_kernel(RopeArgs rope, CacheGeom g,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             FrameTable chunk) {
  constexpr int VE = 8;                      // bf16 per 16-byte input vector
  constexpr int DW = 64;                     // channels per workgroup
  constexpr int VPR = DW / VE;               // vectors per token row piece
  constexpr int NV = kVTileTok * VPR / 256;  // vectors per thread (K and V each)
  static_assert(NV * 256 == kVTileTok * VPR, "whole tile per workgroup");
  __shared__ uint16_t tile[kVTileTok][DW + VE];
  constexpr int parts = D / DW;
  const int tok0 = (blockIdx.x / parts) * kVTileTok;
  const int d0 = (blockIdx.x % parts) * DW;
  const int h = blockIdx.y;
  const int j = blockIdx.z % chunk.n;
  const int b = blockIdx.z / chunk.n;
  const int T = g.T;
  const int64_t src0 = ((static_cast<int64_t>(b) * chunk.n + j) * T * g.H + h) * D + d0;
  const uint64_t src_tok_stride = static_cast<uint64_t>(g.H) * D;
  u32x4 kv[NV], vv[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int r = e / VPR, cv = e % VPR;
    const int tok = min(tok0 + r, T - 1);
    const uint64_t off = static_cast<uint64_t>(tok) * src_tok_stride + cv * VE;
    kv[u] = *reinterpret_cast<const u32x4*>(k + src0 + off);
    vv[u] = *reinterpret_cast<const u32x4*>(v + src0 + off);
  }
  const int slot = chunk.store_slot[j];
  const uint32_t blk = ((static_cast<uint32_t>(slot) * g.B + b) * g.H + h) * static_cast<uint32_t>(T) * D;
  uint8_t* kst = static_cast<uint8_t*>(g.k_store);
  uint8_t* vst = static_cast<uint8_t*>(g.v_store);
  const float kinv = 1.f / g.k_scale, vinv = 1.f / g.v_scale;
  const int64_t t = chunk.t[j];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int r = e / VPR, cv = e % VPR;
    const int tok = tok0 + r;
    *reinterpret_cast<u32x4*>(&tile[r][cv * VE]) = vv[u];
    if (tok < T) {
      float x[8];
      unpack_bf16x8(kv[u], x);
      rope_rotate8(rope, h, d0 / 8 + cv, t, tok / rope.grid_w, tok % rope.grid_w, x);
      *reinterpret_cast<uint2*>(kst + blk + static_cast<uint32_t>(tok) * D + d0 + cv * VE) = to_e4m3x8(x, kinv);
    }
  }
  __syncthreads();
  constexpr int VPC = kVTileTok / VE;  // 8-token output pieces per row
#pragma unroll
  for (int u = 0; u < DW * VPC / 256; ++u) {
    const int e = threadIdx.x + 256 * u;
    const int d = e / VPC, cv = e % VPC;
    const int tok = tok0 + cv * VE;
    if (tok < T) {
      float x[8];
#pragma unroll
      for (int i = 0; i < VE; ++i) x[i] = bf16_bits_to_f32(tile[cv * VE + i][d]);
      *reinterpret_cast<uint2*>(vst + blk + static_cast<uint32_t>(d0 + d) * T + tok) = to_e4m3x8(x, vinv);
    }
  }
}

// Copy one stored frame out in the boundary layout [B, T, H, D].
template <typename E>
__global__ void __launch_bounds__(256) read_kernel(CacheGeom g, int slot, E* __restrict__ k_out,
                                                    E* __restrict__ v_out) {
  const int64_t total = static_cast<int64_t>(g.B) * g.T * g.H * g.D;
  const E* kst = static_cast<const E*>(g.k_store);
  const E* vst = static_cast<const E*>(g.v_store);
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int d = static_cast<int>(idx % g.D);
    int64_t rest = idx / g.D;
    const int h = static_cast<int>(rest % g.H);
    rest /= g.H;
    const int tok = static_cast<int>(rest % g.T);
    const int b = static_cast<int>(rest / g.T);
    const int64_t base = (static_cast<int64_t>(slot) * g.B + b) * g.H + h;
    if (k_out) k_out[idx] = kst[(base * g.T + tok) * g.D + d];
    if (v_out) v_out[idx] = vst[(base * g.D + d) * g.T + tok];
  }
}

inline unsigned grid_for(int64_t work_items) {
  int64_t blocks = (work_items + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return static_cast<unsigned>(blocks);
}

}  // namespace

hipError_t launch_rope3d(const RopeArgs& rope, const void* x, void* y, int dtype, int B, int H,
                         int D, int T, int n_frames, int64_t t0, hipStream_t stream) {
  const int64_t work = static_cast<int64_t>(B) * n_frames * T * H * (D / 8);
  if (work == 0) return hipSuccess;
  if (dtype == kBF16)
    hipLaunchKernelGGL(rope3d_kernel<uint16_t>, dim3(grid_for(work)), dim3(256), 0, stream, rope,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), B, H, D, T,
                       n_frames, t0);
  else
    hipLaunchKernelGGL(rope3d_kernel<float>, dim3(grid_for(work)), dim3(256), 0, stream, rope,
                       static_cast<const float*>(x), static_cast<float*>(y), B, H, D, T, n_frames,
                       t0);
  return hipGetLastError();
}

hipError_t launch_append(const RopeArgs& rope, const CacheGeom& g, const void* k, const void* v,
                         int dtype, const FrameTable& chunk, hipStream_t stream) {
  const int64_t work = static_cast<int64_t>(g.B) * chunk.n * g.T * g.H * (g.D / 8);
  const dim3 vgrid((g.T + kVTileTok - 1) / kVTileTok, g.H, g.B * chunk.n);
  if (dtype == kFP8) {
    const dim3 kvgrid(vgrid.x * (g.D / 64), vgrid.y, vgrid.z);
    if (g.D == 128)
      hipLaunchKernelGGL(append_kv_fp8_kernel<128>, kvgrid, dim3(256), 0, stream, rope, g,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), chunk);
    else
      hipLaunchKernelGGL(append_kv_fp8_kernel<64>, kvgrid, dim3(256), 0, stream, rope, g,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), chunk);
  } else if (dtype == kBF16) {
    const dim3 kvgrid(vgrid.x * (g.D / 64), vgrid.y, vgrid.z);
    if (g.D == 128)
      hipLaunchKernelGGL(append_kv_bf16_kernel<128>, kvgrid, dim3(256), 0, stream, rope, g,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), chunk);
    else
      hipLaunchKernelGGL(append_kv_bf16_kernel<64>, kvgrid, dim3(256), 0, stream, rope, g,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), chunk);
  } else {
    hipLaunchKernelGGL(append_k_kernel<float>, dim3(grid_for(work)), dim3(256), 0, stream, rope, g,
                       static_cast<const float*>(k), chunk);
    if (g.D == 128)
      hipLaunchKernelGGL((append_v_kernel<float, 128>), vgrid, dim3(256), 0, stream, g,
                         static_cast<const float*>(v), chunk);
    else
      hipLaunchKernelGGL((append_v_kernel<float, 64>), vgrid, dim3(256), 0, stream, g,
                         static_cast<const float*>(v), chunk);
  }
  return hipGetLastError();
}

hipError_t launch_read(const CacheGeom& g, int store_slot, void* k_out, void* v_out, int dtype,
                       hipStream_t stream) {
  const int64_t work = static_cast<int64_t>(g.B) * g.T * g.H * g.D;
  if (dtype == kFP8)
    hipLaunchKernelGGL(read_kernel<uint8_t>, dim3(grid_for(work)), dim3(256), 0, stream, g,
                       store_slot, static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out));
  else if (dtype == kBF16)
    hipLaunchKernelGGL(read_kernel<uint16_t>, dim3(grid_for(work)), dim3(256), 0, stream, g,
                       store_slot, static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
  else
    hipLaunchKernelGGL(read_kernel<float>, dim3(grid_for(work)), dim3(256), 0, stream, g,
                       store_slot, static_cast<float*>(k_out), static_cast<float*>(v_out));
  return hipGetLastError();
}

}  // namespace sa
