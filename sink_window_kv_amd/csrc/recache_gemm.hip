// KV recache at a prompt switch (LongLive paper review, section 3 "KV
// Recache": the cached frames' keys and values are recomputed so that the
// cache carries the new prompt, then generation continues).
//
// One GEMM computes both projections for every resident token:
//   out^T[f][n] = sum_c Wt[f][c] x[n][c],  f in [0, 2*H*D): rows 0..H*D-1 are
//   W_k's output channels, the rest W_v's (weights in the [out, in] layout,
//   so both operands are contiguous along the reduction axis, as the matrix
//   cores want).
// Epilogue: key channels are rotated at their frame's time (RoPE, same
// device code as the append kernel) and scattered to [slot][b][h][tok][d];
// value channels go to the transposed store [slot][b][h][d][tok].  The
// feature-major orientation puts 4 consecutive channels of one token in each
// lane, so every RoPE pair is in-lane.
#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace sa {
namespace {

typedef __bf16 mfma_bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float mfma_f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kTM = 128;  // features per workgroup
constexpr int kTN = 128;  // tokens per workgroup
constexpr int kTK = 64;   // reduction slice per LDS tile

struct GemmSmem {
  uint16_t a[kTM][kTK + 8];
  uint16_t b[kTN][kTK + 8];
};

__device__ __forceinline__ mfma_bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(mfma_bf16x8, v);
}

// Map a global token index to (stream, logical frame, token in frame).
__device__ __forceinline__ void token_coords(int64_t n, int per_stream, int T, int* b, int* lf,
                                             int* tok) {
  *b = static_cast<int>(n / per_stream);
  const int rem = static_cast<int>(n - static_cast<int64_t>(*b) * per_stream);
  *lf = rem / T;
  *tok = rem - *lf * T;
}

__global__ void __launch_bounds__(256) recache_bf16_kernel(RecacheArgs a) {
  __shared__ GemmSmem sm;
  const CacheGeom& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int HD = g.H * g.D;
  const int C = a.hidden;
  const int per_stream = a.frames.n * g.T;
  const int64_t n_tok = static_cast<int64_t>(g.B) * per_stream;
  const int m0 = blockIdx.y * kTM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTN;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wk = static_cast<const uint16_t*>(a.wk);
  const uint16_t* wv = static_cast<const uint16_t*>(a.wv);

  mfma_f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int k0 = 0; k0 < C; k0 += kTK) {
    __syncthreads();
    for (int e = threadIdx.x; e < kTM * (kTK / 8); e += 256) {
      const int r = e / (kTK / 8), c = e % (kTK / 8);
      const int f = m0 + r;
      const uint16_t* src = f < HD ? wk + static_cast<int64_t>(f) * C : wv + static_cast<int64_t>(f - HD) * C;
      *reinterpret_cast<u32x4*>(&sm.a[r][c * 8]) = *reinterpret_cast<const u32x4*>(src + k0 + c * 8);
    }
    for (int e = threadIdx.x; e < kTN * (kTK / 8); e += 256) {
      const int r = e / (kTK / 8), c = e % (kTK / 8);
      const int64_t tkn = n0 + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (tkn < n_tok) v = *reinterpret_cast<const u32x4*>(x + tkn * C + k0 + c * 8);
      *reinterpret_cast<u32x4*>(&sm.b[r][c * 8]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kTK / 16; ++s) {
      mfma_bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.a[wm * 64 + i * 32 + n][16 * s + 8 * hh]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.b[wn * 64 + j * 32 + n][16 * s + 8 * hh]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue.  acc[i][j][r]: feature m0 + wm*64 + 32i + 8(r/4) + 4hh + r%4,
  // token n0 + wn*64 + 32j + n.
  uint16_t* kst = static_cast<uint16_t*>(g.k_store);
  uint16_t* vst = static_cast<uint16_t*>(g.v_store);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t tkn = n0 + wn * 64 + 32 * j + n;
    if (tkn >= n_tok) continue;
    int b, lf, tok;
    token_coords(tkn, per_stream, g.T, &b, &lf, &tok);
    const int64_t slot = a.frames.store_slot[lf];
    const int64_t t = a.frames.t[lf];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = m0 + wm * 64 + 32 * i + 8 * q + 4 * hh;  // multiple of 4
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
        if (f < HD) {
          const int head = f / g.D, d = f - head * g.D;
          const double* freq_h = a.rope.freq + static_cast<size_t>(head) * (g.D / 2);
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const int p = d / 2 + pp;
            float sn, cs;
            rope_sincos(rope_pair_pos(a.rope, p, t, tok / a.rope.grid_w, tok % a.rope.grid_w),
                        freq_h[p], &sn, &cs);
            const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
            v[2 * pp] = x0 * cs - x1 * sn;
            v[2 * pp + 1] = x0 * sn + x1 * cs;
          }
          uint2 w;
          w.x = pack_bf16x2(v[0], v[1]);
          w.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(kst + (((slot * g.B + b) * g.H + head) * g.T + tok) * g.D + d) = w;
        } else {
          const int fv = f - HD;
          const int head = fv / g.D, d = fv - head * g.D;
          const int64_t base = ((slot * g.B + b) * g.H + head) * static_cast<int64_t>(g.D);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            vst[(base + d + r) * g.T + tok] = static_cast<uint16_t>(f32_to_bf16_bits(v[r]));
        }
      }
  }
}

// fp32 path (small configurations): one thread per (token, 4 output channels).
__global__ void __launch_bounds__(256) recache_f32_kernel(RecacheArgs a) {
  const CacheGeom& g = a.g;
  const int HD = g.H * g.D;
  const int C = a.hidden;
  const int per_stream = a.frames.n * g.T;
  const int64_t n_tok = static_cast<int64_t>(g.B) * per_stream;
  const int quads = 2 * HD / 4;
  const int64_t total = n_tok * quads;
  const float* x = static_cast<const float*>(a.x);
  const float* wk = static_cast<const float*>(a.wk);
  const float* wv = static_cast<const float*>(a.wv);
  float* kst = static_cast<float*>(g.k_store);
  float* vst = static_cast<float*>(g.v_store);
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int qd = static_cast<int>(idx % quads);
    const int64_t tkn = idx / quads;
    const int f = qd * 4;
    const float* w = f < HD ? wk + static_cast<int64_t>(f) * C : wv + static_cast<int64_t>(f - HD) * C;
    const float* xr = x + tkn * C;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < C; ++c) {
      const float xv = xr[c];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = fmaf(xv, w[static_cast<int64_t>(r) * C + c], v[r]);
    }
    int b, lf, tok;
    token_coords(tkn, per_stream, g.T, &b, &lf, &tok);
    const int64_t slot = a.frames.store_slot[lf];
    if (f < HD) {
      const int head = f / g.D, d = f - head * g.D;
      const double* freq_h = a.rope.freq + static_cast<size_t>(head) * (g.D / 2);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int p = d / 2 + pp;
        float sn, cs;
        rope_sincos(rope_pair_pos(a.rope, p, a.frames.t[lf], tok / a.rope.grid_w, tok % a.rope.grid_w),
                    freq_h[p], &sn, &cs);
        const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
        v[2 * pp] = x0 * cs - x1 * sn;
        v[2 * pp + 1] = x0 * sn + x1 * cs;
      }
      float* dst = kst + (((slot * g.B + b) * g.H + head) * g.T + tok) * g.D + d;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r] = v[r];
    } else {
      const int fv = f - HD;
      const int head = fv / g.D, d = fv - head * g.D;
      const int64_t base = ((slot * g.B + b) * g.H + head) * static_cast<int64_t>(g.D);
#pragma unroll
      for (int r = 0; r < 4; ++r) vst[(base + d + r) * g.T + tok] = v[r];
    }
  }
}

}  // namespace

hipError_t launch_recache(const RecacheArgs& a, int dtype, hipStream_t stream) {
  const int64_t n_tok = static_cast<int64_t>(a.g.B) * a.frames.n * a.g.T;
  const int HD = a.g.H * a.g.D;
  if (dtype == kBF16) {
    const dim3 grid(static_cast<unsigned>((n_tok + kTN - 1) / kTN), (2 * HD) / kTM);
    hipLaunchKernelGGL(recache_bf16_kernel, grid, dim3(256), 0, stream, a);
  } else {
    const int64_t work = n_tok * (2 * HD / 4);
    int64_t blocks = (work + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(recache_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sa
