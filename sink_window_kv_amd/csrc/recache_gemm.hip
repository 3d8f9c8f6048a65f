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

constexpr int kTM = 256;    // features per workgroup
constexpr int kTN = 128;    // tokens per workgroup
constexpr int kTK = 32;     // reduction slice per LDS stage
constexpr int kGWaves = 4;  // waves per workgroup (2 x 2 grid of 128 x 64 wave tiles)
constexpr int kAI = kTM * 4 / (kGWaves * 64);  // feature-tile transfers per wave per slice
constexpr int kBI = kTN * 4 / (kGWaves * 64);  // token-tile transfers per wave per slice
static_assert(kAI * kGWaves * 64 == kTM * 4 && kBI * kGWaves * 64 == kTN * 4, "whole tiles");

// LDS stage: rows of kTK bf16 = 4 chunks of 16 bytes, chunk (r, c) stored at
// r*4 + (c ^ swz(r)) so that the 32 rows of a matrix-core operand read hit
// distinct bank groups.
struct GemmStage {
  u32x4 a[kTM * 4];  // features x reduction slice
  u32x4 b[kTN * 4];  // tokens x reduction slice
};
__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 3; }
// Epilogue tile: the workgroup's results in bf16, [token][feature] (padded
// rows), so that both cache layouts are written in whole 16-byte pieces.
constexpr int kOPad = 8;
struct GemmOut {
  uint16_t o[kTN][kTM + kOPad];
};
union GemmSmem {
  GemmStage stg[2];
  GemmOut out;
};

__device__ __forceinline__ mfma_bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(mfma_bf16x8, v);
}

// Raw buffer descriptor (gfx9 layout) over [base, base + bytes): loads past
// the end return zero.
__device__ __forceinline__ u32x4 gemm_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// 16 bytes per lane, global -> LDS (buffer_load_dwordx4 ... lds): lane L's
// chunk lands at lds_base + 16 L.  M0 is set inside the asm; completion is
// waited for with an explicit vmcnt before the barrier that publishes it.
__device__ __forceinline__ void gemm_dma16(const u32x4 rsrc, uint32_t voff, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_base)));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// Map a global token index to (stream, logical frame, token in frame).
__device__ __forceinline__ void token_coords(int64_t n, int per_stream, int T, int* b, int* lf,
                                             int* tok) {
  *b = static_cast<int>(n / per_stream);
  const int rem = static_cast<int>(n - static_cast<int64_t>(*b) * per_stream);
  *lf = rem / T;
  *tok = rem - *lf * T;
}

// Workgroup: 256 features x 128 tokens, four waves in a 2 x 2 grid, each
// 128 features x 64 tokens (4 x 2 products of 32 x 32); two workgroups per
// CU, so one's epilogue overlaps the other's products.  The reduction runs
// in slices of 32 through two LDS stages filled by direct-to-LDS loads: the
// next slice lands while the current one is multiplied.
__global__ void __launch_bounds__(kGWaves * 64, 2) recache_bf16_kernel(RecacheArgs a) {
  __shared__ GemmSmem sm;
  GemmStage* stg = sm.stg;
  const CacheGeom& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int HD = g.H * g.D;
  const int C = a.hidden;
  const int per_stream = a.frames.n * g.T;
  const int64_t n_tok = static_cast<int64_t>(g.B) * per_stream;
  const int m0 = blockIdx.y * kTM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTN;
  const u32x4 wk_rsrc = gemm_rsrc(a.wk, static_cast<uint32_t>(static_cast<uint64_t>(HD) * C * 2));
  const u32x4 wv_rsrc = gemm_rsrc(a.wv, static_cast<uint32_t>(static_cast<uint64_t>(HD) * C * 2));
  const u32x4 x_rsrc = gemm_rsrc(a.x, static_cast<uint32_t>(static_cast<uint64_t>(n_tok) * C * 2));
  const int w_bytes = static_cast<int>(static_cast<uint32_t>(static_cast<uint64_t>(HD) * C * 2));
  const __amdgpu_buffer_rsrc_t wk_br = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.wk), (short)0, w_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t wv_br = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.wv), (short)0, w_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t x_br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.x), (short)0, static_cast<int>(static_cast<uint32_t>(static_cast<uint64_t>(n_tok) * C * 2)), 0x00020000);

  // Per-lane source offsets (bytes, at reduction offset 0) of this wave's
  // transfers into the feature and token tiles.  A transfer covers 16 rows,
  // all on one side of the K/V boundary (HD % 16 == 0).
  uint32_t aoff[kAI], boff[kBI];
  bool a_is_v[kAI];
#pragma unroll
  for (int u = 0; u < kAI; ++u) {
    const int P = 64 * (wave * kAI + u) + lane;
    const int r = P >> 2, c = (P & 3) ^ gswz(r);
    const int f = m0 + r;
    a_is_v[u] = m0 + 16 * (wave * kAI + u) >= HD;  // first row of the transfer
    const int fl = f < HD ? f : f - HD;
    aoff[u] = static_cast<uint32_t>((static_cast<uint64_t>(fl) * C + c * 8) * 2);
  }
#pragma unroll
  for (int u = 0; u < kBI; ++u) {
    const int P = 64 * (wave * kBI + u) + lane;
    const int r = P >> 2, c = (P & 3) ^ gswz(r);
    const uint64_t tkn = static_cast<uint64_t>(n0 + r);
    // tokens past the end read past the buffer: zero
    const uint64_t off = (tkn * C + c * 8) * 2;
    boff[u] = off >= 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(off);
  }
  auto issue = [&](int k0, GemmStage& st) {
#pragma unroll
    for (int u = 0; u < kAI; ++u)
      gemm_dma16(a_is_v[u] ? wv_rsrc : wk_rsrc, aoff[u] + k0 * 2, &st.a[64 * (wave * kAI + u)]);
#pragma unroll
    for (int u = 0; u < kBI; ++u)
      gemm_dma16(x_rsrc, boff[u] == 0xffffffffu ? boff[u] : boff[u] + k0 * 2, &st.b[64 * (wave * kBI + u)]);
  };

  // operand read addresses (chunk units) for k-chunk 0; the k-chunk enters by XOR
  int arow[4], brow[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = wm * 128 + 32 * i + n;
#pragma unroll
  for (int j = 0; j < 2; ++j) brow[j] = wn * 64 + 32 * j + n;

  mfma_f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Slices go global -> registers -> LDS: step ks writes slice ks+1 (loaded
  // during step ks-1) into the stage that slice ks-1 was read from, loads
  // slice ks+2 into registers and multiplies slice ks; one barrier per step
  // publishes the writes and retires the reads.  (Plain vector loads: the
  // direct-to-LDS path moves far fewer bytes per cycle per CU.)
  const int nk = C / kTK;
  u32x4 R[kAI + kBI];
  auto load_regs = [&](int k0) {
#pragma unroll
    for (int u = 0; u < kAI; ++u)
      R[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                 a_is_v[u] ? wv_br : wk_br, static_cast<int>(aoff[u] + k0 * 2), 0, 0));
#pragma unroll
    for (int u = 0; u < kBI; ++u)
      R[kAI + u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       x_br, static_cast<int>(boff[u] == 0xffffffffu ? boff[u] : boff[u] + k0 * 2), 0, 0));
  };
  auto store_regs = [&](GemmStage& st) {
#pragma unroll
    for (int u = 0; u < kAI; ++u) st.a[64 * (wave * kAI + u) + lane] = R[u];
#pragma unroll
    for (int u = 0; u < kBI; ++u) st.b[64 * (wave * kBI + u) + lane] = R[kAI + u];
  };
  load_regs(0);
  store_regs(stg[0]);
  if (nk > 1) load_regs(kTK);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  for (int ks = 0; ks < nk; ++ks) {
    const GemmStage& st = stg[ks & 1];
    if (ks + 1 < nk) store_regs(stg[(ks + 1) & 1]);
    if (ks + 2 < nk) load_regs((ks + 2) * kTK);
#pragma unroll
    for (int s = 0; s < kTK / 16; ++s) {
      mfma_bf16x8 af[4], bfr[2];
      const int kc = 2 * s + hh;
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = as_bf16x8(st.a[arow[i] * 4 + (kc ^ gswz(arow[i]))]);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = as_bf16x8(st.b[brow[j] * 4 + (kc ^ gswz(brow[j]))]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // Epilogue.  acc[i][j][r]: feature m0 + wm*128 + 32i + 8(r/4) + 4hh + r%4,
  // token n0 + wn*64 + 32j + n.  Key features are rotated at their token's
  // position (4 consecutive features = 2 pairs in-lane), everything is
  // rounded to bf16 into the LDS tile, then written out in 16-byte pieces:
  // key rows [tok][d] directly, value rows [d][tok] gathered per feature.
  asm volatile("s_barrier" ::: "memory");  // every wave is done with the stages
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tl = wn * 64 + 32 * j + n;
    const int64_t tkn = n0 + tl;
    int b = 0, lf = 0, tok = 0;
    if (tkn < n_tok) token_coords(tkn, per_stream, g.T, &b, &lf, &tok);
    const int64_t t = a.frames.t[lf];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int fl = wm * 128 + 32 * i + 8 * q + 4 * hh;
        const int f = m0 + fl;  // multiple of 4
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (f < HD) {
          const int head = f / g.D, d = f - head * g.D;
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const int p = d / 2 + pp;
            float sn, cs;
            rope_cs(a.rope, head, p, t, tok / a.rope.grid_w, tok % a.rope.grid_w, &sn, &cs);
            const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
            v[2 * pp] = x0 * cs - x1 * sn;
            v[2 * pp + 1] = x0 * sn + x1 * cs;
          }
        }
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(&sm.out.o[tl][fl]) = w;
      }
  }
  __syncthreads();
  uint16_t* kst = static_cast<uint16_t*>(g.k_store);
  uint16_t* vst = static_cast<uint16_t*>(g.v_store);
  // 16-byte pieces: (token, 8 features) for keys, (feature, 8 tokens) for values
  for (int e = threadIdx.x; e < kTN * (kTM / 8); e += kGWaves * 64) {
    const int tl = e / (kTM / 8), fl = (e % (kTM / 8)) * 8;
    const int64_t tkn = n0 + tl;
    const int f = m0 + fl;
    if (tkn >= n_tok || f >= HD) continue;
    int b, lf, tok;
    token_coords(tkn, per_stream, g.T, &b, &lf, &tok);
    const int64_t slot = a.frames.store_slot[lf];
    const int head = f / g.D, d = f - head * g.D;
    *reinterpret_cast<u32x4*>(kst + (((slot * g.B + b) * g.H + head) * g.T + tok) * g.D + d) =
        *reinterpret_cast<const u32x4*>(&sm.out.o[tl][fl]);
  }
  for (int e = threadIdx.x; e < kTM * (kTN / 8); e += kGWaves * 64) {
    const int fl = e / (kTN / 8), tl = (e % (kTN / 8)) * 8;
    const int f = m0 + fl;
    const int64_t tkn0 = n0 + tl;
    if (f < HD || f >= 2 * HD || tkn0 >= n_tok) continue;
    // 8 consecutive tokens stay in one frame and stream (T % 8 == 0)
    int b, lf, tok;
    token_coords(tkn0, per_stream, g.T, &b, &lf, &tok);
    const int64_t slot = a.frames.store_slot[lf];
    const int fv = f - HD;
    const int head = fv / g.D, d = fv - head * g.D;
    uint16_t vals[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) vals[r] = sm.out.o[tl + r][fl];
    *reinterpret_cast<u32x4*>(vst + (((slot * g.B + b) * g.H + head) * g.D + d) * g.T + tok) =
        *reinterpret_cast<const u32x4*>(vals);
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
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int p = d / 2 + pp;
        float sn, cs;
        rope_cs(a.rope, head, p, a.frames.t[lf], tok / a.rope.grid_w, tok % a.rope.grid_w, &sn, &cs);
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
    const dim3 grid(static_cast<unsigned>((n_tok + kTN - 1) / kTN), (2 * HD + kTM - 1) / kTM);
    hipLaunchKernelGGL(recache_bf16_kernel, grid, dim3(kGWaves * 64), 0, stream, a);
  } else {
    const int64_t work = n_tok * (2 * HD / 4);
    int64_t blocks = (work + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(recache_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sa
