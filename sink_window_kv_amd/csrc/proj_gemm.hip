// Projection GEMMs around the attention: one matrix-core kernel with three
// kinds of output segment.
//
//   out^T[f][n] = sum_c W[f][c] x[n][c]
//
// Weights are in the [out, in] layout, so both operands are contiguous along
// the reduction axis, as the matrix cores want.  The output features are
// the concatenation of up to three segments of equal width (one weight
// matrix each); a segment's result either goes to a plain row-major matrix
// [token][feature], or straight into the frame cache:
//   * key segment: each key channel pair is rotated at its token's frame
//     time (RoPE, same device code as the append kernel) and the result is
//     scattered to the key store [slot][b][h][tok][d];
//   * value segment: scattered to the transposed value store
//     [slot][b][h][d][tok].
// An e4m3 cache receives the bf16-rounded results divided by its scales and
// rounded to e4m3 (8-byte pieces).
// Operands are bf16, or 8-bit codes (int8 or OCP e4m3) with an fp32 scale per
// token row of x and per weight row, for the 8-bit projections (LongLive
// paper review, "INT8 quantized inference" table; model card FP8 variant):
// the products run on v_mfma_i32_32x32x32_i8 / v_mfma_scale_f32_32x32x64_
// f8f6f4 and the epilogue applies the two scales before everything else.
// Three entry points use it:
//   * KV recache at a prompt switch (LongLive paper review, section 3 "KV
//     Recache"): segments (W_k -> key cache, W_v -> value cache) over every
//     resident token;
//   * per-frame projections of a new chunk (LoL paper review, background
//     "multi-head attention": every head has its own query, key and value
//     projections): (W_q -> q rows, W_k -> key cache, W_v -> value cache),
//     the cache writes being the append of the new frames;
//   * a plain linear map (one row-major segment), e.g. the output
//     projection after the attention.
// The feature-major orientation puts 4 consecutive channels of one token in
// each lane, so every RoPE pair is in-lane.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <type_traits>

#include "device_common.hpp"

namespace sa {
namespace {

typedef __bf16 mfma_bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float mfma_f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// A reduction slice is 64 bytes of every operand row: 32 bf16 or 64 8-bit codes.
constexpr int kSliceBytes = 64;
// Waves per workgroup: a 2 x WN grid of wave tiles of (TM/2) x (TN/WN), each
// (TM/64) x (TN/(32 WN)) products of 32 x 32.  Four waves (two workgroups per
// CU) for the smaller tiles; eight waves and one workgroup per CU for the
// 256 x 256 tile, whose slices carry 1.5 times the products per byte staged.
template <int TM, int TN>
struct GemmShape {
  static constexpr int NW = (TM == 256 && TN == 256) ? 8 : 4;
  static constexpr int WN = NW / 2;
  static constexpr int WG_PER_CU = NW == 8 ? 1 : 2;
};
constexpr int kOPad = 8;    // epilogue tile row padding (bf16 elements)
constexpr int kPre = 3;     // reduction slices in flight in registers

// LDS stage: rows of one 64-byte slice = 4 chunks of 16 bytes, chunk (r, c) stored at
// r*4 + (c ^ swz(r)).  A 16-byte LDS read is served 16 lanes at a time, and
// the 16 lanes of an operand read take 16 consecutive rows at one chunk
// index: 4 rows share each 256-byte line of the 64 banks, and the swizzle
// gives those 4 rows 4 different chunk positions, so every 16-lane group
// hits each bank once.
template <int TM, int TN>
struct GemmStage {
  u32x4 a[TM * 4];  // features x reduction slice
  u32x4 b[TN * 4];  // tokens x reduction slice
};
__device__ __forceinline__ int gswz(int r) { return (r >> 2) & 3; }
// Epilogue tile: the workgroup's results in bf16, [token][feature] (padded
// rows), so that every output layout is written in whole 16-byte pieces; a
// tile made only of value features is kept [feature][token] instead, the
// order of the transposed value store.
template <int TM, int TN>
union GemmOut {
  uint16_t o[TN][TM + kOPad];
  uint16_t ot[TM][TN + kOPad];
};
template <int TM, int TN>
union GemmSmem {
  GemmStage<TM, TN> stg[2];
  GemmOut<TM, TN> out;
};

__device__ __forceinline__ mfma_bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(mfma_bf16x8, v);
}

// Map a global token index to (stream, frame of the table, token in frame).
__device__ __forceinline__ void token_coords(int64_t n, int per_stream, int T, int* b, int* lf,
                                             int* tok) {
  *b = static_cast<int>(n / per_stream);
  const int rem = static_cast<int>(n - static_cast<int64_t>(*b) * per_stream);
  *lf = rem / T;
  *tok = rem - *lf * T;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           static_cast<int>(static_cast<uint32_t>(bytes)), 0x00020000);
}

// Workgroup: TM features x TN tokens, four waves in a 2 x 2 grid, each
// (TM/2) x (TN/2) as (TM/64) x (TN/64) products of 32 x 32; two workgroups
// per CU, so one's epilogue overlaps the other's products.  The reduction
// runs in slices of 64 bytes per row (32 bf16 or 64 8-bit codes): each step
// writes the next slice (already in registers) into the free LDS stage,
// loads the one after into registers and multiplies the current one, with
// one barrier per step.  Plain vector loads stage the slices (the
// direct-to-LDS path moves far fewer bytes per cycle per CU).
template <int TM, int TN, int QT>
__device__ __forceinline__ void proj_body(ProjArgs a) {
  constexpr int EB = QT == kOpBF16 ? 2 : 1;    // operand bytes per element
  constexpr int TKE = kSliceBytes / EB;        // reduction elements per slice
  using Acc = typename std::conditional<QT == kOpI8, i32x16, mfma_f32x16>::type;
  constexpr int NW = GemmShape<TM, TN>::NW;    // waves per workgroup
  constexpr int WN = GemmShape<TM, TN>::WN;    // wave columns (tokens)
  constexpr int MI = TM / 64;                  // 32-row products per wave (features)
  constexpr int NJ = TN / (32 * WN);           // 32-column products per wave (tokens)
  constexpr int kAI = TM * 4 / (NW * 64);      // feature-tile transfers per wave per slice
  constexpr int kBI = TN * 4 / (NW * 64);      // token-tile transfers per wave per slice
  static_assert(kAI * NW * 64 == TM * 4 && kBI * NW * 64 == TN * 4, "whole tiles");
  __shared__ GemmSmem<TM, TN> sm;
  GemmStage<TM, TN>* stg = sm.stg;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
  const int C = a.hidden;
  const int width = a.width;
  const int F = a.n_seg * width;
  const int64_t n_tok = a.n_tok;
  // Workgroup order: token tiles vary fastest.  On a small grid (at most two
  // rounds of workgroups: the per-frame projections) each XCD takes a
  // contiguous range of that order, so the workgroups it runs at once share
  // one feature tile of W and neighbouring x tiles in its L2 (measured 7 -
  // 11 % faster there); on the recache's large grid the hardware's
  // round-robin order measured faster (10 %), so it is kept.
  int m0 = blockIdx.y * TM;
  int64_t n0 = static_cast<int64_t>(blockIdx.x) * TN;
  if (a.xcd_order) {  // one-dimensional grid
    const int n_tt = static_cast<int>((a.n_tok + TN - 1) / TN);
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    m0 = (lid / n_tt) * TM;
    n0 = static_cast<int64_t>(lid % n_tt) * TN;
  }
  const uint64_t w_bytes = static_cast<uint64_t>(width) * C * EB;
  const __amdgpu_buffer_rsrc_t w0 = gemm_rsrc(a.seg[0].w, w_bytes);
  const __amdgpu_buffer_rsrc_t w1 = gemm_rsrc(a.seg[1].w, w_bytes);
  const __amdgpu_buffer_rsrc_t w2 = gemm_rsrc(a.seg[2].w, w_bytes);
  const __amdgpu_buffer_rsrc_t xr = gemm_rsrc(a.x, static_cast<uint64_t>(n_tok) * C * EB);

  // Per-lane source offsets (bytes, at reduction offset 0) of this wave's
  // transfers into the feature and token tiles.  A transfer covers 16 rows,
  // all in one segment (width % 16 == 0); rows past the last segment read
  // past their matrix and load zeros (their results are never stored).
  uint32_t aoff[kAI], boff[kBI];
  __amdgpu_buffer_rsrc_t arsrc[kAI];
#pragma unroll
  for (int u = 0; u < kAI; ++u) {
    const int P = 64 * (wave * kAI + u) + lane;
    const int r = P >> 2, c = (P & 3) ^ gswz(r);
    const int fr = m0 + 16 * (wave * kAI + u);  // first row of the transfer (wave-uniform)
    int s = fr / width;
    s = s < a.n_seg ? s : a.n_seg - 1;
    arsrc[u] = s == 0 ? w0 : (s == 1 ? w1 : w2);
    const int fl = m0 + r - s * width;
    aoff[u] = static_cast<uint32_t>(static_cast<uint64_t>(fl) * C * EB + c * 16);
  }
#pragma unroll
  for (int u = 0; u < kBI; ++u) {
    const int P = 64 * (wave * kBI + u) + lane;
    const int r = P >> 2, c = (P & 3) ^ gswz(r);
    const uint64_t tkn = static_cast<uint64_t>(n0 + r);
    // tokens past the end read past the buffer: zero
    const uint64_t off = tkn * C * EB + c * 16;
    boff[u] = off >= 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(off);
  }

  // operand read addresses (chunk units) for k-chunk 0; the k-chunk enters by XOR
  int arow[MI], brow[NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i) arow[i] = wm * (TM / 2) + 32 * i + n;
#pragma unroll
  for (int j = 0; j < NJ; ++j) brow[j] = wn * (TN / WN) + 32 * j + n;

  Acc acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // Slices go global -> registers -> LDS through kPre register buffers:
  // step ks writes slice ks+1 (loaded kPre steps earlier) into the LDS stage
  // that slice ks-1 was read from, reloads that register buffer with slice
  // ks+1+kPre and multiplies slice ks.  The step loop is unrolled by kPre so
  // that every register buffer index is static.
  const int nk = C / TKE;
  u32x4 R[kPre][kAI + kBI];
  auto load_regs = [&](u32x4 (&Rb)[kAI + kBI], int k0) {
#pragma unroll
    for (int u = 0; u < kAI; ++u)
      Rb[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                  arsrc[u], static_cast<int>(aoff[u] + k0 * EB), 0, 0));
#pragma unroll
    for (int u = 0; u < kBI; ++u)
      Rb[kAI + u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        xr, static_cast<int>(boff[u] == 0xffffffffu ? boff[u] : boff[u] + k0 * EB), 0, 0));
  };
  auto store_regs = [&](const u32x4 (&Rb)[kAI + kBI], GemmStage<TM, TN>& st) {
#pragma unroll
    for (int u = 0; u < kAI; ++u) st.a[64 * (wave * kAI + u) + lane] = Rb[u];
#pragma unroll
    for (int u = 0; u < kBI; ++u) st.b[64 * (wave * kBI + u) + lane] = Rb[kAI + u];
  };
  // Per-token coordinates of the tile for the cache outputs, computed once
  // here (one division per token) instead of per output piece: frame time,
  // grid row and column, and the element offsets of the token's key row and
  // value column at head 0, channel 0.
  const CacheGeom& g = a.g;
  const int dshift = g.D == 128 ? 7 : 6;  // head_dim is 64 or 128
  __shared__ int s_row[TN], s_col[TN];
  __shared__ int64_t s_t[TN], s_kb[TN], s_vb[TN];
  if (a.has_key || a.has_value) {
    const int per_stream = a.frames.n * g.T;
    for (int t = threadIdx.x; t < TN; t += NW * 64) {
      const int64_t tkn = n0 + t;
      int row = 0, col = 0;
      int64_t tt = 0, kb = 0, vb = 0;
      if (tkn < n_tok) {
        const int nn = static_cast<int>(tkn);  // < 2^31: x is below 4 GiB
        const int b = nn / per_stream;
        const int rem = nn - b * per_stream;
        const int lf = rem / g.T;
        const int tok = rem - lf * g.T;
        row = tok / a.rope.grid_w;
        col = tok - row * a.rope.grid_w;
        tt = a.frames.t[lf];
        const int64_t sb = (static_cast<int64_t>(a.frames.store_slot[lf]) * g.B + b) * g.H;  // (slot, b, head 0)
        kb = (sb * g.T + tok) * g.D;
        vb = sb * g.D * g.T + tok;
      }
      s_row[t] = row;
      s_col[t] = col;
      s_t[t] = tt;
      s_kb[t] = kb;
      s_vb[t] = vb;
    }
  }
  // Time-axis cos / sin of the tile's key features.  With T >= TN the tile's
  // tokens carry at most two frame times (its first and last token's), so
  // each (time, head, time pair) is evaluated once here, by the same function
  // as everywhere else, instead of once per output pair.
  constexpr int kTcs = 384;  // 2 times x (TM / D + 1) heads x D / 2 pairs, TM <= 256
  __shared__ float2 s_tcs[kTcs];
  int tcs_h0 = 0, tcs_nh = 0;
  int64_t tcs_t0 = 0;
  if (a.has_key && g.T >= TN && a.rope.pairs_t > 0) {
    int sk = -1;
    for (int i = 0; i < a.n_seg; ++i)
      if (a.seg[i].kind == kOutCacheK) sk = i;
    const int kf0 = max(m0, sk * width), kf1 = min(m0 + TM, min(F, (sk + 1) * width));
    if (sk >= 0 && kf0 < kf1) {
      tcs_h0 = (kf0 - sk * width) >> dshift;
      tcs_nh = ((kf1 - 1 - sk * width) >> dshift) - tcs_h0 + 1;
      if (2 * tcs_nh * a.rope.pairs_t > kTcs) tcs_nh = 0;  // not for these shapes; kept as a guard
      const int per_stream = a.frames.n * g.T;
      auto time_of = [&](int64_t tkn) {
        const int nn = static_cast<int>(tkn);
        const int b = nn / per_stream;
        return a.frames.t[(nn - b * per_stream) / g.T];
      };
      tcs_t0 = time_of(n0);
      const int64_t t1 = time_of(min(n0 + TN, n_tok) - 1);
      const int pt = a.rope.pairs_t;
      for (int i = threadIdx.x; i < 2 * tcs_nh * pt; i += NW * 64) {
        const int fi = i / (tcs_nh * pt), rem = i - fi * tcs_nh * pt;
        const int hh2 = rem / pt, pp = rem - hh2 * pt;
        float sn, cs;
        rope_sincos(static_cast<double>(fi ? t1 : tcs_t0),
                    a.rope.freq[static_cast<size_t>(tcs_h0 + hh2) * a.rope.pairs_all + pp], &sn, &cs);
        s_tcs[i] = float2{cs, sn};
      }
    }
  }
  // Slice s lives in register buffer s % kPre until it is written to LDS.
  // Every load is unconditional (slices past the end reload the last one and
  // are never multiplied), so inside the loop the compiler's load-completion
  // waits stay exact: each step waits only for the slice it stores, not for
  // the kPre - 1 slices loaded after it.
  const int last = (nk - 1) * TKE;
  load_regs(R[0], 0);
  store_regs(R[0], stg[0]);
#pragma unroll
  for (int p = 1; p <= kPre; ++p) load_regs(R[p % kPre], min(p * TKE, last));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // The reduction index of an operand byte only has to be the same for both
  // operands: lane half hh takes chunk 2s + hh of the slice in step s (bf16,
  // int8: 16 bytes per lane per product), or chunks 2hh and 2hh + 1 (e4m3:
  // 32 bytes per lane, one product per slice).
  auto multiply = [&](const GemmStage<TM, TN>& st) {
    if constexpr (QT == kOpE4M3) {
      i32x8 af[MI], bfr[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const u32x4 lo = st.a[arow[i] * 4 + ((2 * hh) ^ gswz(arow[i]))];
        const u32x4 hi = st.a[arow[i] * 4 + ((2 * hh + 1) ^ gswz(arow[i]))];
        af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 lo = st.b[brow[j] * 4 + ((2 * hh) ^ gswz(brow[j]))];
        const u32x4 hi = st.b[brow[j] * 4 + ((2 * hh + 1) ^ gswz(brow[j]))];
        bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0, 127, 0, 127);
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 af[MI], bfr[NJ];
        const int kc = 2 * s + hh;
#pragma unroll
        for (int i = 0; i < MI; ++i) af[i] = st.a[arow[i] * 4 + (kc ^ gswz(arow[i]))];
#pragma unroll
        for (int j = 0; j < NJ; ++j) bfr[j] = st.b[brow[j] * 4 + (kc ^ gswz(brow[j]))];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            if constexpr (QT == kOpI8)
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, af[i]),
                                                                 __builtin_bit_cast(i32x4, bfr[j]), acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[i]), as_bf16x8(bfr[j]), acc[i][j], 0, 0, 0);
          }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // Whole groups of kPre steps, no branch inside.  The store at step nk - 1
  // (when nk % kPre == 0) writes a copy of the last slice into the stage no
  // wave reads any more: harmless.
  const int full = nk / kPre * kPre;
  int kb = 0;
  for (; kb < full; kb += kPre) {
#pragma unroll
    for (int p = 0; p < kPre; ++p) {
      const int ks = kb + p;
      store_regs(R[(p + 1) % kPre], stg[(ks + 1) & 1]);
      load_regs(R[(p + 1) % kPre], min((ks + 1 + kPre) * TKE, last));
      multiply(stg[ks & 1]);
    }
  }
  // The last nk % kPre steps need no more loads.
#pragma unroll
  for (int p = 0; p + 1 < kPre; ++p) {
    const int ks = full + p;
    if (ks < nk) {
      if (ks + 1 < nk) store_regs(R[(p + 1) % kPre], stg[(ks + 1) & 1]);
      multiply(stg[ks & 1]);
    }
  }

  // Epilogue.  acc[i][j][r]: feature m0 + wm*TM/2 + 32i + 8(r/4) + 4hh + r%4,
  // token n0 + wn*TN/WN + 32j + n.  Key features are rotated at their token's
  // position (4 consecutive features = 2 pairs in-lane), everything is
  // rounded to bf16 into the LDS tile, then written out in 16-byte pieces:
  // row-major and key rows [tok][d] directly, value rows [d][tok] gathered
  // per feature.
  // The segment of feature f: at most three, so two compares.
  auto seg_of = [&](int f) { return (f >= width ? 1 : 0) + (f >= 2 * width ? 1 : 0); };
  // Per-segment fields as scalars, selected per lane: indexing the argument
  // array with a lane's segment number would load it from memory each time.
  const int kind0 = a.seg[0].kind, kind1 = a.seg[1].kind, kind2 = a.seg[2].kind;
  auto kind_of = [&](int sg) { return sg == 0 ? kind0 : (sg == 1 ? kind1 : kind2); };
  // A tile of value features only (the recache and per-frame projections put
  // the value segment last and tiles are aligned to it when the width is a
  // multiple of the tile): kept transposed in LDS.
  const bool allv = a.has_value && m0 >= (a.n_seg - 1) * width && a.seg[a.n_seg - 1].kind == kOutCacheV;
  const int pt = a.rope.pairs_t, pth = a.rope.pairs_th;
  const int ph = pth - pt, pw = a.rope.pairs_all - pth;
  asm volatile("s_barrier" ::: "memory");  // every wave is done with the stages
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int tl = wn * (TN / WN) + 32 * j + n;
    const int64_t tkn = n0 + tl;
    int row = 0, col = 0;
    int64_t t = 0;
    if (a.has_key) {
      row = s_row[tl];
      col = s_col[tl];
      t = s_t[tl];
    }
    const int tsel = t == tcs_t0 ? 0 : 1;
    float sx = 1.f;
    if constexpr (QT != kOpBF16) sx = tkn < n_tok ? a.x_scale[tkn] : 0.f;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int fl = wm * (TM / 2) + 32 * i + 8 * q + 4 * hh;
        const int f = m0 + fl;  // multiple of 4
        const int sg = seg_of(f);
        float v[4] = {static_cast<float>(acc[i][j][4 * q]), static_cast<float>(acc[i][j][4 * q + 1]),
                      static_cast<float>(acc[i][j][4 * q + 2]), static_cast<float>(acc[i][j][4 * q + 3])};
        if constexpr (QT != kOpBF16) {
          // (acc * sx[token]) * sw[feature]; the 4 features lie in one segment
          f32x4 sw = {0.f, 0.f, 0.f, 0.f};
          if (f < F) {
            const float* wsc = sg == 0 ? a.w_scale[0] : (sg == 1 ? a.w_scale[1] : a.w_scale[2]);
            sw = *reinterpret_cast<const f32x4*>(wsc + (f - sg * width));
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (v[r] * sx) * sw[r];
        }
        if (a.has_key && f < F && kind_of(sg) == kOutCacheK) {
          // the lane's 4 features are 2 pairs, p0 and p0 + 1
          const int fs = f - sg * width;
          const int head = fs >> dshift, d = fs & (g.D - 1);
          const int p0 = d / 2;
          auto rot = [&](int pp, float cs, float sn) {
            const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
            v[2 * pp] = x0 * cs - x1 * sn;
            v[2 * pp + 1] = x0 * sn + x1 * cs;
          };
          if (tcs_nh > 0 && p0 + 1 < pt) {
            // time axis, both pairs: the tile's table
            const float2* e = &s_tcs[(tsel * tcs_nh + (head - tcs_h0)) * pt + p0];
            const float2 e0 = e[0];
            rot(0, e0.x, e0.y);
            const float2 e1 = e[1];
            rot(1, e1.x, e1.y);
          } else if (p0 >= pt && a.rope.grid_cs != nullptr && (p0 + 1 < pth || p0 >= pth)) {
            // grid axes, both pairs on one axis: neighbouring table entries
            const int idx = p0 < pth ? row * ph + (p0 - pt) : a.rope.grid_h * ph + col * pw + (p0 - pth);
            const float2* e = reinterpret_cast<const float2*>(a.rope.grid_cs) +
                              (a.rope.grid_per_head ? head * a.rope.grid_stride : 0) + idx;
            const float2 e0 = e[0];
            rot(0, e0.x, e0.y);
            const float2 e1 = e[1];
            rot(1, e1.x, e1.y);
          } else {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const int p = p0 + pp;
              float sn, cs;
              if (tcs_nh > 0 && p < pt) {
                const float2 e = s_tcs[(tsel * tcs_nh + (head - tcs_h0)) * pt + p];
                cs = e.x;
                sn = e.y;
              } else {
                rope_cs(a.rope, head, p, t, row, col, &sn, &cs);
              }
              rot(pp, cs, sn);
            }
          }
        }
        if (allv) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.out.ot[fl + r][tl] = static_cast<uint16_t>(f32_to_bf16_bits(v[r]));
        } else {
          uint2 w;
          w.x = pack_bf16x2(v[0], v[1]);
          w.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(&sm.out.o[tl][fl]) = w;
        }
      }
  }
  __syncthreads();
  // Write-out in 16-byte pieces.  A thread's feature column (row-major and
  // key outputs) or token column (values) is the same for all its pieces, so
  // everything that depends only on it is resolved once, before its loop.
  constexpr int kNT = NW * 64;  // threads
  if (!allv) {
    // (token, 8 features) pieces: row-major outputs and keys, kNT / (TM/8)
    // tokens per pass
    constexpr int kPerTok = TM / 8;
    const int fl = (threadIdx.x % kPerTok) * 8;
    const int f = m0 + fl;
    if (f < F) {
      const int sg = seg_of(f);
      const int fs = f - sg * width;
      const int kind = kind_of(sg);
      if (kind == kOutRows) {
        uint16_t* const ybase = static_cast<uint16_t*>(sg == 0 ? a.seg[0].y : (sg == 1 ? a.seg[1].y : a.seg[2].y)) + fs;
        for (int tl = threadIdx.x / kPerTok; tl < TN && n0 + tl < n_tok; tl += kNT / kPerTok)
          *reinterpret_cast<u32x4*>(ybase + (n0 + tl) * width) = *reinterpret_cast<const u32x4*>(&sm.out.o[tl][fl]);
      } else if (kind == kOutCacheK) {
        const int64_t hoff = static_cast<int64_t>(fs >> dshift) * g.T * g.D + (fs & (g.D - 1));
        if (a.cache_fp8) {
          uint8_t* const kb8 = static_cast<uint8_t*>(g.k_store) + hoff;
          const float inv = 1.f / g.k_scale;
          for (int tl = threadIdx.x / kPerTok; tl < TN && n0 + tl < n_tok; tl += kNT / kPerTok) {
            float x[8];
            unpack_bf16x8(*reinterpret_cast<const u32x4*>(&sm.out.o[tl][fl]), x);
            *reinterpret_cast<uint2*>(kb8 + s_kb[tl]) = to_e4m3x8(x, inv);
          }
        } else {
          uint16_t* const kb16 = static_cast<uint16_t*>(g.k_store) + hoff;
          for (int tl = threadIdx.x / kPerTok; tl < TN && n0 + tl < n_tok; tl += kNT / kPerTok)
            *reinterpret_cast<u32x4*>(kb16 + s_kb[tl]) = *reinterpret_cast<const u32x4*>(&sm.out.o[tl][fl]);
        }
      }
    }
  }
  if (!a.has_value) return;
  {
    // (feature, 8 tokens) pieces: values, kNT / (TN/8) features per pass;
    // 8 consecutive tokens stay in one frame and stream (T % 8 == 0)
    constexpr int kPerFeat = TN / 8;
    const int tl = (threadIdx.x % kPerFeat) * 8;
    if (n0 + tl < n_tok) {
      const int64_t vb = s_vb[tl];
      for (int fl = threadIdx.x / kPerFeat; fl < TM; fl += kNT / kPerFeat) {
        const int f = m0 + fl;
        if (f >= F) break;
        const int sg = seg_of(f);
        if (kind_of(sg) != kOutCacheV) continue;
        const int64_t idx = vb + static_cast<int64_t>(f - sg * width) * g.T;  // (head * D + d) * T
        alignas(16) uint16_t vals[8];
        if (allv) {
          *reinterpret_cast<u32x4*>(vals) = *reinterpret_cast<const u32x4*>(&sm.out.ot[fl][tl]);
        } else {
#pragma unroll
          for (int r = 0; r < 8; ++r) vals[r] = sm.out.o[tl + r][fl];
        }
        if (a.cache_fp8) {
          float x[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) x[r] = bf16_bits_to_f32(vals[r]);
          *reinterpret_cast<uint2*>(static_cast<uint8_t*>(g.v_store) + idx) = to_e4m3x8(x, 1.f / g.v_scale);
        } else {
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.v_store) + idx) = *reinterpret_cast<const u32x4*>(vals);
        }
      }
    }
  }
}

template <int TM, int TN>
__global__ void __launch_bounds__((GemmShape<TM, TN>::NW * 64), (GemmShape<TM, TN>::WG_PER_CU))
    proj_bf16_kernel(ProjArgs a) {
  proj_body<TM, TN, kOpBF16>(a);
}

// 8-bit operands (QT = kOpE4M3 or kOpI8), bf16 results.
template <int TM, int TN, int QT>
__global__ void __launch_bounds__((GemmShape<TM, TN>::NW * 64), (GemmShape<TM, TN>::WG_PER_CU))
    proj_q8_kernel(ProjArgs a) {
  proj_body<TM, TN, QT>(a);
}

// fp32 path (small configurations): one thread per (token, 4 output features).
__global__ void __launch_bounds__(256) proj_f32_kernel(ProjArgs a) {
  const CacheGeom& g = a.g;
  const int C = a.hidden;
  const int width = a.width;
  const int per_stream = a.frames.n * g.T;
  const int64_t n_tok = a.n_tok;
  const int quads = a.n_seg * width / 4;
  const int64_t total = n_tok * quads;
  const float* x = static_cast<const float*>(a.x);
  float* kst = static_cast<float*>(g.k_store);
  float* vst = static_cast<float*>(g.v_store);
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int qd = static_cast<int>(idx % quads);
    const int64_t tkn = idx / quads;
    const int f = qd * 4;
    const int s = f / width;
    const int fs = f - s * width;
    const ProjSeg& seg = a.seg[s];
    const float* w = static_cast<const float*>(seg.w) + static_cast<int64_t>(fs) * C;
    const float* xr = x + tkn * C;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < C; ++c) {
      const float xv = xr[c];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = fmaf(xv, w[static_cast<int64_t>(r) * C + c], v[r]);
    }
    if (seg.kind == kOutRows) {
      float* dst = static_cast<float*>(seg.y) + tkn * width + fs;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r] = v[r];
      continue;
    }
    int b, lf, tok;
    token_coords(tkn, per_stream, g.T, &b, &lf, &tok);
    const int64_t slot = a.frames.store_slot[lf];
    const int head = fs / g.D, d = fs - head * g.D;
    if (seg.kind == kOutCacheK) {
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
      const int64_t base = ((slot * g.B + b) * g.H + head) * static_cast<int64_t>(g.D);
#pragma unroll
      for (int r = 0; r < 4; ++r) vst[(base + d + r) * g.T + tok] = v[r];
    }
  }
}

template <int TM, int TN>
void launch_tile(const ProjArgs& a0, int num_cus, hipStream_t stream) {
  const int F = a0.n_seg * a0.width;
  const int64_t n_tt = (a0.n_tok + TN - 1) / TN, n_ft = (F + TM - 1) / TM;
  ProjArgs a = a0;
  a.xcd_order = n_tt * n_ft <= 2 * GemmShape<TM, TN>::WG_PER_CU * static_cast<int64_t>(num_cus);  // <= 2 rounds
  const dim3 grid = a.xcd_order ? dim3(static_cast<unsigned>(n_tt * n_ft))
                                : dim3(static_cast<unsigned>(n_tt), static_cast<unsigned>(n_ft));
  if (a.op == kOpE4M3)
    hipLaunchKernelGGL((proj_q8_kernel<TM, TN, kOpE4M3>), grid, dim3(GemmShape<TM, TN>::NW * 64), 0, stream, a);
  else if (a.op == kOpI8)
    hipLaunchKernelGGL((proj_q8_kernel<TM, TN, kOpI8>), grid, dim3(GemmShape<TM, TN>::NW * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((proj_bf16_kernel<TM, TN>), grid, dim3(GemmShape<TM, TN>::NW * 64), 0, stream, a);
}

int64_t tiles_of(int64_t n_tok, int F, int TM, int TN) { return ((n_tok + TN - 1) / TN) * ((F + TM - 1) / TM); }

}  // namespace

int proj_tile_shape(int64_t n_tok, int F, int num_cus) {
  if (const int v = launch_override(kKnobProjTile)) return v - 1;
  // the largest tile that still gives every CU a workgroup
  if (tiles_of(n_tok, F, 256, 128) >= num_cus) return 0;
  if (tiles_of(n_tok, F, 128, 128) >= num_cus) return 1;
  return 2;
}

hipError_t launch_proj(const ProjArgs& a, int dtype, int num_cus, hipStream_t stream) {
  if (a.n_tok == 0) return hipSuccess;
  const int F = a.n_seg * a.width;
  if (dtype == kBF16) {
    switch (proj_tile_shape(a.n_tok, F, num_cus)) {
      case 0: launch_tile<256, 128>(a, num_cus, stream); break;
      case 1: launch_tile<128, 128>(a, num_cus, stream); break;
      case 3: launch_tile<256, 256>(a, num_cus, stream); break;
      default: launch_tile<128, 64>(a, num_cus, stream); break;
    }
  } else {
    const int64_t work = a.n_tok * (F / 4);
    int64_t blocks = (work + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(proj_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sa
