// Internal interface between the host API (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "cache_plan.hpp"

namespace sa {

enum ElemType : int { kBF16 = 0, kF32 = 1, kFP8 = 2 };  // kFP8: cache only (e4m3)

// Device view of a RoPE handle.
struct RopeArgs {
  const double* freq;   // device [H][D/2], fp64
  const float* grid_cs; // device cos/sin of the grid-axis angles (see build_rope_grid_table), or null
  int32_t pairs_t;      // pairs [0, pairs_t) rotate with the time position
  int32_t pairs_th;     // pairs [pairs_t, pairs_th) with the grid row, the rest with the column
  int32_t pairs_all;    // D / 2
  int32_t grid_h, grid_w;
  int32_t grid_stride;  // entries per head table
  int32_t grid_per_head;
};

// Per-call table of frames, passed by value as a kernel argument.
struct FrameTable {
  int32_t n;
  int32_t store_slot[kMaxFrames];
  int64_t t[kMaxFrames];
};

// Cache geometry and stores.
struct CacheGeom {
  int32_t B, H, D, T;  // streams, heads, head size, tokens per frame
  int32_t n_slots;     // n_sink + n_local
  void* k_store;       // [n_slots][B][H][T][D]
  void* v_store;       // [n_slots][B][H][D][T]
  float k_scale, v_scale;  // e4m3 caches: stored = value / scale
};

struct AttnArgs {
  const void* q;  // [B, n_q*T, H, D]
  void* o;        // [B, n_q*T, H, D]
  CacheGeom g;
  RopeArgs rope;
  FrameTable frames;  // resident frames, logical order; the queries are the last n_q
  int32_t n_q;
  int32_t causal;
  float scale_log2;   // softmax scale * log2(e)
  int32_t n_splits;   // key splits (1 = no workspace)
  float* ws;          // split partials, see attn_workspace_bytes
  uint32_t store_bytes;  // bytes of each cache store (< 4 GiB)
  int32_t variant;       // bf16 kernel variant: 1 default, 2 in-wave pipelined
  int32_t key_limit;     // keys at logical index >= key_limit are hidden (INT32_MAX: none)
  // Per-row statistic, stat[(b*Lq + row)*H + h] (fp32):
  //   kStatNone: not written; kStatLse: the row's log2-sum-exp2 of its scaled
  //   scores; kStatMass: 2^(this call's log2-sum-exp2 - stat), o not written;
  //   kStatZero: 0.
  int32_t stat_mode;
  float* stat;
};
enum AttnStat : int { kStatNone = 0, kStatLse = 1, kStatMass = 2, kStatZero = 3 };

// Projection GEMM: out[n][f] = sum_c x[n][c] W[f][c] over up to three
// output segments of `width` features each (one weight matrix per segment).
enum ProjOut : int {
  kOutRows = 0,    // row-major [n_tok][width] at y
  kOutCacheK = 1,  // rotated at the token's frame time, into the key store
  kOutCacheV = 2,  // into the transposed value store
};
// Operand types: bf16, or 8-bit codes (e4m3 / int8) with an fp32 scale per
// x row (token) and per weight row (output feature):
//   out[n][f] = (float(sum_c qx[n][c] qw[f][c]) * sx[n]) * sw[f].
enum ProjOp : int { kOpBF16 = 0, kOpE4M3 = 1, kOpI8 = 2 };
struct ProjSeg {
  const void* w;  // [width][C]
  void* y;        // kOutRows only
  int32_t kind;   // ProjOut
};
struct ProjArgs {
  const void* x;      // [n_tok][C]
  int64_t n_tok;
  int32_t hidden;     // C
  int32_t width;      // features per segment (multiple of 16)
  int32_t n_seg;      // 1..3; unused entries repeat a valid weight pointer
  ProjSeg seg[3];
  int32_t has_key, has_value;  // some segment is kOutCacheK / kOutCacheV
  int32_t cache_fp8;           // cache outputs go to an e4m3 cache (bf16-rounded results, scaled)
  int32_t op;                  // ProjOp of x and the weights (the output is bf16 unless op and dtype are fp32)
  const float* x_scale;        // [n_tok], 8-bit operands only
  const float* w_scale[3];     // [width] per segment, 8-bit operands only (16-byte aligned)
  int32_t xcd_order;           // set by the launcher: workgroup order contiguous per XCD (small grids)
  // Cache outputs only: token n is token tok of frame j of stream b, with
  // n = (b * frames.n + j) * T + tok.
  CacheGeom g;
  RopeArgs rope;
  FrameTable frames;
};

hipError_t launch_rope3d(const RopeArgs& rope, const void* x, void* y, int dtype, int B, int H,
                         int D, int T, int n_frames, int64_t t0, hipStream_t stream);

hipError_t launch_append(const RopeArgs& rope, const CacheGeom& g, const void* k, const void* v,
                         int dtype, const FrameTable& chunk, hipStream_t stream);

hipError_t launch_read(const CacheGeom& g, int store_slot, void* k_out, void* v_out, int dtype,
                       hipStream_t stream);

// Launch-shape overrides set through sa_set_launch_override (0 = automatic).
enum Knob : int { kKnobAttnKernel = 0, kKnobAttnSplits = 1, kKnobProjTile = 2, kNumKnobs = 3 };
int launch_override(int knob);

// Waves per workgroup and number of key splits the attention launch uses.
int attn_kernel_variant(int dtype, int B, int H, int D, int T, int n_q, int num_cus);
int attn_num_splits(int dtype, int B, int H, int D, int T, int n_q, int n_res, int num_cus);
size_t attn_workspace_bytes(int dtype, int B, int H, int D, int T, int n_q, int n_splits);
// The library's own attention scratch on the current device (sa_window_attn_noalloc):
// kNoAllocScratchBytes at *ptr, resolved once per device; allocates nothing.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t attn_noalloc_scratch(void** ptr);
hipError_t launch_window_attn(const AttnArgs& a, int dtype, hipStream_t stream);
// The e4m3 attention kernel alone (head_dim 128); launch_window_attn adds the split merge.
hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t stream);

// Tile shape the bf16 projection kernel takes for n_tok x F outputs:
// 0 = 256 x 128, 1 = 128 x 128, 2 = 128 x 64 (features x tokens).
int proj_tile_shape(int64_t n_tok, int F, int num_cus);
hipError_t launch_proj(const ProjArgs& a, int dtype, int num_cus, hipStream_t stream);
// Row-wise 8-bit quantisation (op = kOpI8 or kOpE4M3) of x [n_rows][n_cols] bf16.
hipError_t launch_quantize_rows(const void* x, void* codes, float* scales, int op, int64_t n_rows, int n_cols,
                                hipStream_t stream);

}  // namespace sa
