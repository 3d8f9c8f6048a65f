// Sink + short-window attention over an e4m3 (OCP FP8) frame cache, head_dim 128.
//
// Same operation, masks, splits and partial-result layout as the bf16
// kernel (LongLive paper review, section 3 "Short-Window Attention" with
// the pinned frames of "Frame Sink"); the cache holds k / k_scale and
// v / v_scale rounded to e4m3 (the model card's FP8 variant).
//
// The products run on v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 x fp8, fp32
// accumulate).
//   * Operand lane layout of the instruction: lane l holds row (A) or column
//     (B) l % 32 and 32 bytes of the reduction axis, byte j of lane half h
//     being reduction index (h, j) for A and B alike; the accumulator has
//     the 32x32x16 layout.
//   * q is rotated, multiplied by softmax scale * log2(e) * k_scale and
//     rounded to e4m3 with a power-of-two scale per query row (its 128
//     values fill the e4m3 range); the instruction applies that scale (E8M0
//     operand of the B side).
//   * Key tiles never cross a frame: each frame is cut into ceil(T/64)
//     tiles, the last one partial and masked, so every transfer is one frame
//     row piece (T need only be a multiple of 8).
//   * The keys of a tile are permuted when K is read (MFMA row m of key
//     block kb takes key 32((m>>2)&1) + 16kb + 4(m>>3) + (m&3)), so that
//     lane half h holds the scores of keys 32h .. 32h+31 in byte order: they
//     are the P^T operand of O^T += V^T P^T after a pack to e4m3 (p <= 2^8).
//   * The row sum is one more product, of a constant all-ones V^T block
//     with the same packed p, so it matches the quantized numerator.
#include <hip/hip_runtime.h>

#include "attn_common.hpp"

namespace sa {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
constexpr int kF8Rows = 8;  // K chunks (16 bytes) per key row, head_dim 128
struct StageF8 {
  u32x4 k[kKTile * kF8Rows];   // [64 keys][128 bytes]
  u32x4 vt[128 * kKTile / 16];  // [128 channels][64 keys]
};
// K: chunk (r, c) at r*8 + (c ^ kswz8(r)); an operand read takes rows
// {16kb + 0..7, 16kb + 32..39} (or those + 8) at one chunk index, which this
// puts on 16 distinct bank groups.  V^T: chunk (d, c) at d*4 + (c ^ vswz8(d)).
__device__ __forceinline__ int kswz8(int r) { return ((r >> 1) ^ ((r >> 5) << 2)) & 7; }
__device__ __forceinline__ int vswz8(int d) { return (d >> 2) & 3; }

__device__ __forceinline__ v8i_t as_v8i(u32x4 lo, u32x4 hi) {
  v8i_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = static_cast<int>(lo[i]);
    r[4 + i] = static_cast<int>(hi[i]);
  }
  return r;
}

__device__ __forceinline__ mfma_f32x16 mfma_f8(v8i_t a, v8i_t b, mfma_f32x16 c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}

__device__ __forceinline__ uint32_t pk_e4m3(float a, float b, float c, float d) {
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

__global__ void __launch_bounds__(512, 1) attn_fp8_kernel(AttnArgs a) {
  constexpr int D = 128;
  constexpr int kWaves = 8;
  constexpr int kQTile = kWaves * kQW;
  constexpr uint32_t kVtOff8 = kKTile * D;  // byte offset of vt inside a stage
  __shared__ StageF8 f0, f1, f2;
  __shared__ int s_slot[kMaxFrames];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const CacheGeom& g = a.g;
  const int T = g.T;
  const int Lq = a.n_q * T;
  const int n_qt = (Lq + kQTile - 1) / kQTile;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % n_qt;
  const int split = (lid / n_qt) % a.n_splits;
  const int bh = lid / (n_qt * a.n_splits);
  const int b = bh / g.H;
  const int h = bh - b * g.H;
  const int n_res = a.frames.n;
  const int first_q = n_res - a.n_q;
  const int ntf = (T + kKTile - 1) / kKTile;  // key tiles per frame
  if (threadIdx.x < kMaxFrames) s_slot[threadIdx.x] = threadIdx.x < n_res ? a.frames.store_slot[threadIdx.x] : 0;

  // visibility in whole frames: a row sees frames [0, fend)
  const int flim = min(n_res, a.key_limit / T);
  const int row = qt * kQTile + wave * kQW + n;
  const bool row_ok = row < Lq;
  const int qf = row_ok ? row / T : a.n_q - 1;
  const int fend = min(a.causal ? first_q + qf + 1 : n_res, flim);
  const int wave_row0 = qt * kQTile + wave_u * kQW;
  const bool wave_active = wave_row0 < Lq;
  const int wave_last = min(wave_row0 + kQW - 1, Lq - 1);
  const int wave_fend = min(a.causal ? first_q + wave_last / T + 1 : n_res, flim);
  const int wave_fmin = min(a.causal ? first_q + min(wave_row0, Lq - 1) / T + 1 : n_res, flim);
  const int last_row = min(qt * kQTile + kQTile - 1, Lq - 1);
  const int fend_wg = min(a.causal ? first_q + last_row / T + 1 : n_res, flim);
  const int n_tiles = fend_wg * ntf;
  const int tile_lo = static_cast<int>((static_cast<int64_t>(n_tiles) * split) / a.n_splits);
  const int tile_hi = static_cast<int>((static_cast<int64_t>(n_tiles) * (split + 1)) / a.n_splits);

  // ---- Q: rotate, scale, e4m3 with one power-of-two scale per lane.
  v8i_t q8[2];
  int qscale;
  {
    const int tok = row_ok ? row - qf * T : 0;
    const int64_t t = a.frames.t[first_q + qf];
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((static_cast<int64_t>(b) * Lq + (row_ok ? row : 0)) * g.H + h) * D;
    const float qmul = a.scale_log2 * g.k_scale;
    float x[2][32];
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (row_ok) {
          unpack_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 64 * s + 32 * hh + 8 * c), y);
          rope_rotate8(a.rope, h, 8 * s + 4 * hh + c, t, tok / a.rope.grid_w, tok % a.rope.grid_w, y);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          x[s][8 * c + i] = y[i] * qmul;
          amax = fmaxf(amax, fabsf(x[s][8 * c + i]));
        }
      }
    // one scale for the whole row (both lane halves): smallest e with
    // amax * 2^-e <= 448
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int e = 0;
    if (amax > 0.f) {
      e = static_cast<int>(ceilf(log2f(amax * (1.f / 448.f))));
      if (ldexpf(amax, -e) > 448.f) ++e;
      e = max(-126, min(126, e));
    }
    qscale = 127 + e;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float v4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = fminf(fmaxf(ldexpf(x[s][4 * w + i], -e), -448.f), 448.f);
        q8[s][w] = static_cast<int>(pk_e4m3(v4[0], v4[1], v4[2], v4[3]));
      }
  }

  mfma_f32x16 oacc[D / 32], lacc;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) lacc[i] = 0.f;
  float m_run = kNegInf;
  mfma_f32x16 mseed;
#pragma unroll
  for (int i = 0; i < 16; ++i) mseed[i] = 0.f;
  v8i_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;  // e4m3 1.0 in every byte

  // LDS operand addresses (bytes in a stage); key block and channel block
  // enter as immediate offsets (2048 bytes each).
  uint32_t kaddr[2][2];
  {
    const int r = 32 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        kaddr[s][c] = static_cast<uint32_t>((r * kF8Rows + ((4 * s + 2 * hh + c) ^ kswz8(r))) * 16);
  }
  uint32_t vaddr[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) vaddr[c] = kVtOff8 + static_cast<uint32_t>((n * 4 + ((2 * hh + c) ^ vswz8(n))) * 16);

  // ---- global -> LDS: one K and one V^T transfer per wave per tile.  Each
  // goes through a descriptor that covers just the frame's (slot, stream,
  // head) block: the tail tile of a frame reads past the frame's keys, and
  // past the block those bytes may be anything (a slot never written, NaN
  // codes); the range check returns zeros for every dword beyond the block
  // instead (dword by dword, so a piece that straddles the end keeps its
  // valid part).  Beyond-frame keys are masked; their V^T bytes are then
  // finite, so p = 0 contributes nothing.
  const uint8_t* kst8 = static_cast<const uint8_t*>(g.k_store);
  const uint8_t* vst8 = static_cast<const uint8_t*>(g.v_store);
  const int64_t head_off = static_cast<int64_t>(b) * g.H + h;
  const int64_t slot_stride = static_cast<int64_t>(g.B) * g.H;
  const uint32_t blk_bytes = static_cast<uint32_t>(T) * D;
  uint32_t klane, vlane;
  {
    const int P = 64 * wave_u + lane;
    const int r = P / kF8Rows, c = (P % kF8Rows) ^ kswz8(r);
    klane = static_cast<uint32_t>(r * D + c * 16);
    const int d = P / 4, cv = (P % 4) ^ vswz8(d);
    vlane = static_cast<uint32_t>(d * T + cv * 16);
  }
  __syncthreads();  // s_slot visible
  // tiles are planned in non-decreasing order: frame of the tile tracked
  int pl_lf = 0, pl_end = ntf;
  struct Plan8 {
    u32x4 krs, vrs;  // descriptors of the frame's K and V^T blocks
    uint32_t koff, voff;
  };
  auto plan = [&](int kt) {
    while (kt >= pl_end) {
      ++pl_lf;
      pl_end += ntf;
    }
    const int jl0 = (kt - (pl_end - ntf)) * kKTile;
    const int slot = __builtin_amdgcn_readfirstlane(s_slot[min(pl_lf, n_res - 1)]);
    const uint32_t base = static_cast<uint32_t>((static_cast<int64_t>(slot) * slot_stride + head_off) * blk_bytes);
    Plan8 p;
    p.krs = buffer_rsrc(kst8 + base, blk_bytes);
    p.vrs = buffer_rsrc(vst8 + base, blk_bytes);
    p.koff = static_cast<uint32_t>(jl0) * D + klane;
    p.voff = static_cast<uint32_t>(jl0) + vlane;
    return p;
  };
  auto fire = [&](const Plan8& p, int u, StageF8& st) {
    if (u == 0)
      dma16(p.krs, p.koff, &st.k[64 * wave_u]);
    else
      dma16(p.vrs, p.voff, &st.vt[64 * wave_u]);
  };
  auto issue = [&](int kt, StageF8& st) {
    const Plan8 p = plan(kt);
    fire(p, 0, st);
    fire(p, 1, st);
  };
  auto rd = [&](const StageF8& st, uint32_t off) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&st) + off);
  };

  auto compute = [&](int kt, const StageF8& st, const Plan8& np, StageF8& nst) {
    const int lf = kt / ntf;
    const int jl0 = (kt - lf * ntf) * kKTile;
    if (!wave_active || lf >= wave_fend) {
      fire(np, 0, nst);
      fire(np, 1, nst);
      return;
    }
    mfma_f32x16 sacc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = mfma_f8(as_v8i(rd(st, kaddr[s][0] + kb * 2048), rd(st, kaddr[s][1] + kb * 2048)), q8[s],
                           s == 0 ? mseed : sacc[kb], qscale);
      fire(np, s, nst);
    }
    // the frame's tail tile, and frames a row of a causal chunk does not see
    if (jl0 + kKTile > T || lf >= wave_fmin) {
      const int lim = lf >= fend ? 0 : T - jl0 - 32 * hh;  // keys 32hh + 16kb + i with 16kb + i >= lim hidden
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * kb + i >= lim) sacc[kb][i] = kNegInf;
    }
    // lazy, per-row raise of an integer running max (as in the bf16 kernel)
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    const float mx = max_halves(tile_max(sacc)) + m_use;
    if (__any(mx > m_run + 8.f)) {
      const float m_new = mx > m_run + 8.f ? ceilf(mx) : m_run;
      const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      lacc[0] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      const float m_next = m_new == kNegInf ? 0.f : m_new;
      const float shift = m_next - m_use;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] -= shift;
#pragma unroll
      for (int i = 0; i < 16; ++i) mseed[i] = -m_next;
    }
    v8i_t pk;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, i0 = 4 * (w & 3);
      pk[w] = static_cast<int>(pk_e4m3(__builtin_amdgcn_exp2f(sacc[kb][i0]), __builtin_amdgcn_exp2f(sacc[kb][i0 + 1]),
                                       __builtin_amdgcn_exp2f(sacc[kb][i0 + 2]), __builtin_amdgcn_exp2f(sacc[kb][i0 + 3])));
    }
    lacc = mfma_f8(ones, pk, lacc, 127);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      oacc[db] = mfma_f8(as_v8i(rd(st, vaddr[0] + db * 2048), rd(st, vaddr[1] + db * 2048)), pk, oacc[db], 127);
  };

  // three stages, two tiles in flight (as the bf16 eight-wave path)
  const int t_last = tile_hi - 1;
  if (tile_lo < tile_hi) {
    issue(tile_lo, f0);
    issue(min(tile_lo + 1, t_last), f1);
  }
  auto step = [&](int kt, const StageF8& cur, StageF8& nxt2) {
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    barrier();
    compute(kt, cur, plan(min(kt + 2, t_last)), nxt2);
  };
  for (int kt = tile_lo; kt < tile_hi; kt += 3) {
    step(kt, f0, f2);
    if (kt + 1 < tile_hi) step(kt + 1, f1, f0);
    if (kt + 2 < tile_hi) step(kt + 2, f2, f1);
  }
  wait_vmcnt0();

  // ---- epilogue: O^T[d][row] as in the bf16 kernel; l from the ones product
  const float l_tot = lacc[0];
  if (a.n_splits > 1) {
    if (row_ok) {
      const int64_t plane = static_cast<int64_t>(g.B) * g.H * Lq;
      const int64_t prow = static_cast<int64_t>(bh) * Lq + row;
      float* po = a.ws + (split * plane + prow) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 w = {oacc[db][4 * gq] * g.v_scale, oacc[db][4 * gq + 1] * g.v_scale,
                           oacc[db][4 * gq + 2] * g.v_scale, oacc[db][4 * gq + 3] * g.v_scale};
          *reinterpret_cast<f32x4*>(po + 32 * db + 8 * gq + 4 * hh) = w;
        }
      if (hh == 0) {
        float* pml = a.ws + static_cast<int64_t>(a.n_splits) * plane * D + (split * plane + prow) * 2;
        pml[0] = m_run;
        pml[1] = l_tot;
      }
    }
    return;
  }
  if (row_ok) {
    const float inv = g.v_scale / l_tot;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + ((static_cast<int64_t>(b) * Lq + row) * g.H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint2 w;
        w.x = cvt_pk_bf16(oacc[db][4 * gq] * inv, oacc[db][4 * gq + 1] * inv);
        w.y = cvt_pk_bf16(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * gq + 4 * hh) = w;
      }
  }
}

}  // namespace

hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t stream) {
  const int Lq = a.n_q * a.g.T;
  const int64_t wgs = static_cast<int64_t>((Lq + 255) / 256) * a.g.B * a.g.H * a.n_splits;
  hipLaunchKernelGGL(attn_fp8_kernel, dim3(static_cast<unsigned>(wgs)), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
