// Sink + short-window attention over the frame cache.
//
// Computes, per stream b and head h, o = softmax(RoPE(q) K^T * scale) V over
// the resident frames (LongLive paper review, section 3 "Short-Window
// Attention" equation with the pinned frames of "Frame Sink"; LoL paper
// review, background "multi-head attention" equation).  Queries are the
// newest n_q resident frames; with the frame-causal mask a query of frame f
// sees the resident frames up to f.  Because resident frames are kept in
// increasing frame order, every query row sees a prefix [0, kend) of the
// logical key sequence.
//
// bf16 kernel (gfx950 matrix cores).  A workgroup of W waves owns 32 W query
// rows of one (stream, head), and each SIMD runs two waves, so one wave's
// softmax overlaps the other's matrix-core work.  W = 8 (one workgroup per
// CU, three K/V stages, two tiles in flight) by default; W = 4 (two
// workgroups per CU, two stages each) on request.
//   * Each wave owns 32 query rows and computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16, so that every lane holds the scores of ONE
//     query (column) for 16 keys per 32-key block: the row max and row sum are
//     in-lane plus one exchange between the two half-waves.
//   * The keys of each 32-key block are permuted (bits 2 and 3 of the row
//     index swapped) when the K operand is read from LDS, so the score
//     registers are already in the order the P^T operand of the second
//     product needs: O^T += V^T P^T runs straight from registers.
//   * V is stored transposed in the cache ([D][T] per slot, stream and head),
//     so the V^T operand is a plain 16-byte LDS read.
//   * q is rotated (RoPE) in fp32 as it is loaded, scaled by the softmax
//     scale * log2(e), then rounded to bf16.
//   * Online softmax in the exp2 domain with a lazily raised running max m:
//     the S^T accumulators start at -m, so p = exp2 of the product with no
//     per-score arithmetic; the row sum is accumulated from the same
//     bf16-rounded p the PV product uses.
//   * K and V^T tiles of 64 keys go global -> LDS by direct-to-LDS buffer
//     loads into XOR-swizzled stages (no VGPR staging, conflict-free
//     operand reads); per-tile frame bases come from the slot table, so sink
//     and ring frames are read in place with no gather copy.
// For one stream at Wan-1.3B shapes the (q-tile, head) grid alone does not
// fill 256 CUs, so the key range is split; each split writes a partial
// (O, m, l) and a small second kernel merges them in split order
// (deterministic).  The kernel boundary orders the two: a merge inside the
// attention kernel would need device-scope fences, which on this chip write
// back and invalidate whole L2 slices and cost more than the merge itself.
//
// fp32 kernel: one thread per query row, VALU FMA, for the small fp32
// configurations (accuracy 1e-5 against an fp64 reference).
//
// The e4m3-cache kernel is in window_attn_fp8.hip; it writes the same split
// partials and is merged by the kernel here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <type_traits>

#include "attn_common.hpp"

namespace sa {
namespace {

typedef __bf16 mfma_bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));

// Lazy rescaling: the running max used for exp2 is only raised when a new
// score exceeds it by more than this (log2 units), so p <= 2^kLazy.
constexpr float kLazy = 8.f;

// Workspace layout (float units): split partials O [S][B][H][Lq][D] (fp32,
// unnormalised), then (m, l) [S][B][H][Lq][2].  Every call writes all of it
// before reading it, so it needs no initialisation.

__device__ __forceinline__ int key_perm(int m) {  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ mfma_bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(mfma_bf16x8, v); }

// Sum of the two bf16 halves of a packed word, accumulated in fp32.
__device__ __forceinline__ float dot2_ones(uint32_t pk, float acc) {
  const bf16x2_t one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), one, acc, false);
}


// LDS stage: 16-byte chunks, no padding, XOR-swizzled so that the 16 lanes of
// a matrix-core operand read hit 16 distinct bank groups:
//   K   : 64 keys x (D/8) chunks, chunk (r, c) at r*(D/8) + (c ^ kswz(r))
//   V^T : D rows x 8 chunks (8 keys each), chunk (d, c) at d*8 + (c ^ vswz(d))
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

template <int D>
struct StageSmem {
  u32x4 k[kKTile * D / 8];
  u32x4 vt[D * kKTile / 8];
};


template <int D>
__device__ __forceinline__ u32x4 lds_read(const StageSmem<D>& st, uint32_t byte_off) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&st) + byte_off);
}

// BIG_T: every 64-key tile spans at most two frames (T >= 64), so frame and
// slot are resolved once per tile with uniform arithmetic.
// W waves per workgroup (W * 32 query rows).  W = 4: two workgroups per CU,
// two K/V stages each; W = 8: one workgroup per CU, three K/V stages, half
// the K/V traffic per query row.
template <int D, bool BIG_T, int W>
__global__ void __launch_bounds__(W * 64, 8 / W) attn_bf16_kernel(AttnArgs a) {
  constexpr int kWaves = W;
  constexpr int kQTile = W * kQW;  // query rows per workgroup
  __shared__ StageSmem<D> st0, st1;
  __shared__ int s_slot[kMaxFrames];
  constexpr int CPR = D / 8;                      // K chunks per key row
  constexpr int KI = kKTile * CPR / 64 / kWaves;  // K DMA instructions per wave per tile
  constexpr int VI = D * 8 / 64 / kWaves;         // V^T DMA instructions per wave per tile
  constexpr uint32_t kVtOff = kKTile * D * 2;     // byte offset of vt inside a stage

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const CacheGeom& g = a.g;
  const int T = g.T;
  const int Lq = a.n_q * T;
  const int n_qt = (Lq + kQTile - 1) / kQTile;
  // logical id = ((b*H + h) * S + split) * n_qt + qt
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % n_qt;
  const int split = (lid / n_qt) % a.n_splits;
  const int bh = lid / (n_qt * a.n_splits);
  const int b = bh / g.H;
  const int h = bh - b * g.H;
  const int n_res = a.frames.n;
  const int first_q = n_res - a.n_q;  // logical index of the first query frame
  const int n_keys = n_res * T;
  if (threadIdx.x < kMaxFrames) s_slot[threadIdx.x] = threadIdx.x < n_res ? a.frames.store_slot[threadIdx.x] : 0;

  const int row = qt * kQTile + wave * kQW + n;
  const bool row_ok = row < Lq;
  const int qf = row_ok ? row / T : a.n_q - 1;
  const int klim = min(n_keys, a.key_limit);
  const int kend = min(a.causal ? (first_q + qf + 1) * T : n_keys, klim);
  const int wave_row0 = qt * kQTile + wave_u * kQW;  // wave-uniform (scalar) from here on
  const bool wave_active = wave_row0 < Lq;
  const int wave_last = min(wave_row0 + kQW - 1, Lq - 1);
  const int wave_kend = min(a.causal ? (first_q + wave_last / T + 1) * T : n_keys, klim);            // largest kend
  const int wave_kmin = min(a.causal ? (first_q + min(wave_row0, Lq - 1) / T + 1) * T : n_keys, klim);  // smallest
  const int last_row = min(qt * kQTile + kQTile - 1, Lq - 1);
  const int kend_wg = min(a.causal ? (first_q + last_row / T + 1) * T : n_keys, klim);
  const int n_tiles = (kend_wg + kKTile - 1) / kKTile;
  const int tile_lo = static_cast<int>((static_cast<int64_t>(n_tiles) * split) / a.n_splits);
  const int tile_hi = static_cast<int>((static_cast<int64_t>(n_tiles) * (split + 1)) / a.n_splits);

  // ---- Q fragment: rotate in fp32, scale by softmax scale * log2(e), round
  // to bf16 (B operand of S^T = K Q^T).
  mfma_bf16x8 qfrag[D / 16];
  {
    const int tok = row_ok ? row - qf * T : 0;
    const int64_t t = a.frames.t[first_q + qf];
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((static_cast<int64_t>(b) * Lq + (row_ok ? row : 0)) * g.H + h) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) {
        float x[8];
        unpack_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hh), x);
        rope_rotate8(a.rope, h, 2 * s + hh, t, tok / a.rope.grid_w, tok % a.rope.grid_w, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] *= a.scale_log2;  // scores come out in log2 units
        v = pack_bf16x8(x);
      }
      qfrag[s] = as_bf16x8(v);
    }
  }

  mfma_f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = kNegInf;  // running (lazy) max of scaled scores, log2 units
  float l_run = 0.f;      // this half-wave's partial row sum
  // S^T accumulators start at -m_use (m_use = m_run, or 0 while it is -inf),
  // so the products come out as s - m_use and p = exp2 of them directly.
  mfma_f32x16 mseed;
#pragma unroll
  for (int i = 0; i < 16; ++i) mseed[i] = 0.f;

  // Per-lane LDS operand addresses (bytes inside a stage); the key block,
  // channel block and stage enter as immediate offsets.
  uint32_t kaddr[D / 16];
  {
    const int r = key_perm(n);  // key row inside the 32-key block (kb adds 32 rows)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kaddr[s] = static_cast<uint32_t>((r * CPR + ((2 * s + hh) ^ kswz<D>(r))) * 16);
  }
  uint32_t vaddr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) vaddr[q] = kVtOff + static_cast<uint32_t>((n * 8 + (((q << 1) | hh) ^ vswz(n))) * 16);

  // ---- global -> LDS (direct) for one tile.
  const uint16_t* kst = static_cast<const uint16_t*>(g.k_store);
  const uint16_t* vst = static_cast<const uint16_t*>(g.v_store);
  const int64_t head_off = static_cast<int64_t>(b) * g.H + h;  // within a slot
  const int64_t slot_stride = static_cast<int64_t>(g.B) * g.H;
  const uint32_t blk_elems = static_cast<uint32_t>(T) * D;  // one (slot, b, h) block
  const u32x4 krsrc = buffer_rsrc(kst, a.store_bytes);
  const u32x4 vrsrc = buffer_rsrc(vst, a.store_bytes);
  __syncthreads();  // s_slot visible
  auto blk_bytes = [&](int lf) -> uint32_t {
    const int slot = __builtin_amdgcn_readfirstlane(s_slot[lf]);
    return static_cast<uint32_t>((static_cast<int64_t>(slot) * slot_stride + head_off) * blk_elems * 2);
  };
  // Each wave instruction writes 64 consecutive chunks of the stage, lane L
  // landing at chunk (base + L); the lane fetches whichever global chunk the
  // swizzled layout puts there.  Keys past kend_wg are clamped to the tile's
  // first key (resident, finite): their scores are masked, they add nothing.
  // plan_tile resolves a tile's frames and this lane's byte offsets; fire
  // issues one of the wave's KI + VI transfers.  The transfers of the next
  // tiles are spread over the current tile's S^T products: issued together
  // they queue at the CU's texture addresser and stall every wave.
  struct TilePlan {
    uint32_t off[KI + VI];
  };
  // Frame of the tiles being planned (BIG_T): tiles are planned in
  // non-decreasing order, so the frame lf0 of a tile's first key and the
  // store offsets of frames lf0 and lf0+1 are advanced, not recomputed.
  int pl_lf0 = 0, pl_jb = T;
  uint32_t pl_b0 = 0, pl_b1 = 0;
  if (BIG_T) {
    pl_b0 = blk_bytes(0);
    pl_b1 = blk_bytes(min(1, n_res - 1));
  }
  // Lane parts of the byte offsets of a tile that lies inside one frame:
  // key row r, chunk c -> r*D*2 + c*16; V^T row d, key chunk c -> d*T*2 + c*16.
  uint32_t klane[KI], vlane[VI];
#pragma unroll
  for (int u = 0; u < KI; ++u) {
    const int P = 64 * (wave_u * KI + u) + lane;
    const int r = P / CPR, c = (P % CPR) ^ kswz<D>(r);
    klane[u] = static_cast<uint32_t>(r * (D * 2) + c * 16);
  }
#pragma unroll
  for (int u = 0; u < VI; ++u) {
    const int P = 64 * (wave_u * VI + u) + lane;
    const int d = P / 8, c = (P % 8) ^ vswz(d);
    vlane[u] = static_cast<uint32_t>(d * T * 2 + c * 16);
  }
  auto plan_tile = [&](int kt) {
    TilePlan p;
    const int j0 = kt * kKTile;
    uint32_t koff0 = 0, koff1 = 0, voff0 = 0, voff1 = 0;
    int jb = 0;
    if (BIG_T) {
      while (j0 >= pl_jb) {
        ++pl_lf0;
        pl_jb += T;
        pl_b0 = pl_b1;
        pl_b1 = blk_bytes(min(pl_lf0 + 1, n_res - 1));
      }
      const int lf0 = pl_lf0;
      jb = pl_jb;
      const uint32_t b0 = pl_b0, b1 = pl_b1;
      koff0 = b0 - static_cast<uint32_t>(lf0) * blk_elems * 2;
      koff1 = b1 - static_cast<uint32_t>(jb) * D * 2;
      voff0 = b0 - static_cast<uint32_t>(lf0) * T * 2;
      voff1 = b1 - static_cast<uint32_t>(jb) * 2;
      // common case: the whole tile in frame lf0 and before kend_wg -- a
      // scalar tile base plus the lane part (wave-uniform branch)
      if (j0 + kKTile <= jb && j0 + kKTile <= kend_wg) {
        const uint32_t kb = koff0 + static_cast<uint32_t>(j0) * (D * 2);
        const uint32_t vb = voff0 + static_cast<uint32_t>(j0) * 2;
#pragma unroll
        for (int u = 0; u < KI; ++u) p.off[u] = kb + klane[u];
#pragma unroll
        for (int u = 0; u < VI; ++u) p.off[KI + u] = vb + vlane[u];
        return p;
      }
    }
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int P = 64 * (wave_u * KI + u) + lane;
      const int r = P / CPR, c = (P % CPR) ^ kswz<D>(r);
      int j = j0 + r;
      if (j >= kend_wg) j = j0;
      uint32_t off;
      if (BIG_T) {
        off = (j < jb ? koff0 : koff1) + static_cast<uint32_t>(j) * (D * 2);
      } else {
        const int lf = j / T;
        off = static_cast<uint32_t>((static_cast<int64_t>(s_slot[lf]) * slot_stride + head_off) * blk_elems * 2) +
              static_cast<uint32_t>(j - lf * T) * (D * 2);
      }
      p.off[u] = off + c * 16;
    }
#pragma unroll
    for (int u = 0; u < VI; ++u) {
      const int P = 64 * (wave_u * VI + u) + lane;
      const int d = P / 8, c = (P % 8) ^ vswz(d);
      int j = j0 + c * 8;
      if (j >= kend_wg) j = j0;
      uint32_t off;
      if (BIG_T) {
        off = (j < jb ? voff0 : voff1) + static_cast<uint32_t>(d) * T * 2 + static_cast<uint32_t>(j) * 2;
      } else {
        const int lf = j / T;
        off = static_cast<uint32_t>((static_cast<int64_t>(s_slot[lf]) * slot_stride + head_off) * blk_elems * 2) +
              static_cast<uint32_t>(d) * T * 2 + static_cast<uint32_t>(j - lf * T) * 2;
      }
      p.off[KI + u] = off;
    }
    return p;
  };
  auto fire = [&](const TilePlan& p, int u, StageSmem<D>& st) {
    if (u < KI)
      dma16(krsrc, p.off[u], &st.k[64 * (wave_u * KI + u)]);
    else
      dma16(vrsrc, p.off[u], &st.vt[64 * (wave_u * VI + (u - KI))]);
  };
  auto issue_tile = [&](int kt, StageSmem<D>& st) {
    const TilePlan p = plan_tile(kt);
#pragma unroll
    for (int u = 0; u < KI + VI; ++u) fire(p, u, st);
  };
  // one transfer after every kFireStep pairs of S^T products
  constexpr int kFireStep = (D / 16) / (KI + VI) > 0 ? (D / 16) / (KI + VI) : 1;
  static_assert((D / 16) / kFireStep >= KI + VI, "every transfer has a slot in the S^T loop");

  // ---- one 64-key tile: S^T for both 32-key blocks (two independent
  // accumulation chains), softmax of the 32 scores each lane holds, then
  // O^T += V^T P^T over four channel blocks.
  // With do_fire, the wave's transfers of plan np into stage nst are issued
  // in between (or, for a wave with nothing to compute, at once).
  auto compute = [&](int kt, const StageSmem<D>& st, bool do_fire, const TilePlan& np, StageSmem<D>& nst) {
    const int j0 = kt * kKTile;
    if (!wave_active || j0 >= wave_kend) {
      if (do_fire) {
#pragma unroll
        for (int u = 0; u < KI + VI; ++u) fire(np, u, nst);
      }
      return;
    }
    mfma_f32x16 sacc[2];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read(st, kaddr[s] + kb * 32 * CPR * 16)),
                                                            qfrag[s], s == 0 ? mseed : sacc[kb], 0, 0, 0);
      if (do_fire && s % kFireStep == 0 && s / kFireStep < KI + VI) fire(np, s / kFireStep, nst);
    }
    // mask (register i of block kb holds key j0 + 32kb + 16(i/8) + 8hh + i%8)
    if (j0 + kKTile > wave_kmin) {
      const int lim = kend - j0 - 8 * hh;  // keys j0 + 8hh + off with off >= lim are hidden
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 16 * (i >> 3) + (i & 7) >= lim) sacc[kb][i] = kNegInf;
    }
    // sacc holds s - m_use; raise the running max lazily (rare; the branch is
    // wave-uniform, the decision per row).  m stays an integer, so p = 2^(s - m)
    // is rounded exactly as 2^s would be, whatever m a row has reached.
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    const float mx = max_halves(tile_max(sacc)) + m_use;  // the tile's max of s
    if (__any(mx > m_run + kLazy)) {
      const float m_new = mx > m_run + kLazy ? ceilf(mx) : m_run;
      const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      // re-base this tile's scores and the seed of the next tiles
      const float m_next = m_new == kNegInf ? 0.f : m_new;
      const float shift = m_next - m_use;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] -= shift;
#pragma unroll
      for (int i = 0; i < 16; ++i) mseed[i] = -m_next;
    }
    u32x4 pk[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[kb][8 * s2 + 2 * w]);
          const float p1 = __builtin_amdgcn_exp2f(sacc[kb][8 * s2 + 2 * w + 1]);
          pk[kb][s2][w] = cvt_pk_bf16(p0, p1);
          l_run = dot2_ones(pk[kb][s2][w], l_run);
        }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(lds_read(st, vaddr[q] + db * 32 * 8 * 16)), as_bf16x8(pk[q >> 1][q & 1]), oacc[db], 0, 0, 0);
  };

  if constexpr (W == 4) {
    // ---- two stages (two workgroups share a CU's LDS), unrolled by two so
    // both stages are fixed objects: wait for tile kt, barrier (which also
    // retires the stage read at kt-1), compute tile kt while issuing tile
    // kt+1 into that stage.
    if (tile_lo < tile_hi) issue_tile(tile_lo, st0);
    for (int kt = tile_lo; kt < tile_hi; kt += 2) {
      wait_vmcnt0();
      barrier();
      compute(kt, st0, kt + 1 < tile_hi, plan_tile(min(kt + 1, tile_hi - 1)), st1);
      if (kt + 1 < tile_hi) {
        wait_vmcnt0();
        barrier();
        compute(kt + 1, st1, kt + 2 < tile_hi, plan_tile(min(kt + 2, tile_hi - 1)), st0);
      }
    }
  } else {
    // ---- three stages, two tiles in flight (one workgroup per CU).  Each
    // step waits until only the newer tile's loads are outstanding, so tile
    // kt has landed in every wave's share; the barrier also retires the
    // stage that tile kt-1 was read from, which then receives tile kt+2.
    // Past the end the last tile is fetched again into a stage nobody reads,
    // which keeps the outstanding-load count the same in every step.
    __shared__ StageSmem<D> st2;
    const int t_last = tile_hi - 1;
    if (tile_lo < tile_hi) {
      issue_tile(tile_lo, st0);
      issue_tile(min(tile_lo + 1, t_last), st1);
    }
    auto step = [&](int kt, const StageSmem<D>& cur, StageSmem<D>& nxt2) {
      static_assert(KI + VI == 4 || KI + VI == 2, "one tile's DMA count per wave");
      if constexpr (KI + VI == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      barrier();
      compute(kt, cur, true, plan_tile(min(kt + 2, t_last)), nxt2);
    };
    for (int kt = tile_lo; kt < tile_hi; kt += 3) {
      step(kt, st0, st2);
      if (kt + 1 < tile_hi) step(kt + 1, st1, st0);
      if (kt + 2 < tile_hi) step(kt + 2, st2, st1);
    }
    wait_vmcnt0();
  }

  // ---- epilogue: lane holds O^T[d][row] for d = 32db + 8(i/4) + 4hh + i%4.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (a.n_splits > 1) {
    // Publish this split's partial; attn_merge_kernel combines the splits.
    if (row_ok) {
      const int64_t plane = static_cast<int64_t>(g.B) * g.H * Lq;
      const int64_t prow = static_cast<int64_t>(bh) * Lq + row;
      float* po = a.ws + (split * plane + prow) * D;
      if (a.stat_mode != kStatMass) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const f32x4 w = {oacc[db][4 * gq], oacc[db][4 * gq + 1], oacc[db][4 * gq + 2], oacc[db][4 * gq + 3]};
            *reinterpret_cast<f32x4*>(po + 32 * db + 8 * gq + 4 * hh) = w;
          }
      }
      if (hh == 0) {
        float* pml = a.ws + static_cast<int64_t>(a.n_splits) * plane * D + (split * plane + prow) * 2;
        pml[0] = m_run;
        pml[1] = l_tot;
      }
    }
    return;
  }
  if (row_ok && a.stat_mode != kStatNone && hh == 0)
    write_stat(a.stat_mode, a.stat + (static_cast<int64_t>(b) * Lq + row) * g.H + h, m_run, l_tot);
  if (row_ok && a.stat_mode != kStatMass) {
    const float inv = 1.f / l_tot;
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

// ---------------------------------------------------------------------------
// Software-pipelined bf16 kernel, in two shapes: eight waves per workgroup
// (two per SIMD) of 32 query rows each, or four waves (one per SIMD) of 64
// rows each.  A SIMD overlaps matrix-core and vector work only inside one
// wave's instruction stream (an MFMA wave and a VALU wave on one SIMD run
// nearly one after the other), so each wave interleaves its own work: while
// the products S(t+1) = K(t+1) Q^T run, it exponentiates and packs the scores
// of tile t; while O^T += V^T(t) P^T(t) runs, it takes the row maxima of
// S(t+1).  A 64-row wave feeds each K and V^T operand read to two products
// and runs a tile's addressing, transfers and waits once for both row
// blocks.  Q and S sit in ordinary vector registers, O^T too in the 32-row
// shape and in AGPRs in the 64-row one; four K/V stages keep two tiles in
// flight ahead of the one being multiplied.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// QB (1 or 2) row blocks of 32 query rows per wave, 8 / QB waves per
// workgroup (256 query rows, one workgroup per CU, four K/V stages).
template <int D, bool BIG_T, int QB>
__global__ void __launch_bounds__(512 / QB, 1) attn_bf16_pipe_kernel(AttnArgs a) {
  constexpr int kWaves = 8 / QB;
  constexpr int kRowsW = 32 * QB;                 // query rows per wave
  constexpr bool kAgprO = QB > 1;                 // O^T accumulators in AGPRs
  constexpr int kQTile = kWaves * kRowsW;         // 256
  // Four K/V stages, the K tiles of all four in one array and the V^T tiles
  // in another: every operand read then addresses its stage and block with
  // the instruction's 16-bit immediate offset from one per-lane register.
  __shared__ u32x4 kq[4][kKTile * D / 8];
  __shared__ u32x4 vq[4][D * kKTile / 8];
  __shared__ int s_slot[kMaxFrames];
  constexpr int CPR = D / 8;
  constexpr int KI = kKTile * CPR / 64 / kWaves;  // K DMA instructions per wave per tile
  constexpr int VI = D * 8 / 64 / kWaves;         // V^T DMA instructions per wave per tile
  constexpr int NDMA = KI + VI;
  constexpr int KS = D / 16;                      // k-steps of an S product
  constexpr uint32_t kStageBytes = kKTile * D * 2;  // one stage of K, or of V^T
  static_assert(NDMA <= 8, "one transfer per k-step slot");

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
  const int n_keys = n_res * T;
  if (threadIdx.x < kMaxFrames) s_slot[threadIdx.x] = threadIdx.x < n_res ? a.frames.store_slot[threadIdx.x] : 0;

  const int klim = min(n_keys, a.key_limit);
  int row[QB], kend[QB];
  bool row_ok[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    row[qb] = qt * kQTile + wave * kRowsW + 32 * qb + n;
    row_ok[qb] = row[qb] < Lq;
    const int qf = row_ok[qb] ? row[qb] / T : a.n_q - 1;
    kend[qb] = min(a.causal ? (first_q + qf + 1) * T : n_keys, klim);
  }
  const int wave_row0 = qt * kQTile + wave_u * kRowsW;
  const int wave_kmin = min(a.causal ? (first_q + min(wave_row0, Lq - 1) / T + 1) * T : n_keys, klim);
  const int last_row = min(qt * kQTile + kQTile - 1, Lq - 1);
  const int kend_wg = min(a.causal ? (first_q + last_row / T + 1) * T : n_keys, klim);
  const int n_tiles = (kend_wg + kKTile - 1) / kKTile;
  const int tile_lo = static_cast<int>((static_cast<int64_t>(n_tiles) * split) / a.n_splits);
  const int tile_hi = static_cast<int>((static_cast<int64_t>(n_tiles) * (split + 1)) / a.n_splits);

  // ---- Q fragments (rotated, scaled to log2 units, bf16), kept in
  // accumulation registers
  mfma_bf16x8 qfrag[QB][KS];
  {
    u32x4 qv[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qf = row_ok[qb] ? row[qb] / T : a.n_q - 1;
      const int tok = row_ok[qb] ? row[qb] - qf * T : 0;
      const int64_t t = a.frames.t[first_q + qf];
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                             ((static_cast<int64_t>(b) * Lq + (row_ok[qb] ? row[qb] : 0)) * g.H + h) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok[qb]) {
          float x[8];
          unpack_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hh), x);
          rope_rotate8(a.rope, h, 2 * s + hh, t, tok / a.rope.grid_w, tok % a.rope.grid_w, x);
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] *= a.scale_log2;
          v = pack_bf16x8(x);
        }
        qv[qb][s] = v;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < KS; ++s) qfrag[qb][s] = as_bf16x8(qv[qb][s]);
  }

  mfma_f32x16 oacc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
  // With two row blocks per wave the O^T accumulators (128 registers at
  // D = 128) live in AGPRs: the O products are written as inline asm with
  // AGPR accumulators, while the S products stay in VGPR form for the
  // softmax that reads them.  The compiler does not see an asm product's
  // result latency, so every ordinary read of an accumulator waits behind a
  // fence that first pads 24 wait states (more than the product's result
  // latency), and every ordinary write is followed by one before the next
  // product reads it.  A fence is one asm statement per accumulator, with the
  // padding in the first (before reads) or the last (after writes); each
  // statement takes its accumulator as an operand, which orders it with that
  // accumulator's reads and writes, and asm statements keep their order.
  auto acc_fence = [&](bool before_read) {
    if constexpr (kAgprO) {
      if (before_read) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(oacc[0][0]));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          if (before_read ? (qb | db) != 0 : !(qb == QB - 1 && db == D / 32 - 1))
            asm volatile("" : "+a"(oacc[qb][db]));
      if (!before_read) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(oacc[QB - 1][D / 32 - 1]));
    }
  };
  acc_fence(false);
  float m_run[QB], l_run[QB];
  mfma_f32x16 mseed[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) mseed[qb][i] = 0.f;
  }

  uint32_t kaddr[KS];
  {
    const int r = key_perm(n);
#pragma unroll
    for (int s = 0; s < KS; ++s) kaddr[s] = static_cast<uint32_t>((r * CPR + ((2 * s + hh) ^ kswz<D>(r))) * 16);
  }
  // V^T operand addresses as full LDS byte addresses, hidden from constant
  // folding: the V^T stages start 64 KiB into LDS, past what the 16-bit
  // immediate offset can reach, so the stage and channel block offsets must
  // be added to a base register that already holds the array's address.
  typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
  const uint32_t vq_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(&vq[0][0])));
  uint32_t vaddr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    vaddr[q] = vq_base + static_cast<uint32_t>((n * 8 + (((q << 1) | hh) ^ vswz(n))) * 16);
    asm volatile("" : "+v"(vaddr[q]));
  }
  // operand reads: K of stage st, 32-key block kb, k-step s; V^T of stage st,
  // 16-key step q, channel block db
  auto kread = [&](int st, int kb, int s) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&kq[0][0]) + kaddr[s] +
                                                     st * kStageBytes + kb * 32 * CPR * 16));
  };
  auto vread = [&](int st, int q, int db) {
    return as_bf16x8(*reinterpret_cast<lds_u32x4*>(
        static_cast<uintptr_t>(vaddr[q] + st * kStageBytes + db * 32 * 8 * 16)));
  };

  // ---- global -> LDS transfers (as in attn_bf16_kernel: the waves share each tile)
  const uint16_t* kst = static_cast<const uint16_t*>(g.k_store);
  const uint16_t* vst = static_cast<const uint16_t*>(g.v_store);
  const int64_t head_off = static_cast<int64_t>(b) * g.H + h;
  const int64_t slot_stride = static_cast<int64_t>(g.B) * g.H;
  const uint32_t blk_elems = static_cast<uint32_t>(T) * D;
  const u32x4 krsrc = buffer_rsrc(kst, a.store_bytes);
  const u32x4 vrsrc = buffer_rsrc(vst, a.store_bytes);
  __syncthreads();
  auto blk_bytes = [&](int lf) -> uint32_t {
    const int slot = __builtin_amdgcn_readfirstlane(s_slot[lf]);
    return static_cast<uint32_t>((static_cast<int64_t>(slot) * slot_stride + head_off) * blk_elems * 2);
  };
  struct TilePlan {
    uint32_t off[NDMA];
  };
  int pl_lf0 = 0, pl_jb = T;
  uint32_t pl_b0 = 0, pl_b1 = 0;
  if (BIG_T) {
    pl_b0 = blk_bytes(0);
    pl_b1 = blk_bytes(min(1, n_res - 1));
  }
  uint32_t klane[KI], vlane[VI];
#pragma unroll
  for (int u = 0; u < KI; ++u) {
    const int P = 64 * (wave_u * KI + u) + lane;
    const int r = P / CPR, c = (P % CPR) ^ kswz<D>(r);
    klane[u] = static_cast<uint32_t>(r * (D * 2) + c * 16);
  }
#pragma unroll
  for (int u = 0; u < VI; ++u) {
    const int P = 64 * (wave_u * VI + u) + lane;
    const int d = P / 8, c = (P % 8) ^ vswz(d);
    vlane[u] = static_cast<uint32_t>(d * T * 2 + c * 16);
  }
  auto plan_tile = [&](int kt) {
    TilePlan p;
    const int j0 = kt * kKTile;
    uint32_t koff0 = 0, koff1 = 0, voff0 = 0, voff1 = 0;
    int jb = 0;
    if (BIG_T) {
      while (j0 >= pl_jb) {
        ++pl_lf0;
        pl_jb += T;
        pl_b0 = pl_b1;
        pl_b1 = blk_bytes(min(pl_lf0 + 1, n_res - 1));
      }
      const int lf0 = pl_lf0;
      jb = pl_jb;
      const uint32_t b0 = pl_b0, b1 = pl_b1;
      koff0 = b0 - static_cast<uint32_t>(lf0) * blk_elems * 2;
      koff1 = b1 - static_cast<uint32_t>(jb) * D * 2;
      voff0 = b0 - static_cast<uint32_t>(lf0) * T * 2;
      voff1 = b1 - static_cast<uint32_t>(jb) * 2;
      if (j0 + kKTile <= jb && j0 + kKTile <= kend_wg) {
        const uint32_t kb = koff0 + static_cast<uint32_t>(j0) * (D * 2);
        const uint32_t vb = voff0 + static_cast<uint32_t>(j0) * 2;
#pragma unroll
        for (int u = 0; u < KI; ++u) p.off[u] = kb + klane[u];
#pragma unroll
        for (int u = 0; u < VI; ++u) p.off[KI + u] = vb + vlane[u];
        return p;
      }
    }
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int P = 64 * (wave_u * KI + u) + lane;
      const int r = P / CPR, c = (P % CPR) ^ kswz<D>(r);
      int j = j0 + r;
      if (j >= kend_wg) j = j0;
      uint32_t off;
      if (BIG_T) {
        off = (j < jb ? koff0 : koff1) + static_cast<uint32_t>(j) * (D * 2);
      } else {
        const int lf = j / T;
        off = static_cast<uint32_t>((static_cast<int64_t>(s_slot[lf]) * slot_stride + head_off) * blk_elems * 2) +
              static_cast<uint32_t>(j - lf * T) * (D * 2);
      }
      p.off[u] = off + c * 16;
    }
#pragma unroll
    for (int u = 0; u < VI; ++u) {
      const int P = 64 * (wave_u * VI + u) + lane;
      const int d = P / 8, c = (P % 8) ^ vswz(d);
      int j = j0 + c * 8;
      if (j >= kend_wg) j = j0;
      uint32_t off;
      if (BIG_T) {
        off = (j < jb ? voff0 : voff1) + static_cast<uint32_t>(d) * T * 2 + static_cast<uint32_t>(j) * 2;
      } else {
        const int lf = j / T;
        off = static_cast<uint32_t>((static_cast<int64_t>(s_slot[lf]) * slot_stride + head_off) * blk_elems * 2) +
              static_cast<uint32_t>(d) * T * 2 + static_cast<uint32_t>(j - lf * T) * 2;
      }
      p.off[KI + u] = off;
    }
    return p;
  };
  auto fire = [&](const TilePlan& p, int u, int st) {
    if (u < KI)
      dma16_nomem(krsrc, p.off[u], &kq[st][64 * (wave_u * KI + u)]);
    else
      dma16_nomem(vrsrc, p.off[u], &vq[st][64 * (wave_u * VI + (u - KI))]);
  };

  // Mask the keys a row does not see (register i holds key j0 + 16(i/8) +
  // 8hh + i%8), and the row maximum of one row block.
  auto mask_rows = [&](int j0, mfma_f32x16& x, int qb) {
    const int lim = kend[qb] - j0 - 8 * hh;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * (i >> 3) + (i & 7) >= lim) x[i] = kNegInf;
  };
  auto row_max = [&](const mfma_f32x16& x) {
    const float a0 = fmaxf(fmaxf(x[0], x[1]), x[2]), a1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
    const float a2 = fmaxf(fmaxf(x[6], x[7]), x[8]), a3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
    const float a4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
    return max_halves(fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), x[15])));
  };
  // ---- one pipeline step over a block of 32 keys (half a tile), in two
  // interleaved phases separated by scheduling barriers:
  //   phase 1: S^T products of the next block (every row block, D/16
  //            k-steps, K operand reads two steps ahead; the first product
  //            starts from the masked or plain seed), each k-step slot
  //            followed by an eighth of this block's softmax (per row block 2
  //            exp2, 1 pack, 1 row-sum dot) and one of a later tile's
  //            transfers (half of them at each block of a tile);
  //   phase 2: O^T += V^T P^T over this block's two 16-key steps (V^T reads
  //            two ahead), with the row maxima of the next block between the
  //            products of the second half.
  // Operand reads run kLA products ahead, through rings of kLA + 1, and each
  // phase issues the first kLA operand reads of the phase after it in its
  // last kLA slots, so no phase starts by waiting out a full LDS read.
  // Blocks a row does not see are computed and masked, so neither phase has a
  // branch inside; the only data-dependent one is the rare running-max raise.
  constexpr int kLA = 4, kRing = kLA + 1;
  static_assert(kLA <= KS && kLA <= 4 * (D / 32) && kLA <= 8, "read-ahead within a phase");
  mfma_bf16x8 kop[kRing], vop[kRing];
  auto phase1 = [&](int kst_, int kbn, mfma_f32x16 (&sn)[QB], const mfma_f32x16 (&sc)[QB], u32x4 (&pk)[QB][2],
                    const TilePlan* np, int nst, int u0, int nu, int jn, int vst_, int vkb) {
    // kop[0 .. kLA-1] hold (or are loading) k-steps 0 .. kLA-1 of block kbn.
    // First k-step: the accumulator starts at -m of the row (scores come out
    // re-based), or at -inf for the keys the row does not see when the next
    // block reaches past the wave's first row's last visible key.  Deciding
    // here, before the interleaved work, leaves no branch inside it.
    if (jn + 32 > wave_kmin) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        mfma_f32x16 seed = mseed[qb];
        mask_rows(jn, seed, qb);
        sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qfrag[qb][0], seed, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qfrag[qb][0], mseed[qb], 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < KS) {
        if (s + kLA < KS) kop[(s + kLA) % kRing] = kread(kst_, kbn, s + kLA);
        if (s > 0) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s % kRing], qfrag[qb][s], sn[qb], 0, 0, 0);
        }
      }
      // the next phase's first kLA V^T operands
      if (s >= 8 - kLA) {
        const int i = s - (8 - kLA);
        vop[i] = vread(vst_, 2 * vkb + i / (D / 32), i % (D / 32));
      }
      if (np && s < nu) fire(*np, u0 + s, nst);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {  // pair s of row block qb: 16-key half s/4, word s%4
        const int s2 = s >> 2, w = s & 3;
        const float p0 = __builtin_amdgcn_exp2f(sc[qb][8 * s2 + 2 * w]);
        const float p1 = __builtin_amdgcn_exp2f(sc[qb][8 * s2 + 2 * w + 1]);
        pk[qb][s2][w] = cvt_pk_bf16(p0, p1);
        l_run[qb] = dot2_ones(pk[qb][s2][w], l_run[qb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto phase2 = [&](int vst_, int kb, const u32x4 (&pk)[QB][2], const mfma_f32x16 (&sn)[QB], float (&mx)[QB],
                    int kst_next, int kbn_next) {
    constexpr int NR = 2 * (D / 32);  // V^T operand reads: (s2, db) = (r / (D/32), r % (D/32))
    static_assert(NR / 2 + QB <= NR, "a slot for each row block's maximum");
    // vop[0 .. kLA-1] hold (or are loading) the first kLA V^T operands
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int s2 = r / (D / 32), db = r % (D / 32);
      if (r + kLA < NR)
        vop[(r + kLA) % kRing] = vread(vst_, 2 * kb + (r + kLA) / (D / 32), (r + kLA) % (D / 32));
      // the next phase's first kLA K operands
      if (r >= NR - kLA) kop[r - (NR - kLA)] = kread(kst_next, kbn_next, r - (NR - kLA));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (kAgprO)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                       : "+a"(oacc[qb][db])
                       : "v"(vop[r % kRing]), "v"(as_bf16x8(pk[qb][s2])));
        else
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[r % kRing], as_bf16x8(pk[qb][s2]), oacc[qb][db], 0, 0, 0);
      }
      // the next block's scores are complete (and past the MFMA result
      // hazard) from half way on
      if (r >= NR / 2 && r < NR / 2 + QB) mx[r - NR / 2] = row_max(sn[r - NR / 2]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Lazy raise of the running maxima (per row, to an integer; rare, and
  // wave-uniform as a branch), then the re-base of the block's scores.
  // sn holds s - m_use; mxr the block's maxima of s - m_use.
  auto raise_max = [&](mfma_f32x16 (&sn)[QB], const float (&mxr)[QB]) {
    float m_use[QB], mx[QB];
    bool up = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_use[qb] = m_run[qb] == kNegInf ? 0.f : m_run[qb];
      mx[qb] = mxr[qb] + m_use[qb];
      up = up || mx[qb] > m_run[qb] + kLazy;
    }
    if (__any(up)) {
      acc_fence(true);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = mx[qb] > m_run[qb] + kLazy ? ceilf(mx[qb]) : m_run[qb];
        const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
        const float m_next = m_new == kNegInf ? 0.f : m_new;
        const float shift = m_next - m_use[qb];
#pragma unroll
        for (int i = 0; i < 16; ++i) sn[qb][i] -= shift;
#pragma unroll
        for (int i = 0; i < 16; ++i) mseed[qb][i] = -m_next;
      }
      acc_fence(false);
    }
  };

  // ---- the pipeline, in 32-key blocks; block j is half kb = j % 2 of tile
  // t = j / 2, and tile t lives in LDS stage (t - tile_lo) % 4.  Step j runs
  // phase 1 [S(j+1) products | softmax of block j] and phase 2 [PV(j)
  // products | maxima of S(j+1)], then raises the maxima if needed.  At the
  // first block of tile t the wave first waits until tile t+1 has landed
  // (only tile t+2's transfers may still be out) and meets the other waves
  // at a barrier (all are past tile t-1, so its stage is free); tile t+3's
  // transfers then go into that stage during the phase 1 of both blocks.
  // Every K operand a phase 2 reads ahead (blocks of tiles t and t+1) has
  // landed by then.  Past the end the last tile is fetched again into a
  // stage nobody reads (which keeps the count of transfers in flight the
  // same at every wait), and the last step's next-block products are
  // computed and dropped.
  const int t_last = tile_hi - 1;
  mfma_f32x16 sa[QB], sb[QB];
  u32x4 pk[QB][2];
  if (tile_lo < tile_hi) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const TilePlan pl = plan_tile(min(tile_lo + k, t_last));
#pragma unroll
      for (int u = 0; u < NDMA; ++u) fire(pl, u, k);
    }
    wait_vmcnt<2 * NDMA>();
    barrier();
    // S of the first block, with nothing to overlap
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const mfma_bf16x8 k0 = kread(0, 0, s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        sa[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qfrag[qb][s], s == 0 ? mseed[qb] : sa[qb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < kLA; ++i) kop[i] = kread(0, 1, i);
    float mx0[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (tile_lo * kKTile + 32 > wave_kmin) mask_rows(tile_lo * kKTile, sa[qb], qb);
      mx0[qb] = row_max(sa[qb]);
    }
    raise_max(sa, mx0);
  }
  // step over block (t, KB): stage cur holds tile t, nxt tile t+1, fr receives
  // tile t+3, whose transfers are split between the tile's two steps
  constexpr int kFire0 = NDMA / 2;
  TilePlan np_t3;
  auto step = [&](auto kb_c, int t, mfma_f32x16 (&s_cur)[QB], mfma_f32x16 (&s_nxt)[QB], int cur, int nxt, int fr) {
    constexpr int KB = decltype(kb_c)::value;
    const int jn = t * kKTile + 32 * KB + 32;  // first key of the next block
    float mx[QB];
    if constexpr (KB == 0) {
      wait_vmcnt<NDMA>();
      barrier();
      np_t3 = plan_tile(min(t + 3, t_last));
      phase1(cur, 1, s_nxt, s_cur, pk, &np_t3, fr, 0, kFire0, jn, cur, 0);
      phase2(cur, 0, pk, s_nxt, mx, nxt, 0);
      raise_max(s_nxt, mx);
    } else {
      phase1(nxt, 0, s_nxt, s_cur, pk, &np_t3, fr, kFire0, NDMA - kFire0, jn, cur, 1);
      phase2(cur, 1, pk, s_nxt, mx, nxt, 1);
      if (t < t_last) raise_max(s_nxt, mx);
    }
  };
  using KB0 = std::integral_constant<int, 0>;
  using KB1 = std::integral_constant<int, 1>;
  for (int kt = tile_lo; kt < tile_hi; kt += 4) {
    step(KB0{}, kt, sa, sb, 0, 1, 3);
    step(KB1{}, kt, sb, sa, 0, 1, 3);
    if (kt + 1 < tile_hi) {
      step(KB0{}, kt + 1, sa, sb, 1, 2, 0);
      step(KB1{}, kt + 1, sb, sa, 1, 2, 0);
    }
    if (kt + 2 < tile_hi) {
      step(KB0{}, kt + 2, sa, sb, 2, 3, 1);
      step(KB1{}, kt + 2, sb, sa, 2, 3, 1);
    }
    if (kt + 3 < tile_hi) {
      step(KB0{}, kt + 3, sa, sb, 3, 0, 2);
      step(KB1{}, kt + 3, sb, sa, 3, 0, 2);
    }
  }
  wait_vmcnt0();
  acc_fence(true);

  // ---- epilogue: lane holds O^T[d][row] of its row blocks
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (a.n_splits > 1) {
      if (row_ok[qb]) {
        const int64_t plane = static_cast<int64_t>(g.B) * g.H * Lq;
        const int64_t prow = static_cast<int64_t>(bh) * Lq + row[qb];
        float* po = a.ws + (split * plane + prow) * D;
        if (a.stat_mode != kStatMass) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const f32x4 w = {oacc[qb][db][4 * gq], oacc[qb][db][4 * gq + 1], oacc[qb][db][4 * gq + 2],
                               oacc[qb][db][4 * gq + 3]};
              *reinterpret_cast<f32x4*>(po + 32 * db + 8 * gq + 4 * hh) = w;
            }
        }
        if (hh == 0) {
          float* pml = a.ws + static_cast<int64_t>(a.n_splits) * plane * D + (split * plane + prow) * 2;
          pml[0] = m_run[qb];
          pml[1] = l_tot;
        }
      }
      continue;
    }
    if (row_ok[qb] && a.stat_mode != kStatNone && hh == 0)
      write_stat(a.stat_mode, a.stat + (static_cast<int64_t>(b) * Lq + row[qb]) * g.H + h, m_run[qb], l_tot);
    if (row_ok[qb] && a.stat_mode != kStatMass) {
      const float inv = 1.f / l_tot;
      uint16_t* orow = static_cast<uint16_t*>(a.o) + ((static_cast<int64_t>(b) * Lq + row[qb]) * g.H + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          uint2 w;
          w.x = cvt_pk_bf16(oacc[qb][db][4 * gq] * inv, oacc[qb][db][4 * gq + 1] * inv);
          w.y = cvt_pk_bf16(oacc[qb][db][4 * gq + 2] * inv, oacc[qb][db][4 * gq + 3] * inv);
          *reinterpret_cast<uint2*>(orow + 32 * db + 8 * gq + 4 * hh) = w;
        }
    }
  }
}

// fp32 path: one thread per query row, 32-key tiles staged in LDS.
constexpr int kF32Rows = 64;
constexpr int kF32Keys = 32;

// Split merge: o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with
// M = max_s m_s, splits in order.  16 lanes per row, 8 channels each.
template <int D>
__global__ void __launch_bounds__(256) attn_merge_kernel(const float* __restrict__ ws, uint16_t* __restrict__ o,
                                                         int B, int H, int Lq, int n_splits, int stat_mode,
                                                         float* __restrict__ stat) {
  constexpr int kLanes = D / 8;
  constexpr int kRows = 256 / kLanes;
  const int64_t plane = static_cast<int64_t>(B) * H * Lq;
  const int64_t prow = static_cast<int64_t>(blockIdx.x) * kRows + threadIdx.x / kLanes;  // (b*H + h)*Lq + row
  const int c8 = (threadIdx.x % kLanes) * 8;
  if (prow >= plane) return;
  const float* pml = ws + static_cast<int64_t>(n_splits) * plane * D;
  float M = kNegInf;
  for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, pml[(sp * plane + prow) * 2]);
  const int64_t bh = prow / Lq;
  const int row = static_cast<int>(prow - bh * Lq);
  const int b = static_cast<int>(bh / H), h = static_cast<int>(bh - static_cast<int64_t>(b) * H);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (stat_mode == kStatMass) {  // statistics only: the partial O were not written
    for (int sp = 0; sp < n_splits; ++sp) {
      const float ms = pml[(sp * plane + prow) * 2];
      if (ms != kNegInf) l += pml[(sp * plane + prow) * 2 + 1] * __builtin_amdgcn_exp2f(ms - M);
    }
    if (c8 == 0) write_stat(stat_mode, stat + (static_cast<int64_t>(b) * Lq + row) * H + h, M, l);
    return;
  }
  for (int sp = 0; sp < n_splits; ++sp) {
    const float ms = pml[(sp * plane + prow) * 2];
    if (ms == kNegInf) continue;
    const float w = __builtin_amdgcn_exp2f(ms - M);
    l += pml[(sp * plane + prow) * 2 + 1] * w;
    const f32x4* src = reinterpret_cast<const f32x4*>(ws + (sp * plane + prow) * D + c8);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += x0[i] * w;
      acc[4 + i] += x1[i] * w;
    }
  }
  if (stat_mode != kStatNone && c8 == 0)
    write_stat(stat_mode, stat + (static_cast<int64_t>(b) * Lq + row) * H + h, M, l);
  const float inv = 1.f / l;
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = cvt_pk_bf16(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(o + ((static_cast<int64_t>(b) * Lq + row) * H + h) * D + c8) = out;
}

template <int D>
__global__ void __launch_bounds__(kF32Rows) attn_f32_kernel(AttnArgs a) {
  __shared__ float ks[kF32Keys][D + 1];
  __shared__ float vs[kF32Keys][D + 1];
  const CacheGeom& g = a.g;
  const int T = g.T;
  const int b = blockIdx.y / g.H;
  const int h = blockIdx.y - b * g.H;
  const int Lq = a.n_q * T;
  const int n_res = a.frames.n;
  const int first_q = n_res - a.n_q;
  const int row = blockIdx.x * kF32Rows + threadIdx.x;
  const bool row_ok = row < Lq;
  const int qf = row_ok ? row / T : a.n_q - 1;
  const int n_keys = n_res * T;
  const int klim = min(n_keys, a.key_limit);
  const int kend = min(a.causal ? (first_q + qf + 1) * T : n_keys, klim);
  const int last_row = min(static_cast<int>(blockIdx.x) * kF32Rows + kF32Rows - 1, Lq - 1);
  const int kend_wg = min(a.causal ? (first_q + last_row / T + 1) * T : n_keys, klim);

  float q[D];
  {
    const int tok = row_ok ? row - qf * T : 0;
    const int64_t t = a.frames.t[first_q + qf];
    const float* qrow = static_cast<const float*>(a.q) + ((static_cast<int64_t>(b) * Lq + (row_ok ? row : 0)) * g.H + h) * D;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = row_ok ? qrow[c * 8 + i] : 0.f;
      rope_rotate8(a.rope, h, c, t, tok / a.rope.grid_w, tok % a.rope.grid_w, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) q[c * 8 + i] = x[i];
    }
  }
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  const float* kst = static_cast<const float*>(g.k_store);
  const float* vst = static_cast<const float*>(g.v_store);
  const int64_t head_off = static_cast<int64_t>(b) * g.H + h;

  for (int j0 = 0; j0 < kend_wg; j0 += kF32Keys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Keys * D; e += kF32Rows) {
      const int r = e / D, d = e - (e / D) * D;
      const int j = j0 + r;
      float kv = 0.f, vv = 0.f;
      if (j < kend_wg) {
        const int lf = j / T;
        const int tok = j - lf * T;
        const int64_t base = static_cast<int64_t>(a.frames.store_slot[lf]) * g.B * g.H + head_off;
        kv = kst[(base * T + tok) * D + d];
        vv = vst[(base * D + d) * static_cast<int64_t>(T) + tok];
      }
      ks[r][d] = kv;
      vs[r][d] = vv;
    }
    __syncthreads();
    float s[kF32Keys];
    float mx = kNegInf;
#pragma unroll 4
    for (int r = 0; r < kF32Keys; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], ks[r][d], acc);
      s[r] = (j0 + r < kend) ? acc * a.scale_log2 : kNegInf;
      mx = fmaxf(mx, s[r]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
    for (int r = 0; r < kF32Keys; ++r) {
      const float p = exp2f(s[r] - m_use);
      l_run += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, vs[r][d], o[d]);
    }
  }
  if (row_ok && a.stat_mode != kStatNone)
    write_stat(a.stat_mode, a.stat + (static_cast<int64_t>(b) * Lq + row) * g.H + h, m_run, l_run);
  if (row_ok && a.stat_mode != kStatMass) {
    const float inv = 1.f / l_run;
    float* orow = static_cast<float*>(a.o) + ((static_cast<int64_t>(b) * Lq + row) * g.H + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
  }
}

// Device-resident scratch of sa_window_attn_noalloc: the key-split partials,
// for callers that cannot allocate.  In host code this name is only a
// stand-in for the device array; its device address, which differs per GPU,
// comes from hipGetSymbolAddress and is kept in g_scratch_ptr.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

}  // namespace

hipError_t attn_noalloc_scratch(void** ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // once per device, with that device current
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

int attn_kernel_variant(int dtype, int B, int H, int D, int T, int n_q, int num_cus) {
  (void)B; (void)H; (void)D; (void)T; (void)n_q; (void)num_cus;
  if (dtype != kBF16) return 0;
  if (const int v = launch_override(kKnobAttnKernel)) return v;
  // 1: attn_bf16_kernel.  2: attn_bf16_pipe_kernel with eight waves of 32
  // query rows, the in-wave interleaved variant; it measures a few per cent
  // slower on the Wan-1.3B layer (its vector and scalar instruction count per
  // key tile is the larger), so it is not the default.  3: the same kernel
  // with four waves of 64 rows.  All run one workgroup of 256 rows per CU.
  return 1;
}

int attn_num_splits(int dtype, int B, int H, int D, int T, int n_q, int n_res, int num_cus) {
  if (dtype != kBF16 && dtype != kFP8) return 1;
  const int64_t q_tile = 256;  // query rows per workgroup (every bf16 and e4m3 shape)
  const int64_t tiles = static_cast<int64_t>(B) * H * ((static_cast<int64_t>(n_q) * T + q_tile - 1) / q_tile);
  const int64_t key_tiles = (static_cast<int64_t>(n_res) * T + kKTile - 1) / kKTile;
  int64_t max_s = key_tiles / 8;  // at least 8 key tiles per split
  if (max_s > 16) max_s = 16;
  if (max_s < 1) max_s = 1;
  if (const int v = launch_override(kKnobAttnSplits)) return static_cast<int>(v < max_s ? v : max_s);
  // Pick the split count whose workgroup count best fills whole rounds of
  // the CUs' workgroup slots, with a small charge per split for the partial
  // results it writes and merges.
  const double slots = static_cast<double>(num_cus);  // one workgroup per CU
  int best = 1;
  double best_score = -1.0;
  for (int64_t s = 1; s <= max_s; ++s) {
    const double wgs = static_cast<double>(tiles * s);
    const double rounds = std::ceil(wgs / slots);
    const double score = wgs / (rounds * slots) - (s > 1 ? 0.01 * s : 0.0);
    if (score > best_score + 1e-9) {
      best_score = score;
      best = static_cast<int>(s);
    }
  }
  return best;
}

size_t attn_workspace_bytes(int dtype, int B, int H, int D, int T, int n_q, int n_splits) {
  if ((dtype != kBF16 && dtype != kFP8) || n_splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(B) * H * n_q * T;
  return static_cast<size_t>(n_splits) * rows * (D + 2) * sizeof(float);
}

hipError_t launch_window_attn(const AttnArgs& a, int dtype, hipStream_t stream) {
  const int Lq = a.n_q * a.g.T;
  const int BH = a.g.B * a.g.H;
  if (dtype == kFP8) {
    const hipError_t e8 = launch_attn_fp8(a, stream);
    if (e8 != hipSuccess) return e8;
    if (a.n_splits > 1) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t rows = static_cast<int64_t>(a.g.B) * a.g.H * Lq;
      const dim3 mgrid(static_cast<unsigned>((rows + 15) / 16));
      hipLaunchKernelGGL(attn_merge_kernel<128>, mgrid, dim3(256), 0, stream, a.ws, static_cast<uint16_t*>(a.o),
                         a.g.B, a.g.H, Lq, a.n_splits, a.stat_mode, a.stat);
    }
  } else if (dtype == kBF16) {
    const int64_t wgs = static_cast<int64_t>((Lq + 255) / 256) * BH * a.n_splits;  // 256 query rows per workgroup
    const dim3 grid(static_cast<unsigned>(wgs));
    const dim3 block(a.variant == 3 ? 256 : 512);
    const bool big_t = a.g.T >= kKTile;
#define SA_LAUNCH_ATTN(DD, BT, WW) hipLaunchKernelGGL((attn_bf16_kernel<DD, BT, WW>), grid, block, 0, stream, a)
#define SA_LAUNCH_PIPE(DD, BT, QQ) hipLaunchKernelGGL((attn_bf16_pipe_kernel<DD, BT, QQ>), grid, block, 0, stream, a)
    if (a.variant == 2) {
      if (a.g.D == 128) { if (big_t) SA_LAUNCH_PIPE(128, true, 1); else SA_LAUNCH_PIPE(128, false, 1); }
      else { if (big_t) SA_LAUNCH_PIPE(64, true, 1); else SA_LAUNCH_PIPE(64, false, 1); }
    } else if (a.variant == 3) {
      if (a.g.D == 128) { if (big_t) SA_LAUNCH_PIPE(128, true, 2); else SA_LAUNCH_PIPE(128, false, 2); }
      else { if (big_t) SA_LAUNCH_PIPE(64, true, 2); else SA_LAUNCH_PIPE(64, false, 2); }
    } else {
      if (a.g.D == 128) { if (big_t) SA_LAUNCH_ATTN(128, true, 8); else SA_LAUNCH_ATTN(128, false, 8); }
      else { if (big_t) SA_LAUNCH_ATTN(64, true, 8); else SA_LAUNCH_ATTN(64, false, 8); }
    }
#undef SA_LAUNCH_PIPE
#undef SA_LAUNCH_ATTN
    if (a.n_splits > 1) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t rows = static_cast<int64_t>(a.g.B) * a.g.H * Lq;
      const int rows_per_block = 256 / (a.g.D / 8);
      const dim3 mgrid(static_cast<unsigned>((rows + rows_per_block - 1) / rows_per_block));
      if (a.g.D == 128)
        hipLaunchKernelGGL(attn_merge_kernel<128>, mgrid, dim3(256), 0, stream, a.ws, static_cast<uint16_t*>(a.o),
                           a.g.B, a.g.H, Lq, a.n_splits, a.stat_mode, a.stat);
      else
        hipLaunchKernelGGL(attn_merge_kernel<64>, mgrid, dim3(256), 0, stream, a.ws, static_cast<uint16_t*>(a.o),
                           a.g.B, a.g.H, Lq, a.n_splits, a.stat_mode, a.stat);
    }
  } else {
    const dim3 grid((Lq + kF32Rows - 1) / kF32Rows, BH, 1);
    if (a.g.D == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kF32Rows), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kF32Rows), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sa
