// Host side of libsinkattn: handle management, validation, launch.
//
// Every entry point validates its arguments and the handle state before it
// changes anything or launches; on error the handle is unchanged and the
// thread-local last-error string says why.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/sinkattn.h"
#include "cache_plan.hpp"
#include "internal.hpp"
#include "rope_tables.hpp"

struct sa_rope {
  int n_heads, head_dim;
  int dims[3];
  int grid_h, grid_w;
  sa::RopeTables tables;
  sa::RopeGridTable grid_table;
  double* d_freq = nullptr;   // device [H][D/2]
  float* d_grid = nullptr;    // device grid-axis cos/sin table (may stay null)
  int device = 0;
};

struct sa_cache {
  sa_cache_desc desc;
  const sa_rope* rope;
  sa::CachePlan plan;
};

namespace {

thread_local std::string g_last_error;

// Launch-shape overrides (sa_set_launch_override); 0 = automatic.
std::atomic<int> g_knobs[sa::kNumKnobs];

sa_status fail(sa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sa_status ok() {
  g_last_error.clear();
  return SA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Do the byte ranges [p, p + pb) and [q, q + qb) share a byte?
bool overlaps(const void* p, size_t pb, const void* q, size_t qb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
  return pb > 0 && qb > 0 && a0 < b0 + qb && b0 < a0 + pb;
}

size_t elem_size(sa_dtype d) { return d == SA_FP8 ? 1 : (d == SA_BF16 ? 2 : 4); }

sa_status hip_fail(hipError_t e, const char* what) {
  return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// SA_DEBUG_SYNC=1 in the environment (read once, when the library loads):
// every entry point waits for its stream after launching, so a device fault
// is reported by the call that caused it instead of at the caller's next
// synchronisation.  For debugging only: it serialises the stream, and a call
// under HIP graph capture must not synchronise.
const bool g_debug_sync = [] {
  const char* v = std::getenv("SA_DEBUG_SYNC");
  return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}();

// Status of a launch just made on stream (e: the launch's own error).
sa_status launched(hipError_t e, void* stream, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  if (g_debug_sync) {
    const hipError_t es = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (es != hipSuccess) return fail(SA_ERR_HIP, "%s (SA_DEBUG_SYNC): %s", what, hipGetErrorString(es));
  }
  return SA_OK;
}

sa_status check_rope_desc(const sa_rope_desc* d) {
  if (!d) return fail(SA_ERR_NULL, "rope descriptor is NULL");
  if (d->n_heads < 1 || d->n_heads > 1024) return fail(SA_ERR_SHAPE, "n_heads must be in [1, 1024]");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(SA_ERR_SHAPE, "head_dim must be 64 or 128");
  const int dims[3] = {d->dim_t, d->dim_h, d->dim_w};
  for (int a = 0; a < 3; ++a)
    if (dims[a] < 0 || dims[a] % 2) return fail(SA_ERR_SHAPE, "RoPE axis dims must be even and >= 0");
  if (dims[0] + dims[1] + dims[2] != d->head_dim)
    return fail(SA_ERR_SHAPE, "dim_t + dim_h + dim_w (%d) must equal head_dim (%d)",
                dims[0] + dims[1] + dims[2], d->head_dim);
  if (d->grid_h < 1 || d->grid_w < 1) return fail(SA_ERR_SHAPE, "grid must be >= 1x1");
  const long long tf = static_cast<long long>(d->grid_h) * d->grid_w;
  if (tf % 8 != 0 || tf > (1 << 20)) return fail(SA_ERR_SHAPE, "tokens per frame must be a multiple of 8 and <= 2^20");
  if (d->t_scale != 0.0 && !(d->t_scale > 0.0 && std::isfinite(d->t_scale)))
    return fail(SA_ERR_RANGE, "t_scale must be 0 (none) or finite and > 0");
  if (d->theta) {  // theta_hat given per head and axis: theta0, sigma, eps and jitter_axes are unused
    for (int i = 0; i < d->n_heads * 3; ++i)
      if (!(d->theta[i] > 1.0) || !std::isfinite(d->theta[i]))
        return fail(SA_ERR_RANGE, "theta[%d] (head %d, axis %d) must be finite and > 1", i, i / 3, i % 3);
    return SA_OK;
  }
  if (!(d->theta0 > 1.0) || !std::isfinite(d->theta0)) return fail(SA_ERR_RANGE, "theta0 must be finite and > 1");
  if (!(d->sigma >= 0.0) || !std::isfinite(d->sigma)) return fail(SA_ERR_RANGE, "sigma must be finite and >= 0");
  if (d->jitter_axes > 7u) return fail(SA_ERR_RANGE, "jitter_axes must be a SA_AXIS_* mask");
  if (d->eps) {
    for (int h = 0; h < d->n_heads; ++h) {
      const double e = d->eps[h];
      if (!(e >= -1.0 && e <= 1.0)) return fail(SA_ERR_RANGE, "eps[%d] must be in [-1, 1]", h);
      if (!(d->theta0 * (1.0 + d->sigma * e) > 1.0))
        return fail(SA_ERR_RANGE, "jittered base of head %d is not > 1", h);
    }
  }
  return SA_OK;
}

sa::RopeArgs rope_args(const sa_rope* r) {
  sa::RopeArgs a;
  a.freq = r->d_freq;
  a.grid_cs = r->d_grid;
  a.pairs_t = r->dims[0] / 2;
  a.pairs_th = (r->dims[0] + r->dims[1]) / 2;
  a.pairs_all = r->head_dim / 2;
  a.grid_h = r->grid_h;
  a.grid_w = r->grid_w;
  a.grid_stride = r->grid_table.stride;
  a.grid_per_head = r->grid_table.per_head ? 1 : 0;
  return a;
}

sa::CacheGeom geom(const sa_cache* c) {
  sa::CacheGeom g;
  g.B = c->desc.batch;
  g.H = c->desc.n_heads;
  g.D = c->desc.head_dim;
  g.T = c->desc.tokens_per_frame;
  g.n_slots = c->desc.n_sink + c->desc.n_local;
  g.k_store = c->desc.k_store;
  g.v_store = c->desc.v_store;
  g.k_scale = c->desc.dtype == SA_FP8 ? c->desc.k_scale : 1.f;
  g.v_scale = c->desc.dtype == SA_FP8 ? c->desc.v_scale : 1.f;
  return g;
}

sa::FrameTable resident_table(const sa_cache* c) {
  sa::FrameTable ft{};
  const auto res = c->plan.resident();
  ft.n = static_cast<int32_t>(res.size());
  for (size_t i = 0; i < res.size(); ++i) {
    ft.store_slot[i] = res[i].store_slot;
    ft.t[i] = res[i].t;
  }
  return ft;
}

// Chunk rules shared by the two append paths (t0 range checked by the caller).
sa_status check_append_chunk(const sa_cache* c, int32_t n_frames, int64_t t0) {
  switch (c->plan.check_append(n_frames, t0)) {
    case 0: return SA_OK;
    case 1: return fail(SA_ERR_SHAPE, "n_frames must be in [1, %d]", SA_MAX_FRAMES);
    case 2: return fail(SA_ERR_RANGE, "chunk of %d frames does not fit the %d-frame local window", n_frames,
                        c->desc.n_local);
    default: return fail(SA_ERR_RANGE, "t0 (%lld) must exceed the newest cached time (%lld)",
                         static_cast<long long>(t0), static_cast<long long>(c->plan.newest_t()));
  }
}

// Slots and times the next append of n_frames frames at t0 will use.
sa::FrameTable chunk_table(const sa_cache* c, int32_t n_frames, int64_t t0) {
  const auto planned = c->plan.plan_append(n_frames, t0);
  sa::FrameTable chunk{};
  chunk.n = n_frames;
  for (int i = 0; i < n_frames; ++i) {
    chunk.store_slot[i] = planned[i].store_slot;
    chunk.t[i] = planned[i].t;
  }
  return chunk;
}

// Size rules of the projection GEMM: the reduction runs in slices of 32,
// and the bf16 kernel addresses x and each weight matrix with 32-bit byte
// offsets (rows past the end included).
sa_status check_proj_sizes(int64_t n_tok, int32_t hidden, int32_t width, size_t es) {
  if (hidden < 32 || hidden % 32 != 0 || hidden > (1 << 16))
    return fail(SA_ERR_SHAPE, "hidden / in_features must be a multiple of 32 in [32, 65536]");
  const unsigned long long row = static_cast<unsigned long long>(hidden) * es;
  if ((static_cast<unsigned long long>(n_tok) + 256) * row >= (1ull << 32) ||
      (static_cast<unsigned long long>(width) + 256) * row >= (1ull << 32))
    return fail(SA_ERR_SHAPE, "x or a weight matrix reaches 4 GiB");
  return SA_OK;
}

// The projection GEMM's element type for this cache: an e4m3 cache takes
// bf16 x, weights and q.
int proj_dtype(const sa_cache* c) { return c->desc.dtype == SA_FP8 ? sa::kBF16 : static_cast<int>(c->desc.dtype); }
size_t proj_elem_size(const sa_cache* c) { return c->desc.dtype == SA_F32 ? 4 : 2; }

// Does [p, p + bytes) share a byte with either of the cache's stores?
bool hits_stores(const sa_cache* c, const void* p, size_t bytes) {
  const size_t sb = sa_cache_store_bytes(&c->desc);
  return overlaps(p, bytes, c->desc.k_store, sb) || overlaps(p, bytes, c->desc.v_store, sb);
}

// Projection segments into this cache: [q rows,] rotated keys, values.
sa::ProjArgs cache_proj_args(const sa_cache* c, const void* x, const void* w_q, void* q_out, const void* w_k,
                             const void* w_v, int32_t hidden) {
  sa::ProjArgs a{};
  a.x = x;
  a.hidden = hidden;
  a.width = c->desc.n_heads * c->desc.head_dim;
  int n = 0;
  if (w_q) a.seg[n++] = sa::ProjSeg{w_q, q_out, sa::kOutRows};
  a.seg[n++] = sa::ProjSeg{w_k, nullptr, sa::kOutCacheK};
  a.seg[n++] = sa::ProjSeg{w_v, nullptr, sa::kOutCacheV};
  a.n_seg = n;
  for (int i = n; i < 3; ++i) a.seg[i] = a.seg[n - 1];
  a.has_key = 1;
  a.has_value = 1;
  a.cache_fp8 = c->desc.dtype == SA_FP8 ? 1 : 0;
  a.g = geom(c);
  a.rope = rope_args(c->rope);
  return a;
}

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus;
}

}  // namespace

extern "C" {

const char* sa_status_str(sa_status s) {
  switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE";
    case SA_ERR_DTYPE: return "SA_ERR_DTYPE";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN";
    case SA_ERR_STATE: return "SA_ERR_STATE";
    case SA_ERR_RANGE: return "SA_ERR_RANGE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
  }
  return "SA_ERR_UNKNOWN";
}

const char* sa_last_error(void) { return g_last_error.c_str(); }

sa_status sa_set_launch_override(sa_knob knob, int32_t value) {
  bool valid = false;
  switch (knob) {
    case SA_KNOB_ATTN_KERNEL: valid = value >= 0 && value <= 3; break;
    case SA_KNOB_ATTN_SPLITS: valid = value >= 0 && value <= 16; break;
    case SA_KNOB_PROJ_TILE: valid = value >= 0 && value <= 4; break;
    default: return fail(SA_ERR_RANGE, "unknown launch knob %d", static_cast<int>(knob));
  }
  if (!valid) return fail(SA_ERR_RANGE, "value %d is outside the set of knob %d", value, static_cast<int>(knob));
  g_knobs[knob].store(value, std::memory_order_relaxed);
  return ok();
}

const char* sa_version(void) { return "libsinkattn 0.1 (gfx950)"; }

sa_status sa_rope_tables(const sa_rope_desc* desc, double* theta_hat_out, double* freq_out) {
  if (sa_status s = check_rope_desc(desc)) return s;
  const int dims[3] = {desc->dim_t, desc->dim_h, desc->dim_w};
  const sa::RopeTables t = sa::build_rope_tables(desc->n_heads, desc->head_dim, dims, desc->theta0,
                                                 desc->sigma, desc->eps, desc->jitter_axes, desc->t_scale, desc->theta);
  if (theta_hat_out) std::memcpy(theta_hat_out, t.theta_hat.data(), t.theta_hat.size() * sizeof(double));
  if (freq_out) std::memcpy(freq_out, t.freq.data(), t.freq.size() * sizeof(double));
  return ok();
}

sa_status sa_rope_phase_coherence(const sa_rope_desc* desc, const double* deltas, int32_t n, double* re,
                                  double* im) {
  if (sa_status s = check_rope_desc(desc)) return s;
  if (n < 0 || (n > 0 && (!deltas || !re || !im))) return fail(SA_ERR_NULL, "deltas, re and im must be non-NULL");
  if (desc->dim_t == 0) return fail(SA_ERR_SHAPE, "no time-axis channels (dim_t is 0)");
  const int dims[3] = {desc->dim_t, desc->dim_h, desc->dim_w};
  const sa::RopeTables t = sa::build_rope_tables(desc->n_heads, desc->head_dim, dims, desc->theta0,
                                                 desc->sigma, desc->eps, desc->jitter_axes, desc->t_scale, desc->theta);
  const int half = desc->head_dim / 2;
  const int K = desc->dim_t / 2;  // time pairs come first in every head's table
  for (int h = 0; h < desc->n_heads; ++h)
    for (int k = 0; k < n; ++k) {
      double c = 0.0, s = 0.0;
      for (int i = 0; i < K; ++i) {
        const double ph = t.freq[static_cast<size_t>(h) * half + i] * deltas[k];
        c += std::cos(ph);
        s += std::sin(ph);
      }
      re[static_cast<size_t>(h) * n + k] = c / K;
      im[static_cast<size_t>(h) * n + k] = s / K;
    }
  return ok();
}

sa_status sa_rope_create(const sa_rope_desc* desc, sa_rope** out) {
  if (!out) return fail(SA_ERR_NULL, "out is NULL");
  if (sa_status s = check_rope_desc(desc)) return s;
  sa_rope* r = new (std::nothrow) sa_rope();
  if (!r) return fail(SA_ERR_RANGE, "out of host memory");
  r->n_heads = desc->n_heads;
  r->head_dim = desc->head_dim;
  r->dims[0] = desc->dim_t;
  r->dims[1] = desc->dim_h;
  r->dims[2] = desc->dim_w;
  r->grid_h = desc->grid_h;
  r->grid_w = desc->grid_w;
  r->tables = sa::build_rope_tables(desc->n_heads, desc->head_dim, r->dims, desc->theta0,
                                    desc->sigma, desc->eps, desc->jitter_axes, desc->t_scale, desc->theta);
  r->grid_table = sa::build_rope_grid_table(r->tables, desc->n_heads, desc->head_dim, r->dims, desc->grid_h,
                                            desc->grid_w);
  hipError_t e = hipGetDevice(&r->device);
  if (e == hipSuccess) e = hipMalloc(&r->d_freq, r->tables.freq.size() * sizeof(double));
  if (e == hipSuccess)
    e = hipMemcpy(r->d_freq, r->tables.freq.data(), r->tables.freq.size() * sizeof(double),
                  hipMemcpyHostToDevice);
  if (e == hipSuccess && !r->grid_table.cs.empty()) {
    e = hipMalloc(&r->d_grid, r->grid_table.cs.size() * sizeof(float));
    if (e == hipSuccess)
      e = hipMemcpy(r->d_grid, r->grid_table.cs.data(), r->grid_table.cs.size() * sizeof(float),
                    hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    if (r->d_freq) (void)hipFree(r->d_freq);
    if (r->d_grid) (void)hipFree(r->d_grid);
    delete r;
    return hip_fail(e, "sa_rope_create");
  }
  *out = r;
  return ok();
}

void sa_rope_destroy(sa_rope* r) {
  if (!r) return;
  if (r->d_freq) (void)hipFree(r->d_freq);
  if (r->d_grid) (void)hipFree(r->d_grid);
  delete r;
}

sa_status sa_rope3d_apply(const sa_rope* rope, const void* x, void* y, sa_dtype dtype, int32_t batch,
                          int32_t n_frames, int64_t t0, void* stream) {
  if (!rope || !x || !y) return fail(SA_ERR_NULL, "rope, x and y must be non-NULL");
  if (dtype != SA_BF16 && dtype != SA_F32) return fail(SA_ERR_DTYPE, "dtype must be SA_BF16 or SA_F32");
  if (batch < 1 || n_frames < 1) return fail(SA_ERR_SHAPE, "batch and n_frames must be >= 1");
  if (!aligned16(x) || !aligned16(y)) return fail(SA_ERR_ALIGN, "x and y must be 16-byte aligned");
  if (t0 < 0 || t0 > (int64_t(1) << 40) - n_frames) return fail(SA_ERR_RANGE, "t0 out of range [0, 2^40)");
  const int T = rope->grid_h * rope->grid_w;
  const size_t bytes = static_cast<size_t>(batch) * n_frames * T * rope->n_heads * rope->head_dim * elem_size(dtype);
  if (x != y && overlaps(x, bytes, y, bytes))
    return fail(SA_ERR_RANGE, "y must be x itself or not overlap it");
  const hipError_t e = sa::launch_rope3d(rope_args(rope), x, y, dtype, batch, rope->n_heads,
                                         rope->head_dim, T, n_frames, t0,
                                         static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "rope3d launch")) return s_;
  return ok();
}

size_t sa_cache_bytes(const sa_cache_desc* d) { return sa_cache_store_bytes(d); }

size_t sa_cache_store_bytes(const sa_cache_desc* d) {
  if (!d || d->batch < 1 || d->n_heads < 1 || (d->head_dim != 64 && d->head_dim != 128) ||
      d->tokens_per_frame < 8 || d->n_sink < 0 || d->n_local < 1 ||
      d->n_sink + d->n_local > SA_MAX_FRAMES || (d->dtype != SA_BF16 && d->dtype != SA_F32 && d->dtype != SA_FP8))
    return 0;
  return static_cast<size_t>(d->n_sink + d->n_local) * d->batch * d->n_heads * d->tokens_per_frame *
         d->head_dim * elem_size(d->dtype);
}

sa_status sa_cache_create(const sa_cache_desc* d, const sa_rope* rope, sa_cache** out) {
  if (!d || !rope || !out) return fail(SA_ERR_NULL, "desc, rope and out must be non-NULL");
  if (!d->k_store || !d->v_store) return fail(SA_ERR_NULL, "k_store and v_store must be non-NULL");
  if (d->dtype != SA_BF16 && d->dtype != SA_F32 && d->dtype != SA_FP8)
    return fail(SA_ERR_DTYPE, "dtype must be SA_BF16, SA_F32 or SA_FP8");
  if (d->dtype == SA_FP8) {
    if (d->head_dim != 128) return fail(SA_ERR_SHAPE, "an SA_FP8 cache needs head_dim 128");
    if (!(d->k_scale > 0.f) || !std::isfinite(d->k_scale) || !(d->v_scale > 0.f) || !std::isfinite(d->v_scale))
      return fail(SA_ERR_RANGE, "k_scale and v_scale must be finite and > 0 for an SA_FP8 cache");
  }
  if (d->batch < 1 || d->batch > 65535) return fail(SA_ERR_SHAPE, "batch must be in [1, 65535]");
  if (d->n_sink < 0 || d->n_local < 1 || d->n_sink + d->n_local > SA_MAX_FRAMES)
    return fail(SA_ERR_SHAPE, "need n_sink >= 0, n_local >= 1, n_sink + n_local <= %d", SA_MAX_FRAMES);
  if (d->n_heads != rope->n_heads || d->head_dim != rope->head_dim)
    return fail(SA_ERR_SHAPE, "cache heads/head_dim (%d, %d) differ from the rope's (%d, %d)", d->n_heads,
                d->head_dim, rope->n_heads, rope->head_dim);
  if (d->tokens_per_frame != rope->grid_h * rope->grid_w)
    return fail(SA_ERR_SHAPE, "tokens_per_frame (%d) differs from the rope grid (%d x %d)", d->tokens_per_frame,
                rope->grid_h, rope->grid_w);
  if (!aligned16(d->k_store) || !aligned16(d->v_store)) return fail(SA_ERR_ALIGN, "stores must be 16-byte aligned");
  // Every in-kernel index of one stream's queries and keys fits in int32.
  const long long keys = static_cast<long long>(d->n_sink + d->n_local) * d->tokens_per_frame;
  if (keys > (1LL << 30)) return fail(SA_ERR_SHAPE, "too many tokens in the window");
  // The kernels address each store with 32-bit byte offsets.
  if (sa_cache_store_bytes(d) > 0xFFFFFF00ull) return fail(SA_ERR_SHAPE, "each cache store must be below 4 GiB");
  sa_cache* c = new (std::nothrow) sa_cache();
  if (!c) return fail(SA_ERR_RANGE, "out of host memory");
  c->desc = *d;
  c->rope = rope;
  c->plan = sa::CachePlan(d->n_sink, d->n_local);
  *out = c;
  return ok();
}

void sa_cache_destroy(sa_cache* c) { delete c; }

sa_status sa_cache_reset(sa_cache* c) {
  if (!c) return fail(SA_ERR_NULL, "cache is NULL");
  c->plan.reset();
  return ok();
}

sa_status sa_cache_append(sa_cache* c, const void* k, const void* v, int32_t n_frames, int64_t t0,
                          void* stream) {
  if (!c || !k || !v) return fail(SA_ERR_NULL, "cache, k and v must be non-NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(SA_ERR_ALIGN, "k and v must be 16-byte aligned");
  if (t0 < 0 || t0 > (int64_t(1) << 40)) return fail(SA_ERR_RANGE, "t0 out of range [0, 2^40]");
  if (sa_status s = check_append_chunk(c, n_frames, t0)) return s;
  const size_t in_bytes = static_cast<size_t>(c->desc.batch) * n_frames * c->desc.tokens_per_frame * c->desc.n_heads *
                          c->desc.head_dim * proj_elem_size(c);
  if (hits_stores(c, k, in_bytes) || hits_stores(c, v, in_bytes))
    return fail(SA_ERR_RANGE, "k and v must not overlap the cache stores");
  const sa::FrameTable chunk = chunk_table(c, n_frames, t0);
  const hipError_t e = sa::launch_append(rope_args(c->rope), geom(c), k, v, c->desc.dtype, chunk,
                                         static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "append launch")) return s_;
  c->plan.commit_append(n_frames, t0);
  return ok();
}

sa_status sa_cache_recache(sa_cache* c, const void* x, const void* w_k, const void* w_v, int32_t hidden,
                           void* stream) {
  if (!c || !x || !w_k || !w_v) return fail(SA_ERR_NULL, "cache, x, w_k and w_v must be non-NULL");
  if (!aligned16(x) || !aligned16(w_k) || !aligned16(w_v)) return fail(SA_ERR_ALIGN, "x and weights must be 16-byte aligned");
  const int hd = c->desc.n_heads * c->desc.head_dim;
  if (sa_status s = check_proj_sizes(0, hidden, hd, proj_elem_size(c))) return s;
  if (!c->plan.has_frames()) return fail(SA_ERR_STATE, "recache on an empty cache");
  const int64_t n_tok = static_cast<int64_t>(c->desc.batch) * c->plan.resident().size() * c->desc.tokens_per_frame;
  if (sa_status s = check_proj_sizes(n_tok, hidden, hd, proj_elem_size(c))) return s;
  {
    const size_t es = proj_elem_size(c), wb = static_cast<size_t>(hd) * hidden * es;
    if (hits_stores(c, x, static_cast<size_t>(n_tok) * hidden * es) || hits_stores(c, w_k, wb) || hits_stores(c, w_v, wb))
      return fail(SA_ERR_RANGE, "x and the weights must not overlap the cache stores");
  }
  sa::ProjArgs a = cache_proj_args(c, x, nullptr, nullptr, w_k, w_v, hidden);
  a.n_tok = n_tok;
  a.frames = resident_table(c);
  const hipError_t e = sa::launch_proj(a, proj_dtype(c), device_cus(), static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "recache launch")) return s_;
  return ok();
}

sa_status sa_cache_project_append(sa_cache* c, const void* x, const void* w_q, const void* w_k, const void* w_v,
                                  int32_t hidden, void* q_out, int32_t n_frames, int64_t t0, void* stream) {
  if (!c || !x || !w_k || !w_v) return fail(SA_ERR_NULL, "cache, x, w_k and w_v must be non-NULL");
  if (!w_q != !q_out) return fail(SA_ERR_NULL, "w_q and q_out must both be given or both be NULL");
  if (!aligned16(x) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(w_q) || !aligned16(q_out))
    return fail(SA_ERR_ALIGN, "x, weights and q_out must be 16-byte aligned");
  if (t0 < 0 || t0 > (int64_t(1) << 40)) return fail(SA_ERR_RANGE, "t0 out of range [0, 2^40]");
  if (sa_status s = check_append_chunk(c, n_frames, t0)) return s;
  const int hd = c->desc.n_heads * c->desc.head_dim;
  const int64_t n_tok = static_cast<int64_t>(c->desc.batch) * n_frames * c->desc.tokens_per_frame;
  if (sa_status s = check_proj_sizes(n_tok, hidden, hd, proj_elem_size(c))) return s;
  {
    const size_t es = proj_elem_size(c), wb = static_cast<size_t>(hd) * hidden * es;
    const size_t xb = static_cast<size_t>(n_tok) * hidden * es, qb = q_out ? static_cast<size_t>(n_tok) * hd * es : 0;
    if (hits_stores(c, x, xb) || hits_stores(c, w_k, wb) || hits_stores(c, w_v, wb) ||
        (w_q && hits_stores(c, w_q, wb)) || (q_out && hits_stores(c, q_out, qb)))
      return fail(SA_ERR_RANGE, "x, the weights and q_out must not overlap the cache stores");
    if (q_out && (overlaps(q_out, qb, x, xb) || overlaps(q_out, qb, w_q, wb) || overlaps(q_out, qb, w_k, wb) ||
                  overlaps(q_out, qb, w_v, wb)))
      return fail(SA_ERR_RANGE, "q_out must not overlap x or the weights");
  }
  sa::ProjArgs a = cache_proj_args(c, x, w_q, q_out, w_k, w_v, hidden);
  a.n_tok = n_tok;
  a.frames = chunk_table(c, n_frames, t0);
  const hipError_t e = sa::launch_proj(a, proj_dtype(c), device_cus(), static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "projection launch")) return s_;
  c->plan.commit_append(n_frames, t0);
  return ok();
}

sa_status sa_linear(const void* x, const void* w, void* y, sa_dtype dtype, int64_t n_rows, int32_t in_features,
                    int32_t out_features, void* stream) {
  if (!x || !w || !y) return fail(SA_ERR_NULL, "x, w and y must be non-NULL");
  if (dtype != SA_BF16 && dtype != SA_F32) return fail(SA_ERR_DTYPE, "dtype must be SA_BF16 or SA_F32");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(SA_ERR_ALIGN, "x, w and y must be 16-byte aligned");
  if (n_rows < 0) return fail(SA_ERR_SHAPE, "n_rows must be >= 0");
  if (out_features < 16 || out_features % 16 != 0 || out_features > (1 << 20))
    return fail(SA_ERR_SHAPE, "out_features must be a multiple of 16 in [16, 2^20]");
  if (sa_status s = check_proj_sizes(n_rows, in_features, out_features, elem_size(dtype))) return s;
  const size_t es = elem_size(dtype);
  const size_t yb = static_cast<size_t>(n_rows) * out_features * es;
  if (n_rows > 0 && (overlaps(y, yb, x, static_cast<size_t>(n_rows) * in_features * es) ||
                     overlaps(y, yb, w, static_cast<size_t>(out_features) * in_features * es)))
    return fail(SA_ERR_RANGE, "y overlaps x or w");
  sa::ProjArgs a{};
  a.x = x;
  a.n_tok = n_rows;
  a.hidden = in_features;
  a.width = out_features;
  a.n_seg = 1;
  for (int i = 0; i < 3; ++i) a.seg[i] = sa::ProjSeg{w, y, sa::kOutRows};
  const hipError_t e = sa::launch_proj(a, dtype, device_cus(), static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "linear launch")) return s_;
  return ok();
}

static sa_status q8_op(sa_qtype qtype, int* op) {
  if (qtype == SA_Q_INT8) *op = sa::kOpI8;
  else if (qtype == SA_Q_E4M3) *op = sa::kOpE4M3;
  else return fail(SA_ERR_DTYPE, "qtype must be SA_Q_INT8 or SA_Q_E4M3");
  return SA_OK;
}

// 8-bit GEMM operands: slices of 64 codes.
static sa_status check_q8_hidden(int32_t hidden) {
  if (hidden < 64 || hidden % 64 != 0 || hidden > (1 << 16))
    return fail(SA_ERR_SHAPE, "hidden / in_features must be a multiple of 64 in [64, 65536] for 8-bit operands");
  return SA_OK;
}

sa_status sa_quantize_rows(const void* x, void* codes, float* scales, sa_qtype qtype, int64_t n_rows, int32_t n_cols,
                           void* stream) {
  if (!x || !codes || !scales) return fail(SA_ERR_NULL, "x, codes and scales must be non-NULL");
  int op = 0;
  if (sa_status s = q8_op(qtype, &op)) return s;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return fail(SA_ERR_ALIGN, "x, codes and scales must be 16-byte aligned");
  if (n_rows < 0) return fail(SA_ERR_SHAPE, "n_rows must be >= 0");
  if (n_cols < 8 || n_cols % 8 != 0 || n_cols > (1 << 16))
    return fail(SA_ERR_SHAPE, "n_cols must be a multiple of 8 in [8, 65536]");
  {
    // the kernel reads x while other waves write codes and scales: the three must be disjoint
    const size_t xb = static_cast<size_t>(n_rows) * n_cols * 2, cb = static_cast<size_t>(n_rows) * n_cols,
                 sb = static_cast<size_t>(n_rows) * sizeof(float);
    if (overlaps(codes, cb, x, xb) || overlaps(scales, sb, x, xb) || overlaps(codes, cb, scales, sb))
      return fail(SA_ERR_RANGE, "x, codes and scales must not overlap one another");
  }
  const hipError_t e = sa::launch_quantize_rows(x, codes, scales, op, n_rows, n_cols, static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "quantize launch")) return s_;
  return ok();
}

sa_status sa_linear_q8(const void* x_codes, const float* x_scales, const void* w_codes, const float* w_scales, void* y,
                       sa_qtype qtype, int64_t n_rows, int32_t in_features, int32_t out_features, void* stream) {
  if (!x_codes || !x_scales || !w_codes || !w_scales || !y)
    return fail(SA_ERR_NULL, "codes, scales and y must be non-NULL");
  int op = 0;
  if (sa_status s = q8_op(qtype, &op)) return s;
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y))
    return fail(SA_ERR_ALIGN, "codes, scales and y must be 16-byte aligned");
  if (n_rows < 0) return fail(SA_ERR_SHAPE, "n_rows must be >= 0");
  if (out_features < 16 || out_features % 16 != 0 || out_features > (1 << 20))
    return fail(SA_ERR_SHAPE, "out_features must be a multiple of 16 in [16, 2^20]");
  if (sa_status s = check_q8_hidden(in_features)) return s;
  if (sa_status s = check_proj_sizes(n_rows, in_features, out_features, 1)) return s;
  const size_t yb = static_cast<size_t>(n_rows) * out_features * 2;
  if (n_rows > 0 && (overlaps(y, yb, x_codes, static_cast<size_t>(n_rows) * in_features) ||
                     overlaps(y, yb, w_codes, static_cast<size_t>(out_features) * in_features) ||
                     overlaps(y, yb, x_scales, static_cast<size_t>(n_rows) * 4) ||
                     overlaps(y, yb, w_scales, static_cast<size_t>(out_features) * 4)))
    return fail(SA_ERR_RANGE, "y overlaps an input");
  sa::ProjArgs a{};
  a.x = x_codes;
  a.n_tok = n_rows;
  a.hidden = in_features;
  a.width = out_features;
  a.n_seg = 1;
  for (int i = 0; i < 3; ++i) {
    a.seg[i] = sa::ProjSeg{w_codes, y, sa::kOutRows};
    a.w_scale[i] = w_scales;
  }
  a.op = op;
  a.x_scale = x_scales;
  const hipError_t e = sa::launch_proj(a, sa::kBF16, device_cus(), static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "linear launch")) return s_;
  return ok();
}

// Checks shared by the 8-bit cache projections (before any state is read).
static sa_status check_cache_q8(const sa_cache* c, sa_qtype qtype, int* op, int32_t hidden) {
  if (sa_status s = q8_op(qtype, op)) return s;
  if (c->desc.dtype == SA_F32) return fail(SA_ERR_DTYPE, "8-bit projections write bf16 or e4m3 caches only");
  return check_q8_hidden(hidden);
}

sa_status sa_cache_recache_q8(sa_cache* c, const void* x_codes, const float* x_scales, const void* wk_codes,
                              const float* wk_scales, const void* wv_codes, const float* wv_scales, sa_qtype qtype,
                              int32_t hidden, void* stream) {
  if (!c || !x_codes || !x_scales || !wk_codes || !wk_scales || !wv_codes || !wv_scales)
    return fail(SA_ERR_NULL, "cache, codes and scales must be non-NULL");
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(wk_codes) || !aligned16(wk_scales) ||
      !aligned16(wv_codes) || !aligned16(wv_scales))
    return fail(SA_ERR_ALIGN, "codes and scales must be 16-byte aligned");
  int op = 0;
  if (sa_status s = check_cache_q8(c, qtype, &op, hidden)) return s;
  const int hd = c->desc.n_heads * c->desc.head_dim;
  if (sa_status s = check_proj_sizes(0, hidden, hd, 1)) return s;
  if (!c->plan.has_frames()) return fail(SA_ERR_STATE, "recache on an empty cache");
  const int64_t n_tok = static_cast<int64_t>(c->desc.batch) * c->plan.resident().size() * c->desc.tokens_per_frame;
  if (sa_status s = check_proj_sizes(n_tok, hidden, hd, 1)) return s;
  {
    const size_t wb = static_cast<size_t>(hd) * hidden, ws = static_cast<size_t>(hd) * 4;
    if (hits_stores(c, x_codes, static_cast<size_t>(n_tok) * hidden) || hits_stores(c, x_scales, static_cast<size_t>(n_tok) * 4) ||
        hits_stores(c, wk_codes, wb) || hits_stores(c, wk_scales, ws) || hits_stores(c, wv_codes, wb) ||
        hits_stores(c, wv_scales, ws))
      return fail(SA_ERR_RANGE, "codes and scales must not overlap the cache stores");
  }
  sa::ProjArgs a = cache_proj_args(c, x_codes, nullptr, nullptr, wk_codes, wv_codes, hidden);
  a.w_scale[0] = wk_scales;
  a.w_scale[1] = a.w_scale[2] = wv_scales;
  a.op = op;
  a.x_scale = x_scales;
  a.n_tok = n_tok;
  a.frames = resident_table(c);
  const hipError_t e = sa::launch_proj(a, sa::kBF16, device_cus(), static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "recache launch")) return s_;
  return ok();
}

sa_status sa_cache_project_append_q8(sa_cache* c, const void* x_codes, const float* x_scales, const void* wq_codes,
                                     const float* wq_scales, const void* wk_codes, const float* wk_scales,
                                     const void* wv_codes, const float* wv_scales, sa_qtype qtype, int32_t hidden,
                                     void* q_out, int32_t n_frames, int64_t t0, void* stream) {
  if (!c || !x_codes || !x_scales || !wk_codes || !wk_scales || !wv_codes || !wv_scales)
    return fail(SA_ERR_NULL, "cache, codes and scales must be non-NULL");
  if (!wq_codes != !q_out || !wq_codes != !wq_scales)
    return fail(SA_ERR_NULL, "wq_codes, wq_scales and q_out must all be given or all be NULL");
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(wk_codes) || !aligned16(wk_scales) ||
      !aligned16(wv_codes) || !aligned16(wv_scales) || !aligned16(wq_codes) || !aligned16(wq_scales) ||
      !aligned16(q_out))
    return fail(SA_ERR_ALIGN, "codes, scales and q_out must be 16-byte aligned");
  int op = 0;
  if (sa_status s = check_cache_q8(c, qtype, &op, hidden)) return s;
  if (t0 < 0 || t0 > (int64_t(1) << 40)) return fail(SA_ERR_RANGE, "t0 out of range [0, 2^40]");
  if (sa_status s = check_append_chunk(c, n_frames, t0)) return s;
  const int hd = c->desc.n_heads * c->desc.head_dim;
  const int64_t n_tok = static_cast<int64_t>(c->desc.batch) * n_frames * c->desc.tokens_per_frame;
  if (sa_status s = check_proj_sizes(n_tok, hidden, hd, 1)) return s;
  {
    const size_t xb = static_cast<size_t>(n_tok) * hidden, wb = static_cast<size_t>(hd) * hidden;
    const size_t xs = static_cast<size_t>(n_tok) * 4, ws = static_cast<size_t>(hd) * 4;
    const size_t qb = q_out ? static_cast<size_t>(n_tok) * hd * 2 : 0;
    if (hits_stores(c, x_codes, xb) || hits_stores(c, x_scales, xs) || hits_stores(c, wk_codes, wb) ||
        hits_stores(c, wk_scales, ws) || hits_stores(c, wv_codes, wb) || hits_stores(c, wv_scales, ws) ||
        (wq_codes && (hits_stores(c, wq_codes, wb) || hits_stores(c, wq_scales, ws))) ||
        (q_out && hits_stores(c, q_out, qb)))
      return fail(SA_ERR_RANGE, "codes, scales and q_out must not overlap the cache stores");
    if (q_out && (overlaps(q_out, qb, x_codes, xb) || overlaps(q_out, qb, x_scales, xs) ||
                  overlaps(q_out, qb, wq_codes, wb) || overlaps(q_out, qb, wq_scales, ws) ||
                  overlaps(q_out, qb, wk_codes, wb) || overlaps(q_out, qb, wk_scales, ws) ||
                  overlaps(q_out, qb, wv_codes, wb) || overlaps(q_out, qb, wv_scales, ws)))
      return fail(SA_ERR_RANGE, "q_out must not overlap the codes or scales");
  }
  sa::ProjArgs a = cache_proj_args(c, x_codes, wq_codes, q_out, wk_codes, wv_codes, hidden);
  int n = 0;
  if (wq_codes) a.w_scale[n++] = wq_scales;
  a.w_scale[n++] = wk_scales;
  a.w_scale[n++] = wv_scales;
  for (int i = n; i < 3; ++i) a.w_scale[i] = wv_scales;
  a.op = op;
  a.x_scale = x_scales;
  a.n_tok = n_tok;
  a.frames = chunk_table(c, n_frames, t0);
  const hipError_t e = sa::launch_proj(a, sa::kBF16, device_cus(), static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "projection launch")) return s_;
  c->plan.commit_append(n_frames, t0);
  return ok();
}

static sa_status attn_plan(const sa_cache* c, int32_t n_q, int* splits, size_t* bytes) {
  if (!c->plan.has_frames()) return fail(SA_ERR_STATE, "attention on an empty cache");
  const auto res = c->plan.resident();
  if (n_q < 1 || n_q > static_cast<int32_t>(res.size()))
    return fail(SA_ERR_SHAPE, "n_q (%d) must be in [1, resident frames = %d]", n_q, static_cast<int>(res.size()));
  // The query frames are the newest n_q appended frames; they must all still be resident.
  if (res.back().frame - (n_q - 1) != res[res.size() - n_q].frame)
    return fail(SA_ERR_RANGE, "the newest %d frames are not all resident", n_q);
  const long long lq = static_cast<long long>(n_q) * c->desc.tokens_per_frame;
  if (lq * c->desc.batch > (1LL << 31) / 4) return fail(SA_ERR_SHAPE, "query chunk too large");
  const int s = sa::attn_num_splits(c->desc.dtype, c->desc.batch, c->desc.n_heads, c->desc.head_dim,
                                    c->desc.tokens_per_frame, n_q, static_cast<int>(res.size()), device_cus());
  *splits = s;
  *bytes = sa::attn_workspace_bytes(c->desc.dtype, c->desc.batch, c->desc.n_heads, c->desc.head_dim,
                                    c->desc.tokens_per_frame, n_q, s);
  return SA_OK;
}

sa_status sa_window_attn_workspace(const sa_cache* c, int32_t n_q, size_t* bytes) {
  if (!c || !bytes) return fail(SA_ERR_NULL, "cache and bytes must be non-NULL");
  int splits = 1;
  if (sa_status s = attn_plan(c, n_q, &splits, bytes)) return s;
  return ok();
}

}  // extern "C"

namespace {

sa_status check_attn(const sa_cache* c, const void* q, void* o, int32_t n_q, float scale, sa_mask mask,
                     void* workspace, size_t workspace_bytes) {
  if (!c || !q || !o) return fail(SA_ERR_NULL, "cache, q and o must be non-NULL");
  if (!aligned16(q) || !aligned16(o) || !aligned16(workspace)) return fail(SA_ERR_ALIGN, "q, o and workspace must be 16-byte aligned");
  if (q == o) return fail(SA_ERR_RANGE, "o must not alias q");
  if (mask != SA_MASK_NONE && mask != SA_MASK_FRAME_CAUSAL) return fail(SA_ERR_RANGE, "unknown mask");
  if (!(scale >= 0.f) || !std::isfinite(scale)) return fail(SA_ERR_RANGE, "scale must be finite and >= 0");
  int splits = 1;
  size_t need = 0;
  if (sa_status s = attn_plan(c, n_q, &splits, &need)) return s;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SA_ERR_RANGE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  // q and o [B, n_q*T, H, D]; o, q and the workspace must be disjoint from
  // each other and from the cache's stores.
  const size_t io = static_cast<size_t>(c->desc.batch) * n_q * c->desc.tokens_per_frame * c->desc.n_heads *
                    c->desc.head_dim * (c->desc.dtype == SA_F32 ? 4 : 2);
  const size_t sb = sa_cache_store_bytes(&c->desc);
  if (overlaps(o, io, q, io)) return fail(SA_ERR_RANGE, "o must not overlap q");
  if (overlaps(o, io, c->desc.k_store, sb) || overlaps(o, io, c->desc.v_store, sb) ||
      overlaps(q, io, c->desc.k_store, sb) || overlaps(q, io, c->desc.v_store, sb))
    return fail(SA_ERR_RANGE, "q and o must not overlap the cache stores");
  if (need > 0 && (overlaps(workspace, need, q, io) || overlaps(workspace, need, o, io) ||
                   overlaps(workspace, need, c->desc.k_store, sb) || overlaps(workspace, need, c->desc.v_store, sb)))
    return fail(SA_ERR_RANGE, "the workspace must not overlap q, o or the cache stores");
  return SA_OK;
}

sa::AttnArgs attn_args(const sa_cache* c, const void* q, void* o, int32_t n_q, float scale, sa_mask mask,
                       void* workspace) {
  int splits = 1;
  size_t need = 0;
  (void)attn_plan(c, n_q, &splits, &need);
  sa::AttnArgs a;
  a.q = q;
  a.o = o;
  a.g = geom(c);
  a.rope = rope_args(c->rope);
  a.frames = resident_table(c);
  a.n_q = n_q;
  a.causal = mask == SA_MASK_FRAME_CAUSAL ? 1 : 0;
  const float sc = scale == 0.f ? 1.f / std::sqrt(static_cast<float>(c->desc.head_dim)) : scale;
  a.scale_log2 = static_cast<float>(static_cast<double>(sc) * 1.4426950408889634);
  a.n_splits = splits;
  a.ws = static_cast<float*>(workspace);
  a.store_bytes = static_cast<uint32_t>(sa_cache_store_bytes(&c->desc));
  a.variant = sa::attn_kernel_variant(c->desc.dtype, c->desc.batch, c->desc.n_heads, c->desc.head_dim,
                             c->desc.tokens_per_frame, n_q, device_cus());
  a.key_limit = INT32_MAX;
  a.stat_mode = sa::kStatNone;
  a.stat = nullptr;
  return a;
}

}  // namespace

extern "C" {

sa_status sa_window_attn(const sa_cache* c, const void* q, void* o, int32_t n_q, float scale, sa_mask mask,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (sa_status s = check_attn(c, q, o, n_q, scale, mask, workspace, workspace_bytes)) return s;
  const sa::AttnArgs a = attn_args(c, q, o, n_q, scale, mask, workspace);
  const hipError_t e = sa::launch_window_attn(a, c->desc.dtype, static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "attention launch")) return s_;
  return ok();
}

sa_status sa_window_attn_noalloc(const sa_cache* c, const void* q, void* o, int32_t n_q, float scale, sa_mask mask,
                                 void* stream) {
  if (!c || !q || !o) return fail(SA_ERR_NULL, "cache, q and o must be non-NULL");
  int splits = 1;
  size_t need = 0;
  if (sa_status s = attn_plan(c, n_q, &splits, &need)) return s;
  if (need > sa::kNoAllocScratchBytes)
    return fail(SA_ERR_RANGE, "this call needs %zu bytes of key-split scratch; the library holds %zu "
                "(use sa_window_attn with a workspace)", need, sa::kNoAllocScratchBytes);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = sa::attn_noalloc_scratch(&scratch);
    if (e != hipSuccess || !scratch) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch address");
  }
  if (sa_status s = check_attn(c, q, o, n_q, scale, mask, scratch, need)) return s;
  const sa::AttnArgs a = attn_args(c, q, o, n_q, scale, mask, scratch);
  const hipError_t e = sa::launch_window_attn(a, c->desc.dtype, static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "attention launch")) return s_;
  return ok();
}

sa_status sa_window_attn_sink_mass(const sa_cache* c, const void* q, void* o, float* sink_mass, int32_t n_q,
                                   float scale, sa_mask mask, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!sink_mass) return fail(SA_ERR_NULL, "sink_mass must be non-NULL");
  if (c && c->desc.dtype == SA_FP8) return fail(SA_ERR_DTYPE, "the sink mass is not supported for an SA_FP8 cache");
  if (!aligned16(sink_mass)) return fail(SA_ERR_ALIGN, "sink_mass must be 16-byte aligned");
  if (sa_status s = check_attn(c, q, o, n_q, scale, mask, workspace, workspace_bytes)) return s;
  {
    // sink_mass [B, n_q*T, H] fp32 is a fourth output: disjoint from q, o, the workspace and the stores
    const size_t rows = static_cast<size_t>(c->desc.batch) * n_q * c->desc.tokens_per_frame * c->desc.n_heads;
    const size_t io = rows * c->desc.head_dim * (c->desc.dtype == SA_F32 ? 4 : 2);
    const size_t sb = sa_cache_store_bytes(&c->desc);
    int splits = 1;
    size_t need = 0;
    (void)attn_plan(c, n_q, &splits, &need);
    const size_t mb = rows * sizeof(float);
    if (overlaps(sink_mass, mb, q, io) || overlaps(sink_mass, mb, o, io) ||
        (need > 0 && overlaps(sink_mass, mb, workspace, need)) || overlaps(sink_mass, mb, c->desc.k_store, sb) ||
        overlaps(sink_mass, mb, c->desc.v_store, sb))
      return fail(SA_ERR_RANGE, "sink_mass must not overlap q, o, the workspace or the cache stores");
  }
  sa::AttnArgs a = attn_args(c, q, o, n_q, scale, mask, workspace);
  int n_sink_res = 0;
  for (const auto& f : c->plan.resident()) n_sink_res += f.segment == 0 ? 1 : 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // pass 1: the attention itself, plus each row's log2-sum-exp2 (or 0 when no sink is resident)
  a.stat_mode = n_sink_res > 0 ? sa::kStatLse : sa::kStatZero;
  a.stat = sink_mass;
  hipError_t e = sa::launch_window_attn(a, c->desc.dtype, st);
  if (sa_status s_ = launched(e, stream, "attention launch")) return s_;
  if (n_sink_res > 0) {
    // pass 2: the same rows over the sink keys only (the first n_sink_res
    // resident frames); the mass is 2^(LSE_sink - LSE_all).  At most as many
    // key splits as the shortest row has key tiles, so no split is empty.
    const int T = c->desc.tokens_per_frame;
    const int n_res = static_cast<int>(c->plan.resident().size());
    a.key_limit = n_sink_res * T;
    const int shortest = mask == SA_MASK_FRAME_CAUSAL ? (n_res - n_q + 1) * T : n_res * T;
    const int min_tiles = (std::min(shortest, a.key_limit) + 63) / 64;
    a.n_splits = std::max(1, std::min(a.n_splits, min_tiles));
    a.o = nullptr;
    a.stat_mode = sa::kStatMass;
    e = sa::launch_window_attn(a, c->desc.dtype, st);
    if (sa_status s_ = launched(e, st, "sink-mass launch")) return s_;
  }
  return ok();
}

sa_status sa_cache_slots(const sa_cache* c, sa_slot* out, int32_t cap, int32_t* n_valid) {
  if (!c || !n_valid) return fail(SA_ERR_NULL, "cache and n_valid must be non-NULL");
  if (cap > 0 && !out) return fail(SA_ERR_NULL, "out is NULL with cap > 0");
  const auto res = c->plan.resident();
  *n_valid = static_cast<int32_t>(res.size());
  for (int32_t i = 0; i < cap && i < static_cast<int32_t>(res.size()); ++i) {
    out[i].frame = res[i].frame;
    out[i].t = res[i].t;
    out[i].segment = res[i].segment;
    out[i].slot = res[i].slot;
  }
  return ok();
}

sa_status sa_cache_read(const sa_cache* c, int32_t index, void* k_out, void* v_out, void* stream) {
  if (!c) return fail(SA_ERR_NULL, "cache is NULL");
  if (!k_out && !v_out) return fail(SA_ERR_NULL, "k_out and v_out are both NULL");
  const auto res = c->plan.resident();
  if (index < 0 || index >= static_cast<int32_t>(res.size()))
    return fail(SA_ERR_RANGE, "index %d outside the %d resident frames", index, static_cast<int>(res.size()));
  const size_t ob = static_cast<size_t>(c->desc.batch) * c->desc.tokens_per_frame * c->desc.n_heads * c->desc.head_dim *
                    elem_size(c->desc.dtype);
  if ((k_out && hits_stores(c, k_out, ob)) || (v_out && hits_stores(c, v_out, ob)))
    return fail(SA_ERR_RANGE, "k_out and v_out must not overlap the cache stores");
  const hipError_t e = sa::launch_read(geom(c), res[index].store_slot, k_out, v_out, c->desc.dtype,
                                       static_cast<hipStream_t>(stream));
  if (sa_status s_ = launched(e, stream, "read launch")) return s_;
  return ok();
}

sa_status sa_cache_counts(const sa_cache* c, int64_t* n_appended, int32_t* n_resident) {
  if (!c) return fail(SA_ERR_NULL, "cache is NULL");
  if (n_appended) *n_appended = c->plan.n_appended();
  if (n_resident) *n_resident = static_cast<int32_t>(c->plan.resident().size());
  return ok();
}

}  // extern "C"

namespace sa {
int launch_override(int knob) {
  return knob >= 0 && knob < kNumKnobs ? g_knobs[knob].load(std::memory_order_relaxed) : 0;
}
}  // namespace sa
