// Row-wise 8-bit quantisation for the W8A8 projections (LongLive paper
// review, "INT8 quantized inference" table; model card FP8 variant).
//
// One wave per row of bf16 values: pass 1 finds a = max |x| (16-byte loads,
// wave reduction through cross-lane swaps), pass 2 reads the row again (from
// L2) and writes codes = round(x * (Q / a)) 8 per lane and step, Q = 127
// (int8, nearest with ties to even) or 448 (e4m3, the converter's nearest
// even after a clamp to +-448), and the scale a / Q.  Divisions and the
// product are single fp32 operations rounded to nearest, so the codes are
// exactly those of the same steps on the host in fp32.  HBM-bound: 2 bytes
// read (twice, the second from L2 for rows up to a few hundred KB) and 1
// byte written per element.
#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace sa {
namespace {

constexpr int kQRowsPerBlock = 4;  // one wave per row

template <int QT>
__global__ void __launch_bounds__(64 * kQRowsPerBlock) quant_rows_kernel(const uint16_t* __restrict__ x,
                                                                         uint8_t* __restrict__ codes,
                                                                         float* __restrict__ scales,
                                                                         int64_t n_rows, int n_cols) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kQRowsPerBlock + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * n_cols);
  const int chunks = n_cols / 8;
  float amax = 0.f;
  for (int c = lane; c < chunks; c += 64) {
    float v[8];
    unpack_bf16x8(src[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  constexpr float Q = QT == kOpI8 ? 127.f : 448.f;
  const float inv = amax > 0.f ? __fdiv_rn(Q, amax) : 0.f;
  if (lane == 0) scales[row] = amax > 0.f ? __fdiv_rn(amax, Q) : 0.f;
  uint2* dst = reinterpret_cast<uint2*>(codes + row * n_cols);
  for (int c = lane; c < chunks; c += 64) {
    float v[8];
    unpack_bf16x8(src[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __fmul_rn(v[i], inv);
    uint2 out;
    if constexpr (QT == kOpI8) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = static_cast<int>(fminf(fmaxf(rintf(v[i]), -127.f), 127.f));
        w[i >> 2] |= (static_cast<uint32_t>(q) & 0xffu) << (8 * (i & 3));
      }
      out.x = w[0];
      out.y = w[1];
    } else {
      out = to_e4m3x8(v, 1.f);  // clamp to +-448, nearest even
    }
    dst[c] = out;
  }
}

}  // namespace

hipError_t launch_quantize_rows(const void* x, void* codes, float* scales, int op, int64_t n_rows, int n_cols,
                                hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n_rows + kQRowsPerBlock - 1) / kQRowsPerBlock));
  const dim3 block(64 * kQRowsPerBlock);
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* cs = static_cast<uint8_t*>(codes);
  if (op == kOpI8)
    hipLaunchKernelGGL(quant_rows_kernel<kOpI8>, grid, block, 0, stream, xs, cs, scales, n_rows, n_cols);
  else
    hipLaunchKernelGGL(quant_rows_kernel<kOpE4M3>, grid, block, 0, stream, xs, cs, scales, n_rows, n_cols);
  return hipGetLastError();
}

}  // namespace sa
