// Host-side fp64 tables for 3D RoPE with LoL's per-head jittered base.
//
// LoL paper review, "method steps": (3) one eps_h in [-1, 1] per head,
// (4) theta_hat_h = theta0 (1 + sigma eps_h), (5) the head's frequencies are
// theta_hat_h raised to the exponents -2j/d of (2); background "Rotary
// Position Embedding": base frequency theta^(-2i/d) per channel pair.
// The head dimension is split into [t | h | w] segments; segment a uses its
// own sub-dimension d_a in the exponent and the jittered base only when the
// axis is selected in jitter_axes.
#pragma once

#include <cmath>
#include <cstdint>
#include <vector>

namespace sa {

struct RopeTables {
  std::vector<double> theta_hat;  // [H][3]
  std::vector<double> freq;       // [H][D/2]
};

// t_scale: position interpolation on the time axis (LoL review, PI baseline),
// folded into the time-axis frequencies: angle t * (w * t_scale).
// theta: optional per-head, per-axis bases [H][3] given directly (theta_hat
// itself); theta0, sigma, eps and jitter_axes are then unused.
inline RopeTables build_rope_tables(int n_heads, int head_dim, const int dims[3], double theta0,
                                    double sigma, const double* eps, uint32_t jitter_axes,
                                    double t_scale = 1.0, const double* theta = nullptr) {
  if (jitter_axes == 0) jitter_axes = 1u;
  if (t_scale == 0.0) t_scale = 1.0;
  RopeTables t;
  t.theta_hat.resize(static_cast<size_t>(n_heads) * 3);
  t.freq.resize(static_cast<size_t>(n_heads) * (head_dim / 2));
  for (int h = 0; h < n_heads; ++h) {
    double e = eps ? eps[h] : 0.0;
    for (int a = 0; a < 3; ++a) {
      bool jit = (jitter_axes >> a) & 1u;
      t.theta_hat[h * 3 + a] = theta ? theta[h * 3 + a] : (jit ? theta0 * (1.0 + sigma * e) : theta0);
    }
    int p = 0;
    for (int a = 0; a < 3; ++a) {
      double base = t.theta_hat[h * 3 + a];
      for (int j = 0; j < dims[a] / 2; ++j, ++p) {
        // base^(-2j/d_a); j = 0 gives exactly 1.
        t.freq[static_cast<size_t>(h) * (head_dim / 2) + p] =
            std::pow(base, -2.0 * static_cast<double>(j) / static_cast<double>(dims[a])) * (a == 0 ? t_scale : 1.0);
      }
    }
  }
  return t;
}

// cos and sin of the grid-axis angles, which do not depend on the frame:
// for every head table (one per head when the h or w axis is jittered, else
// one shared), entries [row][pairs_h] then [col][pairs_w], each (cos, sin) of
// pos * w formed and evaluated in fp64, rounded to fp32.  Empty when the
// table would exceed max_bytes (the kernels then evaluate sin/cos directly).
struct RopeGridTable {
  std::vector<float> cs;  // [n_tab][stride][2]
  int stride = 0;         // entries per head table
  bool per_head = false;
};

// One table per head when some head's grid-axis (h or w) base differs from
// head 0's, else one shared table.
inline RopeGridTable build_rope_grid_table(const RopeTables& t, int n_heads, int head_dim, const int dims[3],
                                           int grid_h, int grid_w, size_t max_bytes = size_t(32) << 20) {
  RopeGridTable g;
  const int pt = dims[0] / 2, ph = dims[1] / 2, pw = dims[2] / 2;
  g.per_head = false;
  for (int h = 1; h < n_heads; ++h)
    for (int a = 1; a < 3; ++a)
      if (t.theta_hat[h * 3 + a] != t.theta_hat[a]) g.per_head = true;
  g.stride = grid_h * ph + grid_w * pw;
  const int n_tab = g.per_head ? n_heads : 1;
  if (static_cast<size_t>(n_tab) * g.stride * 2 * sizeof(float) > max_bytes) {
    g.stride = 0;
    return g;
  }
  g.cs.resize(static_cast<size_t>(n_tab) * g.stride * 2);
  const size_t hp = static_cast<size_t>(head_dim / 2);
  for (int h = 0; h < n_tab; ++h) {
    float* out = g.cs.data() + static_cast<size_t>(h) * g.stride * 2;
    for (int row = 0; row < grid_h; ++row)
      for (int j = 0; j < ph; ++j, out += 2) {
        const double a = static_cast<double>(row) * t.freq[h * hp + pt + j];
        out[0] = static_cast<float>(std::cos(a));
        out[1] = static_cast<float>(std::sin(a));
      }
    for (int col = 0; col < grid_w; ++col)
      for (int j = 0; j < pw; ++j, out += 2) {
        const double a = static_cast<double>(col) * t.freq[h * hp + pt + ph + j];
        out[0] = static_cast<float>(std::cos(a));
        out[1] = static_cast<float>(std::sin(a));
      }
  }
  return g;
}

}  // namespace sa
