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

inline RopeTables build_rope_tables(int n_heads, int head_dim, const int dims[3], double theta0,
                                    double sigma, const double* eps, uint32_t jitter_axes) {
  if (jitter_axes == 0) jitter_axes = 1u;
  RopeTables t;
  t.theta_hat.resize(static_cast<size_t>(n_heads) * 3);
  t.freq.resize(static_cast<size_t>(n_heads) * (head_dim / 2));
  for (int h = 0; h < n_heads; ++h) {
    double e = eps ? eps[h] : 0.0;
    for (int a = 0; a < 3; ++a) {
      bool jit = (jitter_axes >> a) & 1u;
      t.theta_hat[h * 3 + a] = jit ? theta0 * (1.0 + sigma * e) : theta0;
    }
    int p = 0;
    for (int a = 0; a < 3; ++a) {
      double base = t.theta_hat[h * 3 + a];
      for (int j = 0; j < dims[a] / 2; ++j, ++p) {
        // base^(-2j/d_a); j = 0 gives exactly 1.
        t.freq[static_cast<size_t>(h) * (head_dim / 2) + p] =
            std::pow(base, -2.0 * static_cast<double>(j) / static_cast<double>(dims[a]));
      }
    }
  }
  return t;
}

}  // namespace sa
