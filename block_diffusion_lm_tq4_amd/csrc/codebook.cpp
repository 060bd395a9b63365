// The fixed TQ4_1S codebook: the 16-level Lloyd-Max quantizer of N(0,1)
// (Nemotron-TheHobbit-30B-A3B model card, section What "Config-I" means:
// "16-level Lloyd-Max" with one fixed codebook for every tensor), rounded to
// fp32 and stored ascending.
//
// The standard normal density is even, so the optimal quantizer is symmetric:
// only the eight positive levels are iterated, with the middle threshold held
// at 0.  Each sweep applies the two Lloyd-Max conditions:
//   thresholds  t_i = (c_{i-1} + c_i) / 2          (t_0 = 0, t_8 = +inf)
//   levels      c_i = E[X | t_i < X < t_{i+1}]
//                   = (phi(t_i) - phi(t_{i+1})) / (Q(t_i) - Q(t_{i+1})),
// where Q(x) = erfc(x / sqrt 2) / 2 is the upper tail, which keeps the
// denominators free of cancellation.
#include <cmath>
#include <mutex>

#include "tq4_internal.h"

namespace tq4 {
namespace {

double density(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }
double upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }

Codebook compute() {
  double c[8];
  for (int i = 0; i < 8; ++i) c[i] = 0.35 * (i + 0.5);
  for (int sweep = 0; sweep < 1000000; ++sweep) {
    double t[9];
    t[0] = 0.0;
    for (int i = 1; i < 8; ++i) t[i] = 0.5 * (c[i - 1] + c[i]);
    t[8] = INFINITY;
    double next[8], moved = 0.0;
    for (int i = 0; i < 8; ++i) {
      const double hi_density = std::isinf(t[i + 1]) ? 0.0 : density(t[i + 1]);
      const double hi_tail = std::isinf(t[i + 1]) ? 0.0 : upper_tail(t[i + 1]);
      next[i] = (density(t[i]) - hi_density) / (upper_tail(t[i]) - hi_tail);
      moved = std::fmax(moved, std::fabs(next[i] - c[i]));
    }
    for (int i = 0; i < 8; ++i) c[i] = next[i];
    if (moved < 1e-15) break;
  }
  Codebook cb;
  for (int i = 0; i < 8; ++i) {
    cb.c[8 + i] = static_cast<float>(c[i]);
    cb.c[7 - i] = -static_cast<float>(c[i]);
  }
  return cb;
}

}  // namespace

const Codebook &codebook() {
  static std::once_flag once;
  static Codebook cb;
  std::call_once(once, [] { cb = compute(); });
  return cb;
}

}  // namespace tq4
