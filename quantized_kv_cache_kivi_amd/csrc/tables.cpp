// Host-side generation of the format tables written into the cache at create time:
//  * the TurboQuant sign diagonal and Lloyd-Max Beta(d/2, d/2) codebooks
//    ("TurboQuant KV Cache Compression — Spec", "Step 1: Random Orthogonal
//    Rotation", "Step 2: Lloyd-Max Scalar Quantization", "Codebook Generation");
//  * the 4-level Lloyd-Max quantizer of N(0, 1) used by q2k keys (q2k pull
//    request page, "Reference papers": Lloyd-Max codebook over block RMS
//    fitted to the Gaussian grid).
#include <cmath>
#include <cstring>

#include "kvq_internal.h"

namespace kvq {
namespace {

// splitmix64 (Steele, Lea, Flood, OOPSLA 2014): x += golden gamma, then the
// two xor-shift-multiply mixing rounds.
uint64_t splitmix64_next(uint64_t& x) {
  x += 0x9E3779B97F4A7C15ull;
  uint64_t z = x;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Continued fraction of the incomplete beta function (Abramowitz & Stegun
// 26.5.8), evaluated with the modified Lentz algorithm.
double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double c = 1.0, d = 1.0 - (a + b) * x / (a + 1.0);
  if (std::fabs(d) < tiny) d = tiny;
  d = 1.0 / d;
  double h = d;
  for (int m = 1; m <= 10000; ++m) {
    const double m2 = 2.0 * m;
    double num = m * (b - m) * x / ((a - 1.0 + m2) * (a + m2));
    d = 1.0 + num * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    h *= d * c;
    num = -(a + m) * (a + b + m) * x / ((a + m2) * (a + 1.0 + m2));
    d = 1.0 + num * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    const double del = d * c;
    h *= del;
    if (std::fabs(del - 1.0) < 1e-16) break;
  }
  return h;
}

// Regularised incomplete beta I_x(a, b).
double inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double lbt = std::lgamma(a + b) - std::lgamma(a) - std::lgamma(b) + a * std::log(x) + b * std::log1p(-x);
  const double bt = std::exp(lbt);
  if (x < (a + 1.0) / (a + b + 2.0)) return bt * beta_cf(a, b, x) / a;
  return 1.0 - bt * beta_cf(b, a, 1.0 - x) / b;
}

// Lloyd-Max quantizer of Beta(d/2, d/2) on [0, 1]; results in t = 2u - 1 space, fp32.
// Lloyd's conditions: each centroid is the conditional mean of its cell,
// E[X | lo < X < hi] = (1/2)(I_hi(a+1, a) - I_lo(a+1, a)) / (I_hi(a, a) - I_lo(a, a)),
// and each boundary is the midpoint of its two centroids.  Starts from levels
// spread evenly over mean +- 3 sd and stops once the fp32 tables have not
// changed for 100 iterations and the last step is below 1e-13.
void beta_lloyd_max(int d, int bits, float* bnd_t, float* cen_t) {
  const int L = 1 << bits;
  const double a = d / 2.0;
  const double mu = 0.5, sd = 1.0 / (2.0 * std::sqrt(2.0 * a + 1.0));
  double c[16], nc[16], e[17];
  for (int i = 0; i < L; ++i) c[i] = mu - 3.0 * sd + 6.0 * sd * (i + 0.5) / L;
  float last[16];
  for (int i = 0; i < 16; ++i) last[i] = NAN;
  int same = 0;
  for (int it = 0; it < 400000; ++it) {
    e[0] = 0.0;
    e[L] = 1.0;
    for (int i = 1; i < L; ++i) e[i] = 0.5 * (c[i - 1] + c[i]);
    for (int i = 0; i < L; ++i) {
      const double mass = inc_beta(a, a, e[i + 1]) - inc_beta(a, a, e[i]);
      const double mom = 0.5 * (inc_beta(a + 1.0, a, e[i + 1]) - inc_beta(a + 1.0, a, e[i]));
      nc[i] = mom / mass;
    }
    double step = 0.0;
    bool stable = it > 0;
    for (int i = 0; i < L; ++i) {
      const double s = 0.5 * (nc[i] + (1.0 - nc[L - 1 - i]));
      step = std::fmax(step, std::fabs(s - c[i]));
      c[i] = s;
    }
    for (int i = 0; i < L; ++i) {
      const float f = (float)(2.0 * c[i] - 1.0);
      if (f != last[i]) stable = false;
      last[i] = f;
    }
    same = stable ? same + 1 : 0;
    if (same >= 100 && step < 1e-13) break;
  }
  for (int i = 0; i < L; ++i) cen_t[i] = (float)(2.0 * c[i] - 1.0);
  for (int i = 1; i < L; ++i) {
    const double b = (i == L / 2) ? 0.5 : 0.5 * (c[i - 1] + c[i]);
    bnd_t[i - 1] = (float)(2.0 * b - 1.0);
  }
}

double phi(double x) { return std::isfinite(x) ? std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI) : 0.0; }
double Phi(double x) {
  if (x == INFINITY) return 1.0;
  if (x == -INFINITY) return 0.0;
  return 0.5 * std::erfc(-x / std::sqrt(2.0));
}

// 4-level Lloyd-Max quantizer of N(0, 1): level_i = (phi(a) - phi(b)) / (Phi(b) - Phi(a)) over its cell.
void gaussian_lloyd_max4(float* thr, float* lvl) {
  double l[4] = {-1.5, -0.5, 0.5, 1.5}, n[4];
  for (int it = 0; it < 100000; ++it) {
    const double e[5] = {-INFINITY, 0.5 * (l[0] + l[1]), 0.5 * (l[1] + l[2]), 0.5 * (l[2] + l[3]), INFINITY};
    for (int i = 0; i < 4; ++i) n[i] = (phi(e[i]) - phi(e[i + 1])) / (Phi(e[i + 1]) - Phi(e[i]));
    double step = 0.0;
    for (int i = 0; i < 4; ++i) {
      const double s = 0.5 * (n[i] - n[3 - i]);
      step = std::fmax(step, std::fabs(s - l[i]));
      l[i] = s;
    }
    if (step < 1e-15) break;
  }
  for (int i = 0; i < 4; ++i) lvl[i] = (float)l[i];
  thr[0] = (float)(0.5 * (l[0] + l[1]));
  thr[1] = 0.0f;
  thr[2] = (float)(0.5 * (l[2] + l[3]));
  thr[3] = 0.0f;
}

}  // namespace

void make_tables(const kvq_config& cfg, Tables* t) {
  std::memset(t, 0, sizeof(*t));
  uint64_t x = cfg.seed;
  // one sign per stored (padded) coordinate; the codebooks follow Beta(head_dim/2, head_dim/2)
  for (int i = 0; i < stored_dim(cfg); ++i) t->signs[i] = (splitmix64_next(x) >> 63) ? -1.0f : 1.0f;
  if (cfg.format == KVQ_FMT_TQ) {
    beta_lloyd_max(cfg.head_dim, cfg.k_bits, t->k_bnd, t->k_cen);
    beta_lloyd_max(cfg.head_dim, cfg.v_bits, t->v_bnd, t->v_cen);
    // boundaries past a narrower codebook never count (3-bit codes live in 4-bit slots, whose
    // quantizer counts 15 boundaries); centroids past it are never read
    for (int j = (1 << cfg.k_bits) - 1; j < 15; ++j) t->k_bnd[j] = INFINITY;
    for (int j = (1 << cfg.v_bits) - 1; j < 15; ++j) t->v_bnd[j] = INFINITY;
  }
  gaussian_lloyd_max4(t->q2k_thr, t->q2k_lvl);
  const double base = cfg.rope_base > 0.f ? (double)cfg.rope_base : 10000.0;
  const int nrope = cfg.head_dim <= MAX_D ? cfg.head_dim / 2 : 0;  // RoPE is for the block formats (<= 128)
  for (int c = 0; c < nrope; ++c) t->rope_inv[c] = (float)std::pow(base, -2.0 * c / cfg.head_dim);
  if (cfg.rope)
    for (int i = 0; i < 16; ++i)
      for (int c = 0; c < nrope; ++c) {
        const double ang = (double)i * (double)t->rope_inv[c];
        t->rope_row[i][c][0] = (float)std::cos(ang);
        t->rope_row[i][c][1] = (float)std::sin(ang);
      }
}

}  // namespace kvq
