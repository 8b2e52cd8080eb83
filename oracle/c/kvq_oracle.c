/*
 * kvq_oracle.c — plain C99 CPU oracle of the quantized KV cache hot path (TEST INFRASTRUCTURE ONLY).
 * See kvq_oracle.h for what it computes and the pages each step follows.  Built as its own shared
 * library with -std=c99 -O2 -ffp-contract=off -fno-fast-math (and OpenMP for decode attention); it
 * shares no code, header or table with the HIP library.
 */
#define _POSIX_C_SOURCE 200809L
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define G 32           /* token-block length and V channel-group length */
#define MAXD 256       /* widest stored row: TurboQuant head_dim 160 padded to 256 */
#define MAXSINK 16
#define EPS 1e-5f      /* eps of the affine scale: StreamingLLM + KIVI page, "Affine quantisation formula" */

/* ------------------------------------------------------------------------------------------------- */
/* fp16 <-> fp32, from the IEEE-754 binary16 definition                                              */
/* ------------------------------------------------------------------------------------------------- */

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* Round to nearest, ties to even; subnormals kept; overflow to infinity. */
static uint16_t f16_bits(float f) {
  const uint32_t x = bits_of(f);
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  const int e = (int)(ax >> 23) - 127;  /* unbiased exponent (normal fp32) */
  if (ax < 0x00800000u) return sign;   /* fp32 subnormal: far below half the smallest fp16 subnormal */
  const uint32_t m = (ax & 0x7fffffu) | 0x800000u; /* 24-bit significand, value m * 2^(e - 23) */
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  if (e >= -14) {  /* normal binary16: keep 10 fraction bits, round the 13 dropped */
    uint32_t r = ((uint32_t)(e + 15) << 10) | ((m >> 13) & 0x3ffu);
    const uint32_t rem = m & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) r += 1u; /* a carry moves to the next binade / inf */
    return (uint16_t)(sign | r);
  }
  /* subnormal binary16: value in units of 2^-24 is m * 2^(e + 1) */
  const int s = -(e + 1); /* >= 14 */
  if (s > 25) return sign;
  uint32_t r = m >> s;
  const uint32_t rem = m & ((1u << s) - 1u), half = 1u << (s - 1);
  if (rem > half || (rem == half && (r & 1u))) r += 1u;
  return (uint16_t)(sign | r);
}

static float f16_val(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu, f = h & 0x3ffu;
  float v;
  if (e == 0) {
    v = ldexpf((float)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexpf((float)(f | 0x400u), (int)e - 25);
  }
  uint32_t u = bits_of(v) | sign;
  memcpy(&v, &u, 4);
  return v;
}

void ko_f32_to_f16(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_bits(x[i]);
}

static float canon0(float x) { return x + 0.0f; } /* -0 -> +0 */

/* Canonical sum of squares of a power-of-two-length vector: pair products, then halving. */
static float sumsq(const float* x, int d) {
  float a[MAXD / 2];
  for (int l = 0; l < d / 2; ++l) {
    const float p0 = x[2 * l] * x[2 * l];
    const float p1 = x[2 * l + 1] * x[2 * l + 1];
    a[l] = p0 + p1;
  }
  for (int h = d / 4; h >= 1; h /= 2)
    for (int l = 0; l < h; ++l) a[l] = a[l] + a[l + h];
  return a[0];
}

/* ------------------------------------------------------------------------------------------------- */
/* Tables                                                                                            */
/* ------------------------------------------------------------------------------------------------- */

/* splitmix64 (Steele, Lea and Flood, 2014): sigma_i = -1 where bit 63 of draw i is set. */
int ko_tq_signs(uint64_t seed, int d, float* out) {
  uint64_t x = seed;
  for (int i = 0; i < d; ++i) {
    x += 0x9E3779B97F4A7C15ull;
    uint64_t z = x;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    out[i] = (z >> 63) ? -1.0f : 1.0f;
  }
  return 0;
}

/* Regularized incomplete beta I_x(a, b) from its hypergeometric series
 *   I_x(a, b) = x^a (1 - x)^b / (a B(a, b)) * sum_n [(a + b)_n / (a + 1)_n] x^n
 * (all terms positive), used for x <= a / (a + b) and mirrored I_x(a, b) = 1 - I_{1-x}(b, a) above. */
static double lbeta(double a, double b) { return lgamma(a) + lgamma(b) - lgamma(a + b); }
static double ibeta_series(double x, double a, double b) {
  if (x <= 0.0) return 0.0;
  double term = 1.0, sum = 1.0;
  for (int n = 0; n < 100000; ++n) {
    term *= (a + b + n) / (a + 1.0 + n) * x;
    sum += term;
    if (term < 1e-17 * sum) break;
  }
  return exp(a * log(x) + b * log1p(-x) - log(a) - lbeta(a, b)) * sum;
}
static double ibeta(double x, double a, double b) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  if (x <= a / (a + b)) return ibeta_series(x, a, b);
  return 1.0 - ibeta_series(1.0 - x, b, a);
}

/* Lloyd-Max quantizer of Beta(d/2, d/2) on [0, 1] (TurboQuant spec, "Codebook Generation"): cell
 * centroids E[X | cell] = (1/2)(I(a+1, a) differences) / (I(a, a) differences), boundaries at midpoints,
 * symmetric about 1/2; started from levels spread evenly over mean +- 3 sd (the printed uniform start
 * leaves cells without mass at 16 levels) and run until the fp32 tables have not changed for 100
 * iterations and the step is below 1e-13.  Tables in t = 2u - 1. */
int ko_tq_codebook(int d, int bits, float* bnd, float* cen) {
  if (bits < 1 || bits > 4 || d < 2) return -1;
  const int L = 1 << bits;
  const double a = d / 2.0, mu = 0.5, sd = 1.0 / (2.0 * sqrt(2.0 * a + 1.0));
  double c[16], nc[16], edges[17];
  float last32[16], cur32[16];
  for (int i = 0; i < L; ++i) c[i] = mu - 3 * sd + 6 * sd * (i + 0.5) / L;
  int same = 0, have_last = 0;
  for (int it = 1; it <= 400000; ++it) {
    edges[0] = 0.0;
    edges[L] = 1.0;
    for (int i = 1; i < L; ++i) edges[i] = 0.5 * (c[i] + c[i - 1]);
    for (int i = 0; i < L; ++i) {
      const double mass = ibeta(edges[i + 1], a, a) - ibeta(edges[i], a, a);
      const double mom = 0.5 * (ibeta(edges[i + 1], a + 1.0, a) - ibeta(edges[i], a + 1.0, a));
      nc[i] = mom / mass;
    }
    double step = 0.0;
    for (int i = 0; i < L; ++i) {
      const double v = 0.5 * (nc[i] + (1.0 - nc[L - 1 - i]));
      const double dlt = fabs(v - c[i]);
      if (dlt > step) step = dlt;
      c[i] = v;
    }
    int eq = have_last;
    for (int i = 0; i < L; ++i) {
      cur32[i] = (float)(2.0 * c[i] - 1.0);
      if (have_last && cur32[i] != last32[i]) eq = 0;
    }
    same = eq ? same + 1 : 0;
    memcpy(last32, cur32, sizeof(cur32));
    have_last = 1;
    if (same >= 100 && step < 1e-13) break;
  }
  for (int i = 0; i < L; ++i) cen[i] = (float)(2.0 * c[i] - 1.0);
  for (int i = 1; i < L; ++i) {
    const double b = (i == L / 2) ? 0.5 : 0.5 * (c[i] + c[i - 1]);
    bnd[i - 1] = (float)(2.0 * b - 1.0);
  }
  return 0;
}

/* Gaussian 4-level Lloyd-Max quantizer (the q2k grid): levels are conditional means
 * (phi(a) - phi(b)) / (Phi(b) - Phi(a)) of their cells, thresholds midpoints, symmetric. */
static double phi_pdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846); }
static double phi_cdf(double x) {
  if (isinf(x)) return x > 0 ? 1.0 : 0.0;
  return 0.5 * erfc(-x / sqrt(2.0));
}
int ko_q2k_grid(float* thresholds, float* levels) {
  double lv[4] = {-1.5, -0.5, 0.5, 1.5}, nl[4];
  for (int it = 0; it < 100000; ++it) {
    double e[5] = {-INFINITY, 0, 0, 0, INFINITY};
    for (int i = 1; i < 4; ++i) e[i] = 0.5 * (lv[i] + lv[i - 1]);
    for (int i = 0; i < 4; ++i) nl[i] = (phi_pdf(e[i]) - phi_pdf(e[i + 1])) / (phi_cdf(e[i + 1]) - phi_cdf(e[i]));
    double step = 0.0;
    double sym[4];
    for (int i = 0; i < 4; ++i) sym[i] = 0.5 * (nl[i] - nl[3 - i]);
    for (int i = 0; i < 4; ++i) {
      if (fabs(sym[i] - lv[i]) > step) step = fabs(sym[i] - lv[i]);
      lv[i] = sym[i];
    }
    if (step < 1e-15) break;
  }
  for (int i = 0; i < 4; ++i) levels[i] = (float)lv[i];
  thresholds[0] = (float)(0.5 * (lv[0] + lv[1]));
  thresholds[1] = 0.0f;
  thresholds[2] = (float)(0.5 * (lv[2] + lv[3]));
  return 0;
}

/* ------------------------------------------------------------------------------------------------- */
/* Model                                                                                             */
/* ------------------------------------------------------------------------------------------------- */

typedef struct {
  float* k; /* [cap][D] fp32 copies of the input rows (exact for fp16 input) */
  float* v;
  int64_t cap;
} Rows;

struct ko_model {
  ko_config c;
  int dp;                                  /* stored width: TurboQuant pads head_dim to a power of two */
  int kslot, vslot;                        /* bits a stored code occupies */
  int kc, vc, km, vm, rec;                 /* record section sizes */
  int cap_b;
  float signs[MAXD], kbnd[16], kcen[16], vbnd[16], vcen[16];
  float q2k_th[3], q2k_lv[4];
  int64_t *P, *lo, *pend_P;
  int* pend_n;
  int* ncommit;                            /* [L][B] */
  int64_t* cpos;                           /* [L][B][MAXSINK] */
  float* cscore;
  Rows* rows;                              /* [L][B][H] */
};

static int slot_bits(int bits, int dense3) { return bits == 3 ? (dense3 ? 3 : 4) : bits; }

ko_model* ko_create(const ko_config* cfg) {
  const ko_config c = *cfg;
  if (c.n_layers < 1 || c.batch < 1 || c.n_kv_heads < 1 || c.n_q_heads < 1) return NULL;
  if (c.n_q_heads % c.n_kv_heads) return NULL;
  if (c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128 &&
      !(c.fmt == 2 && (c.head_dim == 96 || c.head_dim == 160)))
    return NULL;
  if (c.n_sink < 0 || c.n_sink > MAXSINK || c.capacity < G || c.capacity % G) return NULL;
  if (c.rope && c.fmt == 2) return NULL;
  if (c.fmt == 0) {
    if ((c.k_bits != 2 && c.k_bits != 4 && c.k_bits != 8) || (c.v_bits != 2 && c.v_bits != 4 && c.v_bits != 8))
      return NULL;
  } else if (c.fmt == 1) {
    if (c.k_bits != 2 || c.v_bits != 4) return NULL;
  } else if (c.fmt == 2) {
    if (c.k_bits < 2 || c.k_bits > 4 || c.v_bits < 2 || c.v_bits > 4) return NULL;
  } else {
    return NULL;
  }
  ko_model* m = (ko_model*)calloc(1, sizeof(ko_model));
  if (!m) return NULL;
  m->c = c;
  int dp = c.head_dim;
  if (c.fmt == 2)
    while (dp & (dp - 1)) dp += dp & -dp;  /* next power of two (TurboQuant spec, "Hadamard Transform Detail") */
  m->dp = dp;
  const int D = dp;
  const int dense = c.fmt == 2 && c.tq_dense3;
  m->kslot = slot_bits(c.k_bits, dense);
  m->vslot = slot_bits(c.v_bits, dense);
  m->kc = G * D * m->kslot / 8;
  m->vc = G * D * m->vslot / 8;
  if (c.fmt == 0) {
    m->km = 2 * 2 * D;
    m->vm = 2 * 2 * G * (D / 32);
  } else if (c.fmt == 1) {
    m->km = 2 * D;
    m->vm = 2 * G * (D / 32);
  } else {
    m->km = 4 * G;
    m->vm = 4 * G;
  }
  m->rec = m->kc + m->vc + m->km + m->vm;
  m->cap_b = c.capacity / G;
  if (c.fmt == 2) {  /* one sign per stored coordinate; codebooks of Beta(head_dim/2, head_dim/2) */
    ko_tq_signs(c.seed, dp, m->signs);
    ko_tq_codebook(c.head_dim, c.k_bits, m->kbnd, m->kcen);
    ko_tq_codebook(c.head_dim, c.v_bits, m->vbnd, m->vcen);
  }
  ko_q2k_grid(m->q2k_th, m->q2k_lv);
  const int L = c.n_layers, B = c.batch, H = c.n_kv_heads;
  m->P = (int64_t*)calloc(L, sizeof(int64_t));
  m->lo = (int64_t*)calloc(L, sizeof(int64_t));
  m->pend_P = (int64_t*)calloc(L, sizeof(int64_t));
  m->pend_n = (int*)calloc(L, sizeof(int));
  m->ncommit = (int*)calloc((size_t)L * B, sizeof(int));
  m->cpos = (int64_t*)calloc((size_t)L * B * MAXSINK, sizeof(int64_t));
  m->cscore = (float*)calloc((size_t)L * B * MAXSINK, sizeof(float));
  m->rows = (Rows*)calloc((size_t)L * B * H, sizeof(Rows));
  if (!m->P || !m->lo || !m->pend_P || !m->pend_n || !m->ncommit || !m->cpos || !m->cscore || !m->rows) {
    ko_destroy(m);
    return NULL;
  }
  for (int l = 0; l < L; ++l) {
    m->pend_P[l] = -1;
    m->pend_n[l] = -1;
  }
  return m;
}

void ko_destroy(ko_model* m) {
  if (!m) return;
  if (m->rows) {
    for (int64_t i = 0; i < (int64_t)m->c.n_layers * m->c.batch * m->c.n_kv_heads; ++i) {
      free(m->rows[i].k);
      free(m->rows[i].v);
    }
  }
  free(m->rows);
  free(m->P);
  free(m->lo);
  free(m->pend_P);
  free(m->pend_n);
  free(m->ncommit);
  free(m->cpos);
  free(m->cscore);
  free(m);
}

static Rows* rows_of(const ko_model* m, int layer, int b, int h) {
  return &m->rows[((int64_t)layer * m->c.batch + b) * m->c.n_kv_heads + h];
}

/* Input element i of a chunk, as fp32. */
static float in_val(const ko_model* m, const void* p, int64_t i) {
  return m->c.in_f32 ? ((const float*)p)[i] : f16_val(((const uint16_t*)p)[i]);
}

int ko_state(const ko_model* m, int layer, int64_t* P, int64_t* lo) {
  if (!m || layer < 0 || layer >= m->c.n_layers) return -1;
  if (P) *P = m->P[layer];
  if (lo) *lo = m->lo[layer];
  return 0;
}

int ko_record_layout(const ko_model* m, int32_t* out6) {
  out6[0] = m->rec;
  out6[1] = 0;
  out6[2] = m->kc;
  out6[3] = m->kc + m->vc;
  out6[4] = m->kc + m->vc + m->km;
  out6[5] = m->cap_b;
  return 0;
}

/* ---- sinks (kivi_sink page, "How it works" 1; "Fidelity to the paper") ---- */

typedef struct {
  int64_t pos;
  float score;
  int is_new;
} Cand;

/* a ranks before b: score descending, position ascending */
static int ranks_before(const Cand* a, const Cand* b) {
  if (a->score != b->score) return a->score > b->score;
  return a->pos < b->pos;
}

int ko_select(ko_model* m, int layer, const void* k, int n) {
  if (!m || layer < 0 || layer >= m->c.n_layers || !k || n < 1) return -1;
  const ko_config* c = &m->c;
  const int64_t P = m->P[layer];
  if (c->sink_mode == 2 && c->n_sink > 0) {
    const int H = c->n_kv_heads, D = c->head_dim, ns = c->n_sink;
    float* sc = (float*)malloc(sizeof(float) * n);
    Cand* cand = (Cand*)malloc(sizeof(Cand) * (n + MAXSINK));
    if (!sc || !cand) {
      free(sc);
      free(cand);
      return -1;
    }
    for (int b = 0; b < c->batch; ++b) {
      int* nc = &m->ncommit[layer * c->batch + b];
      if (*nc >= ns) continue;
      float row[MAXD];
      for (int t = 0; t < n; ++t) {
        float acc = 0.0f;
        for (int h = 0; h < H; ++h) {
          const int64_t base = (((int64_t)b * H + h) * n + t) * D;
          for (int ch = 0; ch < D; ++ch) row[ch] = in_val(m, k, base + ch);
          acc = acc + sqrtf(sumsq(row, D));
        }
        sc[t] = acc / (float)H;
      }
      int64_t* cp = &m->cpos[((int64_t)layer * c->batch + b) * MAXSINK];
      float* cs = &m->cscore[((int64_t)layer * c->batch + b) * MAXSINK];
      int nn = 0;
      for (int i = 0; i < *nc; ++i) cand[nn++] = (Cand){cp[i], cs[i], 0};
      for (int t = 0; t < n; ++t) cand[nn++] = (Cand){P + t, sc[t], 1};
      /* the top n_sink of the candidates, in rank order; new members join while there is room */
      for (int r = 0; r < ns && r < nn; ++r) {
        int best = r;
        for (int i = r + 1; i < nn; ++i)
          if (ranks_before(&cand[i], &cand[best])) best = i;
        const Cand tmp = cand[r];
        cand[r] = cand[best];
        cand[best] = tmp;
        if (cand[r].is_new && *nc < ns) {
          cp[*nc] = cand[r].pos;
          cs[*nc] = cand[r].score;
          ++*nc;
        }
      }
    }
    free(sc);
    free(cand);
  }
  m->pend_P[layer] = P;
  m->pend_n[layer] = n;
  return 0;
}

int ko_append(ko_model* m, int layer, const void* k, const void* v, int n) {
  if (!m || layer < 0 || layer >= m->c.n_layers || !k || !v || n < 1) return -1;
  const ko_config* c = &m->c;
  const int64_t P = m->P[layer];
  if (c->sink_mode == 2 && c->n_sink > 0 && (m->pend_P[layer] != P || m->pend_n[layer] != n)) return -4;
  if (c->window == 0) {
    if (P + n > c->capacity) return -3;
  } else {
    const int64_t last = (P + n - 1) / G;
    if ((last - m->cap_b + 1) * G > m->lo[layer]) return -3;
  }
  const int H = c->n_kv_heads, D = c->head_dim;
  for (int b = 0; b < c->batch; ++b)
    for (int h = 0; h < H; ++h) {
      Rows* r = rows_of(m, layer, b, h);
      if (P + n > r->cap) {
        int64_t nc = r->cap ? r->cap : 64;
        while (nc < P + n) nc *= 2;
        float* nk = (float*)realloc(r->k, sizeof(float) * nc * D);
        if (!nk) return -1;
        r->k = nk;
        float* nv = (float*)realloc(r->v, sizeof(float) * nc * D);
        if (!nv) return -1;
        r->v = nv;
        r->cap = nc;
      }
      for (int t = 0; t < n; ++t) {
        const int64_t base = (((int64_t)b * H + h) * n + t) * D;
        for (int ch = 0; ch < D; ++ch) {
          r->k[(P + t) * D + ch] = in_val(m, k, base + ch);
          r->v[(P + t) * D + ch] = in_val(m, v, base + ch);
        }
      }
    }
  m->P[layer] = P + n;
  m->pend_P[layer] = -1;
  m->pend_n[layer] = -1;
  if (c->sink_mode == 1 && c->n_sink > 0)
    for (int b = 0; b < c->batch; ++b) {
      const int64_t np = P + n < c->n_sink ? P + n : c->n_sink;
      int64_t* cp = &m->cpos[((int64_t)layer * c->batch + b) * MAXSINK];
      float* cs = &m->cscore[((int64_t)layer * c->batch + b) * MAXSINK];
      for (int64_t p = 0; p < np; ++p) {
        cp[p] = p;
        cs[p] = 0.0f;
      }
      m->ncommit[layer * c->batch + b] = (int)np;
    }
  return 0;
}

/* StreamingLLM eviction (StreamingLLM + KIVI page, "Implementation"): lo = max(lo, P - W). */
int ko_evict(ko_model* m, int layer) {
  if (!m || layer < 0 || layer >= m->c.n_layers) return -1;
  if (m->c.window > 0 && m->P[layer] - m->c.window > m->lo[layer]) m->lo[layer] = m->P[layer] - m->c.window;
  return 0;
}

int ko_sink_state(const ko_model* m, int layer, int b, int32_t* pos, float* score, int32_t* count) {
  if (!m || layer < 0 || layer >= m->c.n_layers || b < 0 || b >= m->c.batch) return -1;
  const int nc = m->ncommit[layer * m->c.batch + b];
  const int64_t* cp = &m->cpos[((int64_t)layer * m->c.batch + b) * MAXSINK];
  const float* cs = &m->cscore[((int64_t)layer * m->c.batch + b) * MAXSINK];
  for (int i = 0; i < m->c.n_sink; ++i) {
    if (pos) pos[i] = i < nc ? (int32_t)cp[i] : -1;
    if (score) score[i] = i < nc ? cs[i] : 0.0f;
  }
  if (count) *count = nc;
  return 0;
}

/* committed sinks of (layer, b) that have been appended */
static int sinks_of(const ko_model* m, int layer, int b, int64_t* out) {
  const int nc = m->ncommit[layer * m->c.batch + b];
  const int64_t* cp = &m->cpos[((int64_t)layer * m->c.batch + b) * MAXSINK];
  int n = 0;
  for (int i = 0; i < nc; ++i)
    if (cp[i] < m->P[layer]) out[n++] = cp[i];
  return n;
}
static int is_sink(const int64_t* s, int ns, int64_t p) {
  for (int i = 0; i < ns; ++i)
    if (s[i] == p) return 1;
  return 0;
}

/* ---- quantization of one 32-token block of one stream ---- */

typedef struct {
  uint8_t kcode[G][MAXD], vcode[G][MAXD];
  uint16_t ks[MAXD], kz[MAXD];          /* KIVI K scale and zero; q2k: ks = block RMS */
  uint16_t vs[G][MAXD / 32], vz[G][MAXD / 32];
  float kn[G], vn[G];                    /* TurboQuant norms */
} Block;

/* Fast Walsh-Hadamard transform, stages len = 1, 2, ..., d/2 (TurboQuant spec, "Hadamard Transform
 * Detail"): each stage maps (u, v) = (x[i + j], x[i + j + len]) to (u + v, u - v). */
static void fwht32(float* x, int d) {
  for (int len = 1; len < d; len *= 2)
    for (int i = 0; i < d; i += 2 * len)
      for (int j = 0; j < len; ++j) {
        const float u = x[i + j], v = x[i + j + len];
        x[i + j] = u + v;
        x[i + j + len] = u - v;
      }
}
static void fwht64(double* x, int d) {
  for (int len = 1; len < d; len *= 2)
    for (int i = 0; i < d; i += 2 * len)
      for (int j = 0; j < len; ++j) {
        const double u = x[i + j], v = x[i + j + len];
        x[i + j] = u + v;
        x[i + j + len] = u - v;
      }
}

/* TurboQuant row: y = c_d * FWHT(sigma * x); n = sqrt(sumsq(y)); code = #{boundaries <= y / n}. */
static void tq_row(const ko_model* m, const float* x, const float* bnd, int bits, uint8_t* code, float* norm) {
  const int D = m->dp, Din = m->c.head_dim;  /* the row, zero-padded from Din to D channels */
  const float cd = (float)(1.0 / sqrt((double)D));
  float y[MAXD];
  for (int i = 0; i < D; ++i) y[i] = (i < Din ? x[i] : 0.0f) * m->signs[i];
  fwht32(y, D);
  for (int i = 0; i < D; ++i) y[i] = y[i] * cd;
  const float n = sqrtf(sumsq(y, D));
  const int nb = (1 << bits) - 1;
  for (int i = 0; i < D; ++i) {
    const float t = n > 0.0f ? y[i] / n : 0.0f;
    int u = 0;
    for (int j = 0; j < nb; ++j) u += t >= bnd[j];
    code[i] = (uint8_t)u;
  }
  *norm = n;
}

static void quantize_block(const ko_model* m, int layer, int b, int h, int64_t beta, Block* o) {
  const ko_config* c = &m->c;
  const int D = c->head_dim, ng = D / 32;
  const Rows* r = rows_of(m, layer, b, h);
  const int64_t P = m->P[layer], p0 = beta * G;
  int64_t s[MAXSINK];
  const int ns = sinks_of(m, layer, b, s);
  int calib[G];
  for (int t = 0; t < G; ++t) calib[t] = p0 + t < P && !is_sink(s, ns, p0 + t);
  memset(o, 0, sizeof(*o));
  if (c->fmt == 0) {
    /* K per channel over the block's calibration rows; V per row over 32-channel groups
     * (StreamingLLM + KIVI page, "Affine quantisation formula") */
    const float Lk = (float)((1 << c->k_bits) - 1), Lv = (float)((1 << c->v_bits) - 1);
    for (int ch = 0; ch < D; ++ch) {
      float mn = INFINITY, mx = -INFINITY;
      int has = 0;
      for (int t = 0; t < G; ++t)
        if (calib[t]) {
          const float x = r->k[(p0 + t) * D + ch];
          if (x < mn) mn = x;
          if (x > mx) mx = x;
          has = 1;
        }
      if (!has) mn = mx = 0.0f;
      mn = canon0(mn);
      mx = canon0(mx);
      float s32 = (mx - mn) / Lk;
      if (!(s32 >= EPS)) s32 = EPS;
      o->ks[ch] = f16_bits(s32);
      o->kz[ch] = f16_bits(mn);
      const float sv = f16_val(o->ks[ch]), zv = f16_val(o->kz[ch]);
      for (int t = 0; t < G; ++t)
        if (calib[t]) {
          float q = rintf((r->k[(p0 + t) * D + ch] - zv) / sv);
          if (q < 0.0f) q = 0.0f;
          if (q > Lk) q = Lk;
          o->kcode[t][ch] = (uint8_t)q;
        }
    }
    for (int t = 0; t < G; ++t) {
      if (!calib[t]) continue;
      for (int g = 0; g < ng; ++g) {
        const float* x = &r->v[(p0 + t) * D + 32 * g];
        float mn = x[0], mx = x[0];
        for (int i = 1; i < 32; ++i) {
          if (x[i] < mn) mn = x[i];
          if (x[i] > mx) mx = x[i];
        }
        mn = canon0(mn);
        mx = canon0(mx);
        float s32 = (mx - mn) / Lv;
        if (!(s32 >= EPS)) s32 = EPS;
        o->vs[t][g] = f16_bits(s32);
        o->vz[t][g] = f16_bits(mn);
        const float sv = f16_val(o->vs[t][g]), zv = f16_val(o->vz[t][g]);
        for (int i = 0; i < 32; ++i) {
          float q = rintf((x[i] - zv) / sv);
          if (q < 0.0f) q = 0.0f;
          if (q > Lv) q = Lv;
          o->vcode[t][32 * g + i] = (uint8_t)q;
        }
      }
    }
  } else if (c->fmt == 1) {
    /* q2k (q2k page, "Summary"): K code = #{Gaussian Lloyd-Max thresholds <= x / fp16(block RMS)};
     * V symmetric 4-bit, s = absmax / 7, u = clamp(rint(x / s), -8, 7) + 8 */
    int n = 0;
    for (int t = 0; t < G; ++t) n += calib[t];
    for (int ch = 0; ch < D; ++ch) {
      float ss = 0.0f;
      for (int t = 0; t < G; ++t)
        if (calib[t]) {
          const float x = r->k[(p0 + t) * D + ch];
          const float sq = x * x;
          ss = ss + sq;
        }
      float r32 = EPS;
      if (n > 0) {
        const float rr = sqrtf(ss / (float)n);
        r32 = rr >= EPS ? rr : EPS;
      }
      o->ks[ch] = f16_bits(r32);
      const float rv = f16_val(o->ks[ch]);
      for (int t = 0; t < G; ++t)
        if (calib[t]) {
          const float tt = r->k[(p0 + t) * D + ch] / rv;
          o->kcode[t][ch] = (uint8_t)((tt >= m->q2k_th[0]) + (tt >= m->q2k_th[1]) + (tt >= m->q2k_th[2]));
        }
    }
    for (int t = 0; t < G; ++t) {
      if (!calib[t]) continue;
      for (int g = 0; g < ng; ++g) {
        const float* x = &r->v[(p0 + t) * D + 32 * g];
        float am = fabsf(x[0]);
        for (int i = 1; i < 32; ++i)
          if (fabsf(x[i]) > am) am = fabsf(x[i]);
        am = canon0(am);
        float s32 = am / 7.0f;
        if (!(s32 >= EPS)) s32 = EPS;
        o->vs[t][g] = f16_bits(s32);
        const float sv = f16_val(o->vs[t][g]);
        for (int i = 0; i < 32; ++i) {
          float q = rintf(x[i] / sv);
          if (q < -8.0f) q = -8.0f;
          if (q > 7.0f) q = 7.0f;
          o->vcode[t][32 * g + i] = (uint8_t)(q + 8.0f);
        }
      }
    }
  } else {
    for (int t = 0; t < G; ++t) {
      if (!calib[t]) continue;
      tq_row(m, &r->k[(p0 + t) * D], m->kbnd, c->k_bits, o->kcode[t], &o->kn[t]);
      tq_row(m, &r->v[(p0 + t) * D], m->vbnd, c->v_bits, o->vcode[t], &o->vn[t]);
    }
  }
}

/* ---- packing in the documented storage format (include/kvq.h) ---- */

/* code k of a 32-bit little-endian word of b-bit codes sits at bit 16*(k%2) + b*(k/2) */
static void put_word_code(uint8_t* sec, int64_t seq, int b, uint32_t code) {
  const int per = 32 / b;
  const int64_t w = seq / per;
  const int k = (int)(seq % per);
  const int bit = 16 * (k % 2) + b * (k / 2);
  uint32_t word;
  memcpy(&word, sec + 4 * w, 4);
  word |= code << bit;
  memcpy(sec + 4 * w, &word, 4);
}
/* dense 3-bit stream: code i at bits [3i, 3i + 3), least significant bit first */
static void put_dense3(uint8_t* sec, int64_t i, uint32_t code) {
  for (int j = 0; j < 3; ++j)
    if ((code >> j) & 1u) sec[(3 * i + j) / 8] |= (uint8_t)(1u << ((3 * i + j) % 8));
}
static void put_code(uint8_t* sec, int64_t seq, int slot, uint32_t code) {
  if (slot == 3) put_dense3(sec, seq, code);
  else put_word_code(sec, seq, slot, code);
}
static void put_f16(uint8_t* p, uint16_t h) { memcpy(p, &h, 2); }

static void pack_record(const ko_model* m, const Block* o, uint8_t* rec) {
  const int D = m->dp, ng = D / 32;
  memset(rec, 0, m->rec);
  uint8_t* kc = rec;
  uint8_t* vc = rec + m->kc;
  uint8_t* km = rec + m->kc + m->vc;
  uint8_t* vm = km + m->km;
  for (int t = 0; t < G; ++t)
    for (int ch = 0; ch < D; ++ch) {
      if (m->kslot == 3) put_dense3(kc, (int64_t)t * D + ch, o->kcode[t][ch]);
      else put_word_code(kc + (int64_t)t * D * m->kslot / 8, ch, m->kslot, o->kcode[t][ch]);
    }
  /* V tile order: chunk 16*kg + i holds, at sequence index 8*mu + e, channel 16*mu + i of token
   * 16*(e/4) + 4*kg + e%4 */
  const int per_chunk = D / 2;
  for (int q = 0; q < 64; ++q) {
    const int kg = q / 16, i = q % 16;
    for (int s = 0; s < per_chunk; ++s) {
      const int mu = s / 8, e = s % 8;
      const int t = 16 * (e / 4) + 4 * kg + e % 4, ch = 16 * mu + i;
      if (m->vslot == 3) put_code(vc, (int64_t)q * per_chunk + s, 3, o->vcode[t][ch]);
      else put_code(vc + (int64_t)q * (D * m->vslot / 16), s, m->vslot, o->vcode[t][ch]);
    }
  }
  if (m->c.fmt == 0) {
    for (int ch = 0; ch < D; ++ch) {
      put_f16(km + 2 * ch, o->ks[ch]);
      put_f16(km + 2 * (D + ch), o->kz[ch]);
    }
    for (int t = 0; t < G; ++t)
      for (int g = 0; g < ng; ++g) {
        const int idx = (t / 2) * 2 * ng + 2 * g + t % 2;
        put_f16(vm + 2 * idx, o->vs[t][g]);
        put_f16(vm + 2 * (G * ng + idx), o->vz[t][g]);
      }
  } else if (m->c.fmt == 1) {
    for (int ch = 0; ch < D; ++ch) put_f16(km + 2 * ch, o->ks[ch]);
    for (int t = 0; t < G; ++t)
      for (int g = 0; g < ng; ++g) put_f16(vm + 2 * ((t / 2) * 2 * ng + 2 * g + t % 2), o->vs[t][g]);
  } else {
    memcpy(km, o->kn, 4 * G);
    memcpy(vm, o->vn, 4 * G);
  }
}

/* Block formats with fp16 input and residual >= 32 quantize a block once, when its last row arrives (KIVI
 * groups keys per channel over full groups of tokens; while a block is open all its rows are in the fp16
 * window, which serves every read of them): an open block's record holds zero bytes until then.  Otherwise
 * an open block's record holds its rows so far, re-quantized on every append. */
static int defers_open_block(const ko_config* c) { return c->fmt != 2 && !c->in_f32 && c->residual >= G; }

int ko_stream_image(ko_model* m, int layer, int b, int h, uint8_t* bulk, uint16_t* win_k, uint16_t* win_v,
                    uint16_t* sink_k, uint16_t* sink_v) {
  if (!m || layer < 0 || layer >= m->c.n_layers || b < 0 || b >= m->c.batch || h < 0 || h >= m->c.n_kv_heads)
    return -1;
  const int D = m->dp, Din = m->c.head_dim, R = m->c.residual;  /* fp16 rows stored padded to D */
  const int64_t P = m->P[layer];
  const Rows* r = rows_of(m, layer, b, h);
  if (bulk) {
    memset(bulk, 0, (size_t)m->cap_b * m->rec);
    if (P > 0) {
      Block* o = (Block*)malloc(sizeof(Block));
      if (!o) return -1;
      const int64_t last = (P - 1) / G;
      for (int64_t slot = 0; slot < m->cap_b && slot <= last; ++slot) {
        const int64_t beta = slot + m->cap_b * ((last - slot) / m->cap_b); /* the latest block in the slot */
        if (beta == last && P % G != 0 && defers_open_block(&m->c)) continue;  /* open block: zero bytes */
        quantize_block(m, layer, b, h, beta, o);
        pack_record(m, o, bulk + slot * m->rec);
      }
      free(o);
    }
  }
  for (int rho = 0; rho < R; ++rho) {
    const int64_t p = rho <= P - 1 ? rho + R * ((P - 1 - rho) / R) : -1;
    for (int ch = 0; ch < D; ++ch) {
      if (win_k) win_k[rho * D + ch] = p >= 0 && ch < Din ? f16_bits(r->k[p * Din + ch]) : 0;
      if (win_v) win_v[rho * D + ch] = p >= 0 && ch < Din ? f16_bits(r->v[p * Din + ch]) : 0;
    }
  }
  int64_t s[MAXSINK];
  const int ns = sinks_of(m, layer, b, s);
  for (int i = 0; i < m->c.n_sink; ++i)
    for (int ch = 0; ch < D; ++ch) {
      if (sink_k) sink_k[i * D + ch] = i < ns && ch < Din ? f16_bits(r->k[s[i] * Din + ch]) : 0;
      if (sink_v) sink_v[i * D + ch] = i < ns && ch < Din ? f16_bits(r->v[s[i] * Din + ch]) : 0;
    }
  return 0;
}

/* ---- values and attention ---- */

/* Read source of position p: 0 not valid, 1 sink, 2 window, 3 bulk. */
static int source_of(const ko_model* m, int layer, const int64_t* s, int ns, int64_t p) {
  const int64_t P = m->P[layer], lo = m->lo[layer];
  if (p < 0 || p >= P) return 0;
  if (is_sink(s, ns, p)) return 1;
  if (p < lo) return 0;
  return p >= P - m->c.residual ? 2 : 3;
}

/* Dequantized bulk row t of block o (which 0 = K, 1 = V): exact fp64 and the fp32 formula. */
static void bulk_row(const ko_model* m, const Block* o, int t, int which, double* x64, float* x32) {
  const int D = m->c.head_dim;
  const uint8_t* u = which ? o->vcode[t] : o->kcode[t];
  if (m->c.fmt == 0) {
    for (int ch = 0; ch < D; ++ch) {
      const uint16_t s = which ? o->vs[t][ch / 32] : o->ks[ch], z = which ? o->vz[t][ch / 32] : o->kz[ch];
      if (x64) x64[ch] = (double)u[ch] * (double)f16_val(s) + (double)f16_val(z);
      if (x32) {
        const float pr = (float)u[ch] * f16_val(s);
        x32[ch] = pr + f16_val(z);
      }
    }
  } else if (m->c.fmt == 1) {
    for (int ch = 0; ch < D; ++ch) {
      if (which) {
        const float s = f16_val(o->vs[t][ch / 32]);
        if (x64) x64[ch] = ((double)u[ch] - 8.0) * (double)s;
        if (x32) x32[ch] = ((float)u[ch] - 8.0f) * s;
      } else {
        const float rr = f16_val(o->ks[ch]);
        if (x64) x64[ch] = (double)m->q2k_lv[u[ch]] * (double)rr;
        if (x32) x32[ch] = m->q2k_lv[u[ch]] * rr;
      }
    }
  } else {
    /* R^T (n c[u]) = sigma * (FWHT(n c[u]) / sqrt(d)) (TurboQuant spec, "Step 2"; inverse rotation: the
     * transform first, then the signs) */
    const float* cen = which ? m->vcen : m->kcen;
    const float n = which ? o->vn[t] : o->kn[t];
    const int Dp = m->dp;  /* the inverse over every stored coordinate, then the first head_dim channels */
    if (x64) {
      double w[MAXD];
      for (int ch = 0; ch < Dp; ++ch) w[ch] = (double)n * (double)cen[u[ch]];
      fwht64(w, Dp);
      for (int ch = 0; ch < D; ++ch) x64[ch] = (double)m->signs[ch] * (w[ch] / sqrt((double)Dp));
    }
    if (x32) {
      const float cd = (float)(1.0 / sqrt((double)Dp));
      float w[MAXD];
      for (int ch = 0; ch < Dp; ++ch) w[ch] = n * cen[u[ch]];
      fwht32(w, Dp);
      for (int ch = 0; ch < D; ++ch) x32[ch] = m->signs[ch] * (w[ch] * cd);
    }
  }
}

int ko_values(ko_model* m, int layer, int b, int h, int which, const int64_t* pos, int n, double* out64,
              uint16_t* out16) {
  if (!m || layer < 0 || layer >= m->c.n_layers || b < 0 || b >= m->c.batch || h < 0 || h >= m->c.n_kv_heads)
    return -1;
  const int D = m->c.head_dim;
  int64_t s[MAXSINK];
  const int ns = sinks_of(m, layer, b, s);
  const Rows* r = rows_of(m, layer, b, h);
  Block* o = (Block*)malloc(sizeof(Block));
  if (!o) return -1;
  int64_t have = -1;
  for (int i = 0; i < n; ++i) {
    const int src = source_of(m, layer, s, ns, pos[i]);
    if (src == 0) {
      free(o);
      return -2;
    }
    if (src != 3) {
      const float* x = (which ? r->v : r->k) + pos[i] * D;
      for (int ch = 0; ch < D; ++ch) {
        const uint16_t hb = f16_bits(x[ch]);
        if (out64) out64[(int64_t)i * D + ch] = (double)f16_val(hb);
        if (out16) out16[(int64_t)i * D + ch] = hb;
      }
      continue;
    }
    const int64_t beta = pos[i] / G;
    if (beta != have) {
      quantize_block(m, layer, b, h, beta, o);
      have = beta;
    }
    float x32[MAXD];
    bulk_row(m, o, (int)(pos[i] % G), which, out64 ? out64 + (int64_t)i * D : NULL, x32);
    if (out16)
      for (int ch = 0; ch < D; ++ch) out16[(int64_t)i * D + ch] = f16_bits(x32[ch]);
  }
  free(o);
  return 0;
}

/* Values of every valid position of stream (layer, b, h) in position order, block by block. */
typedef struct {
  int64_t* pos;
  int n;
} Valid;

static Valid valid_positions(const ko_model* m, int layer, int b) {
  int64_t s[MAXSINK];
  const int ns = sinks_of(m, layer, b, s);
  const int64_t P = m->P[layer], lo = m->lo[layer];
  Valid v;
  v.pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(P - lo + ns + 1));
  v.n = 0;
  if (!v.pos) return v;
  /* committed sinks below lo, ascending, then every position of [lo, P) */
  for (int i = 0; i < ns; ++i)
    if (s[i] < lo) {
      int k = v.n++;
      while (k > 0 && v.pos[k - 1] > s[i]) {
        v.pos[k] = v.pos[k - 1];
        --k;
      }
      v.pos[k] = s[i];
    }
  for (int64_t p = lo; p < P; ++p) v.pos[v.n++] = p;
  return v;
}

/* RoPE on read: row x [D] turned by the exact angles idx * theta_c (rotate-half pairs). */
static void rope_turn(double* x, int D, int64_t idx, const float* theta) {
  const int h = D / 2;
  for (int f = 0; f < h; ++f) {
    const double a = (double)idx * (double)theta[f], cs = cos(a), sn = sin(a);
    const double x0 = x[f], x1 = x[f + h];
    x[f] = x0 * cs - x1 * sn;
    x[f + h] = x1 * cs + x0 * sn;
  }
}

/* One stream (b, g): scores of its r query heads over every valid position, then the weighted values. */
static int attend_stream(ko_model* m, int layer, int b, int g, const void* q, double alpha, double* out) {
  const ko_config* c = &m->c;
  const int D = c->head_dim, r = c->n_q_heads / c->n_kv_heads;
  Valid v = valid_positions(m, layer, b);
  if (!v.pos) return -1;
  int64_t s[MAXSINK];
  const int ns = sinks_of(m, layer, b, s);
  const Rows* rows = rows_of(m, layer, b, g);
  double* sc = (double*)malloc(sizeof(double) * (size_t)r * (v.n > 0 ? v.n : 1));
  Block* o = (Block*)malloc(sizeof(Block));
  if (!sc || !o) {
    free(sc);
    free(o);
    free(v.pos);
    return -1;
  }
  double qv[16][MAXD];
  for (int j = 0; j < r; ++j)
    for (int ch = 0; ch < D; ++ch) {
      const int64_t qi = ((int64_t)b * c->n_q_heads + (int64_t)g * r + j) * D + ch;
      qv[j][ch] = c->in_f32 ? (double)((const float*)q)[qi] : (double)f16_val(((const uint16_t*)q)[qi]);
    }
  float theta[MAXD / 2];
  if (c->rope) {  /* the query's index: valid positions before its own, P - 1 (the last valid one) */
    const double base = c->rope_base > 0.f ? (double)c->rope_base : 10000.0;
    for (int f = 0; f < D / 2; ++f) theta[f] = (float)pow(base, -2.0 * f / D);
    int64_t qidx = 0;
    while (qidx < v.n && v.pos[qidx] < m->P[layer] - 1) ++qidx;
    for (int j = 0; j < r; ++j) rope_turn(qv[j], D, qidx, theta);
  }
  for (int pass = 0; pass < 2; ++pass) {  /* pass 0: K and scores; pass 1: V and the output */
    int64_t have = -1;
    double acc[16][MAXD], wsum[16], mx[16];
    if (pass == 1) {
      for (int j = 0; j < r; ++j) {
        mx[j] = -INFINITY;
        for (int i = 0; i < v.n; ++i)
          if (sc[(int64_t)j * v.n + i] > mx[j]) mx[j] = sc[(int64_t)j * v.n + i];
        wsum[j] = 0.0;
        for (int ch = 0; ch < D; ++ch) acc[j][ch] = 0.0;
      }
    }
    for (int i = 0; i < v.n; ++i) {
      const int64_t p = v.pos[i];
      const int src = source_of(m, layer, s, ns, p);
      double x[MAXD];
      if (src != 3) {
        const float* xr = (pass ? rows->v : rows->k) + p * D;
        for (int ch = 0; ch < D; ++ch) x[ch] = (double)f16_val(f16_bits(xr[ch]));
      } else {
        if (p / G != have) {
          quantize_block(m, layer, b, g, p / G, o);
          have = p / G;
        }
        bulk_row(m, o, (int)(p % G), pass, x, NULL);
      }
      if (c->rope && pass == 0) rope_turn(x, D, i, theta);  /* row i of the ascending valid list has index i */
      for (int j = 0; j < r; ++j) {
        if (pass == 0) {
          double d = 0.0;
          for (int ch = 0; ch < D; ++ch) d += x[ch] * qv[j][ch];
          sc[(int64_t)j * v.n + i] = alpha * d;
        } else {
          const double w = exp(sc[(int64_t)j * v.n + i] - mx[j]);
          wsum[j] += w;
          for (int ch = 0; ch < D; ++ch) acc[j][ch] += w * x[ch];
        }
      }
    }
    if (pass == 1)
      for (int j = 0; j < r; ++j)
        for (int ch = 0; ch < D; ++ch)
          out[((int64_t)b * c->n_q_heads + (int64_t)g * r + j) * D + ch] = v.n > 0 ? acc[j][ch] / wsum[j] : 0.0;
  }
  free(sc);
  free(o);
  free(v.pos);
  return 0;
}

int ko_decode_attention(ko_model* m, int layer, const void* q, double scale, double* out, int threads) {
  if (!m || layer < 0 || layer >= m->c.n_layers || !q || !out || m->P[layer] == 0) return -1;
  const double alpha = scale > 0.0 ? scale : 1.0 / sqrt((double)m->c.head_dim);
  const int S = m->c.batch * m->c.n_kv_heads;
  int err = 0;
  (void)threads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1) reduction(| : err)
  for (int st = 0; st < S; ++st) err |= attend_stream(m, layer, st / m->c.n_kv_heads, st % m->c.n_kv_heads, q, alpha, out) != 0;
  return err ? -1 : 0;
}

/* ---- accounting (kivi_sink page, "How it works" 4; StreamingLLM + KIVI page, "Caveats") ---- */

int ko_account(const ko_model* m, int layer, int b, int64_t* out8) {
  if (!m || layer < 0 || layer >= m->c.n_layers || b < 0 || b >= m->c.batch) return -1;
  int64_t s[MAXSINK];
  const int ns = sinks_of(m, layer, b, s);
  const int64_t P = m->P[layer];
  int64_t n_s = 0, n_w = 0, n_q = 0, nblk = 0, last_blk = -1;
  for (int64_t p = 0; p < P; ++p) {
    const int src = source_of(m, layer, s, ns, p);
    if (src == 1) ++n_s;
    if (src == 2) ++n_w;
    if (src == 3) {
      ++n_q;
      if (p / G != last_blk) {  /* positions ascend: a new block index is a new block */
        ++nblk;
        last_blk = p / G;
      }
    }
  }
  const int64_t H = m->c.n_kv_heads, D = m->dp;  /* stored width */
  const int64_t meta = m->c.fmt == 2 ? n_q * 8 * H : nblk * m->km * H + n_q * (m->vm / G) * H;
  out8[0] = n_s + n_w + n_q;
  out8[1] = n_q;
  out8[2] = n_s;
  out8[3] = n_w;
  out8[4] = P;
  out8[5] = n_q * H * D * (m->kslot + m->vslot) / 8 + meta;
  out8[6] = n_s * H * D * 2 * 2;
  out8[7] = n_w * H * D * 2 * 2;
  return 0;
}
