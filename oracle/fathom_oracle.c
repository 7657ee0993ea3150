/*
 * fathom_oracle.c — plain CPU oracle of the Fathom key scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  The GPU library
 * shares no code, header, table or helper with it; the two meet only through
 * the seeded input generator and the arrays each side produces.
 *
 * Method: "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
 * Caches" (papers.paperslantern.ai/papers/2609.17652) and its review at
 * jaehun.me/en/posts/paper-2609-17652 (which restores the equations the first
 * page lost).  Each function names the passage it follows.
 *
 * Written for clarity, not speed: no blocking, no fusion, no SIMD.  Floating
 * point is fp64 except where the fp32 evaluation order of the scan is
 * reproduced on purpose (fo_scan_ref32), so that top-k decisions are taken in
 * the same precision as the kernel.  Build: gcc -O2 -ffp-contract=off
 * (-fopenmp optional; threads only split independent groups/rows).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define FO_PLANES 4
#define FO_BLOCK 64

/* ------------------------------------------------------------------------ */
/* binary16 helpers (IEEE 754-2008 binary16, written from the format)       */
/* ------------------------------------------------------------------------ */

/* Every finite binary16 value is an integer multiple of 2^-24.  Return that
 * integer (exact in int64: |value| <= 65504 = 2047 * 2^5). */
static int64_t f16_units(uint16_t h) {
  int e = (h >> 10) & 0x1f;
  int64_t m = h & 0x3ff;
  int64_t u = (e == 0) ? m : ((m | 0x400) << (e - 1));
  return (h & 0x8000) ? -u : u;
}

static int f16_is_finite(uint16_t h) { return ((h >> 10) & 0x1f) != 0x1f; }

double fo_f16_to_f64(uint16_t h) {
  if (!f16_is_finite(h)) return (h & 0x3ff) ? NAN : ((h & 0x8000) ? -INFINITY : INFINITY);
  return ldexp((double)f16_units(h), -24);
}

/* ------------------------------------------------------------------------ */
/* Encode: §3.2 "Bit-Plane K Cache"                                          */
/* ------------------------------------------------------------------------ */

/* 4-bit code of one key value.  §3.2: block maximum a, cell width s = a/8,
 * code = floor(k/s) + 8 so that code 8 is zero and the MSB is the sign; the
 * Appendix A codes (4,12,9,14,0,3) for (-0.2,0.3,0.1,0.4,-0.5,-0.3) at a=0.5
 * fix floor.  k = +a falls outside [-a, a) and is clamped to 15.  With both k
 * and a counted in units of 2^-24, floor(k/s) = floor(8K/A) in exact integer
 * arithmetic.  a = 0 (all-zero block) gives code 8. */
static int fo_code(int64_t K, int64_t A) {
  if (A == 0) return 8;
  int64_t num = 8 * K;
  int64_t q = num / A;              /* C division truncates toward zero */
  if ((num % A != 0) && (num < 0)) q -= 1; /* -> floor */
  int64_t c = q + 8;
  if (c < 0) c = 0;
  if (c > 15) c = 15;
  return (int)c;
}

/* K [groups][n][d] fp16 bits -> planes [groups][d][4][nb_store] and scales
 * [groups][d][nb_store] (fp16 bits of a), blocks written at slot
 * block_offset + b.  Token i of a block goes to bit i of the plane word; bit p
 * of the code (p = 0 the MSB) goes to plane p (§3.2).  Returns the number of
 * blocks that held a non-finite value. */
int64_t fo_encode(const uint16_t* k, int64_t groups, int64_t n, int d,
                  int64_t nb_store, int64_t block_offset, uint64_t* planes,
                  uint16_t* scales, int nthreads) {
  int64_t nb = n / FO_BLOCK;
  int64_t bad = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) reduction(+ : bad) num_threads(nthreads > 0 ? nthreads : 1)
#endif
  for (int64_t g = 0; g < groups; ++g) {
    for (int64_t b = 0; b < nb; ++b) {
      for (int j = 0; j < d; ++j) {
        uint16_t amax_bits = 0;
        int64_t amax = 0;
        int nonfinite = 0;
        for (int i = 0; i < FO_BLOCK; ++i) {
          uint16_t h = k[(g * n + b * FO_BLOCK + i) * d + j];
          if (!f16_is_finite(h)) { nonfinite = 1; continue; }
          int64_t u = llabs(f16_units(h));
          if (u > amax) { amax = u; amax_bits = (uint16_t)(h & 0x7fff); }
        }
        if (nonfinite) bad++;
        uint64_t w[FO_PLANES] = {0, 0, 0, 0};
        for (int i = 0; i < FO_BLOCK; ++i) {
          uint16_t h = k[(g * n + b * FO_BLOCK + i) * d + j];
          int c = f16_is_finite(h) ? fo_code(f16_units(h), amax) : 8;
          for (int p = 0; p < FO_PLANES; ++p)
            if ((c >> (3 - p)) & 1) w[p] |= (uint64_t)1 << i;
        }
        int64_t slot = block_offset + b;
        for (int p = 0; p < FO_PLANES; ++p)
          planes[((g * d + j) * FO_PLANES + p) * nb_store + slot] = w[p];
        scales[(g * d + j) * nb_store + slot] = amax_bits;
      }
    }
  }
  (void)nthreads;
  return bad;
}

/* Prefix code of depth t read back from the planes: c' = c >> (4 - t)
 * (§3.2: the first t planes are the top t bits of the code). */
static int fo_prefix_code(const uint64_t* planes, int64_t nb_store, int64_t gj,
                          int64_t blk, int i, int t) {
  int c = 0;
  for (int p = 0; p < t; ++p)
    c = 2 * c + (int)((planes[(gj * FO_PLANES + p) * nb_store + blk] >> i) & 1);
  return c;
}

/* Dequantized prefix value (§3.2): (c' + 0.5 - 2^(t-1)) * a / 2^(t-1), in
 * fp64 (exact: at most 15 significant bits).  t = 0 gives 0. */
double fo_dequant(uint16_t a_bits, int cprefix, int t) {
  if (t == 0) return 0.0;
  double a = fo_f16_to_f64(a_bits);
  return ((double)cprefix + 0.5 - ldexp(1.0, t - 1)) * a / ldexp(1.0, t - 1);
}

/* Decode every token of planes/scales at depth t into fp64 (test helper). */
void fo_decode(const uint64_t* planes, const uint16_t* scales, int64_t groups,
               int64_t n, int d, int64_t nb_store, int t, double* out) {
  int64_t nb = n / FO_BLOCK;
  for (int64_t g = 0; g < groups; ++g)
    for (int64_t b = 0; b < nb; ++b)
      for (int j = 0; j < d; ++j) {
        int64_t gj = g * d + j;
        uint16_t a = scales[gj * nb_store + b];
        for (int i = 0; i < FO_BLOCK; ++i)
          out[(g * n + b * FO_BLOCK + i) * d + j] =
              fo_dequant(a, fo_prefix_code(planes, nb_store, gj, b, i, t), t);
      }
}

/* ------------------------------------------------------------------------ */
/* Plan: §3.3 "Per-Query Read Depth", Eq. 4, Appendix A                     */
/* ------------------------------------------------------------------------ */

/* Importance of channel j for a query group (§3.3):
 *   g_j = sum_h (q_j^(h))^2 * Var(k_j),
 * in fp64, heads summed in order h = 0..G-1, then one multiply. */
void fo_importance(const float* q, const float* var, int G, int d, double* g) {
  for (int j = 0; j < d; ++j) {
    double s = 0.0;
    for (int h = 0; h < G; ++h) {
      double x = (double)q[h * d + j];
      s = s + x * x;
    }
    g[j] = s * (double)var[j];
  }
}

/* Depth of one channel at water line theta (Eq. 4): t = clip(round(log4(g /
 * theta)), 0, 4).  round(x) >= m  <=>  x >= m - 1/2 (halves rounded up), and
 * log4(g/theta) >= m - 1/2  <=>  g >= 2^(2m-1) * theta, so t counts the m in
 * 1..4 that pass; the power-of-two product is exact in fp64.  g = 0 -> 0. */
int fo_depth_one(double g, double theta) {
  if (!(g > 0.0)) return 0;
  int t = 0;
  for (int m = 1; m <= 4; ++m)
    if (g >= ldexp(theta, 2 * m - 1)) t++;
  return t;
}

int fo_depths_at(const double* g, int d, double theta, uint8_t* t) {
  int sum = 0;
  for (int j = 0; j < d; ++j) {
    int tj = fo_depth_one(g[j], theta);
    if (t) t[j] = (uint8_t)tj;
    sum += tj;
  }
  return sum;
}

/* Water line by log-bisection (§3.3; Appendix A: geometric-mean midpoints,
 * 30 steps): keep hi feasible (sum t <= B) and lo infeasible; mid =
 * sqrt(lo * hi); return the depths at hi.  The caller supplies the bracket. */
void fo_bisect(const double* g, int d, int B, double lo, double hi, int steps,
               uint8_t* t, double* theta, int* bits) {
  for (int s = 0; s < steps; ++s) {
    double mid = sqrt(lo * hi);
    if (fo_depths_at(g, d, mid, NULL) <= B) hi = mid;
    else lo = mid;
  }
  int used = fo_depths_at(g, d, hi, t);
  if (theta) *theta = hi;
  if (bits) *bits = used;
}

/* Plan of one group with the general bracket [min_{g>0} g / 256, max g]:
 * at max g every channel has t = 0 (feasible), at min g / 256 every g > 0 has
 * t = 4 (infeasible unless the budget covers all of them, handled first). */
void fo_plan_group(const double* g, int d, int B, uint8_t* t, double* theta,
                   int* bits) {
  double gmax = 0.0, gmin = 0.0;
  int npos = 0;
  for (int j = 0; j < d; ++j) {
    if (g[j] > 0.0) {
      if (npos == 0 || g[j] < gmin) gmin = g[j];
      if (g[j] > gmax) gmax = g[j];
      npos++;
    }
  }
  if (npos == 0 || B == 0) {
    for (int j = 0; j < d; ++j) t[j] = 0;
    *theta = gmax;
    *bits = 0;
    return;
  }
  if (B >= 4 * npos) {
    int used = 0;
    for (int j = 0; j < d; ++j) { t[j] = (g[j] > 0.0) ? 4 : 0; used += t[j]; }
    *theta = gmin / 256.0;
    *bits = used;
    return;
  }
  fo_bisect(g, d, B, gmin / 256.0, gmax, 30, t, theta, bits);
}

/* q [groups][G][d], var [groups][d] -> depths [groups][d] (+ theta, bits). */
void fo_plan(const float* q, const float* var, int64_t groups, int G, int d,
             int B, uint8_t* depths, double* theta, int* bits, int nthreads) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
  for (int64_t gi = 0; gi < groups; ++gi) {
    double* g = (double*)malloc(sizeof(double) * (size_t)d);
    double th;
    int used;
    fo_importance(q + gi * G * d, var + gi * d, G, d, g);
    fo_plan_group(g, d, B, depths + gi * d, &th, &used);
    if (theta) theta[gi] = th;
    if (bits) bits[gi] = used;
    free(g);
  }
  (void)nthreads;
}

/* ------------------------------------------------------------------------ */
/* Scan: §3.2 prefix dequantization, §3.3 active channels                    */
/* ------------------------------------------------------------------------ */

/* Depth values above 4 read as 4 (a channel has four planes). */
static int fo_depth_clamped(uint8_t t) { return t > FO_PLANES ? FO_PLANES : (int)t; }

/* Plain definition in fp64: S_hi = sum_{j : t_j > 0} q_hj * khat_ij with the
 * prefix value of §3.2 (each product is exact in fp64).  Also returns
 * l1_hi = sum_j |q_hj * khat_ij|, the magnitude the tolerance is relative to.
 * Per token the prefix values of the active channels are read back first, then
 * each head's sum runs over them by ascending channel.  Threads split the
 * (group, block) pairs, which are independent.  Output [groups][G][n]. */
void fo_scan_f64(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                 const uint8_t* depths, const float* q, int64_t groups, int G,
                 int d, int64_t n, double* scores, double* l1, int nthreads) {
  int64_t nb = n / FO_BLOCK;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
  for (int64_t gb = 0; gb < groups * nb; ++gb) {
    int64_t g = gb / nb, b = gb % nb;
    const uint8_t* t = depths + g * d;
    double* kh = (double*)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < FO_BLOCK; ++i) {
      for (int j = 0; j < d; ++j) {
        int tj = fo_depth_clamped(t[j]);
        int64_t gj = g * d + j;
        kh[j] = tj == 0 ? 0.0
                        : fo_dequant(scales[gj * nb_store + b],
                                     fo_prefix_code(planes, nb_store, gj, b, i, tj), tj);
      }
      for (int h = 0; h < G; ++h) {
        double s = 0.0, m = 0.0;
        for (int j = 0; j < d; ++j) {
          if (fo_depth_clamped(t[j]) == 0) continue;
          double prod = (double)q[(g * G + h) * d + j] * kh[j];
          s += prod;
          m += fabs(prod);
        }
        int64_t o = (g * G + h) * n + b * FO_BLOCK + i;
        scores[o] = s;
        if (l1) l1[o] = m;
      }
    }
    free(kh);
  }
  (void)nthreads;
}

/* The same scores in the fp32 order the GPU kernel uses (the pages fix no
 * fp32 order; this one is stated in fathom.h).  Splitting the §3.2 value as
 *   khat = a * (c' * 2^(1-t) + 2^-t - 1)
 * gives, per block b, head h and token i of the block,
 *   U  = +0;  for each active j: U = fmaf(w_hj, m_ij, U),
 *             w_hj = q_hj * 2^(11-t_j), m_ij = a_bj * c'_ij * 2^-10 (both exact)
 *   o  = +0;  for each active j: o = fmaf(e_hj, a_bj, o),
 *             e_hj = fl32(q_hj * (2^-t_j - 1))
 *   S  = fl32(U + o),
 * where "each active j" visits the channels with t_j = 4 first, then 3, 2
 * and 1, ascending j within one depth.  Depth values above 4 read as 4.
 * Threads split the (group, block) pairs.  Output [groups][G][n]. */
void fo_scan_ref32(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                   const uint8_t* depths, const float* q, int64_t groups, int G,
                   int d, int64_t n, float* scores, int nthreads) {
  int64_t nb = n / FO_BLOCK;
  /* The visiting order of every group: by depth 4, 3, 2, 1, then by channel. */
  int* order = (int*)malloc(sizeof(int) * (size_t)(groups * d));
  int* nact = (int*)malloc(sizeof(int) * (size_t)groups);
  for (int64_t g = 0; g < groups; ++g) {
    nact[g] = 0;
    for (int depth = FO_PLANES; depth >= 1; --depth)
      for (int j = 0; j < d; ++j)
        if (fo_depth_clamped(depths[g * d + j]) == depth) order[g * d + nact[g]++] = j;
  }
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
  for (int64_t gb = 0; gb < groups * nb; ++gb) {
    int64_t g = gb / nb, b = gb % nb;
    const int* og = order + g * d;
    for (int h = 0; h < G; ++h) {
      const float* qh = q + (g * G + h) * d;
      float o = 0.0f;
      for (int k = 0; k < nact[g]; ++k) {
        int j = og[k];
        int t = fo_depth_clamped(depths[g * d + j]);
        float a = (float)fo_f16_to_f64(scales[(g * d + j) * nb_store + b]);
        float e = qh[j] * (ldexpf(1.0f, -t) - 1.0f);
        o = fmaf(e, a, o);
      }
      for (int i = 0; i < FO_BLOCK; ++i) {
        float u = 0.0f;
        for (int k = 0; k < nact[g]; ++k) {
          int j = og[k];
          int t = fo_depth_clamped(depths[g * d + j]);
          int64_t gj = g * d + j;
          float a = (float)fo_f16_to_f64(scales[gj * nb_store + b]);
          int c = fo_prefix_code(planes, nb_store, gj, b, i, t);
          float w = ldexpf(qh[j], 11 - t);
          float m = ldexpf(a * (float)c, -10);
          u = fmaf(w, m, u);
        }
        scores[(g * G + h) * n + b * FO_BLOCK + i] = u + o;
      }
    }
  }
  free(order);
  free(nact);
  (void)nthreads;
}

/* ------------------------------------------------------------------------ */
/* Top-k: per query head (§2: top-k by the method's score, per head)         */
/* ------------------------------------------------------------------------ */

typedef struct { float s; int32_t i; } fo_pair;

/* Total order of the selection: score descending, then index ascending
 * (-0 and +0 compare equal as floats). */
static int fo_cmp_rank(const void* x, const void* y) {
  const fo_pair* a = (const fo_pair*)x;
  const fo_pair* b = (const fo_pair*)y;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->i < b->i) ? -1 : (a->i > b->i);
}

static int fo_cmp_int(const void* x, const void* y) {
  int32_t a = *(const int32_t*)x, b = *(const int32_t*)y;
  return (a < b) ? -1 : (a > b);
}

/* Full sort of each row by the order above, first k taken, returned in
 * ascending index order.  scores [rows][n] -> idx [rows][k]. */
void fo_topk(const float* scores, int64_t rows, int64_t n, int k, int32_t* idx,
             int nthreads) {
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
#endif
  for (int64_t r = 0; r < rows; ++r) {
    fo_pair* v = (fo_pair*)malloc(sizeof(fo_pair) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) { v[i].s = scores[r * n + i]; v[i].i = (int32_t)i; }
    qsort(v, (size_t)n, sizeof(fo_pair), fo_cmp_rank);
    for (int i = 0; i < k; ++i) idx[r * k + i] = v[i].i;
    qsort(idx + r * k, (size_t)k, sizeof(int32_t), fo_cmp_int);
    free(v);
  }
  (void)nthreads;
}

/* ------------------------------------------------------------------------ */
/* KLT-rotated store (§3.5; calibration-free fit in Appendix D)              */
/* ------------------------------------------------------------------------ */

/* Rotated key coordinates, the store's input in the rotated variant: the
 * planes hold codes of (k - mu) V instead of k.  For each token i and output
 * coordinate j, in fp32:
 *   d_c  = fl32(k_ic - mu_c)                      (k_ic binary16, exact in fp32)
 *   acc  = +0;  for c = 0 .. d-1 ascending: acc = fmaf(d_c, V[c][j], acc)
 * k [groups][n][d] binary16 bits, mu [groups][d], V [groups][d][d] (row c,
 * column j), out [groups][n][d] fp32 (the caller rounds it to binary16,
 * nearest-even). */
void fo_klt_rotate(const uint16_t* k, const float* mu, const float* V, int64_t groups,
                   int64_t n, int d, float* out, int nthreads) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
  for (int64_t gi = 0; gi < groups * n; ++gi) {
    int64_t g = gi / n;
    const uint16_t* row = k + gi * d;
    const float* m = mu + g * d;
    const float* Vg = V + g * (int64_t)d * d;
    float* dst = out + gi * d;
    float* dc = (float*)malloc(sizeof(float) * (size_t)d);
    for (int c = 0; c < d; ++c) dc[c] = (float)fo_f16_to_f64(row[c]) - m[c];
    for (int j = 0; j < d; ++j) {
      float acc = 0.0f;
      for (int c = 0; c < d; ++c) acc = fmaf(dc[c], Vg[(int64_t)c * d + j], acc);
      dst[j] = acc;
    }
    free(dc);
  }
  (void)nthreads;
}

/* Rotated queries q V, the same fold without a mean:
 *   acc = +0;  for c ascending: acc = fmaf(q_hc, V[c][j], acc).
 * q [groups][G][d] fp32 -> out [groups][G][d] fp32. */
void fo_klt_rotate_q(const float* q, const float* V, int64_t groups, int G, int d, float* out) {
  for (int64_t g = 0; g < groups; ++g)
    for (int h = 0; h < G; ++h) {
      const float* qh = q + (g * G + h) * d;
      const float* Vg = V + g * (int64_t)d * d;
      for (int j = 0; j < d; ++j) {
        float acc = 0.0f;
        for (int c = 0; c < d; ++c) acc = fmaf(qh[c], Vg[(int64_t)c * d + j], acc);
        out[(g * G + h) * d + j] = acc;
      }
    }
}

int fo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
