/*
 * fa_oracle.c -- CPU oracle for frame-aligned attention.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the CPU
 * baseline of bench.py; never by the product library.  It shares no code,
 * header or table with the HIP path.
 *
 * Plain definition, row by row: decide visibility key by key with the
 * pages' rule (see fa_oracle.h for the cited passages), then a masked
 * softmax accumulated in double.  No tiling, no block map, no ring buffer:
 * past target frames are held in one flat array indexed by absolute frame.
 * OpenMP only spreads independent rows over threads.
 */
#include "fa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int fa_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static int ref_total(const fa_oracle_problem *p) {
  int r, n = 0;
  for (r = 0; r < p->n_ref; ++r) n += p->ref_tokens[r];
  return n;
}

static int rows_of(const fa_oracle_problem *p, int kind) {
  return kind == FAO_REF ? ref_total(p) : p->C * p->T;
}

/* Lowest absolute target frame a target row may read.  Block-wise causal
 * streaming: every row of the chunk sees the same history, the last
 * `window` frames before the chunk (all of it for window = -1). */
static int history_lo(const fa_oracle_problem *p) {
  if (p->window < 0) return 0;
  return p->cs - p->window > 0 ? p->cs - p->window : 0;
}

/* The visibility rule.  qframe / kframe are absolute frame indices; for a
 * reference key kframe carries the image index instead. */
static int sees(const fa_oracle_problem *p, int qkind, int qframe, int kkind, int kframe) {
  if (qkind == FAO_TGT) {
    if (kkind == FAO_TGT)
      return (kframe >= history_lo(p) || kframe < p->sink) && kframe < p->cs + p->C;
    if (kkind == FAO_SRC) return kframe == qframe;
    return qframe >= p->ref_t0[kframe];
  }
  if (qkind == FAO_SRC) {
    if (kkind == FAO_SRC) return kframe == qframe;
    if (kkind == FAO_REF) return qframe >= p->ref_t0[kframe];
    return 0;
  }
  /* reference rows: reference tokens only, every image */
  return kkind == FAO_REF;
}

static const float *query_ptr(const fa_oracle_problem *p, int kind) {
  return kind == FAO_TGT ? p->q_tgt : kind == FAO_SRC ? p->q_src : p->q_ref;
}

/* Calls fn(key pointer, value pointer, ctx) for every visible key of one row. */
typedef void (*key_fn)(const float *k, const float *v, void *ctx);

static int for_visible_keys(const fa_oracle_problem *p, int kind, int row, int h, key_fn fn,
                            void *ctx) {
  const int T = p->T, H = p->H, D = p->D;
  const int qframe = kind == FAO_REF ? -1 : p->cs + row / T;
  int g, t, r;
  /* target keys, absolute frames 0 .. cs+C-1 */
  for (g = 0; g < p->cs + p->C; ++g) {
    if (!sees(p, kind, qframe, FAO_TGT, g)) continue;
    if (g < p->hist_first) return -1; /* visible but not supplied */
    for (t = 0; t < T; ++t) {
      const long tok = (long)(g - p->hist_first) * T + t;
      fn(p->k_hist + (tok * H + h) * D, p->v_hist + (tok * H + h) * D, ctx);
    }
  }
  /* source keys, absolute frames cs .. cs+C-1 */
  for (g = p->cs; g < p->cs + p->C; ++g) {
    if (!sees(p, kind, qframe, FAO_SRC, g)) continue;
    for (t = 0; t < T; ++t) {
      const long tok = (long)(g - p->cs) * T + t;
      fn(p->k_src + (tok * H + h) * D, p->v_src + (tok * H + h) * D, ctx);
    }
  }
  /* reference keys, image by image */
  {
    long base = 0;
    for (r = 0; r < p->n_ref; ++r) {
      if (sees(p, kind, qframe, FAO_REF, r)) {
        for (t = 0; t < p->ref_tokens[r]; ++t) {
          const long tok = base + t;
          fn(p->k_ref + (tok * H + h) * D, p->v_ref + (tok * H + h) * D, ctx);
        }
      }
      base += p->ref_tokens[r];
    }
  }
  return 0;
}

/* Pass 1: the row maximum of the scores. */
typedef struct {
  const float *q;
  int D;
  double scale, m;
  long n;
} max_ctx;

static double score(const float *q, const float *k, int D, double scale) {
  double acc = 0.0;
  int d;
  for (d = 0; d < D; ++d) acc += (double)q[d] * (double)k[d];
  return scale * acc;
}

static void max_fn(const float *k, const float *v, void *vctx) {
  max_ctx *c = (max_ctx *)vctx;
  const double s = score(c->q, k, c->D, c->scale);
  (void)v;
  if (c->n == 0 || s > c->m) c->m = s;
  c->n++;
}

/* Pass 2: l = sum exp(s - m) and the weighted sum of values. */
typedef struct {
  const float *q;
  int D;
  double scale, m, l;
  double *acc;
} sum_ctx;

static void sum_fn(const float *k, const float *v, void *vctx) {
  sum_ctx *c = (sum_ctx *)vctx;
  const double w = exp(score(c->q, k, c->D, c->scale) - c->m);
  int d;
  c->l += w;
  for (d = 0; d < c->D; ++d) c->acc[d] += w * (double)v[d];
}

static int one_row(const fa_oracle_problem *p, int kind, int h, int row, float *o, float *lse) {
  const int D = p->D;
  const float *q;
  max_ctx mc;
  sum_ctx sc;
  double acc[1024];
  int d, rc;
  if (D > 1024) return -2;
  if (kind < 0 || kind > 2 || h < 0 || h >= p->H || row < 0 || row >= rows_of(p, kind)) return -2;
  q = query_ptr(p, kind) + ((long)row * p->H + h) * D;
  mc.q = q; mc.D = D; mc.scale = p->scale; mc.m = 0.0; mc.n = 0;
  rc = for_visible_keys(p, kind, row, h, max_fn, &mc);
  if (rc) return rc;
  if (mc.n == 0) {
    for (d = 0; d < D; ++d) o[d] = 0.0f;
    *lse = -INFINITY;
    return 0;
  }
  memset(acc, 0, sizeof(double) * D);
  sc.q = q; sc.D = D; sc.scale = p->scale; sc.m = mc.m; sc.l = 0.0; sc.acc = acc;
  for_visible_keys(p, kind, row, h, sum_fn, &sc);
  for (d = 0; d < D; ++d) o[d] = (float)(acc[d] / sc.l);
  *lse = (float)(mc.m + log(sc.l));
  return 0;
}

static int check(const fa_oracle_problem *p) {
  int r;
  if (p->T <= 0 || p->C < 0 || p->cs < 0 || p->H <= 0 || p->D <= 0 || p->D > 1024) return -2;
  if (p->n_ref < 0 || (p->n_ref > 0 && (!p->ref_tokens || !p->ref_t0))) return -2;
  for (r = 0; r < p->n_ref; ++r)
    if (p->ref_tokens[r] < 0) return -2;
  if (p->hist_first < 0 || p->hist_first > p->cs) return -2;
  return 0;
}

int fa_oracle_attn(const fa_oracle_problem *p, int kind_mask, float *o_tgt, float *lse_tgt,
                   float *o_src, float *lse_src, float *o_ref, float *lse_ref) {
  int kind, err = check(p);
  if (err) return err;
  for (kind = 0; kind < 3; ++kind) {
    float *o = kind == FAO_TGT ? o_tgt : kind == FAO_SRC ? o_src : o_ref;
    float *lse = kind == FAO_TGT ? lse_tgt : kind == FAO_SRC ? lse_src : lse_ref;
    const int rows = rows_of(p, kind);
    const long work = (long)rows * p->H;
    long i;
    if (!(kind_mask & (1 << kind)) || !o || !lse) continue;
#pragma omp parallel for schedule(dynamic, 16) reduction(min : err)
    for (i = 0; i < work; ++i) {
      const int h = (int)(i / rows), row = (int)(i % rows);
      const int rc = one_row(p, kind, h, row, o + ((long)row * p->H + h) * p->D,
                             lse + (long)h * rows + row);
      if (rc < err) err = rc;
    }
    if (err) return err;
  }
  return 0;
}

int fa_oracle_attn_rows(const fa_oracle_problem *p, int n, const int *kind, const int *head,
                        const int *row, float *o, float *lse) {
  int i, err = check(p);
  if (err) return err;
  for (i = 0; i < n; ++i)
    if (kind[i] < 0 || kind[i] > 2 || head[i] < 0 || head[i] >= p->H || row[i] < 0 ||
        row[i] >= rows_of(p, kind[i]))
      return -2;
#pragma omp parallel for schedule(dynamic, 4) reduction(min : err)
  for (i = 0; i < n; ++i) {
    const int rc = one_row(p, kind[i], head[i], row[i], o + (long)i * p->D, lse + i);
    if (rc < err) err = rc;
  }
  return err;
}

static void count_fn(const float *k, const float *v, void *vctx) {
  (void)k; (void)v;
  (*(long *)vctx)++;
}

long fa_oracle_count(const fa_oracle_problem *p, int kind, int row) {
  long n = 0;
  if (check(p)) return -2;
  if (for_visible_keys(p, kind, row, 0, count_fn, &n)) return -1;
  return n;
}

/* ---- quantiser ---------------------------------------------------------- */

static void quant_blocks(const float *x, int N, int H, int D, const float *mean, float qmax,
                         int is_fp8, void *codes, float *scales) {
  const int nblk = (N + 127) / 128;
  int h, b;
  for (h = 0; h < H; ++h) {
    for (b = 0; b < nblk; ++b) {
      const int t0 = b * 128, t1 = (b + 1) * 128 < N ? (b + 1) * 128 : N;
      float absmax = 0.0f, scale, inv;
      int t, d;
      for (t = t0; t < t1; ++t)
        for (d = 0; d < D; ++d) {
          const float v = x[((long)t * H + h) * D + d] - (mean ? mean[h * D + d] : 0.0f);
          const float a = fabsf(v);
          if (a > absmax) absmax = a;
        }
      if (is_fp8) {
        /* power-of-two scale: absmax = f * 2^k with f in [0.5, 1); 448 * 2^e >= absmax holds
         * from e = k - 9 on when f <= 448/512, else from e = k - 8 */
        int k, e;
        const float f = frexpf(absmax, &k);
        e = k - 9 + (f > 0.875f ? 1 : 0);
        if (e < -126) e = -126;
        scale = absmax > 0.0f ? ldexpf(1.0f, e) : 0.0f;
        inv = absmax > 0.0f ? ldexpf(1.0f, -e) : 0.0f;
      } else {
        scale = absmax / qmax;
        inv = absmax > 0.0f ? qmax / absmax : 0.0f;
      }
      scales[(long)h * nblk + b] = scale;
      for (t = t0; t < t1; ++t)
        for (d = 0; d < D; ++d) {
          const long idx = ((long)t * H + h) * D + d;
          const float v = x[idx] - (mean ? mean[h * D + d] : 0.0f);
          const float y = v * inv;
          if (is_fp8) {
            ((uint8_t *)codes)[idx] = fa_oracle_e4m3_encode(y);
          } else {
            float r = nearbyintf(y); /* default rounding mode: nearest, ties to even */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            ((int8_t *)codes)[idx] = (int8_t)r;
          }
        }
    }
  }
}

void fa_oracle_quant_int8(const float *x, int N, int H, int D, const float *mean, int8_t *codes,
                          float *scales) {
  quant_blocks(x, N, H, D, mean, 127.0f, 0, codes, scales);
}

void fa_oracle_quant_e4m3(const float *x, int N, int H, int D, const float *mean, uint8_t *codes,
                          float *scales) {
  quant_blocks(x, N, H, D, mean, 0.0f, 1, codes, scales);
}

void fa_oracle_quant_int8_2d(const float *x, int rows, int cols, int br, int bc, int8_t *codes,
                             float *scales) {
  const int nbr = (rows + br - 1) / br, nbc = (cols + bc - 1) / bc;
  int bi, bj, i, j;
  for (bi = 0; bi < nbr; ++bi)
    for (bj = 0; bj < nbc; ++bj) {
      const int i0 = bi * br, i1 = i0 + br < rows ? i0 + br : rows;
      const int j0 = bj * bc, j1 = j0 + bc < cols ? j0 + bc : cols;
      float absmax = 0.0f, inv;
      for (i = i0; i < i1; ++i)
        for (j = j0; j < j1; ++j) {
          const float a = fabsf(x[(long)i * cols + j]);
          if (a > absmax) absmax = a;
        }
      scales[(long)bi * nbc + bj] = absmax / 127.0f;
      inv = absmax > 0.0f ? 127.0f / absmax : 0.0f;
      for (i = i0; i < i1; ++i)
        for (j = j0; j < j1; ++j) {
          float r = nearbyintf(x[(long)i * cols + j] * inv); /* ties to even */
          if (r > 127.0f) r = 127.0f;
          if (r < -127.0f) r = -127.0f;
          codes[(long)i * cols + j] = (int8_t)r;
        }
    }
}

void fa_oracle_w8a8_gemm(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw,
                         int m, int n, int k, double *y) {
  const int kb = (k + 127) / 128;
  int i, j, b, t;
#pragma omp parallel for private(j, b, t) schedule(static)
  for (i = 0; i < m; ++i)
    for (j = 0; j < n; ++j) {
      double acc = 0.0;
      for (b = 0; b < kb; ++b) {
        long dot = 0;
        const int t1 = (b + 1) * 128 < k ? (b + 1) * 128 : k;
        for (t = b * 128; t < t1; ++t) dot += (long)xq[(long)i * k + t] * wq[(long)j * k + t];
        acc += (double)sx[(long)i * kb + b] * (double)sw[(long)(j / 128) * kb + b] * (double)dot;
      }
      y[(long)i * n + j] = acc;
    }
}

void fa_oracle_norm_rope(const float *x, int N, int H, int D, const float *gamma, double eps,
                         const int *pos, double base, float *out) {
  const int P = D / 2, py = D / 6, pt = P - 2 * py;
  const int gsize[3] = {pt, py, py}, gstart[3] = {0, pt, pt + py};
  int n, h;
#pragma omp parallel for private(h) schedule(static)
  for (n = 0; n < N; ++n)
    for (h = 0; h < H; ++h) {
      const float *xv = x + ((long)n * H + h) * D;
      float *ov = out + ((long)n * H + h) * D;
      double ss = 0.0, y[1024];
      int d, g, j;
      for (d = 0; d < D; ++d) ss += (double)xv[d] * (double)xv[d];
      {
        const double r = sqrt(ss / D + eps);
        for (d = 0; d < D; ++d) y[d] = (double)xv[d] / r * (double)gamma[d];
      }
      for (g = 0; g < 3; ++g)
        for (j = 0; j < gsize[g]; ++j) {
          const int i = gstart[g] + j;
          const double ang = (double)pos[n * 3 + g] * pow(base, -(double)j / gsize[g]);
          const double a = y[i], b = y[i + P];
          ov[i] = (float)(a * cos(ang) - b * sin(ang));
          ov[i + P] = (float)(a * sin(ang) + b * cos(ang));
        }
    }
}

/* OCP e4m3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.  Normal
 * values 2^(e-7) * (1 + m/8) for e = 1..15 (except e=15,m=7 which is NaN),
 * subnormals 2^-6 * m/8.  Largest finite 448.  Encoding here: round to the
 * nearest representable value, ties to the even code, values beyond 448
 * saturate to 448. */
uint8_t fa_oracle_e4m3_encode(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  int best = 0, c;
  double best_err;
  if (isnan(x)) return 0x7f;
  if (a >= 448.0) return sign | 0x7e;
  /* exhaustive search over the 127 non-negative finite codes 0x00..0x7e */
  best_err = a;
  for (c = 1; c <= 0x7e; ++c) {
    const double v = fa_oracle_e4m3_decode((uint8_t)c);
    const double err = fabs(v - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best_err = err;
      best = c;
    }
  }
  return sign | (uint8_t)best;
}

float fa_oracle_e4m3_decode(uint8_t c) {
  const int e = (c >> 3) & 0xf, m = c & 7;
  double v;
  if ((c & 0x7f) == 0x7f) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return (float)((c & 0x80) ? -v : v);
}

void fa_oracle_kmean(int n_seg, const float *const *seg, const int *n_tok, int H, int D,
                     float *mean) {
  int h, d, s, t;
  for (h = 0; h < H; ++h)
    for (d = 0; d < D; ++d) {
      double acc = 0.0;
      long n = 0;
      for (s = 0; s < n_seg; ++s)
        for (t = 0; t < n_tok[s]; ++t) {
          acc += (double)seg[s][((long)t * H + h) * D + d];
          n++;
        }
      mean[h * D + d] = n ? (float)(acc / (double)n) : 0.0f;
    }
}
