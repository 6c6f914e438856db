/*
 * Plain fp64 CPU oracle for Kimi K2's latent-attention (MLA) attend-and-combine
 * step.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the smoke
 * check and by the benchmark's CPU-baseline leg, never by the product path.
 * It shares no code, header, table or constant with the HIP library.
 *
 * What it computes is the plain definition of the step, evaluated in double
 * precision on bf16 inputs that are widened exactly.  Sources (the pages):
 *   [MIX]    page "Kimi K2 · Mix and project": the I/O header (A, V -> delta_attn),
 *            the output-projection parameter table (8,192 x 7,168), the remark
 *            that no step before the projection combines heads, and the code
 *            excerpts "mla-prefill" (rotary, query/key join with the shared
 *            rotary key, scaled scores, additive mask, fp32 softmax, value mix)
 *            and "mla-output" (head transpose, flatten to 64*128, o_proj).
 *   [BLOCKS] page "Kimi K2 · Transformer blocks": block-stack I/O header
 *            (R [T positions, 32 pairs], M [T queries, T keys]) and the model-body
 *            excerpt, whose position ids start after the already cached
 *            tokens and which builds the causal mask.
 *   [CONFIG] page "Block input", config.json excerpt: 64 heads, nope 128,
 *            rope 64, value 128, hidden 7168, attention_bias false, bfloat16.
 *
 * Rounding points (where the eager model holds a tensor in bf16 and the value
 * is a model-visible input of the next step):
 *   R1  rotated q_pe / k_pe are stored in the bf16 query/key tensors ([MIX],
 *       "mla-prefill": query_states / key_states are built from them).
 *   R2  the flattened attention output enters o_proj as bf16 ([MIX], "mla-output").
 *   R3  (latent decode only) the nope keys and values up-projected from the
 *       cached latent fill the bf16 key and value tensors.
 * Every other intermediate (scores, softmax weights, sums) stays in fp64.
 * Rounding is round-to-nearest-even, done directly from double.
 *
 * Threads: independent output rows are handed out to pthreads through an
 * atomic counter.  Each row is computed exactly as the definition states, in
 * key order; threads change nothing in the arithmetic of a row.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Head widths, from [CONFIG]: qk_nope_head_dim, qk_rope_head_dim, v_head_dim. */
#define OR_NOPE 128
#define OR_ROPE 64
#define OR_PAIRS 32
#define OR_VDIM 128

int oracle_dims(int *d_nope, int *d_rope, int *d_v) {
  *d_nope = OR_NOPE;
  *d_rope = OR_ROPE;
  *d_v = OR_VDIM;
  return 0;
}

/* ---------------------------------------------------------------- bf16 ---- */

/* Exact widening of a bf16 bit pattern (the upper half of an IEEE binary32). */
static double widen(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, without passing
 * through binary32 (which could round twice).  bf16 keeps 8 significant bits
 * and binary32's exponent range: spacing 2^(e-8) for |x| in [2^(e-1), 2^e),
 * and 2^-133 for subnormals. */
double oracle_bf16_round(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  frexp(x, &e);
  int es = e - 8;
  if (es < -133) es = -133;
  double q = ldexp(x, -es);
  double r = nearbyint(q); /* default rounding mode: nearest, ties to even */
  return ldexp(r, es);
}

/* bf16 bit pattern of oracle_bf16_round(x); finite inputs only. */
static uint16_t bf16_bits(double x) {
  float f = (float)oracle_bf16_round(x); /* exact: the value is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

void oracle_bf16_round_array(const double *x, double *y, size_t n) {
  for (size_t i = 0; i < n; i++) y[i] = oracle_bf16_round(x[i]);
}

void oracle_bf16_widen_array(const uint16_t *x, double *y, size_t n) {
  for (size_t i = 0; i < n; i++) y[i] = widen(x[i]);
}

/* ------------------------------------------------------------- rotary ---- */

/* Rotary step of [MIX] "mla-prefill" (the rotary embedding and its
 * application to q_pe and k_pe; the bodies are not printed).  Reading used:
 * pair i couples elements i and i+32 of the 64-wide rotary part ("rotate
 * half"), the angle of pair i at position t is R[t][i] (the [BLOCKS] input
 * R [T positions, 32 pairs]), and the pair turns by that angle:
 *   y_i    = x_i cos - x_{i+32} sin
 *   y_{i+32} = x_{i+32} cos + x_i sin
 * cos and sin are taken in double of the binary32 angle.  `out` receives the
 * double result before rounding point R1. */
void oracle_rotate_row(const double *x, const float *R_row, double *out) {
  for (int i = 0; i < OR_PAIRS; i++) {
    double a = (double)R_row[i];
    double c = cos(a), s = sin(a);
    double lo = x[i], hi = x[i + OR_PAIRS];
    out[i] = lo * c - hi * s;
    out[i + OR_PAIRS] = hi * c + lo * s;
  }
}

/* Rotate n rows of 64 bf16 values, row r at position pos[r]; writes both the
 * unrounded double result and its bf16 (R1) bit pattern.  Returns 1 if a
 * position is outside the table. */
int oracle_rope_rotate(const uint16_t *x, const float *R, int r_rows, const int *pos, int n,
                       double *out_f64, uint16_t *out_bf16) {
  double row[OR_ROPE], rot[OR_ROPE];
  for (int r = 0; r < n; r++) {
    if (pos[r] < 0 || pos[r] >= r_rows) return 1;
    for (int d = 0; d < OR_ROPE; d++) row[d] = widen(x[(size_t)r * OR_ROPE + d]);
    oracle_rotate_row(row, R + (size_t)pos[r] * OR_PAIRS, rot);
    for (int d = 0; d < OR_ROPE; d++) {
      if (out_f64) out_f64[(size_t)r * OR_ROPE + d] = rot[d];
      if (out_bf16) out_bf16[(size_t)r * OR_ROPE + d] = bf16_bits(rot[d]);
    }
  }
  return 0;
}

/* ------------------------------------------------------ thread helper ---- */

typedef void (*unit_fn)(void *ctx, long unit, double *scratch);

typedef struct {
  unit_fn fn;
  void *ctx;
  long n_units;
  long next; /* atomic */
  size_t scratch_doubles;
  int failed;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  double *scratch = (double *)malloc(p->scratch_doubles * sizeof(double) + 64);
  if (!scratch) {
    __atomic_store_n(&p->failed, 1, __ATOMIC_SEQ_CST);
    return NULL;
  }
  for (;;) {
    long u = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
    if (u >= p->n_units) break;
    p->fn(p->ctx, u, scratch);
  }
  free(scratch);
  return NULL;
}

static int run_units(unit_fn fn, void *ctx, long n_units, size_t scratch_doubles, int nthreads) {
  pool_t p = {fn, ctx, n_units, 0, scratch_doubles, 0};
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((long)nthreads > n_units) nthreads = (int)(n_units > 0 ? n_units : 1);
  pthread_t th[256];
  int started = 0;
  for (int i = 1; i < nthreads; i++) {
    if (pthread_create(&th[i], NULL, pool_worker, &p) != 0) break;
    started = i;
  }
  pool_worker(&p);
  for (int i = 1; i <= started; i++) pthread_join(th[i], NULL);
  return p.failed ? 2 : 0;
}

/* ---------------------------------------------------------- attention ---- */

/* One query row against keys 0..n_keys-1, the plain definition of [MIX]
 * "mla-prefill" from the scores on:
 *   s_j  = scale * (sum_{d<128} qn_d kn_jd + sum_{d<64} qr_d kr_jd)
 *   p_j  = exp(s_j - m) / sum_k exp(s_k - m),   m = max_j s_j
 *   o    = sum_j p_j v_j
 *   lse  = m + log sum_k exp(s_k - m)
 * qn (128) and qr (64, rotated and rounded) are doubles; key j's parts are
 * kn(j), kr(j) and its value row v(j).  Masked keys are simply absent: the
 * caller passes only the visible ones (a masked weight is exactly 0).
 * s holds n_keys scratch doubles. */
typedef struct {
  const uint16_t *base;
  long stride; /* elements between consecutive key rows */
} rows_t;

static void attend_row(const double *qn, const double *qr, rows_t kn, const double *kr_rot,
                       long kr_stride, rows_t v, long n_keys, double scale, double *s,
                       double *o, double *lse) {
  double m = -INFINITY;
  for (long j = 0; j < n_keys; j++) {
    const uint16_t *knj = kn.base + j * kn.stride;
    const double *krj = kr_rot + j * kr_stride;
    double dot_n = 0.0, dot_r = 0.0;
    for (int d = 0; d < OR_NOPE; d++) dot_n += qn[d] * widen(knj[d]);
    for (int d = 0; d < OR_ROPE; d++) dot_r += qr[d] * krj[d];
    s[j] = scale * (dot_n + dot_r);
    if (s[j] > m) m = s[j];
  }
  double denom = 0.0;
  for (long j = 0; j < n_keys; j++) denom += exp(s[j] - m);
  for (int d = 0; d < OR_VDIM; d++) o[d] = 0.0;
  for (long j = 0; j < n_keys; j++) {
    double p = exp(s[j] - m) / denom;
    const uint16_t *vj = v.base + j * v.stride;
    for (int d = 0; d < OR_VDIM; d++) o[d] += p * widen(vj[d]);
  }
  if (lse) *lse = m + log(denom);
}

/* ------------------------------------------------------------ prefill ---- */

typedef struct {
  const uint16_t *q_nope, *q_pe, *k_nope, *v;
  const double *kr_rot; /* [B][T][64]: rotated shared key, already rounded (R1) */
  const float *R;
  double scale;
  int B, H, T;
  const int *sel; /* NULL: every (b,h,t); else n_sel triples */
  double *out;    /* full: [B][T][H*128]; rows: [n_sel][128] */
  double *lse;    /* full: [B][H][T]; rows: [n_sel] */
} prefill_ctx;

static void prefill_unit(void *vctx, long unit, double *scratch) {
  prefill_ctx *c = (prefill_ctx *)vctx;
  int b, h, t;
  if (c->sel) {
    b = c->sel[3 * unit];
    h = c->sel[3 * unit + 1];
    t = c->sel[3 * unit + 2];
  } else {
    t = (int)(unit % c->T);
    h = (int)((unit / c->T) % c->H);
    b = (int)(unit / ((long)c->T * c->H));
  }
  const long bh = (long)b * c->H + h;
  double qn[OR_NOPE], qpe[OR_ROPE], qr[OR_ROPE], o[OR_VDIM], l;
  const uint16_t *qn_src = c->q_nope + (bh * c->T + t) * OR_NOPE;
  const uint16_t *qp_src = c->q_pe + (bh * c->T + t) * OR_ROPE;
  for (int d = 0; d < OR_NOPE; d++) qn[d] = widen(qn_src[d]);
  for (int d = 0; d < OR_ROPE; d++) qpe[d] = widen(qp_src[d]);
  /* The query sits at position t (position ids start after the cached tokens, here
   * 0, [BLOCKS] model body); rotate, then round (R1). */
  oracle_rotate_row(qpe, c->R + (size_t)t * OR_PAIRS, qr);
  for (int d = 0; d < OR_ROPE; d++) qr[d] = oracle_bf16_round(qr[d]);
  /* Causal mask ([BLOCKS] M [T queries, T keys]; [MIX] additive mask): the
   * query at t sees keys 0..t. */
  rows_t kn = {c->k_nope + bh * c->T * OR_NOPE, OR_NOPE};
  rows_t vv = {c->v + bh * c->T * OR_VDIM, OR_VDIM};
  const double *kr = c->kr_rot + (size_t)b * c->T * OR_ROPE; /* shared by all heads */
  attend_row(qn, qr, kn, kr, OR_ROPE, vv, (long)t + 1, c->scale, scratch, o, &l);
  if (c->sel) {
    for (int d = 0; d < OR_VDIM; d++) c->out[unit * OR_VDIM + d] = o[d];
    if (c->lse) c->lse[unit] = l;
  } else {
    /* Head-major flatten ([MIX] "mla-output"): out[b][t][h*128 + d]. */
    double *dst = c->out + ((size_t)b * c->T + t) * ((size_t)c->H * OR_VDIM) + (size_t)h * OR_VDIM;
    for (int d = 0; d < OR_VDIM; d++) dst[d] = o[d];
    if (c->lse) c->lse[bh * c->T + t] = l;
  }
}

/* Rotate and round the shared rotary key k_pe [B][1][T][64] once per (b, t):
 * one key rotary part serves every head ([MIX] "mla-prefill" and its
 * description: the key's rotated part is the shared rotary key). */
static double *rotate_shared_keys(const uint16_t *k_pe, const float *R, int B, int T) {
  double *kr = (double *)malloc((size_t)B * T * OR_ROPE * sizeof(double));
  if (!kr) return NULL;
  double row[OR_ROPE], rot[OR_ROPE];
  for (int b = 0; b < B; b++)
    for (int t = 0; t < T; t++) {
      const uint16_t *src = k_pe + ((size_t)b * T + t) * OR_ROPE;
      for (int d = 0; d < OR_ROPE; d++) row[d] = widen(src[d]);
      oracle_rotate_row(row, R + (size_t)t * OR_PAIRS, rot);
      double *dst = kr + ((size_t)b * T + t) * OR_ROPE;
      for (int d = 0; d < OR_ROPE; d++) dst[d] = oracle_bf16_round(rot[d]);
    }
  return kr;
}

/* Full prefill: out [B][T][H*128] (double, before rounding point R2),
 * lse [B][H][T] (natural log) or NULL.  Inputs are bf16 bit patterns:
 * q_nope [B][H][T][128], q_pe [B][H][T][64] (unrotated), k_nope [B][H][T][128],
 * k_pe [B][1][T][64] (unrotated, shared), v [B][H][T][128]; R [r_rows][32].
 * Returns 0, 1 on a bad size, 2 on allocation failure. */
int oracle_prefill(const uint16_t *q_nope, const uint16_t *q_pe, const uint16_t *k_nope,
                   const uint16_t *k_pe, const uint16_t *v, const float *R, int r_rows,
                   double scale, int B, int H, int T, double *out, double *lse, int nthreads) {
  if (B <= 0 || H <= 0 || T <= 0 || T > r_rows) return 1;
  double *kr = rotate_shared_keys(k_pe, R, B, T);
  if (!kr) return 2;
  prefill_ctx c = {q_nope, q_pe, k_nope, v, kr, R, scale, B, H, T, NULL, out, lse};
  int rc = run_units(prefill_unit, &c, (long)B * H * T, (size_t)T, nthreads);
  free(kr);
  return rc;
}

/* Selected rows only: sel holds n_sel (b, h, t) triples; out [n_sel][128],
 * lse [n_sel] or NULL.  Each row is the same exact computation as in
 * oracle_prefill. */
int oracle_prefill_rows(const uint16_t *q_nope, const uint16_t *q_pe, const uint16_t *k_nope,
                        const uint16_t *k_pe, const uint16_t *v, const float *R, int r_rows,
                        double scale, int B, int H, int T, int n_sel, const int *sel,
                        double *out, double *lse, int nthreads) {
  if (B <= 0 || H <= 0 || T <= 0 || T > r_rows || n_sel < 0) return 1;
  for (int i = 0; i < n_sel; i++)
    if (sel[3 * i] < 0 || sel[3 * i] >= B || sel[3 * i + 1] < 0 || sel[3 * i + 1] >= H ||
        sel[3 * i + 2] < 0 || sel[3 * i + 2] >= T)
      return 1;
  double *kr = rotate_shared_keys(k_pe, R, B, T);
  if (!kr) return 2;
  prefill_ctx c = {q_nope, q_pe, k_nope, v, kr, R, scale, B, H, T, sel, out, lse};
  int rc = run_units(prefill_unit, &c, (long)n_sel, (size_t)T, nthreads);
  free(kr);
  return rc;
}

/* ------------------------------------------------------------- decode ---- */

/* One new query per sequence against a cache of L keys that are already
 * rotated (the cache stores the keys after rotation: in [MIX] "mla-prefill"
 * the cache update comes after the rotary step).  Cache rows are
 * [nope(128) | rope(64)] for keys and 128 for values.  The query is rotated at
 * position q_pos.  All L cached keys are visible. */
typedef struct {
  const uint16_t *q_nope, *q_pe, *k_cache, *v_cache;
  const float *R;
  int q_pos;
  double scale;
  int B, H, L;
  const int *sel; /* NULL or n_sel (b, h) pairs */
  double *out;    /* full: [B][H*128]; rows: [n_sel][128] */
  double *lse;    /* full: [B][H]; rows: [n_sel] */
  /* NULL: k_cache rows are [nope | rope] (192).  Otherwise the shared-rotary
   * layout: k_cache rows are the 128 nope dims of each head and kpe_cache
   * [B][L][64] holds the one rotated rope key per position, shared by every
   * head ([MIX] the rotated key part is one tensor for all heads). */
  const uint16_t *kpe_cache;
} decode_ctx;

static void decode_unit(void *vctx, long unit, double *scratch) {
  decode_ctx *c = (decode_ctx *)vctx;
  int b, h;
  if (c->sel) {
    b = c->sel[2 * unit];
    h = c->sel[2 * unit + 1];
  } else {
    h = (int)(unit % c->H);
    b = (int)(unit / c->H);
  }
  const long bh = (long)b * c->H + h;
  double qn[OR_NOPE], qpe[OR_ROPE], qr[OR_ROPE], o[OR_VDIM], l;
  for (int d = 0; d < OR_NOPE; d++) qn[d] = widen(c->q_nope[bh * OR_NOPE + d]);
  for (int d = 0; d < OR_ROPE; d++) qpe[d] = widen(c->q_pe[bh * OR_ROPE + d]);
  oracle_rotate_row(qpe, c->R + (size_t)c->q_pos * OR_PAIRS, qr);
  for (int d = 0; d < OR_ROPE; d++) qr[d] = oracle_bf16_round(qr[d]);
  double *kr = scratch + c->L;
  rows_t kn;
  if (c->kpe_cache) {
    /* Nope rows of this head; the rotated rope key of position j is row j of
     * the sequence's shared table (already bf16 values). */
    kn.base = c->k_cache + bh * c->L * OR_NOPE;
    kn.stride = OR_NOPE;
    const uint16_t *kp = c->kpe_cache + (long)b * c->L * OR_ROPE;
    for (long j = 0; j < c->L; j++)
      for (int d = 0; d < OR_ROPE; d++) kr[j * OR_ROPE + d] = widen(kp[j * OR_ROPE + d]);
  } else {
    const long krow = OR_NOPE + OR_ROPE;
    const uint16_t *kc = c->k_cache + bh * c->L * krow;
    /* Widen the cached rotary parts of this head (already bf16 values). */
    for (long j = 0; j < c->L; j++)
      for (int d = 0; d < OR_ROPE; d++) kr[j * OR_ROPE + d] = widen(kc[j * krow + OR_NOPE + d]);
    kn.base = kc;
    kn.stride = krow;
  }
  rows_t vv = {c->v_cache + bh * c->L * OR_VDIM, OR_VDIM};
  attend_row(qn, qr, kn, kr, OR_ROPE, vv, c->L, c->scale, scratch, o, &l);
  if (c->sel) {
    for (int d = 0; d < OR_VDIM; d++) c->out[unit * OR_VDIM + d] = o[d];
    if (c->lse) c->lse[unit] = l;
  } else {
    double *dst = c->out + (size_t)b * c->H * OR_VDIM + (size_t)h * OR_VDIM;
    for (int d = 0; d < OR_VDIM; d++) dst[d] = o[d];
    if (c->lse) c->lse[bh] = l;
  }
}

/* Full decode: q_nope [B][H][128], q_pe [B][H][64] (unrotated), k_cache
 * [B][H][L][192] (rotated), v_cache [B][H][L][128]; out [B][H*128] double;
 * lse [B][H] or NULL. */
int oracle_decode(const uint16_t *q_nope, const uint16_t *q_pe, const uint16_t *k_cache,
                  const uint16_t *v_cache, const float *R, int r_rows, int q_pos, double scale,
                  int B, int H, int L, double *out, double *lse, int nthreads) {
  if (B <= 0 || H <= 0 || L <= 0 || q_pos < 0 || q_pos >= r_rows) return 1;
  decode_ctx c = {q_nope, q_pe, k_cache, v_cache, R, q_pos, scale, B, H, L, NULL, out, lse, NULL};
  return run_units(decode_unit, &c, (long)B * H, (size_t)L * (1 + OR_ROPE), nthreads);
}

/* Selected (b, h) pairs only: out [n_sel][128], lse [n_sel] or NULL. */
int oracle_decode_rows(const uint16_t *q_nope, const uint16_t *q_pe, const uint16_t *k_cache,
                       const uint16_t *v_cache, const float *R, int r_rows, int q_pos,
                       double scale, int B, int H, int L, int n_sel, const int *sel, double *out,
                       double *lse, int nthreads) {
  if (B <= 0 || H <= 0 || L <= 0 || q_pos < 0 || q_pos >= r_rows || n_sel < 0) return 1;
  for (int i = 0; i < n_sel; i++)
    if (sel[2 * i] < 0 || sel[2 * i] >= B || sel[2 * i + 1] < 0 || sel[2 * i + 1] >= H) return 1;
  decode_ctx c = {q_nope, q_pe, k_cache, v_cache, R, q_pos, scale, B, H, L, sel, out, lse, NULL};
  return run_units(decode_unit, &c, (long)n_sel, (size_t)L * (1 + OR_ROPE), nthreads);
}

/* Decode against the shared-rotary cache layout: k_nope_cache [B][H][L][128],
 * kpe_cache [B][L][64] (rotated, one per position for all heads), v_cache
 * [B][H][L][128].  Same scores and softmax as oracle_decode: the score of key
 * j is the nope dot product plus the rope dot product with row j of the
 * shared table. */
int oracle_decode_shared_kpe(const uint16_t *q_nope, const uint16_t *q_pe,
                             const uint16_t *k_nope_cache, const uint16_t *kpe_cache,
                             const uint16_t *v_cache, const float *R, int r_rows, int q_pos,
                             double scale, int B, int H, int L, double *out, double *lse,
                             int nthreads) {
  if (B <= 0 || H <= 0 || L <= 0 || q_pos < 0 || q_pos >= r_rows || !kpe_cache) return 1;
  decode_ctx c = {q_nope, q_pe, k_nope_cache, v_cache, R, q_pos, scale, B, H, L, NULL, out, lse,
                  kpe_cache};
  return run_units(decode_unit, &c, (long)B * H, (size_t)L * (1 + OR_ROPE), nthreads);
}

int oracle_decode_shared_kpe_rows(const uint16_t *q_nope, const uint16_t *q_pe,
                                  const uint16_t *k_nope_cache, const uint16_t *kpe_cache,
                                  const uint16_t *v_cache, const float *R, int r_rows, int q_pos,
                                  double scale, int B, int H, int L, int n_sel, const int *sel,
                                  double *out, double *lse, int nthreads) {
  if (B <= 0 || H <= 0 || L <= 0 || q_pos < 0 || q_pos >= r_rows || n_sel < 0 || !kpe_cache)
    return 1;
  for (int i = 0; i < n_sel; i++)
    if (sel[2 * i] < 0 || sel[2 * i] >= B || sel[2 * i + 1] < 0 || sel[2 * i + 1] >= H) return 1;
  decode_ctx c = {q_nope, q_pe, k_nope_cache, v_cache, R, q_pos, scale, B, H, L, sel, out, lse,
                  kpe_cache};
  return run_units(decode_unit, &c, (long)n_sel, (size_t)L * (1 + OR_ROPE), nthreads);
}

/* ------------------------------------------------------ latent decode ---- */

/* Decode against a latent cache.  [CONFIG] fixes kv_lora_rank = 512 and the
 * dense-block parameter total (pinned in the tests) fixes the up-projection as
 * one 512 -> 64*(128+128) linear map, kv_b_proj, stored [out][in] like every
 * linear layer of the model.  Reading of its output order (its code is not on
 * the pages): per head, 128 nope-key features then 128 value features, heads
 * in order, so head h's key rows are h*256 .. h*256+127 and its value rows
 * h*256+128 .. h*256+255.  The cache keeps, per position, the 512-wide latent
 * c and the rotated shared rope key (as in the shared-rotary layout).
 *
 * The plain definition: k_nope_j = W_uk,h c_j and v_j = W_uv,h c_j, each
 * rounded to bf16 (rounding point R3: they fill the bf16 key and value tensors
 * the attention reads), then the same scores, softmax and value mix as every
 * other decode here.  round_kv = 0 skips R3 (used by a test that checks the
 * algebra against an independent evaluation). */
typedef struct {
  const uint16_t *q_nope, *q_pe, *ckv, *kpe, *w_kv_b;
  const float *R;
  int q_pos;
  double scale;
  int B, H, L;
  const int *sel;
  double *out, *lse;
  int round_kv;
} latent_ctx;

#define OR_LATENT 512

/* Values of the up-projected row, rounded to bf16 (R3) unless round_kv is 0. */
static void up_project(const uint16_t *w_rows, const uint16_t *c, int n_out, int round_kv,
                       double *dst) {
  for (int r = 0; r < n_out; r++) {
    const uint16_t *w = w_rows + (size_t)r * OR_LATENT;
    double acc = 0.0;
    for (int k = 0; k < OR_LATENT; k++) acc += widen(w[k]) * widen(c[k]);
    dst[r] = round_kv ? oracle_bf16_round(acc) : acc;
  }
}

static void latent_unit(void *vctx, long unit, double *scratch) {
  latent_ctx *c = (latent_ctx *)vctx;
  int b, h;
  if (c->sel) {
    b = c->sel[2 * unit];
    h = c->sel[2 * unit + 1];
  } else {
    h = (int)(unit % c->H);
    b = (int)(unit / c->H);
  }
  const long bh = (long)b * c->H + h;
  const long L = c->L;
  double qn[OR_NOPE], qpe[OR_ROPE], qr[OR_ROPE], o[OR_VDIM];
  for (int d = 0; d < OR_NOPE; d++) qn[d] = widen(c->q_nope[bh * OR_NOPE + d]);
  for (int d = 0; d < OR_ROPE; d++) qpe[d] = widen(c->q_pe[bh * OR_ROPE + d]);
  oracle_rotate_row(qpe, c->R + (size_t)c->q_pos * OR_PAIRS, qr);
  for (int d = 0; d < OR_ROPE; d++) qr[d] = oracle_bf16_round(qr[d]);
  /* scratch: scores [L] | k_nope [L][128] | v [L][128] | rope keys [L][64] */
  double *s = scratch, *kn = s + L, *vv = kn + L * OR_NOPE, *kr = vv + L * OR_VDIM;
  const uint16_t *wk = c->w_kv_b + (size_t)h * (OR_NOPE + OR_VDIM) * OR_LATENT;
  const uint16_t *wv = wk + (size_t)OR_NOPE * OR_LATENT;
  for (long j = 0; j < L; j++) {
    const uint16_t *cj = c->ckv + ((long)b * L + j) * OR_LATENT;
    up_project(wk, cj, OR_NOPE, c->round_kv, kn + j * OR_NOPE);
    up_project(wv, cj, OR_VDIM, c->round_kv, vv + j * OR_VDIM);
    for (int d = 0; d < OR_ROPE; d++) kr[j * OR_ROPE + d] = widen(c->kpe[((long)b * L + j) * OR_ROPE + d]);
  }
  /* The definition of attend_row, on double key and value rows. */
  double m = -INFINITY;
  for (long j = 0; j < L; j++) {
    double dot_n = 0.0, dot_r = 0.0;
    for (int d = 0; d < OR_NOPE; d++) dot_n += qn[d] * kn[j * OR_NOPE + d];
    for (int d = 0; d < OR_ROPE; d++) dot_r += qr[d] * kr[j * OR_ROPE + d];
    s[j] = c->scale * (dot_n + dot_r);
    if (s[j] > m) m = s[j];
  }
  double denom = 0.0;
  for (long j = 0; j < L; j++) denom += exp(s[j] - m);
  for (int d = 0; d < OR_VDIM; d++) o[d] = 0.0;
  for (long j = 0; j < L; j++) {
    const double pj = exp(s[j] - m) / denom;
    for (int d = 0; d < OR_VDIM; d++) o[d] += pj * vv[j * OR_VDIM + d];
  }
  const double l = m + log(denom);
  if (c->sel) {
    for (int d = 0; d < OR_VDIM; d++) c->out[unit * OR_VDIM + d] = o[d];
    if (c->lse) c->lse[unit] = l;
  } else {
    double *dst = c->out + (size_t)b * c->H * OR_VDIM + (size_t)h * OR_VDIM;
    for (int d = 0; d < OR_VDIM; d++) dst[d] = o[d];
    if (c->lse) c->lse[bh] = l;
  }
}

/* q_nope [B][H][128], q_pe [B][H][64] (unrotated), ckv [B][L][512], kpe
 * [B][L][64] (rotated), w_kv_b [H*256][512]; out [B][H*128] double, lse [B][H]
 * or NULL.  sel NULL: every (b, h); else n_sel (b, h) pairs and out
 * [n_sel][128], lse [n_sel]. */
int oracle_decode_latent(const uint16_t *q_nope, const uint16_t *q_pe, const uint16_t *ckv,
                         const uint16_t *kpe, const uint16_t *w_kv_b, const float *R, int r_rows,
                         int q_pos, double scale, int B, int H, int L, int n_sel, const int *sel,
                         int round_kv, double *out, double *lse, int nthreads) {
  if (B <= 0 || H <= 0 || L <= 0 || q_pos < 0 || q_pos >= r_rows) return 1;
  if (sel) {
    if (n_sel < 0) return 1;
    for (int i = 0; i < n_sel; i++)
      if (sel[2 * i] < 0 || sel[2 * i] >= B || sel[2 * i + 1] < 0 || sel[2 * i + 1] >= H) return 1;
  }
  latent_ctx c = {q_nope, q_pe, ckv, kpe, w_kv_b, R, q_pos, scale, B, H, L, sel, out, lse, round_kv};
  const long units = sel ? (long)n_sel : (long)B * H;
  return run_units(latent_unit, &c, units, (size_t)L * (1 + OR_NOPE + OR_VDIM + OR_ROPE), nthreads);
}

/* ------------------------------------------------------------- o_proj ---- */

/* Output projection ([MIX] "mla-output" and the parameter table: an
 * 8,192 -> 7,168 linear map without bias, [CONFIG] attention_bias false).
 * The weight is held as a linear layer holds it, w [N][K] (one row of K
 * inputs per output feature), and y[m][n] = sum_k x[m][k] w[n][k], summed in
 * k order in double.  x is the bf16 attention output (rounding point R2). */
typedef struct {
  const uint16_t *x, *w;
  int M, K, N;
  const int *rows; /* NULL: all rows; else n_rows indices into x */
  double *y;       /* [M or n_rows][N] */
} oproj_ctx;

static void oproj_unit(void *vctx, long unit, double *scratch) {
  oproj_ctx *c = (oproj_ctx *)vctx;
  long m = c->rows ? c->rows[unit] : unit;
  const uint16_t *xr = c->x + m * (long)c->K;
  for (int k = 0; k < c->K; k++) scratch[k] = widen(xr[k]);
  for (int n = 0; n < c->N; n++) {
    const uint16_t *wr = c->w + (long)n * c->K;
    double acc = 0.0;
    for (int k = 0; k < c->K; k++) acc += scratch[k] * widen(wr[k]);
    c->y[unit * (long)c->N + n] = acc;
  }
}

int oracle_out_proj(const uint16_t *x, const uint16_t *w, int M, int K, int N, double *y,
                    int nthreads) {
  if (M <= 0 || K <= 0 || N <= 0) return 1;
  oproj_ctx c = {x, w, M, K, N, NULL, y};
  return run_units(oproj_unit, &c, (long)M, (size_t)K, nthreads);
}

int oracle_out_proj_rows(const uint16_t *x, const uint16_t *w, int M, int K, int N, int n_rows,
                         const int *rows, double *y, int nthreads) {
  if (M <= 0 || K <= 0 || N <= 0 || n_rows < 0) return 1;
  for (int i = 0; i < n_rows; i++)
    if (rows[i] < 0 || rows[i] >= M) return 1;
  oproj_ctx c = {x, w, M, K, N, rows, y};
  return run_units(oproj_unit, &c, (long)n_rows, (size_t)K, nthreads);
}

/* ------------------------------------------------------ up-projection ---- */

/* The MLA up-projection in front of the attention ([CONFIG]: q_lora_rank
 * 1536, kv_lora_rank 512, 64 heads of nope 128 + rope 64 query features and
 * 128 value features; the pages omit its code, and [MIX] "mla-prefill" joins
 * each head's query as nope then rope and reads the key's nope part and the
 * value per head).  Two linear maps without bias, held as linear layers hold
 * them (one row of inputs per output feature):
 *   q  = q_lat · w_q_bᵀ,  w_q_b [H*192][1536]: head h owns rows h*192 ..,
 *        the first 128 its q_nope features, the last 64 its (unrotated) q_pe;
 *   kv = ckv · w_kv_bᵀ,   w_kv_b [H*256][512]: head h owns rows h*256 ..,
 *        the first 128 its nope key features, the last 128 its value.
 * Sums in k order in double, unrounded (the model rounds the products to its
 * bf16 tensors; the tests do so where they compare bf16).  q_lat [B][T][1536],
 * ckv [B][T][512].  rows NULL: every (b, t), outputs q_nope [B][H][T][128],
 * q_pe [B][H][T][64], k_nope [B][H][T][128], v [B][H][T][128]; else n_rows
 * flat row indices b*T + t and outputs [n_rows][H][d]. */
#define OR_QRANK 1536

typedef struct {
  const uint16_t *q_lat, *ckv, *w_q_b, *w_kv_b;
  int B, T, H;
  const int *rows;
  double *q_nope, *q_pe, *k_nope, *v;
} upproj_ctx;

static double dot_bf16(const double *x, const uint16_t *w, int n) {
  double acc = 0.0;
  for (int k = 0; k < n; k++) acc += x[k] * widen(w[k]);
  return acc;
}

static void upproj_unit(void *vctx, long unit, double *scratch) {
  upproj_ctx *c = (upproj_ctx *)vctx;
  const long m = c->rows ? c->rows[unit] : unit;
  const long b = m / c->T, t = m % c->T;
  double *xq = scratch, *xc = scratch + OR_QRANK;
  for (int k = 0; k < OR_QRANK; k++) xq[k] = widen(c->q_lat[m * OR_QRANK + k]);
  for (int k = 0; k < OR_LATENT; k++) xc[k] = widen(c->ckv[m * OR_LATENT + k]);
  for (int h = 0; h < c->H; h++) {
    /* destination row of (b, h, t) in each output */
    const long r = c->rows ? unit * c->H + h : ((long)b * c->H + h) * c->T + t;
    const uint16_t *wq = c->w_q_b + (size_t)h * (OR_NOPE + OR_ROPE) * OR_QRANK;
    const uint16_t *wkv = c->w_kv_b + (size_t)h * (OR_NOPE + OR_VDIM) * OR_LATENT;
    for (int d = 0; d < OR_NOPE; d++) c->q_nope[r * OR_NOPE + d] = dot_bf16(xq, wq + (size_t)d * OR_QRANK, OR_QRANK);
    for (int d = 0; d < OR_ROPE; d++)
      c->q_pe[r * OR_ROPE + d] = dot_bf16(xq, wq + (size_t)(OR_NOPE + d) * OR_QRANK, OR_QRANK);
    for (int d = 0; d < OR_NOPE; d++)
      c->k_nope[r * OR_NOPE + d] = dot_bf16(xc, wkv + (size_t)d * OR_LATENT, OR_LATENT);
    for (int d = 0; d < OR_VDIM; d++)
      c->v[r * OR_VDIM + d] = dot_bf16(xc, wkv + (size_t)(OR_NOPE + d) * OR_LATENT, OR_LATENT);
  }
}

int oracle_up_project(const uint16_t *q_lat, const uint16_t *ckv, const uint16_t *w_q_b,
                      const uint16_t *w_kv_b, int B, int T, int H, int n_rows, const int *rows,
                      double *q_nope, double *q_pe, double *k_nope, double *v, int nthreads) {
  if (B <= 0 || T <= 0 || H <= 0) return 1;
  if (rows) {
    if (n_rows < 0) return 1;
    for (int i = 0; i < n_rows; i++)
      if (rows[i] < 0 || (long)rows[i] >= (long)B * T) return 1;
  }
  upproj_ctx c = {q_lat, ckv, w_q_b, w_kv_b, B, T, H, rows, q_nope, q_pe, k_nope, v};
  const long units = rows ? (long)n_rows : (long)B * T;
  return run_units(upproj_unit, &c, units, (size_t)(OR_QRANK + OR_LATENT), nthreads);
}

/* ----------------------------------------------------------- fp8 weights ---- */

/* The checkpoint stores projection weights in FP8 with one float32 scale per
 * 128 x 128 block (page "Kimi K2 · Transformer blocks" and "Kimi K2 · Mix and
 * project": parameter counts exclude the FP8 block scales).  The format is
 * e4m3 of the OCP "fn" variant: sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities, S.1111.111 is NaN, largest finite value 448.
 * Decoded exactly to double. */
double oracle_e4m3_to_double(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return NAN;
  /* normal: (1 + m/8) 2^(e-7) = (8 + m) 2^(e-10); subnormal: (m/8) 2^-6 = m 2^-9 */
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

void oracle_e4m3_to_double_array(const uint8_t *b, double *out, size_t n) {
  for (size_t i = 0; i < n; i++) out[i] = oracle_e4m3_to_double(b[i]);
}

/* Dequantized weight (reading of the checkpoint format for a bf16 model): the
 * fp8 value times its block's scale, computed in float32 (the exact product
 * fits a double, so one rounding to float32), then rounded to bf16.
 * w8 [N][K], scale [ceil(N/128)][ceil(K/128)], out [N][K] bf16 bits. */
int oracle_dequant_fp8(const uint8_t *w8, const float *scale, int N, int K, uint16_t *out) {
  if (N <= 0 || K <= 0) return 1;
  const int KB = (K + 127) / 128;
  for (long n = 0; n < N; n++)
    for (long k = 0; k < K; k++) {
      const float s = scale[(n / 128) * KB + k / 128];
      const float prod = (float)(oracle_e4m3_to_double(w8[n * K + k]) * (double)s);
      out[n * K + k] = bf16_bits((double)prod);
    }
  return 0;
}

/* ------------------------------------ FP8 activations (dynamic scheme) ---- */

/* Page "Block input", config.json quantization_config: fmt e4m3, weight blocks
 * of 128 x 128, activation_scheme "dynamic" -- the activations are quantized
 * at run time.  The pages give no recipe for the dynamic activation scales;
 * the reading here is the public recipe of the model family's FP8 format
 * (DeepSeek-V3 technical report, fine-grained quantization: activations in
 * 1 x 128 tiles per token, weights in 128 x 128 blocks; its reference
 * per-token cast in the DeepGEMM repository): per row and 128-column block,
 * amax = max |x| in float32, clamped below at 1e-4; scale = amax / 448 (the
 * largest e4m3 value), in float32; q = e4m3(x / scale), the division in
 * float32, the conversion rounding to nearest even.  The projection is then
 * the plain product of the dequantized operands (q times its scale, for x and
 * for the weight), here in double. */

/* e4m3 ("fn") code of a float: round to nearest even on the format's grid
 * (spacing 2^(E-3) for |v| in [2^E, 2^(E+1)), E >= -6; 2^-9 below 2^-6); a
 * magnitude that rounds above 448 has no code and gives NaN (0x7F with the
 * sign), as does NaN. */
uint8_t oracle_e4m3_from_float(float v) {
  const double x = (double)v;
  if (isnan(x)) return 0x7F;
  const uint8_t sign = signbit(x) ? 0x80 : 0;
  const double a = fabs(x);
  if (a == 0.0) return sign;
  int E;
  frexp(a, &E); /* a = f 2^E, f in [0.5, 1): a in [2^(E-1), 2^E) */
  E -= 1;       /* a in [2^E, 2^(E+1)) */
  if (E < -6) E = -6;
  const double spacing = ldexp(1.0, E - 3);
  const double r = nearbyint(a / spacing) * spacing; /* exact: a/spacing is a scaled float */
  if (r > 448.0) return (uint8_t)(sign | 0x7F);
  if (r < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9))); /* subnormal */
  int E2;
  frexp(r, &E2);
  E2 -= 1;
  const int m = (int)(r / ldexp(1.0, E2 - 3)) - 8;
  return (uint8_t)(sign | ((E2 + 7) << 3) | m);
}

void oracle_e4m3_from_float_array(const float *v, uint8_t *out, size_t n) {
  for (size_t i = 0; i < n; i++) out[i] = oracle_e4m3_from_float(v[i]);
}

/* Activation quantization of x [M][K] (bf16 bits): q [M][K] e4m3 codes and
 * scale [M][KB] float32, KB = ceil(K/128) (the last block may be shorter). */
int oracle_act_quant(const uint16_t *x, int M, int K, uint8_t *q, float *scale) {
  if (M <= 0 || K <= 0) return 1;
  const int KB = (K + 127) / 128;
  for (long m = 0; m < M; m++)
    for (int kb = 0; kb < KB; kb++) {
      const int k0 = kb * 128, k1 = k0 + 128 < K ? k0 + 128 : K;
      float amax = 0.0f;
      for (int k = k0; k < k1; k++) {
        const float a = fabsf((float)widen(x[m * K + k]));
        if (a > amax) amax = a;
      }
      if (amax < 1e-4f) amax = 1e-4f;
      const float s = amax / 448.0f;
      scale[m * KB + kb] = s;
      for (int k = k0; k < k1; k++) q[m * K + k] = oracle_e4m3_from_float((float)widen(x[m * K + k]) / s);
    }
  return 0;
}

typedef struct {
  const double *xd, *wd; /* dequantized operands [M][K], [N][K] */
  int M, K, N;
  double *y;
} fp8dyn_ctx;

static void fp8dyn_unit(void *vctx, long unit, double *scratch) {
  (void)scratch;
  fp8dyn_ctx *c = (fp8dyn_ctx *)vctx;
  const double *xr = c->xd + unit * c->K;
  for (int n = 0; n < c->N; n++) {
    const double *wr = c->wd + (long)n * c->K;
    double acc = 0.0;
    for (int k = 0; k < c->K; k++) acc += xr[k] * wr[k];
    c->y[unit * c->N + n] = acc;
  }
}

/* y [M][N] = dequant(act_quant(x)) · dequant(w8, w_scale)ᵀ in double, no bias:
 * x [M][K] bf16 bits, w8 [N][K] e4m3 codes, w_scale [ceil(N/128)][ceil(K/128)]. */
int oracle_out_proj_fp8_dyn(const uint16_t *x, const uint8_t *w8, const float *w_scale, int M,
                            int K, int N, double *y, int nthreads) {
  if (M <= 0 || K <= 0 || N <= 0) return 1;
  const int KB = (K + 127) / 128;
  uint8_t *q = (uint8_t *)malloc((size_t)M * K);
  float *sx = (float *)malloc((size_t)M * KB * sizeof(float));
  double *xd = (double *)malloc((size_t)M * K * sizeof(double));
  double *wd = (double *)malloc((size_t)N * K * sizeof(double));
  int rc = 2;
  if (q && sx && xd && wd) {
    oracle_act_quant(x, M, K, q, sx);
    for (long m = 0; m < M; m++)
      for (int k = 0; k < K; k++)
        xd[m * K + k] = oracle_e4m3_to_double(q[m * K + k]) * (double)sx[m * KB + k / 128];
    for (long n = 0; n < N; n++)
      for (int k = 0; k < K; k++)
        wd[n * K + k] = oracle_e4m3_to_double(w8[n * K + k]) * (double)w_scale[(n / 128) * KB + k / 128];
    fp8dyn_ctx c = {xd, wd, M, K, N, y};
    rc = run_units(fp8dyn_unit, &c, (long)M, 1, nthreads);
  }
  free(q);
  free(sx);
  free(xd);
  free(wd);
  return rc;
}

/* ------------------------------------------------ chunked prefill, append ---- */

/* Page "Kimi K2 · Transformer blocks", model-body excerpt: positions of a new
 * chunk start after the cached tokens (position_ids = past .. past+T-1) and
 * the causal mask is built with that past length; page "Kimi K2 · Mix and
 * project", excerpt "mla-prefill": the cache is updated with the new keys after
 * the rotary step, and the scores run over every cached and new key.  Query t
 * of the chunk (position past + t) sees keys 0 .. past + t.
 *
 * Append: the new chunk's keys and values go to rows past .. past+T-1 of the
 * shared-rotary cache layout; the rope key is rotated at its position and
 * rounded to bf16 (R1).  k_nope [B][H][T][128], k_pe [B][T][64] (unrotated),
 * v [B][H][T][128]; caches k_nope_cache [B][H][Lc][128], kpe_cache [B][Lc][64],
 * v_cache [B][H][Lc][128]. */
int oracle_append_kv(const uint16_t *k_nope, const uint16_t *k_pe, const uint16_t *v,
                     const float *R, int r_rows, int past, int B, int H, int T, int Lc,
                     uint16_t *k_nope_cache, uint16_t *kpe_cache, uint16_t *v_cache) {
  if (B <= 0 || H <= 0 || T <= 0 || past < 0 || past + T > Lc || past + T > r_rows) return 1;
  for (long b = 0; b < B; b++)
    for (long h = 0; h < H; h++)
      for (long t = 0; t < T; t++) {
        memcpy(k_nope_cache + ((b * H + h) * Lc + past + t) * OR_NOPE,
               k_nope + ((b * H + h) * T + t) * OR_NOPE, OR_NOPE * sizeof(uint16_t));
        memcpy(v_cache + ((b * H + h) * Lc + past + t) * OR_VDIM,
               v + ((b * H + h) * T + t) * OR_VDIM, OR_VDIM * sizeof(uint16_t));
      }
  for (long b = 0; b < B; b++)
    for (long t = 0; t < T; t++) {
      double x[OR_ROPE], y[OR_ROPE];
      for (int d = 0; d < OR_ROPE; d++) x[d] = widen(k_pe[(b * T + t) * OR_ROPE + d]);
      oracle_rotate_row(x, R + (size_t)(past + t) * OR_PAIRS, y);
      for (int d = 0; d < OR_ROPE; d++) kpe_cache[(b * Lc + past + t) * OR_ROPE + d] = bf16_bits(y[d]);
    }
  return 0;
}

typedef struct {
  const uint16_t *q_nope, *q_pe, *k_nope_cache, *kpe_cache, *v_cache;
  const float *R;
  int past;
  double scale;
  int B, H, T, Lc;
  const int *sel; /* NULL: every (b,h,t); else n_sel (b, h, t) triples */
  double *out, *lse;
} chunk_ctx;

static void chunk_unit(void *vctx, long unit, double *scratch) {
  chunk_ctx *c = (chunk_ctx *)vctx;
  long t, b, h;
  if (c->sel) {
    b = c->sel[3 * unit];
    h = c->sel[3 * unit + 1];
    t = c->sel[3 * unit + 2];
  } else {
    t = unit % c->T;
    h = (unit / c->T) % c->H;
    b = unit / ((long)c->T * c->H);
  }
  const long bh = b * c->H + h;
  const long nk = c->past + t + 1; /* keys 0 .. past + t */
  double qn[OR_NOPE], qpe[OR_ROPE], qr[OR_ROPE], o[OR_VDIM], l;
  const long qrow = bh * c->T + t;
  for (int d = 0; d < OR_NOPE; d++) qn[d] = widen(c->q_nope[qrow * OR_NOPE + d]);
  for (int d = 0; d < OR_ROPE; d++) qpe[d] = widen(c->q_pe[qrow * OR_ROPE + d]);
  oracle_rotate_row(qpe, c->R + (size_t)(c->past + t) * OR_PAIRS, qr);
  for (int d = 0; d < OR_ROPE; d++) qr[d] = oracle_bf16_round(qr[d]);
  double *kr = scratch + nk;
  const uint16_t *kp = c->kpe_cache + b * c->Lc * OR_ROPE;
  for (long j = 0; j < nk; j++)
    for (int d = 0; d < OR_ROPE; d++) kr[j * OR_ROPE + d] = widen(kp[j * OR_ROPE + d]);
  rows_t kn = {c->k_nope_cache + bh * c->Lc * OR_NOPE, OR_NOPE};
  rows_t vv = {c->v_cache + bh * c->Lc * OR_VDIM, OR_VDIM};
  attend_row(qn, qr, kn, kr, OR_ROPE, vv, nk, c->scale, scratch, o, &l);
  if (c->sel) {
    for (int d = 0; d < OR_VDIM; d++) c->out[unit * OR_VDIM + d] = o[d];
    if (c->lse) c->lse[unit] = l;
    return;
  }
  double *dst = c->out + ((size_t)b * c->T + t) * ((size_t)c->H * OR_VDIM) + (size_t)h * OR_VDIM;
  for (int d = 0; d < OR_VDIM; d++) dst[d] = o[d];
  if (c->lse) c->lse[qrow] = l;
}

/* Chunked prefill over the cache: q_nope [B][H][T][128], q_pe [B][H][T][64]
 * (unrotated, rotated at past + t); caches as for oracle_append_kv, holding
 * rows 0 .. past+T-1 (the chunk's own keys already appended); out
 * [B][T][H*128], lse [B][H][T] or NULL. */
int oracle_prefill_chunk(const uint16_t *q_nope, const uint16_t *q_pe, const uint16_t *k_nope_cache,
                         const uint16_t *kpe_cache, const uint16_t *v_cache, const float *R,
                         int r_rows, int past, double scale, int B, int H, int T, int Lc,
                         double *out, double *lse, int nthreads) {
  if (B <= 0 || H <= 0 || T <= 0 || past < 0 || past + T > Lc || past + T > r_rows) return 1;
  chunk_ctx c = {q_nope, q_pe, k_nope_cache, kpe_cache, v_cache, R, past, scale, B, H, T, Lc,
                 NULL, out, lse};
  return run_units(chunk_unit, &c, (long)B * H * T, (size_t)(past + T) * (1 + OR_ROPE), nthreads);
}

/* Selected rows of the chunked prefill: sel holds n_sel (b, h, t) triples;
 * out [n_sel][128], lse [n_sel] or NULL.  Each row is the same computation as
 * in oracle_prefill_chunk (query at position past + t over cache rows
 * 0 .. past + t). */
int oracle_prefill_chunk_rows(const uint16_t *q_nope, const uint16_t *q_pe,
                              const uint16_t *k_nope_cache, const uint16_t *kpe_cache,
                              const uint16_t *v_cache, const float *R, int r_rows, int past,
                              double scale, int B, int H, int T, int Lc, int n_sel, const int *sel,
                              double *out, double *lse, int nthreads) {
  if (B <= 0 || H <= 0 || T <= 0 || past < 0 || past + T > Lc || past + T > r_rows || n_sel < 0)
    return 1;
  for (int i = 0; i < n_sel; i++)
    if (sel[3 * i] < 0 || sel[3 * i] >= B || sel[3 * i + 1] < 0 || sel[3 * i + 1] >= H ||
        sel[3 * i + 2] < 0 || sel[3 * i + 2] >= T)
      return 1;
  chunk_ctx c = {q_nope, q_pe, k_nope_cache, kpe_cache, v_cache, R, past, scale, B, H, T, Lc,
                 sel, out, lse};
  return run_units(chunk_unit, &c, (long)n_sel, (size_t)(past + T) * (1 + OR_ROPE), nthreads);
}
