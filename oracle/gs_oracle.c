/*
 * gs_oracle.c -- CPU oracle for the block-local multi-head self-attention
 * sub-layer of the Granite-Speech-4.1-2B-NAR conformer encoder.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The HIP product path
 * never calls, links or includes anything from this directory, and this file
 * shares no code, header or table with it.
 *
 * What it computes (the plain definition, written out):
 *   IBM model card, "Model Architecture" (1) CTC Speech Encoder: each conformer
 *   layer uses block attention over 4-second audio blocks; the model card's
 *   usage section runs the model with sequence packing and non-causal
 *   (bidirectional) attention.  The sub-layer is therefore, for packed rows
 *   x[N][d] split into sequences by cu_seqlens[S+1]:
 *
 *   (1) projections   q|k|v [t][c] = sum_k x[t][k] * Wqkv[c][k],  c in [0, 3d)
 *                     (Wqkv is [3d][d], nn.Linear [out][in]; rows 0..d-1 are
 *                      Q, d..2d-1 are K, 2d..3d-1 are V; head h owns rows
 *                      h*dh .. h*dh+dh-1 inside each of the three)
 *   (2) blocks        each sequence s is cut into non-overlapping runs of B rows
 *                     starting at its first row cu[s]; the last run holds the
 *                     remainder.  Blocks never cross a sequence boundary.
 *   (3) attention     inside one block R, for head h and query row i in R:
 *                       z[i][l] = (sum_e q[i][h,e] * k[l][h,e]) / sqrt(dh), l in R
 *                       p[i][l] = exp(z[i][l] - max_l z[i][l])
 *                       o[i][h,e] = sum_l p[i][l] * v[l][h,e] / sum_l p[i][l]
 *                     (no mask inside the block: bidirectional)
 *   (4) output        out[t][c] = x[t][c] + sum_j o[t][j] * Wo[c][j]
 *                     (Wo is [d][d], [out][in]; o columns in head-concat order)
 *
 * No bias, normalisation, dropout or positional term is part of this sub-layer.
 *
 * Arithmetic: IEEE double throughout, every sum accumulated left to right in
 * its natural index order, exp() from libm, a two-pass softmax (max, then exp
 * and sum).  Each output value is produced by exactly one thread in a fixed
 * order, so results are bitwise identical for any thread count.
 *
 * Threads: POSIX threads over independent work items (rows for the
 * projections, (block, head) pairs for attention).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GSO_OK 0
#define GSO_EINVAL 1
#define GSO_ENOMEM 2

/* ------------------------------------------------------------------------ */
/* a tiny static-partition thread runner                                     */

typedef void (*gso_item_fn)(void* ctx, int64_t item);

typedef struct {
  gso_item_fn fn;
  void* ctx;
  int64_t n_items;
  int tid, nthreads;
} gso_job;

static void* gso_worker(void* arg) {
  gso_job* j = (gso_job*)arg;
  /* contiguous ranges: thread tid takes [lo, hi) */
  int64_t lo = j->n_items * j->tid / j->nthreads;
  int64_t hi = j->n_items * (j->tid + 1) / j->nthreads;
  for (int64_t i = lo; i < hi; ++i) j->fn(j->ctx, i);
  return NULL;
}

static int gso_parallel(gso_item_fn fn, void* ctx, int64_t n_items, int nthreads) {
  if (n_items <= 0) return GSO_OK;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n_items) nthreads = (int)n_items;
  pthread_t th[256];
  gso_job jobs[256];
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn; jobs[t].ctx = ctx; jobs[t].n_items = n_items;
    jobs[t].tid = t; jobs[t].nthreads = nthreads;
  }
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, gso_worker, &jobs[t]) != 0) break;
    started = t;
  }
  gso_worker(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  /* any range whose thread failed to start runs here */
  for (int t = started + 1; t < nthreads; ++t) gso_worker(&jobs[t]);
  return GSO_OK;
}

/* ------------------------------------------------------------------------ */
/* step (2): the block list                                                  */

/* Number of blocks over all sequences; -1 if cu_seqlens is malformed. */
int64_t gso_count_blocks(const int32_t* cu, int32_t S, int32_t B) {
  if (!cu || S < 0 || B < 1) return -1;
  if (cu[0] != 0) return -1;
  int64_t n = 0;
  for (int32_t s = 0; s < S; ++s) {
    int64_t len = (int64_t)cu[s + 1] - (int64_t)cu[s];
    if (len < 0) return -1;
    n += (len + B - 1) / B;
  }
  return n;
}

/* Fills start[] and len[] (each of gso_count_blocks() entries). */
int gso_block_table(const int32_t* cu, int32_t S, int32_t B, int64_t* start, int64_t* len) {
  if (gso_count_blocks(cu, S, B) < 0 || !start || !len) return GSO_EINVAL;
  int64_t b = 0;
  for (int32_t s = 0; s < S; ++s) {
    int64_t a = cu[s], end = cu[s + 1];
    for (int64_t r = a; r < end; r += B) {
      start[b] = r;
      len[b] = (r + B <= end) ? B : end - r;
      ++b;
    }
  }
  return GSO_OK;
}

/* ------------------------------------------------------------------------ */
/* step (1): projections                                                     */

typedef struct {
  const double* x; const double* W; double* y;
  int32_t d_in, d_out;
  const int64_t* rows;     /* rows to compute */
} gso_proj_ctx;

/* y[t][c] = sum_k x[t][k] * W[c][k] for one row t */
static void gso_proj_row(void* vctx, int64_t i) {
  const gso_proj_ctx* c = (const gso_proj_ctx*)vctx;
  int64_t t = c->rows[i];
  const double* xr = c->x + t * (int64_t)c->d_in;
  double* yr = c->y + t * (int64_t)c->d_out;
  for (int32_t o = 0; o < c->d_out; ++o) {
    const double* wr = c->W + (int64_t)o * c->d_in;
    double acc = 0.0;
    for (int32_t k = 0; k < c->d_in; ++k) acc += xr[k] * wr[k];
    yr[o] = acc;
  }
}

static int64_t* gso_rows_from_mask(const uint8_t* mask, int64_t N, int64_t* count) {
  int64_t n = 0;
  for (int64_t t = 0; t < N; ++t) n += (!mask || mask[t]) ? 1 : 0;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  if (!rows) return NULL;
  n = 0;
  for (int64_t t = 0; t < N; ++t)
    if (!mask || mask[t]) rows[n++] = t;
  *count = n;
  return rows;
}

/* qkv[N][3d] = x[N][d] . Wqkv[3d][d]^T for rows with mask[t] != 0 (all if NULL) */
int gso_qkv_proj(const double* x, const double* Wqkv, int64_t N, int32_t d,
                 const uint8_t* mask, double* qkv, int nthreads) {
  if (N < 0 || d < 1 || (N > 0 && (!x || !Wqkv || !qkv))) return GSO_EINVAL;
  int64_t n;
  int64_t* rows = gso_rows_from_mask(mask, N, &n);
  if (!rows) return GSO_ENOMEM;
  gso_proj_ctx c = {x, Wqkv, qkv, d, 3 * d, rows};
  gso_parallel(gso_proj_row, &c, n, nthreads);
  free(rows);
  return GSO_OK;
}

/* ------------------------------------------------------------------------ */
/* step (3): attention inside each block, per head                           */

typedef struct {
  const double* qkv;      /* [N][3d] */
  double* o;              /* [N][d]  */
  int32_t d, H, dh;
  const int64_t* bstart; const int64_t* blen;
  const uint8_t* mask;    /* query rows to produce (NULL = all) */
} gso_attn_ctx;

/* one (block, head) work item: item = block * H + head */
static void gso_attn_item(void* vctx, int64_t item) {
  const gso_attn_ctx* c = (const gso_attn_ctx*)vctx;
  int64_t b = item / c->H;
  int32_t h = (int32_t)(item % c->H);
  int64_t a = c->bstart[b], L = c->blen[b];
  int32_t dh = c->dh;
  int64_t ld = 3 * (int64_t)c->d;
  double scale = 1.0 / sqrt((double)dh);
  double* z = (double*)malloc(sizeof(double) * (size_t)L);
  if (!z) abort();
  for (int64_t i = a; i < a + L; ++i) {
    if (c->mask && !c->mask[i]) continue;
    const double* qi = c->qkv + i * ld + (int64_t)h * dh;               /* Q block */
    /* logits against every key row of the same block */
    for (int64_t l = 0; l < L; ++l) {
      const double* kl = c->qkv + (a + l) * ld + c->d + (int64_t)h * dh; /* K block */
      double s = 0.0;
      for (int32_t e = 0; e < dh; ++e) s += qi[e] * kl[e];
      z[l] = s * scale;
    }
    /* two-pass softmax: max, then exp and sum */
    double m = z[0];
    for (int64_t l = 1; l < L; ++l) if (z[l] > m) m = z[l];
    double den = 0.0;
    for (int64_t l = 0; l < L; ++l) { z[l] = exp(z[l] - m); den += z[l]; }
    /* weighted sum of the value rows, normalised */
    double* oi = c->o + i * (int64_t)c->d + (int64_t)h * dh;
    for (int32_t e = 0; e < dh; ++e) {
      double acc = 0.0;
      for (int64_t l = 0; l < L; ++l)
        acc += z[l] * c->qkv[(a + l) * ld + 2 * (int64_t)c->d + (int64_t)h * dh + e]; /* V */
      oi[e] = acc / den;
    }
  }
  free(z);
}

/* o[N][d] from qkv[N][3d] for query rows with mask != 0 (all if NULL).
 * Requires qkv for every row of each block that holds a selected row. */
int gso_block_attn(const double* qkv, const int32_t* cu, int32_t S, int32_t d, int32_t H,
                   int32_t B, const uint8_t* mask, double* o, int nthreads) {
  if (!cu || S < 1 || d < 1 || H < 1 || d % H != 0 || B < 1) return GSO_EINVAL;
  int64_t nb = gso_count_blocks(cu, S, B);
  if (nb < 0) return GSO_EINVAL;
  if (nb == 0) return GSO_OK;
  if (!qkv || !o) return GSO_EINVAL;
  int64_t* bs = (int64_t*)malloc(sizeof(int64_t) * (size_t)nb);
  int64_t* bl = (int64_t*)malloc(sizeof(int64_t) * (size_t)nb);
  if (!bs || !bl) { free(bs); free(bl); return GSO_ENOMEM; }
  gso_block_table(cu, S, B, bs, bl);
  /* keep only blocks that hold a selected row */
  int64_t kept = 0;
  for (int64_t b = 0; b < nb; ++b) {
    int any = 0;
    for (int64_t r = bs[b]; r < bs[b] + bl[b] && !any; ++r) any = !mask || mask[r];
    if (any) { bs[kept] = bs[b]; bl[kept] = bl[b]; ++kept; }
  }
  gso_attn_ctx c = {qkv, o, d, H, d / H, bs, bl, mask};
  gso_parallel(gso_attn_item, &c, kept * H, nthreads);
  free(bs); free(bl);
  return GSO_OK;
}

/* ------------------------------------------------------------------------ */
/* step (4): output projection plus residual                                 */

typedef struct {
  const double* o; const double* Wo; const double* x; double* out;
  int32_t d;
  const int64_t* rows;
} gso_out_ctx;

static void gso_out_row(void* vctx, int64_t i) {
  const gso_out_ctx* c = (const gso_out_ctx*)vctx;
  int64_t t = c->rows[i];
  const double* orow = c->o + t * (int64_t)c->d;
  for (int32_t n = 0; n < c->d; ++n) {
    const double* wr = c->Wo + (int64_t)n * c->d;
    double acc = 0.0;
    for (int32_t j = 0; j < c->d; ++j) acc += orow[j] * wr[j];
    c->out[t * (int64_t)c->d + n] = c->x[t * (int64_t)c->d + n] + acc;
  }
}

int gso_out_proj_residual(const double* o, const double* Wo, const double* x, int64_t N,
                          int32_t d, const uint8_t* mask, double* out, int nthreads) {
  if (N < 0 || d < 1 || (N > 0 && (!o || !Wo || !x || !out))) return GSO_EINVAL;
  int64_t n;
  int64_t* rows = gso_rows_from_mask(mask, N, &n);
  if (!rows) return GSO_ENOMEM;
  gso_out_ctx c = {o, Wo, x, out, d, rows};
  gso_parallel(gso_out_row, &c, n, nthreads);
  free(rows);
  return GSO_OK;
}

/* ------------------------------------------------------------------------ */
/* the whole sub-layer                                                       */

/* out[N][d] for rows with mask != 0 (all rows if mask is NULL); other rows of
 * out are left untouched.  Scratch (qkv, o) is allocated here. */
int gso_block_mhsa(const double* x, const int32_t* cu, int32_t S, int32_t d, int32_t H,
                   int32_t B, const double* Wqkv, const double* Wo, const uint8_t* mask,
                   double* out, int nthreads) {
  if (!cu || S < 1 || d < 1 || H < 1 || d % H != 0 || B < 1) return GSO_EINVAL;
  int64_t nb = gso_count_blocks(cu, S, B);
  if (nb < 0) return GSO_EINVAL;
  int64_t N = cu[S];
  if (N == 0) return GSO_OK;
  if (!x || !Wqkv || !Wo || !out) return GSO_EINVAL;

  /* rows whose q|k|v are needed: every row of a block holding a selected row */
  uint8_t* need = NULL;
  if (mask) {
    need = (uint8_t*)calloc((size_t)N, 1);
    if (!need) return GSO_ENOMEM;
    for (int32_t s = 0; s < S; ++s)
      for (int64_t a = cu[s]; a < cu[s + 1]; a += B) {
        int64_t e = a + B < cu[s + 1] ? a + B : cu[s + 1];
        int any = 0;
        for (int64_t r = a; r < e && !any; ++r) any = mask[r] != 0;
        if (any) memset(need + a, 1, (size_t)(e - a));
      }
  }
  double* qkv = (double*)malloc(sizeof(double) * (size_t)N * 3 * (size_t)d);
  double* o = (double*)malloc(sizeof(double) * (size_t)N * (size_t)d);
  int rc = GSO_ENOMEM;
  if (qkv && o) {
    rc = gso_qkv_proj(x, Wqkv, N, d, need, qkv, nthreads);
    if (rc == GSO_OK) rc = gso_block_attn(qkv, cu, S, d, H, B, mask, o, nthreads);
    if (rc == GSO_OK) rc = gso_out_proj_residual(o, Wo, x, N, d, mask, out, nthreads);
  }
  free(qkv); free(o); free(need);
  return rc;
}
