/*
 * msa_oracle.c -- plain, slow, fp64 CPU oracle for the MSA forward pass.
 *
 * TEST INFRASTRUCTURE ONLY (see msa_oracle.h).  Written as the definition of
 * the method, step by step, with no blocking, fusion or reordering beyond
 * what that definition states.  OpenMP only splits independent
 * (query, group) or (query, head) rows across threads; each row is computed
 * by one thread in a fixed order, so results do not depend on the thread
 * count.
 *
 * Sources (page title, section):
 *   - "MiniMax Sparse Attention" paper summary (hyper.ai), Method: token score
 *     is the index-q / index-k dot product over visible keys, block score is
 *     the max over the block, Top-k per GQA group, the local block always
 *     kept; Main Branch is standard scaled-dot-product attention over the
 *     gathered tokens of the chosen blocks.
 *   - zhichai.net write-up, section 2 (architecture): one index-q and one
 *     index-k head per GQA group; Bk = 128, k = 16, budget k*Bk tokens (so k
 *     counts the local block); every query head of a group shares the
 *     group's block set but keeps its own query.
 *   - same write-up, section 4.1 (exp-free Top-k): only the order of the
 *     scores matters, so no exponential is taken before selection.
 * Readings where the pages are silent: ties go to the lowest block id,
 * the output list is ascending with -1 padding, key t is visible to the
 * query at position p iff t <= p.
 */
#include "msa_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Exact widening of one stored element to fp64. */
static double widen(const void* base, int dtype, int64_t idx) {
  if (dtype == MO_F64) return ((const double*)base)[idx];
  if (dtype == MO_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16; /* bf16 -> fp32 */
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int check_problem(const mo_problem* p, int dtype) {
  if (!p) return -1;
  if (p->batch < 1 || p->n_q < 1 || p->n_k < 1 || p->h_q < 1 || p->h_kv < 1) return -2;
  if (p->d < 1 || p->d_idx < 1 || p->block_size < 1 || p->topk < 1) return -3;
  if (p->h_q % p->h_kv) return -4;
  if (p->q_offset < 0 || p->q_offset + p->n_q > p->n_k) return -5;
  if (dtype != MO_F32 && dtype != MO_BF16 && dtype != MO_F64) return -6;
  return 0;
}

static int64_t num_blocks(const mo_problem* p) {
  return ((int64_t)p->n_k + p->block_size - 1) / p->block_size;
}

static void row_of(const mo_problem* p, const int64_t* rows, int64_t r, int64_t* b, int64_t* i) {
  if (rows) {
    *b = rows[2 * r];
    *i = rows[2 * r + 1];
  } else {
    *b = r / p->n_q;
    *i = r % p->n_q;
  }
}

static int check_rows(const mo_problem* p, const int64_t* rows, int64_t n_rows) {
  if (n_rows < 0) return -7;
  if (!rows) return n_rows == (int64_t)p->batch * p->n_q ? 0 : -8;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[2 * r] < 0 || rows[2 * r] >= p->batch || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= p->n_q)
      return -9;
  return 0;
}

int mo_num_threads(void) { return omp_get_max_threads(); }

void mo_set_num_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

/* Steps 1 and 2: token scores and Block Max Pooling. */
int mo_block_scores(const mo_problem* p, const void* iq, const void* ik, int dtype,
                    const int64_t* rows, int64_t n_rows, double* scores) {
  int rc = check_problem(p, dtype);
  if (rc) return rc;
  if ((rc = check_rows(p, rows, n_rows))) return rc;
  if (!iq || !ik || !scores) return -1;
  const int64_t nblk = num_blocks(p), H = p->h_kv, D = p->d_idx, Bk = p->block_size;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t rg = 0; rg < n_rows * H; ++rg) {
    const int64_t r = rg / H, g = rg % H;
    int64_t b, i;
    row_of(p, rows, r, &b, &i);
    const int64_t pos = p->q_offset + i;
    const int64_t L = pos / Bk; /* local block */
    double* S = scores + (r * H + g) * nblk;
    for (int64_t j = 0; j < nblk; ++j) S[j] = -INFINITY;
    const int64_t qbase = ((b * p->n_q + i) * H + g) * D;
    for (int64_t j = 0; j < L; ++j) {
      double best = -INFINITY;
      for (int64_t t = j * Bk; t < (j + 1) * Bk; ++t) {
        if (t > pos || t >= p->n_k) continue; /* visible tokens only */
        const int64_t kbase = ((b * p->n_k + t) * H + g) * D;
        double s = 0.0;
        for (int64_t c = 0; c < D; ++c) s += widen(iq, dtype, qbase + c) * widen(ik, dtype, kbase + c);
        if (s > best) best = s;
      }
      S[j] = best;
    }
  }
  return 0;
}

typedef struct {
  double s;
  int32_t j;
} cand_t;

/* Order for Top-k: higher score first; equal scores -> lower block id first. */
static int by_score_desc_id_asc(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int by_int_asc(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Step 3: the local block plus the top-(k-1) candidates; no exponential. */
int mo_select(const mo_problem* p, const double* scores, const int64_t* rows, int64_t n_rows,
              int32_t* ids) {
  int rc = check_problem(p, MO_F64);
  if (rc) return rc;
  if ((rc = check_rows(p, rows, n_rows))) return rc;
  if (!scores || !ids) return -1;
  const int64_t nblk = num_blocks(p), H = p->h_kv, K = p->topk, Bk = p->block_size;

#pragma omp parallel
  {
    cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(nblk > 0 ? nblk : 1));
    int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
#pragma omp for schedule(static)
    for (int64_t rg = 0; rg < n_rows * H; ++rg) {
      const int64_t r = rg / H;
      int64_t b, i;
      row_of(p, rows, r, &b, &i);
      const int64_t L = (p->q_offset + i) / Bk;
      const double* S = scores + rg * nblk;
      int32_t* out = ids + rg * K;
      int64_t n = 0;
      if (L <= K - 1) {
        for (int64_t j = 0; j < L; ++j) chosen[n++] = (int32_t)j; /* every candidate */
      } else {
        for (int64_t j = 0; j < L; ++j) {
          /* a NaN score ranks with -inf (lowest, ties to the lower id), as the
             max-pool's NaN token scores are dropped */
          cand[j].s = isnan(S[j]) ? -INFINITY : S[j];
          cand[j].j = (int32_t)j;
        }
        qsort(cand, (size_t)L, sizeof(cand_t), by_score_desc_id_asc);
        for (int64_t m = 0; m < K - 1; ++m) chosen[n++] = cand[m].j;
      }
      chosen[n++] = (int32_t)L; /* the local block is always kept */
      qsort(chosen, (size_t)n, sizeof(int32_t), by_int_asc);
      for (int64_t m = 0; m < K; ++m) out[m] = m < n ? chosen[m] : -1;
    }
    free(cand);
    free(chosen);
  }
  return 0;
}

/* Block -> query lists by plain counting: count, exclusive prefix, then place
 * every pick walking the queries and slots in ascending order. */
int mo_invert(const mo_problem* p, const int32_t* ids, int32_t* offsets, int32_t* entries) {
  int rc = check_problem(p, MO_F64);
  if (rc) return rc;
  if (!ids || !offsets || !entries) return -1;
  const int64_t nblk = num_blocks(p), H = p->h_kv, K = p->topk, Nq = p->n_q;
  for (int64_t b = 0; b < p->batch; ++b)
    for (int64_t g = 0; g < H; ++g) {
      int32_t* off = offsets + (b * H + g) * (nblk + 1);
      int32_t* ent = entries + (b * H + g) * (Nq * K);
      for (int64_t j = 0; j <= nblk; ++j) off[j] = 0;
      for (int64_t i = 0; i < Nq; ++i)
        for (int64_t s = 0; s < K; ++s) {
          const int32_t j = ids[((b * Nq + i) * H + g) * K + s];
          if (j >= 0 && j < nblk) off[j + 1] += 1;
        }
      for (int64_t j = 0; j < nblk; ++j) off[j + 1] += off[j];
      int32_t* fill = (int32_t*)calloc((size_t)nblk, sizeof(int32_t));
      if (!fill) return -10;
      for (int64_t i = 0; i < Nq; ++i)
        for (int64_t s = 0; s < K; ++s) {
          const int32_t j = ids[((b * Nq + i) * H + g) * K + s];
          if (j >= 0 && j < nblk) ent[off[j] + fill[j]++] = (int32_t)(i * K + s);
        }
      free(fill);
    }
  return 0;
}

/* Step 4: exact softmax attention restricted to the selected blocks. */
/* Query head h belongs to GQA group h / G (contiguous heads per group). */
static int64_t group_of(const mo_problem* p, int64_t h) { return h / (p->h_q / p->h_kv); }

/* The attention scale: 1/sqrt(d) unless the problem gives one. */
static double softmax_scale(const mo_problem* p) {
  const int64_t D = p->d;
  return p->softmax_scale > 0 ? p->softmax_scale : 1.0 / sqrt((double)D);
}

/* T: the visible tokens (t <= pos, t < n_k) of the blocks listed in sel
 * (topk entries; ids outside [0, nblk) ignored), in list order: a block listed
 * twice puts its tokens in T twice.  Returns |T|. */
static int64_t visible_tokens(const mo_problem* p, const int32_t* sel, int64_t pos, int64_t* tok) {
  const int64_t Bk = p->block_size, nblk = num_blocks(p);
  int64_t n = 0;
  for (int64_t s = 0; s < p->topk; ++s) {
    const int64_t j = sel[s];
    if (j < 0 || j >= nblk) continue;
    for (int64_t t = j * Bk; t < (j + 1) * Bk; ++t)
      if (t <= pos && t < p->n_k) tok[n++] = t;
  }
  return n;
}

/* Softmax attention of query head h of (b, i) over the tokens tok[0..n):
 * x[a] = probability of token a, o = output row; returns the log-sum-exp of
 * the scaled logits (-inf when n == 0, o then 0). */
static double attend_row(const mo_problem* p, const void* q, const void* k, const void* v, int dtype, int64_t b,
                         int64_t i, int64_t h, const int64_t* tok, int64_t n, double* x, double* o) {
  const int64_t Hq = p->h_q, Hkv = p->h_kv, D = p->d, g = group_of(p, h);
  const double scale = softmax_scale(p);
  const int64_t qbase = ((b * p->n_q + i) * Hq + h) * D;
  if (n == 0) { /* no visible selected token: zero output, empty sum */
    for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
    return -INFINITY;
  }
  double m = -INFINITY;
  for (int64_t a = 0; a < n; ++a) {
    const int64_t kbase = ((b * p->n_k + tok[a]) * Hkv + g) * D;
    double s = 0.0;
    for (int64_t c = 0; c < D; ++c) s += widen(q, dtype, qbase + c) * widen(k, dtype, kbase + c);
    x[a] = scale * s;
    if (x[a] > m) m = x[a];
  }
  double l = 0.0;
  for (int64_t a = 0; a < n; ++a) {
    x[a] = exp(x[a] - m);
    l += x[a];
  }
  for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
  for (int64_t a = 0; a < n; ++a) {
    const int64_t vbase = ((b * p->n_k + tok[a]) * Hkv + g) * D;
    for (int64_t c = 0; c < D; ++c) o[c] += x[a] * widen(v, dtype, vbase + c);
  }
  for (int64_t c = 0; c < D; ++c) o[c] /= l;
  for (int64_t a = 0; a < n; ++a) x[a] /= l;
  return m + log(l);
}

int mo_attend(const mo_problem* p, const void* q, const void* k, const void* v, int dtype,
              const int32_t* ids, const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  int rc = check_problem(p, dtype);
  if (rc) return rc;
  if ((rc = check_rows(p, rows, n_rows))) return rc;
  if (!q || !k || !v || !ids || !out) return -1;
  const int64_t Hq = p->h_q, Hkv = p->h_kv, D = p->d, K = p->topk, Bk = p->block_size;

#pragma omp parallel
  {
    /* Worst case: every block selected. */
    const int64_t cap = K * Bk; /* a block listed twice contributes its tokens twice */
    double* x = (double*)malloc(sizeof(double) * (size_t)cap);
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
#pragma omp for schedule(dynamic, 4)
    for (int64_t rh = 0; rh < n_rows * Hq; ++rh) {
      const int64_t r = rh / Hq, h = rh % Hq, g = group_of(p, h);
      int64_t b, i;
      row_of(p, rows, r, &b, &i);
      const int64_t pos = p->q_offset + i;
      const int32_t* sel = ids + (r * Hkv + g) * K;
      const int64_t n = visible_tokens(p, sel, pos, tok);
      const double row_lse = attend_row(p, q, k, v, dtype, b, i, h, tok, n, x, out + rh * D);
      if (lse) lse[rh] = row_lse;
    }
    free(x);
    free(tok);
  }
  return 0;
}

/* Chain rule through the softmax attention of mo_attend, written out per
 * (b, i, h).  Each OpenMP thread owns whole (b, g) groups and walks the listed
 * rows in list order, so the dk / dv sums are formed by one thread in a fixed
 * order. */
int mo_attend_backward(const mo_problem* p, const void* q, const void* k, const void* v, const void* dout,
                       int dtype, const int32_t* ids, const int64_t* rows, int64_t n_rows, double* dq, double* dk,
                       double* dv) {
  int rc = check_problem(p, dtype);
  if (rc) return rc;
  if (!q || !k || !v || !dout || !ids || !dq || !dk || !dv) return -1;
  rc = check_rows(p, rows, n_rows);
  if (rc) return rc;
  const int64_t Hq = p->h_q, Hkv = p->h_kv, G = Hq / Hkv, D = p->d, K = p->topk, Bk = p->block_size;
  const double scale = softmax_scale(p);
  memset(dk, 0, sizeof(double) * (size_t)(p->batch * p->n_k * Hkv * D));
  memset(dv, 0, sizeof(double) * (size_t)(p->batch * p->n_k * Hkv * D));

#pragma omp parallel
  {
    const int64_t cap = K * Bk; /* a block listed twice contributes its tokens twice */
    double* x = (double*)malloc(sizeof(double) * (size_t)cap);
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < p->batch * Hkv; ++bg) {
      const int64_t g = bg % Hkv;
      for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b, i;
        row_of(p, rows, r, &b, &i);
        if (b != bg / Hkv) continue;
        const int64_t pos = p->q_offset + i;
        const int32_t* sel = ids + (r * Hkv + g) * K;
        const int64_t n = visible_tokens(p, sel, pos, tok);
        for (int64_t h = g * G; h < (g + 1) * G; ++h) {
          const int64_t qbase = ((b * p->n_q + i) * Hq + h) * D;
          double* dqr = dq + (r * Hq + h) * D;
          for (int64_t c = 0; c < D; ++c) dqr[c] = 0.0;
          if (n == 0) continue;
          attend_row(p, q, k, v, dtype, b, i, h, tok, n, x, o); /* x = P, o = O */
          double dot_do_o = 0.0;
          for (int64_t c = 0; c < D; ++c) dot_do_o += widen(dout, dtype, qbase + c) * o[c];
          /* backward */
          for (int64_t a = 0; a < n; ++a) {
            const int64_t kvbase = ((b * p->n_k + tok[a]) * Hkv + g) * D;
            double dp = 0.0;
            for (int64_t c = 0; c < D; ++c) dp += widen(dout, dtype, qbase + c) * widen(v, dtype, kvbase + c);
            const double ds = x[a] * (dp - dot_do_o);
            for (int64_t c = 0; c < D; ++c) {
              dqr[c] += scale * ds * widen(k, dtype, kvbase + c);
              dk[kvbase + c] += scale * ds * widen(q, dtype, qbase + c);
              dv[kvbase + c] += x[a] * widen(dout, dtype, qbase + c);
            }
          }
        }
      }
    }
    free(x);
    free(tok);
    free(o);
  }
  return 0;
}

/* Index-Branch alignment loss (paper summary page, "Method"; zhichai.net
 * write-up, section 5.1): per (b, i, g) over the visible selected tokens T,
 * the Main Branch's group-averaged distribution pm(t) = (1/G) sum_h P_h(t)
 * (P_h the softmax of mo_attend, a fixed target) against the Index Branch's
 * distribution pi(t) = softmax over T of the raw token scores s_t.
 *   kl = sum_t pm(t) (log pm(t) - log pi(t))        (terms with pm = 0 vanish)
 *   d kl / d s_t = pi(t) - pm(t)                    (sum_t pm = 1)
 * and through s_t = <iq, ik_t> the gradients of loss_scale * sum kl. */
int mo_indexer_kl(const mo_problem* p, const void* q, const void* k, const void* iq, const void* ik, int dtype,
                  const int32_t* ids, const int64_t* rows, int64_t n_rows, double loss_scale, double* kl,
                  double* d_iq, double* d_ik) {
  int rc = check_problem(p, dtype);
  if (rc) return rc;
  if (!q || !k || !iq || !ik || !ids || !kl || !d_iq || !d_ik) return -1;
  rc = check_rows(p, rows, n_rows);
  if (rc) return rc;
  const int64_t Hq = p->h_q, Hkv = p->h_kv, G = Hq / Hkv, D = p->d, DI = p->d_idx, K = p->topk;
  const int64_t Bk = p->block_size;
  memset(d_ik, 0, sizeof(double) * (size_t)(p->batch * p->n_k * Hkv * DI));

#pragma omp parallel
  {
    const int64_t cap = K * Bk; /* a block listed twice contributes its tokens twice */
    double* x = (double*)malloc(sizeof(double) * (size_t)cap);
    double* pm = (double*)malloc(sizeof(double) * (size_t)cap);
    double* si = (double*)malloc(sizeof(double) * (size_t)cap);
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < p->batch * Hkv; ++bg) {
      const int64_t g = bg % Hkv;
      for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b, i;
        row_of(p, rows, r, &b, &i);
        if (b != bg / Hkv) continue;
        const int32_t* sel = ids + (r * Hkv + g) * K;
        const int64_t n = visible_tokens(p, sel, p->q_offset + i, tok);
        const int64_t qi = ((b * p->n_q + i) * Hkv + g) * DI;
        double* dq = d_iq + (r * Hkv + g) * DI;
        for (int64_t c = 0; c < DI; ++c) dq[c] = 0.0;
        kl[r * Hkv + g] = 0.0;
        if (n == 0) continue;
        /* the Main Branch target: mean over the group's heads */
        for (int64_t a = 0; a < n; ++a) pm[a] = 0.0;
        for (int64_t h = g * G; h < (g + 1) * G; ++h) {
          attend_row(p, q, k, k, dtype, b, i, h, tok, n, x, o); /* x = P_h */
          for (int64_t a = 0; a < n; ++a) pm[a] += x[a] / (double)G;
        }
        /* the Index Branch distribution over the same tokens */
        double m = -INFINITY;
        for (int64_t a = 0; a < n; ++a) {
          const int64_t ki = ((b * p->n_k + tok[a]) * Hkv + g) * DI;
          double sc = 0.0;
          for (int64_t c = 0; c < DI; ++c) sc += widen(iq, dtype, qi + c) * widen(ik, dtype, ki + c);
          si[a] = sc;
          if (sc > m) m = sc;
        }
        double l = 0.0;
        for (int64_t a = 0; a < n; ++a) l += exp(si[a] - m);
        const double lse = m + log(l);
        double acc = 0.0;
        for (int64_t a = 0; a < n; ++a) {
          const double logpi = si[a] - lse;
          if (pm[a] > 0.0) acc += pm[a] * (log(pm[a]) - logpi);
          const double gs = loss_scale * (exp(logpi) - pm[a]);
          const int64_t ki = ((b * p->n_k + tok[a]) * Hkv + g) * DI;
          for (int64_t c = 0; c < DI; ++c) {
            dq[c] += gs * widen(ik, dtype, ki + c);
            d_ik[ki + c] += gs * widen(iq, dtype, qi + c);
          }
        }
        kl[r * Hkv + g] = acc;
      }
    }
    free(x);
    free(pm);
    free(si);
    free(tok);
    free(o);
  }
  return 0;
}

/* ---- MXFP8: OCP Microscaling Formats v1.0 (E4M3 elements, E8M0 scales) ---- */

double mo_e4m3_value(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  /* exponent field 0: subnormal m/8 * 2^(1-7); otherwise (1 + m/8) * 2^(e-7) */
  const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

uint8_t mo_e4m3_encode(double y) {
  const uint8_t sign = signbit(y) ? 0x80 : 0x00;
  const double a = fabs(y);
  if (a >= 448.0) return sign | 0x7E; /* saturate at the largest finite value */
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; rounding up to 8 lands on 2^-6 */
    const double m = nearbyint(ldexp(a, 9)); /* round half to even */
    return sign | (uint8_t)m;
  }
  int ex;
  frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;  /* a in [2^e, 2^(e+1)) */
  double q = nearbyint(ldexp(a, 3 - e)); /* in [8, 16]: 1.mmm in eighths */
  if (q == 16.0) {
    q = 8.0;
    e += 1;
  }
  return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

int mo_mxfp8_quantize(const void* src, int dtype, int64_t n_rows, int32_t row_len, uint8_t* codes,
                      uint8_t* scales) {
  if (!src || !codes || !scales || n_rows < 0 || row_len <= 0 || row_len % 32) return -1;
  if (dtype != MO_F32 && dtype != MO_BF16 && dtype != MO_F64) return -6;
  const int64_t nblocks = n_rows * (row_len / 32);
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < nblocks; ++blk) {
    const int64_t base = blk * 32;
    double amax = 0.0;
    for (int c = 0; c < 32; ++c) {
      const double a = fabs(widen(src, dtype, base + c));
      if (a > amax) amax = a;
    }
    int e = -127;
    if (amax > 0.0) {
      int ex;
      frexp(amax, &ex);
      e = (ex - 1) - 8; /* floor(log2(amax)) - emax(E4M3) */
      if (e < -127) e = -127;
      if (e > 127) e = 127;
    }
    scales[blk] = (uint8_t)(e + 127);
    for (int c = 0; c < 32; ++c) codes[base + c] = mo_e4m3_encode(ldexp(widen(src, dtype, base + c), -e));
  }
  return 0;
}

int mo_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n_rows, int32_t row_len, double* out) {
  if (!codes || !scales || !out || n_rows < 0 || row_len <= 0 || row_len % 32) return -1;
  const int64_t n = n_rows * row_len;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = ldexp(mo_e4m3_value(codes[i]), (int)scales[i / 32] - 127);
  return 0;
}
