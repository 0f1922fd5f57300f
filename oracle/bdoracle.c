/*
 * bdoracle.c — plain fp64 CPU reference for BDLM attention (see bdoracle.h).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.
 *
 * Every function is a direct transcription of a definition on the pages,
 * evaluated one query row (or one key row) at a time, with no tiling, no
 * fusion and no reordering beyond the definition.  Threads split the
 * independent rows only, so each output element has exactly one writer and
 * the result does not depend on the thread count.
 */
#include "bdoracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* One input element as a double.  bf16 is the top half of an IEEE float. */
static inline double ld(const orc_problem* p, const void* base, int64_t idx) {
  if (p->in_dtype == ORC_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

static inline int64_t qoff(const orc_problem* p, int64_t b, int64_t i, int64_t h) {
  return ((b * 2 * (int64_t)p->L + i) * p->hq + h) * p->d;
}
static inline int64_t koff(const orc_problem* p, int64_t b, int64_t j, int64_t g) {
  return ((b * 2 * (int64_t)p->L + j) * p->hkv + g) * p->d;
}

/*
 * Mask predicate over the doubled input.
 *  - Corrupted query of block b reads exactly [K_b ; K^clean_{<b}]: its own
 *    corrupted block (bidirectionally) and the clean blocks before it —
 *    "CSBP 完全拆解", section "传统上下文并行为什么会传错东西", the key/value
 *    set equation of target block b; restated in the CSBP forward equation
 *    O_b = Attn(Q_b, [K_b; K^clean_<b], [V_b; V^clean_<b]).
 *  - The clean copy is the complete clean context and runs causal attention
 *    over itself ("CSBP 完全拆解", same section, and Turbo-dLLM page,
 *    "Load balancing: pairing early and late blocks", "clean causal
 *    attention").  Read here as block-causal (a clean token sees every clean
 *    token of its own and earlier blocks); token-causal is a parameter.
 *  - Clean queries never read corrupted keys: corrupted K/V are read only by
 *    their own block (Turbo-dLLM page, "Method").
 */
/*  - Sliding window (optional): "CSBP 完全拆解", section "实验数字：256K 上下
 *    文下的主结果", and the Turbo-dLLM page, "Where does the time go?", name
 *    a 1,024-token sliding window over the clean context for most layers of
 *    one model without defining it further.  Read here on token distance: a
 *    query at token position t (the clean token t, or the corrupted token
 *    at offset i of block b, t = b*M + i) sees clean token j only if
 *    t - j < window.  Corrupted keys of the query's own block are not
 *    windowed.  window = 0: no window.
 */
int orc_visible(const orc_problem* p, int64_t i, int64_t j) {
  const int64_t L = p->L, M = p->M;
  if (i < L) {
    if (j >= L) return 0;
    if (p->window > 0 && i - j >= p->window) return 0;
    if (p->token_causal) return j <= i;
    return j / M <= i / M;
  }
  {
    const int64_t b = (i - L) / M, t = i - L;
    if (j < L) return j / M < b && !(p->window > 0 && t - j >= p->window);
    return (j - L) / M == b;
  }
}

static int key_in(const orc_problem* p, const orc_keys* ks, int64_t j) {
  int r;
  if (j >= p->L) return ks->local != 0;
  if (ks->n_ranges < 0) return 1;
  for (r = 0; r < ks->n_ranges && r < 2; ++r)
    if (j >= ks->lo[r] && j < ks->hi[r]) return 1;
  return 0;
}

static int row_in(const orc_problem* p, const orc_share* sh, int64_t i) {
  int r;
  if (sh->all) return 1;
  if (i < p->L) {
    for (r = 0; r < sh->n_clean && r < 2; ++r)
      if (i >= sh->clean_lo[r] && i < sh->clean_hi[r]) return 1;
    return 0;
  }
  return sh->owned != NULL && sh->owned[(i - p->L) / p->M] != 0;
}

static double score(const orc_problem* p, const void* q, const void* k,
                    int64_t b, int64_t h, int64_t i, int64_t j) {
  const int64_t g = h / (p->hq / p->hkv);
  const int64_t qo = qoff(p, b, i, h), ko = koff(p, b, j, g);
  double s = 0.0;
  int t;
  for (t = 0; t < p->d; ++t) s += ld(p, q, qo + t) * ld(p, k, ko + t);
  return p->scale * s;
}

/*
 * One row of O_r = softmax(Q_r K^T / sqrt(d_h) + M_r) V ("CSBP 完全拆解",
 * section "传统上下文并行为什么会传错东西", the CP attention equation), with
 * the mask M_r given by orc_visible and the key set restricted to `keys`.
 * LSE is the natural log of the softmax denominator of the scaled logits.
 * A row that sees no key gets O = 0 and LSE = -inf.
 * `s` is caller scratch of 2L doubles.
 */
static void fwd_row(const orc_problem* p, const orc_keys* keys, const void* q,
                    const void* k, const void* v, int64_t b, int64_t h,
                    int64_t i, double* s, double* o, double* lse) {
  const int64_t n2 = 2 * (int64_t)p->L;
  const int64_t g = h / (p->hq / p->hkv);
  double m = -INFINITY, l = 0.0;
  int64_t j;
  int t;
  for (t = 0; t < p->d; ++t) o[t] = 0.0;
  for (j = 0; j < n2; ++j) {
    if (orc_visible(p, i, j) && key_in(p, keys, j)) {
      s[j] = score(p, q, k, b, h, i, j);
      if (s[j] > m) m = s[j];
    } else {
      s[j] = -INFINITY;
    }
  }
  if (m == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  for (j = 0; j < n2; ++j) {
    if (s[j] == -INFINITY) continue;
    {
      const double e = exp(s[j] - m);
      const int64_t vo = koff(p, b, j, g);
      l += e;
      for (t = 0; t < p->d; ++t) o[t] += e * ld(p, v, vo + t);
    }
  }
  for (t = 0; t < p->d; ++t) o[t] /= l;
  *lse = m + log(l);
}

void orc_fwd_rows(const orc_problem* p, const orc_keys* keys, const void* q,
                  const void* k, const void* v, int64_t n, const int32_t* b,
                  const int32_t* h, const int64_t* i, double* o, double* lse) {
  const int64_t n2 = 2 * (int64_t)p->L;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n2);
    int64_t r;
#pragma omp for schedule(dynamic, 1)
    for (r = 0; r < n; ++r)
      fwd_row(p, keys, q, k, v, b[r], h[r], i[r], s, o + r * p->d, lse + r);
    free(s);
  }
}

void orc_fwd(const orc_problem* p, const orc_keys* keys, const void* q,
             const void* k, const void* v, double* o, double* lse) {
  const int64_t n2 = 2 * (int64_t)p->L;
  const int64_t nrows = (int64_t)p->batch * n2 * p->hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n2);
    int64_t r;
#pragma omp for schedule(dynamic, 16)
    for (r = 0; r < nrows; ++r) {
      const int64_t h = r % p->hq, i = (r / p->hq) % n2, b = r / (p->hq * n2);
      fwd_row(p, keys, q, k, v, b, h, i, s, o + r * p->d, lse + r);
    }
    free(s);
  }
}

/*
 * Backward of the loss l = sum(O * dO) through one softmax row (the pages'
 * "exact fused backward", Turbo-dLLM page, "Block Diffusion Optimizations"
 * table; the row equations are the chain rule of the CP attention equation):
 *   D_i = sum_t dO_i[t] O_i[t]
 *   P_ij = exp(s_ij - LSE_i)
 *   dV_j += P_ij dO_i ;  dP_ij = dO_i . v_j ;  dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i += scale dS_ij k_j ;  dK_j += scale dS_ij q_i
 * LSE and O are taken over keys_norm (the full key set of the softmax); only
 * pairs whose key lies in keys_grad contribute, which is how one streamed
 * shard's share of the gradient is expressed ("CSBP 完全拆解", section
 * "CSBP：BP 管损坏块，CP 管干净上下文": clean dK/dV collect contributions
 * from many blocks).
 */
static void dq_row(const orc_problem* p, const orc_keys* kn,
                   const orc_keys* kg, const void* q, const void* k,
                   const void* v, const void* dO, int64_t b, int64_t h,
                   int64_t i, double* s, double* dq, double* o, double* lse) {
  const int64_t n2 = 2 * (int64_t)p->L;
  const int64_t g = h / (p->hq / p->hkv);
  const int64_t qo = qoff(p, b, i, h);
  double D = 0.0;
  int64_t j;
  int t;
  fwd_row(p, kn, q, k, v, b, h, i, s, o, lse);
  for (t = 0; t < p->d; ++t) dq[t] = 0.0;
  if (*lse == -INFINITY) return;
  for (t = 0; t < p->d; ++t) D += ld(p, dO, qo + t) * o[t];
  for (j = 0; j < n2; ++j) {
    if (s[j] == -INFINITY || !key_in(p, kg, j)) continue;
    {
      const int64_t ko = koff(p, b, j, g);
      const double P = exp(s[j] - *lse);
      double dP = 0.0, dS;
      for (t = 0; t < p->d; ++t) dP += ld(p, dO, qo + t) * ld(p, v, ko + t);
      dS = P * (dP - D);
      for (t = 0; t < p->d; ++t) dq[t] += p->scale * dS * ld(p, k, ko + t);
    }
  }
}

void orc_dq_rows(const orc_problem* p, const orc_keys* keys_norm,
                 const orc_keys* keys_grad, const void* q, const void* k,
                 const void* v, const void* dO, int64_t n, const int32_t* b,
                 const int32_t* h, const int64_t* i, double* dq, double* o,
                 double* lse) {
  const int64_t n2 = 2 * (int64_t)p->L;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n2);
    int64_t r;
#pragma omp for schedule(dynamic, 1)
    for (r = 0; r < n; ++r)
      dq_row(p, keys_norm, keys_grad, q, k, v, dO, b[r], h[r], i[r], s,
             dq + r * p->d, o + r * p->d, lse + r);
    free(s);
  }
}

/* Per-row statistics (LSE_i, D_i) over keys_norm, computed on demand for the
 * query rows that a set of key rows needs.  Index: (b*2L + i)*hq + h. */
typedef struct row_stats {
  double* lse;
  double* D;
  uint8_t* need;
} row_stats;

static void stats_compute(const orc_problem* p, const orc_keys* kn,
                          const void* q, const void* k, const void* v,
                          const void* dO, row_stats* st) {
  const int64_t n2 = 2 * (int64_t)p->L;
  const int64_t nrows = (int64_t)p->batch * n2 * p->hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n2);
    double* o = (double*)malloc(sizeof(double) * (size_t)p->d);
    int64_t r;
#pragma omp for schedule(dynamic, 4)
    for (r = 0; r < nrows; ++r) {
      if (!st->need[r]) continue;
      {
        const int64_t h = r % p->hq, i = (r / p->hq) % n2,
                      b = r / (p->hq * n2);
        const int64_t qo = qoff(p, b, i, h);
        double lse, D = 0.0;
        int t;
        fwd_row(p, kn, q, k, v, b, h, i, s, o, &lse);
        if (lse != -INFINITY)
          for (t = 0; t < p->d; ++t) D += ld(p, dO, qo + t) * o[t];
        st->lse[r] = lse;
        st->D[r] = D;
      }
    }
    free(o);
    free(s);
  }
}

/* dK_j, dV_j of one key row: the same per-pair terms as dq_row, summed over
 * every query head of KV head g (query head h uses KV head h / (hq/hkv)) and
 * every share row that sees key j. */
static void dkdv_key(const orc_problem* p, const orc_share* sh,
                     const orc_keys* kn, const orc_keys* kg, const void* q,
                     const void* k, const void* v, const void* dO,
                     const row_stats* st, int64_t b, int64_t g, int64_t j,
                     double* dk, double* dv) {
  const int64_t n2 = 2 * (int64_t)p->L;
  const int64_t G = p->hq / p->hkv;
  const int64_t ko = koff(p, b, j, g);
  int64_t h, i;
  int t;
  for (t = 0; t < p->d; ++t) dk[t] = dv[t] = 0.0;
  if (!key_in(p, kn, j) || !key_in(p, kg, j)) return;
  for (h = g * G; h < (g + 1) * G; ++h) {
    for (i = 0; i < n2; ++i) {
      if (!row_in(p, sh, i) || !orc_visible(p, i, j)) continue;
      {
        const int64_t r = (b * n2 + i) * p->hq + h;
        const int64_t qo = qoff(p, b, i, h);
        const double P = exp(score(p, q, k, b, h, i, j) - st->lse[r]);
        double dP = 0.0, dS;
        for (t = 0; t < p->d; ++t) dP += ld(p, dO, qo + t) * ld(p, v, ko + t);
        dS = P * (dP - st->D[r]);
        for (t = 0; t < p->d; ++t) {
          dv[t] += P * ld(p, dO, qo + t);
          dk[t] += p->scale * dS * ld(p, q, qo + t);
        }
      }
    }
  }
}

static void stats_alloc(const orc_problem* p, row_stats* st) {
  const size_t nrows = (size_t)p->batch * 2 * (size_t)p->L * (size_t)p->hq;
  st->lse = (double*)malloc(sizeof(double) * nrows);
  st->D = (double*)malloc(sizeof(double) * nrows);
  st->need = (uint8_t*)calloc(nrows, 1);
}

static void stats_free(row_stats* st) {
  free(st->lse);
  free(st->D);
  free(st->need);
}

void orc_dkdv_rows(const orc_problem* p, const orc_share* share,
                   const orc_keys* keys_norm, const orc_keys* keys_grad,
                   const void* q, const void* k, const void* v, const void* dO,
                   int64_t n, const int32_t* b, const int32_t* g,
                   const int64_t* j, double* dk, double* dv) {
  const int64_t n2 = 2 * (int64_t)p->L;
  const int64_t G = p->hq / p->hkv;
  row_stats st;
  int64_t r;
  stats_alloc(p, &st);
  /* mark the query rows the requested keys need */
  for (r = 0; r < n; ++r) {
    int64_t h, i;
    for (h = g[r] * G; h < (g[r] + 1) * G; ++h)
      for (i = 0; i < n2; ++i)
        if (row_in(p, share, i) && orc_visible(p, i, j[r]))
          st.need[((int64_t)b[r] * n2 + i) * p->hq + h] = 1;
  }
  stats_compute(p, keys_norm, q, k, v, dO, &st);
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < n; ++r)
    dkdv_key(p, share, keys_norm, keys_grad, q, k, v, dO, &st, b[r], g[r],
             j[r], dk + r * p->d, dv + r * p->d);
  stats_free(&st);
}

void orc_bwd(const orc_problem* p, const orc_share* share,
             const orc_keys* keys_norm, const orc_keys* keys_grad,
             const void* q, const void* k, const void* v, const void* dO,
             double* dq, double* dk, double* dv) {
  const int64_t n2 = 2 * (int64_t)p->L;
  const int64_t nq = (int64_t)p->batch * n2 * p->hq;
  const int64_t nk = (int64_t)p->batch * n2 * p->hkv;
  row_stats st;
  int64_t r;
  stats_alloc(p, &st);
  for (r = 0; r < nq; ++r) st.need[r] = (uint8_t)row_in(p, share, (r / p->hq) % n2);
  stats_compute(p, keys_norm, q, k, v, dO, &st);
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n2);
    double* o = (double*)malloc(sizeof(double) * (size_t)p->d);
    double lse;
    int64_t rr;
#pragma omp for schedule(dynamic, 4)
    for (rr = 0; rr < nq; ++rr) {
      const int64_t h = rr % p->hq, i = (rr / p->hq) % n2,
                    b = rr / (p->hq * n2);
      if (st.need[rr])
        dq_row(p, keys_norm, keys_grad, q, k, v, dO, b, h, i, s,
               dq + rr * p->d, o, &lse);
      else
        memset(dq + rr * p->d, 0, sizeof(double) * (size_t)p->d);
    }
#pragma omp for schedule(dynamic, 4)
    for (rr = 0; rr < nk; ++rr) {
      const int64_t g = rr % p->hkv, j = (rr / p->hkv) % n2,
                    b = rr / (p->hkv * n2);
      dkdv_key(p, share, keys_norm, keys_grad, q, k, v, dO, &st, b, g, j,
               dk + rr * p->d, dv + rr * p->d);
    }
    free(o);
    free(s);
  }
  stats_free(&st);
}

/*
 * Log-sum-exp merge of two partial attention results over disjoint key sets
 * ("CSBP 完全拆解", section "在线 softmax 合并：为什么分两段算仍是同一个注意力",
 * the equations for m, w_1, w_2, O and z):
 *   m = max(z1, z2);  w_k = exp(z_k - m);
 *   O = (w1 O1 + w2 O2) / (w1 + w2);  z = m + log(w1 + w2).
 * An empty part is (O = 0, z = -inf); two empty parts merge to (0, -inf).
 */
void orc_merge(int64_t n, int32_t d, const double* o1, const double* z1,
               const double* o2, const double* z2, double* o, double* z) {
  int64_t r;
  for (r = 0; r < n; ++r) {
    const double m = z1[r] > z2[r] ? z1[r] : z2[r];
    int t;
    if (m == -INFINITY) {
      for (t = 0; t < d; ++t) o[r * d + t] = 0.0;
      z[r] = -INFINITY;
      continue;
    }
    {
      const double w1 = exp(z1[r] - m), w2 = exp(z2[r] - m);
      for (t = 0; t < d; ++t)
        o[r * d + t] = (w1 * o1[r * d + t] + w2 * o2[r * d + t]) / (w1 + w2);
      z[r] = m + log(w1 + w2);
    }
  }
}

/*
 * Dual-end block assignment: block b and block B+1-b (1-indexed; b and
 * B-1-b 0-indexed) always go to the same rank ("CSBP 完全拆解", section
 * "负载均衡：为什么要首尾块配对"; Turbo-dLLM page, "Load balancing: pairing
 * early and late blocks").  Rank r of P takes the c = B/(2P) pairs
 * r*c .. r*c+c-1 (consecutive pairs per rank: the "dual-end zigzag layout
 * pairs early and late regions", Turbo-dLLM page, "Block Diffusion
 * Optimizations" table).  Output sorted ascending.  Returns B/P, or -1.
 */
int orc_assign_blocks(int32_t B, int32_t P, int32_t r, int32_t* out) {
  int32_t c, t, n = 0;
  if (B <= 0 || P <= 0 || r < 0 || r >= P || B % (2 * P) != 0) return -1;
  c = B / (2 * P);
  for (t = 0; t < c; ++t) out[n++] = r * c + t;               /* early member */
  for (t = c - 1; t >= 0; --t) out[n++] = B - 1 - (r * c + t); /* its late mate */
  return n;
}

/*
 * Zigzag clean shard s of P: the clean sequence in 2P equal chunks, shard s
 * holding an early chunk and its late mate, chunks s and 2P-1-s (the same
 * early/late pairing applied to clean-sequence sharding; Turbo-dLLM page,
 * "Load balancing: pairing early and late blocks").  Returns 2, or -1.
 */
int orc_clean_shard(int64_t L, int32_t P, int32_t s, int64_t lo[2],
                    int64_t hi[2]) {
  int64_t w;
  if (L <= 0 || P <= 0 || s < 0 || s >= P || L % (2 * P) != 0) return -1;
  w = L / (2 * P);
  lo[0] = s * w;
  hi[0] = lo[0] + w;
  lo[1] = (2 * (int64_t)P - 1 - s) * w;
  hi[1] = lo[1] + w;
  return 2;
}
