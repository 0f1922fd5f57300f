/*
 * bdoracle — plain, slow, fp64 CPU reference for block-diffusion (BDLM)
 * attention and its context-sharded block-parallel (CSBP) per-rank form.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (libbdattn) never links, loads or calls it, and it shares no code with it.
 *
 * Layout ("doubled input"): every example holds 2L positions.  Positions
 * [0, L) are the clean copy (token t at position t); positions [L, 2L) are
 * the corrupted copy (token t at position L + t).  Blocks have M tokens.
 *   q, dO : [batch][2L][hq][d]
 *   k, v  : [batch][2L][hkv][d]
 * Inputs are float32 or bf16 bit patterns (uint16), chosen by `in_dtype`;
 * every product and sum is taken in double.
 *
 * Sources (cited by page title and section):
 *  - "CSBP 完全拆解：块并行如何让长上下文扩散语言模型少传无效 KV"
 *    (pinghaoyang.com.cn), sections on the block factorisation, the CP
 *    attention equation, the corrupted-query key set, BP, the CSBP forward,
 *    the online-softmax merge and dual-end load balancing.
 *  - "Block Parallelism for Efficient Distributed Long-Context Diffusion
 *    Language Model Training" (Turbo-dLLM project page), sections
 *    "Background", "Method" and "Load balancing: pairing early and late
 *    blocks".
 */
#ifndef BDORACLE_H
#define BDORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };

typedef struct orc_problem {
  int32_t batch, L, M, hq, hkv, d;
  int32_t token_causal; /* clean-copy mask: 0 block-causal, 1 token-causal */
  int32_t in_dtype;     /* ORC_F32 or ORC_BF16 */
  double scale;         /* logit scale, normally 1/sqrt(d) */
  int32_t window;       /* clean-key sliding window in tokens; 0 = none (see orc_visible) */
} orc_problem;

/* Key subset of one call.  n_ranges < 0: every clean key; otherwise the
 * clean keys are the union of n_ranges (<= 2) half-open token ranges.
 * local != 0 adds the corrupted keys (each query still only sees its own
 * block's corrupted keys through the mask). */
typedef struct orc_keys {
  int32_t n_ranges;
  int32_t local;
  int64_t lo[2], hi[2];
} orc_keys;

/* Query rows a rank owns.  all != 0: every row.  Otherwise clean rows in
 * the n_clean (<= 2) token ranges plus the corrupted rows of every block b
 * with owned[b] != 0. */
typedef struct orc_share {
  int32_t all;
  int32_t n_clean;
  int64_t clean_lo[2], clean_hi[2];
  const uint8_t* owned; /* [L/M] or NULL */
} orc_share;

int orc_visible(const orc_problem* p, int64_t i, int64_t j);
int orc_num_threads(void);

/* O and LSE of n selected query rows (batch b[r], head h[r], position i[r]). */
void orc_fwd_rows(const orc_problem* p, const orc_keys* keys, const void* q,
                  const void* k, const void* v, int64_t n, const int32_t* b,
                  const int32_t* h, const int64_t* i, double* o, double* lse);

/* O and LSE of every position: o [batch][2L][hq][d], lse [batch][2L][hq]. */
void orc_fwd(const orc_problem* p, const orc_keys* keys, const void* q,
             const void* k, const void* v, double* o, double* lse);

/* dQ (and O, LSE) of n selected query rows for the loss sum(O * dO).
 * Softmax over keys_norm; only pairs with the key in keys_grad contribute. */
void orc_dq_rows(const orc_problem* p, const orc_keys* keys_norm,
                 const orc_keys* keys_grad, const void* q, const void* k,
                 const void* v, const void* dO, int64_t n, const int32_t* b,
                 const int32_t* h, const int64_t* i, double* dq, double* o,
                 double* lse);

/* dK, dV of n selected key rows (batch b[r], KV head g[r], position j[r]),
 * summed over the query heads of the group and the share's query rows. */
void orc_dkdv_rows(const orc_problem* p, const orc_share* share,
                   const orc_keys* keys_norm, const orc_keys* keys_grad,
                   const void* q, const void* k, const void* v, const void* dO,
                   int64_t n, const int32_t* b, const int32_t* g,
                   const int64_t* j, double* dk, double* dv);

/* Full backward over a share: dq [batch][2L][hq][d] (zero outside the
 * share), dk, dv [batch][2L][hkv][d]. */
void orc_bwd(const orc_problem* p, const orc_share* share,
             const orc_keys* keys_norm, const orc_keys* keys_grad,
             const void* q, const void* k, const void* v, const void* dO,
             double* dq, double* dk, double* dv);

/* Log-sum-exp merge of two partial results over disjoint key sets. */
void orc_merge(int64_t n, int32_t d, const double* o1, const double* z1,
               const double* o2, const double* z2, double* o, double* z);

/* Dual-end block assignment and zigzag clean shard. */
int orc_assign_blocks(int32_t B, int32_t P, int32_t r, int32_t* out);
int orc_clean_shard(int64_t L, int32_t P, int32_t s, int64_t lo[2],
                    int64_t hi[2]);

#ifdef __cplusplus
}
#endif
#endif
