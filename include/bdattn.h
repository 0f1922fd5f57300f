/*
 * bdattn.h — C ABI of libbdattn: block-diffusion (BDLM) attention over the
 * doubled clean + corrupted input, and its context-sharded block-parallel
 * (CSBP) per-rank form, for AMD MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *  [P1] "CSBP 完全拆解：块并行如何让长上下文扩散语言模型少传无效 KV"
 *       (pinghaoyang.com.cn).
 *  [P3] "Block Parallelism for Efficient Distributed Long-Context Diffusion
 *       Language Model Training" (Turbo-dLLM project page).
 *
 * What is computed.  An example of L clean tokens in blocks of M tokens
 * (B = L/M blocks) is processed as 2L positions: the clean copy and the
 * corrupted copy ([P1] "块扩散模型到底多了哪一种并行机会", factorisation
 * p(x) = prod_b p(x^(b) | x^(<b)); [P3] "Background", every token appears
 * twice).  Attention is O = softmax(Q K^T * scale + mask) V
 * ([P1] "传统上下文并行为什么会传错东西", CP attention equation) with:
 *   - a corrupted query of block b seeing its own corrupted block
 *     (bidirectionally) and the clean tokens of blocks < b, nothing else
 *     ([P1] same section, key/value set [K_b; K^clean_<b]; [P1] "CSBP：BP 管
 *     损坏块，CP 管干净上下文", CSBP forward equation);
 *   - a clean query of block c seeing the clean tokens of blocks <= c
 *     (block-causal; BDATTN_CLEAN_TOKEN_CAUSAL gives token-causal instead);
 *     clean queries never see corrupted keys ([P3] "Method": corrupted K/V
 *     are only read by their own block).
 * LSE is the natural-log softmax denominator of the scaled logits.
 *
 * Row spaces.
 *   - A *share* is the set of query rows one rank owns: up to two clean token
 *     ranges and a sorted list of corrupted blocks B_r ([P1] "BP：把损坏块留
 *     在本地", block set B_r).  Its rows, in order: the clean rows of range
 *     0, of range 1, then M rows per block of B_r in list order.  R is the
 *     row count.  o, lse, d_o, delta and dq use this order.
 *   - q_clean holds the share's clean rows in share order (packed).
 *   - q_corr, k_corr, v_corr hold the share's corrupted rows packed: block
 *     blocks[i] occupies rows [i*M, (i+1)*M).
 *   - k_clean, v_clean are indexed by clean token (row t = token t); only the
 *     rows in the call's key ranges are read.
 *   The whole-mask case (one launch for the whole structured mask, [P3]
 *   "Block Diffusion Optimizations" table) is blocks = 0..B-1, clean query
 *   range [0, L), key range [0, L) and include_local = 1; on a
 *   [batch, 2L, h, d] tensor, the corrupted views are the base pointer plus
 *   L rows with the same strides.
 *   - A *call's key set* is up to two clean token ranges plus, when
 *     include_local != 0, the corrupted keys of the share (each query still
 *     sees only its own block's).  A call computes exactly the visible pairs
 *     (query of the share, key of the call).  A row with no visible key in a
 *     call gets O = 0 and LSE = -inf.
 *
 * Tensors.  bdattn_tensor gives a base pointer (device memory) and strides
 * in elements for batch, row and head; the head dimension d is contiguous.
 * dtype BDATTN_BF16 or BDATTN_F32 as stated per argument.  Values of bf16
 * inputs must lie within the IEEE half range (|x| <= 65504): products with
 * probabilities run in fp16 matrix cores, on operands converted from bf16
 * (exact in that range).  A value outside it (or NaN) is clamped to the
 * range (NaN stays NaN) and raises the call's range flag, which
 * bdattn_workspace_status reports as BDATTN_ERANGE; such a call's results
 * are not those of the inputs.  The backward also needs each per-pair term
 * |dO_i . v_j - D_i| below 65504 * 2^c_i (c_i the row's probability scale,
 * see bdattn_bwd).
 *
 * Conventions for every entry point.
 *   - Device buffers are caller-owned; the library allocates no device
 *     memory.  Scratch comes from `workspace` (size from
 *     bdattn_workspace_bytes).
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL =
 *     the null stream); buffers must stay valid until it completes.  Calls on
 *     one stream are ordered; calls that share output buffers, or a
 *     workspace (it holds the call's range flag and the work-queue heads its
 *     kernels take items from), must not run concurrently on different
 *     streams.
 *   - Every argument is validated on the host before any HIP call; an invalid
 *     argument returns BDATTN_EINVAL (or ENOTSUP / EWORKSPACE) and enqueues
 *     nothing.  A failed launch returns BDATTN_EHIP.  Nothing aborts or
 *     throws across the ABI.
 */
#ifndef BDATTN_H
#define BDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bdattn_status {
  BDATTN_OK = 0,
  BDATTN_EINVAL = -1,     /* invalid argument                          */
  BDATTN_ENOTSUP = -2,    /* valid but not supported (dtype, d, ...)    */
  BDATTN_EHIP = -3,       /* a HIP runtime call or launch failed        */
  BDATTN_EWORKSPACE = -4, /* workspace NULL or smaller than required    */
  BDATTN_ERANGE = -5,     /* an input value lay outside the fp16 range  */
  BDATTN_ESCRATCH = -6    /* bdattn_fwd_static: problem needs more than
                             BDATTN_STATIC_SCRATCH_BYTES of scratch      */
} bdattn_status;

typedef enum bdattn_dtype { BDATTN_BF16 = 0, BDATTN_F32 = 1 } bdattn_dtype;

typedef enum bdattn_clean_mask {
  BDATTN_CLEAN_BLOCK_CAUSAL = 0, /* clean token of block c sees clean blocks <= c */
  BDATTN_CLEAN_TOKEN_CAUSAL = 1  /* clean token t sees clean tokens <= t          */
} bdattn_clean_mask;

/* Problem statement: L clean tokens, block size M (M divides L), hq query
 * heads sharing hkv key/value heads (query head h uses KV head
 * h / (hq/hkv)), head dimension d (64 or 128), input dtype, clean-copy
 * mask, logit scale (<= 0 selects 1/sqrt(d); [P1] CP attention equation),
 * and an optional sliding window over the clean keys.
 *
 * Sliding window ([P1] "实验数字：256K 上下文下的主结果" and [P3] "Under the
 * hood", "Where does the time go?": most layers of one of the pages' models
 * attend through a 1,024-token sliding window, and the sharded form then
 * exchanges only the clean rows a rank's queries can see).  window = 0 means
 * none.  Otherwise a query at token position t -- clean token t, or the
 * corrupted token at offset i of block b, t = b*M + i -- sees clean key j
 * only if t - j < window, in addition to the rules above.  The corrupted
 * keys of the query's own block are not windowed. */
typedef struct bdattn_problem {
  int32_t batch, L, M, hq, hkv, d;
  int32_t dtype;      /* bdattn_dtype of q, k, v, d_o */
  int32_t clean_mask; /* bdattn_clean_mask */
  float scale;
  int32_t window;     /* clean-key sliding window in tokens; 0 = none */
} bdattn_problem;

/* Maximum number of runs of consecutive block ids in a share's block list. */
#define BDATTN_MAX_RUNS 8

/* Query rows owned by one rank: sorted block list B_r (host pointer,
 * strictly increasing ids in [0, B), at most BDATTN_MAX_RUNS runs of
 * consecutive ids) and up to two disjoint increasing clean token ranges
 * (ranges need not be block aligned). */
typedef struct bdattn_share {
  const int32_t* blocks;
  int32_t n_blocks;
  int32_t n_clean;
  int32_t clean_lo[2], clean_hi[2];
} bdattn_share;

/* Key set of one call: up to two disjoint increasing clean token ranges and
 * whether the share's corrupted keys take part ([P1] "在线 softmax 合并",
 * the local block-diagonal part and the clean-prefix part are separate
 * launches merged by LSE). */
typedef struct bdattn_kv {
  int32_t n;
  int32_t lo[2], hi[2];
  int32_t include_local;
} bdattn_kv;

typedef struct bdattn_tensor {
  void* ptr;
  int64_t batch_stride, row_stride, head_stride; /* in elements */
} bdattn_tensor;

/* Dual-end block assignment ([P1] "负载均衡：为什么要首尾块配对"; [P3]
 * "Load balancing: pairing early and late blocks"): block b and block
 * B-1-b (0-indexed) go to the same rank; rank r of P takes the B/(2P)
 * consecutive pairs starting at pair r*B/(2P).  Writes B/P sorted ids to
 * `out` (host).  Requires B % (2P) == 0.  Pure host function. */
int bdattn_assign_blocks(int32_t B, int32_t P, int32_t r, int32_t* out);

/* Zigzag clean shard s of P ([P3] "Load balancing": the same early-late
 * pairing applied to clean-sequence sharding): clean chunks s and 2P-1-s of
 * 2P equal chunks, as a key set with include_local = 0.  Requires
 * L % (2P) == 0.  Pure host function. */
int bdattn_clean_shard(int32_t L, int32_t P, int32_t s, bdattn_kv* out);

/* Work items of the query-major kernels (forward and dQ) for this call
 * (bit-exact contract), four int32 values each (batch, query head, first
 * query tile, second query tile or -1), in queue order: item w is the
 * (w / 8)-th item of the queue of XCD w % 8, and each XCD's queue holds a
 * contiguous block of the logical order described next.  A workgroup takes the next item of its own
 * XCD's queue, or, when that is empty, of the other queues in turn (a
 * launch has a quarter more workgroups than items, so a die that finishes
 * early takes over the others' remaining items).  Query
 * tiles are numbered over the share rows in tiles of 128 rows, clean
 * ranges first; within each kind, tile t is paired with its mirror n-1-t so
 * that every workgroup does the same work (dual-end pairing applied to the
 * query tiles of one GPU).  `cap` is the capacity of `items` in int32s;
 * `*n` receives the number of work items.  Pure host function. */
int bdattn_plan_order(const bdattn_problem* problem, const bdattn_share* share,
                      const bdattn_kv* kv, int32_t* items, int64_t cap,
                      int64_t* n);

/* Work items of the key-major backward kernel (dK/dV) for this call
 * (bit-exact contract; queues and dynamic assignment as for
 * bdattn_plan_order, except that each queue hands out its block longest
 * first: item w is the (w / 8)-th item queue w % 8 hands out, its block's
 * clean-tile pairs in logical order, then its corrupted-key tiles), by the
 * same dual-end rule applied to key tiles
 * ([P1] "负载均衡：为什么要首尾块配对"; [P3] "Load balancing: pairing early
 * and late blocks"): for each work item, four int32 values
 * (batch, KV head, first key tile, second key tile or -1).  Key tiles hold
 * 128 keys of one key segment: the call's clean ranges in order, then its
 * corrupted keys, each segment starting a new tile.  Clean tile t (counted
 * over the clean segments) is paired with clean tile n-1-t, the earlier one
 * first, so each workgroup's two tiles together are seen by the same number
 * of query rows wherever the rows seeing a key fall linearly with its
 * position (the whole mask); tiles of corrupted keys, each seen only by its
 * own block's rows, are single.  `cap`, `*n` as in bdattn_plan_order.
 * Pure host function. */
int bdattn_plan_order_keys(const bdattn_problem* problem,
                           const bdattn_share* share, const bdattn_kv* kv,
                           int32_t* items, int64_t cap, int64_t* n);

/* Workspace bytes for one bdattn_fwd (bwd = 0) or bdattn_bwd (bwd = 1) call
 * with these arguments; 0 on invalid arguments. */
size_t bdattn_workspace_bytes(const bdattn_problem* problem,
                              const bdattn_share* share, const bdattn_kv* kv,
                              int bwd);

/* Forward over the call's key set ([P1] "CSBP：BP 管损坏块，CP 管干净上下文",
 * CSBP forward equation; [P1] "在线 softmax 合并", steps 2 and 3 of the
 * schedule).
 *   q_clean, q_corr, k_clean, v_clean, k_corr, v_corr: problem dtype.
 *   o: share rows x hq heads, o_dtype BDATTN_BF16 (final output) or
 *      BDATTN_F32 (normalised partial for bdattn_shard_merge).
 *   lse: fp32 [batch][R][hq] contiguous.
 * For dtype BDATTN_F32 only o_dtype BDATTN_F32 is supported. */
int bdattn_fwd(const bdattn_problem* problem, const bdattn_share* share,
               const bdattn_kv* kv, bdattn_tensor q_clean, bdattn_tensor q_corr,
               bdattn_tensor k_clean, bdattn_tensor v_clean,
               bdattn_tensor k_corr, bdattn_tensor v_corr, bdattn_tensor o,
               int32_t o_dtype, float* lse, void* workspace, size_t ws_bytes,
               void* hip_stream);

/* Forward with no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and results as
 * bdattn_fwd; the scratch bdattn_fwd takes from `workspace` comes instead
 * from a static device buffer of BDATTN_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  Problems
 * whose bdattn_workspace_bytes(..., 0) exceed it return BDATTN_ESCRATCH
 * before any device work.  The call allocates nothing (its first call on a
 * device looks up the buffer's address once).  Every call on one GPU uses
 * the same buffer: calls that overlap on one GPU (concurrent streams or
 * threads) race and must be serialised by the caller; calls on one stream
 * are ordered.  bdattn_workspace_status(NULL, stream) reads its range
 * flag. */
#define BDATTN_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
int bdattn_fwd_static(const bdattn_problem* problem, const bdattn_share* share,
                      const bdattn_kv* kv, bdattn_tensor q_clean,
                      bdattn_tensor q_corr, bdattn_tensor k_clean,
                      bdattn_tensor v_clean, bdattn_tensor k_corr,
                      bdattn_tensor v_corr, bdattn_tensor o, int32_t o_dtype,
                      float* lse, void* hip_stream);

/* Range flag of the last bf16 bdattn_fwd / bdattn_bwd call that used
 * `workspace` (device pointer, as passed to that call; NULL: the last
 * bdattn_fwd_static call on the current device).  Synchronises
 * `hip_stream` (the stream of that call), then returns BDATTN_ERANGE if
 * that call clamped an input value to the fp16 range, else BDATTN_OK
 * (BDATTN_EINVAL for a misaligned workspace, BDATTN_EHIP on a HIP
 * error). */
int bdattn_workspace_status(const void* workspace, void* hip_stream);

/* Log-sum-exp merge of a partial result into an accumulator, in fp32
 * ([P1] "在线 softmax 合并", equations for m, w1, w2, O and z; numerator,
 * max and normaliser kept in fp32 to the last step):
 *   m = max(z_acc, z_part); w = exp(z - m);
 *   o_acc = (w_acc o_acc + w_part o_part) / (w_acc + w_part);
 *   z_acc = m + log(w_acc + w_part);  (0, -inf) is the empty result.
 * o_acc, o_part: fp32 [rows][d] contiguous; lse_acc, lse_part: fp32 [rows]
 * (rows = batch * R * hq for a share).  o_acc and lse_acc are updated in
 * place.  o_final_bf16 (nullable): also writes bf16(o_acc) [rows][d]. */
int bdattn_shard_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc,
                       const float* o_part, const float* lse_part,
                       void* o_final_bf16, void* hip_stream);

/* Backward over the call's key set for the loss sum(O * dO) ([P1] "CSBP：BP
 * 管损坏块，CP 管干净上下文": corrupted dQ/dK/dV stay with the block owner,
 * clean dK/dV collect contributions from every later block; [P3] "exact
 * fused backward").  The softmax is the FINAL one: o_final and lse_final
 * are the merged forward results over every key the rows see, so the
 * per-call contributions of a sharded key set sum to the full gradient.
 * Precision: the kernels form each probability as P * 2^c_i and the row's
 * dO and D times 2^-c_i (c_i = ceil(log2 n_i) - 7 within [0, 15], n_i the
 * number of keys row i sees in the whole mask), which keeps P out of fp16's
 * subnormal range on long rows and leaves every product unchanged.
 *   q_*, k_*, v_*: as in bdattn_fwd (bf16 only).
 *   o_final: share rows x hq, o_dtype BDATTN_BF16 or BDATTN_F32; read only
 *          when D is formed here (flags without BDATTN_BWD_DELTA_READY),
 *          otherwise not validated.
 *   lse_final: fp32 [batch][R][hq].   d_o: share rows x hq, bf16.
 *   delta: fp32 [batch][R][hq], D = rowsum(dO * O).  Without
 *          BDATTN_BWD_DELTA_READY: computed here and stored; with it: read
 *          as given (reuse across the calls of one step).
 *   flags: BDATTN_BWD_DELTA_READY (1) as above; BDATTN_BWD_OVERWRITE (2):
 *          the gradients are written, not added, so they need no zeroing.
 *          Only for the whole-mask form (every block, clean query range
 *          [0, L), key range [0, L) and include_local), where this one call
 *          produces every element; any other call with it is BDATTN_EINVAL.
 *   dq_acc: fp32 [batch][R][hq][d] contiguous, += this call's part.
 *   dk_clean_acc, dv_clean_acc: fp32 [batch][L][hkv][d] contiguous (token
 *          rows), += (may be NULL when the call has no clean key range).
 *   dk_corr_acc, dv_corr_acc: fp32 [batch][n_blocks*M][hkv][d] contiguous
 *          (packed corrupted rows), += (may be NULL when include_local == 0).
 * Without BDATTN_BWD_OVERWRITE the accumulators must be zeroed by the caller
 * before the first call. */
enum { BDATTN_BWD_DELTA_READY = 1, BDATTN_BWD_OVERWRITE = 2 };
int bdattn_bwd(const bdattn_problem* problem, const bdattn_share* share,
               const bdattn_kv* kv, bdattn_tensor q_clean, bdattn_tensor q_corr,
               bdattn_tensor k_clean, bdattn_tensor v_clean,
               bdattn_tensor k_corr, bdattn_tensor v_corr,
               bdattn_tensor o_final, int32_t o_dtype, const float* lse_final,
               bdattn_tensor d_o, float* delta, int32_t flags,
               float* dq_acc, float* dk_clean_acc, float* dv_clean_acc,
               float* dk_corr_acc, float* dv_corr_acc, void* workspace,
               size_t ws_bytes, void* hip_stream);

/* Human-readable text for a status code (static storage). */
const char* bdattn_status_string(int status);

/* Kernel timing: when enabled, every kernel launch made by the library is
 * bracketed by HIP events on its stream.  bdattn_profile_read synchronises
 * the recorded events and writes, per kernel kind k < *n (at most cap),
 * its name (static storage), launch count and summed milliseconds; then
 * clears the record.  Returns BDATTN_OK or BDATTN_EHIP. */
int bdattn_profile_enable(int enable);
int bdattn_profile_read(const char** names, int64_t* counts, double* ms,
                        int32_t cap, int32_t* n);

#ifdef __cplusplus
}
#endif
#endif
