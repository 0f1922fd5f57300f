/*
 * bdvocab.h — C ABI of libbdvocab: the streaming vocabulary loss of BDLM
 * training on AMD MI355X (gfx950).
 *
 * Source (cited by page title and section):
 *  [P3] "Block Parallelism for Efficient Distributed Long-Context Diffusion
 *       Language Model Training" (Turbo-dLLM project page), "Library"
 *       section, tables "Speculative Decoding Optimizations" and "Block
 *       Diffusion Optimizations", row "Vocabulary loss": rows are streamed
 *       through the frozen LM head in token chunks, with projection and
 *       cross-entropy done per chunk, so the logits of the whole sequence
 *       are never held.
 *
 * What is computed.  For the R rows that carry the loss (the masked
 * positions of the corrupted copy, chosen by the caller), with hidden row
 * h_r (length d), target y_r and weight w_r, and the frozen head W [V, d]:
 *   s_r    = h_r W^T                         (the row's V logits)
 *   lse_r  = log sum_v exp(s_rv)
 *   loss_r = w_r (lse_r - s_r[y_r])
 *   g_r    = w_r (softmax(s_r) - e_{y_r})     (gradient of loss_r wrt s_r)
 *   dh_r   = g_r W                            (gradient of loss_r wrt h_r)
 *   dW     = sum_r g_r^T h_r                  (gradient of the summed loss wrt W)
 * dW is optional: the speculative-decoding row streams through a frozen
 * head (no dW), the block-diffusion row does not say the head is frozen.
 * A row whose target is outside [0, V) is ignored: loss_r = 0, dh_r = 0,
 * no dW term (lse_r is still written).
 *
 * How.  Rows go in chunks of C.  Per chunk: the chunk's logits in fp32
 * (a plain library GEMM, bf16 inputs, fp32 accumulation) into the
 * workspace; one fused pass per row forms lse, the loss and the logit
 * gradient, written in bf16 over the same workspace rows; a second library
 * GEMM forms dh from a transposed copy of the head made once per call, and
 * a third, when dW is requested, adds the chunk's G^T H to dW (from
 * transposed copies of G and H, so that both operands run along the
 * contraction).
 * Device memory for logits is C * V * 4 bytes, never R * V.  bdvocab_tune
 * (a set-up call) times the GEMM library's candidate algorithms for the
 * shapes of a loss call and keeps the fastest per shape; bdvocab_loss never
 * times or synchronises, and a shape nobody tuned takes the library's first
 * candidate.
 *
 * Conventions.
 *   - Device buffers are caller-owned and scratch comes from `workspace`
 *     (size from bdvocab_workspace_bytes).  bdvocab_loss allocates no
 *     device memory itself; the GEMM library (hipBLASLt) creates its handle
 *     once per device on the first call of either entry point and may
 *     allocate inside it, so a caller that captures bdvocab_loss into a
 *     graph calls bdvocab_tune (or bdvocab_loss) once before.
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL =
 *     the null stream); buffers must stay valid until it completes.  Calls
 *     sharing a workspace must not overlap.
 *   - Return value: BDVOCAB_OK or a negative bdvocab_status.  Argument
 *     errors are found on the host before anything is enqueued; device
 *     contents (targets, row indices) are not checked on the host.
 */
#ifndef BDVOCAB_H
#define BDVOCAB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BDVOCAB_OK = 0,
  BDVOCAB_EINVAL = -1,     /* bad argument (sizes, strides, missing buffer) */
  BDVOCAB_ENOTSUP = -2,    /* valid but unsupported (hidden size not a multiple of 8, dtype) */
  BDVOCAB_EHIP = -3,       /* a HIP runtime call failed */
  BDVOCAB_EWORKSPACE = -4, /* workspace too small or misaligned */
  BDVOCAB_EBLAS = -5       /* the GEMM library refused or failed */
} bdvocab_status;

typedef enum { BDVOCAB_BF16 = 0, BDVOCAB_F32 = 1 } bdvocab_dtype;

typedef struct {
  int64_t n_rows;   /* R >= 0: rows that carry the loss */
  int32_t vocab;    /* V >= 1 */
  int32_t hidden;   /* d >= 8, multiple of 8 */
  int32_t chunk;    /* C: rows per chunk, >= 1; 0 picks the default (8192) */
  int32_t dh_dtype; /* BDVOCAB_BF16 or BDVOCAB_F32 */
} bdvocab_problem;

/* Bytes of device workspace bdvocab_loss needs for `problem` (256-byte
 * aligned base required): the chunk's logits, the transposed head, and the
 * GEMM library's 64 MiB.  `flags`: BDVOCAB_WS_ROW_LIST when the call passes
 * a row index list (adds the gathered chunk of hidden rows and of dh);
 * BDVOCAB_WS_HEAD_GRAD when it passes dw (adds transposed copies of a
 * chunk's logit gradient and hidden rows, V x C and d x C bf16).  Returns 0
 * for an invalid problem or unknown flag bits. */
enum { BDVOCAB_WS_ROW_LIST = 1, BDVOCAB_WS_HEAD_GRAD = 2 };
size_t bdvocab_workspace_bytes(const bdvocab_problem* problem, int flags);

/* Loss, lse and dh of the R loss rows.
 *   h        bf16, device.  Row r is read at h + idx_r * h_stride elements,
 *            idx_r = rows[r] when `rows` is given, else r; the d values of a
 *            row are contiguous.  h_stride >= d.
 *   w_head   bf16 [V, d] row-major, contiguous, device.
 *   rows     int32 [R] device, or NULL.  Distinct, each in [0, 2^31); the
 *            caller guarantees h and dh hold row idx_r (not checked).
 *   targets  int32 [R] device.
 *   weights  fp32 [R] device, or NULL for weight 1.
 *   lse      fp32 [R] device, or NULL.
 *   loss     fp32 [R] device (per-row weighted loss), required.
 *   loss_sum fp32 device scalar, or NULL: sum of loss over the rows, in a
 *            fixed order (deterministic).
 *   dh       device, dtype problem->dh_dtype, or NULL to skip the gradient.
 *            Row idx_r of dh (at dh + idx_r * dh_stride elements) is
 *            written for every r; other rows are not touched.  dh_stride
 *            >= d.
 *   dw       fp32 [V, d] row-major, contiguous, device, or NULL.  The call
 *            ADDS its gradient (dw += sum_r g_r^T h_r), so the caller
 *            clears it before the first call of a step.
 *   workspace / ws_bytes: at least bdvocab_workspace_bytes(problem,
 *            (rows ? BDVOCAB_WS_ROW_LIST : 0) | (dw ? BDVOCAB_WS_HEAD_GRAD
 *            : 0)); the contents need not be initialised.
 * R = 0 enqueues only the zeroing of loss_sum. */
int bdvocab_loss(const bdvocab_problem* problem, const void* h, int64_t h_stride,
                 const void* w_head, const int32_t* rows, const int32_t* targets,
                 const float* weights, float* lse, float* loss, float* loss_sum,
                 void* dh, int64_t dh_stride, float* dw, void* workspace, size_t ws_bytes,
                 void* hip_stream);

/* Set-up call: times the GEMM library's candidate algorithms for every GEMM
 * shape a bdvocab_loss call with the same problem and the same kind of
 * arguments runs (full chunks and the last, shorter chunk; the head
 * gradient GEMM on a scratch output, since its runs accumulate) and keeps
 * the fastest per shape for the process.
 *   flags     BDVOCAB_WS_ROW_LIST when the loss calls pass a row list,
 *             BDVOCAB_WS_HEAD_GRAD when they pass dw.
 *   h, h_stride, w_head: as in bdvocab_loss (only their addresses, strides
 *             and the shapes are used; the values are not read for
 *             results).
 *   dh_stride the loss calls' dh_stride, or 0 when they pass no dh.
 *   workspace / ws_bytes: as in bdvocab_loss for these flags; its contents
 *             are overwritten.
 * Unlike bdvocab_loss it synchronises `hip_stream` and allocates (and
 * frees) scratch device memory for the outputs it must not write: the dh
 * rows (without a row list) and a V x d fp32 head gradient.  Calling it is
 * optional; calling it again re-times.  R = 0 does nothing. */
int bdvocab_tune(const bdvocab_problem* problem, int flags, const void* h, int64_t h_stride,
                 const void* w_head, int64_t dh_stride, void* workspace, size_t ws_bytes,
                 void* hip_stream);

/* Static text for a bdvocab_status value. */
const char* bdvocab_status_string(int status);

/* Kernel timing for measurement: when enabled (nonzero), every launch of
 * bdvocab_loss is bracketed by HIP events on its stream, per kind:
 * "logits_gemm", "rows", "grad_gemm", "gather", "scatter", "loss_sum",
 * "transpose", "head_grad_gemm".
 * bdvocab_profile_read synchronises the recorded events, writes up to `cap`
 * (name, launch count, total milliseconds) entries for the kinds that ran,
 * sets *n to their number and clears the record. */
int bdvocab_profile_enable(int enable);
int bdvocab_profile_read(const char** names, int64_t* counts, double* ms, int32_t cap, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* BDVOCAB_H */
