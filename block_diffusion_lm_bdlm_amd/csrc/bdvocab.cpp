// bdvocab.cpp — host side of libbdvocab (include/bdvocab.h): argument
// checks, workspace layout, the two library GEMMs per chunk (hipBLASLt,
// bf16 inputs, fp32 accumulation) and the launches of the hand-written
// kernels in vocab_rows.hip.
//
// Chunk loop ([P3] Turbo-dLLM project page, "Library" section, "Vocabulary
// loss" rows: token-chunked projection and cross-entropy, no
// full-sequence logits):
//   (gather)      listed hidden rows -> packed bf16 chunk [n, d]
//   logits GEMM   S[n, V] = H_chunk W^T            (fp32, pitch ld)
//   rows          lse, loss, G = w (softmax - onehot) in bf16 over S
//   grad GEMM     dH_chunk[n, d] = G W              (bf16 or fp32)
//   (scatter)     packed dh rows -> their positions
//   head GEMM     dW[V, d] += G^T H_chunk           (fp32, when requested; on
//                 transposed copies of G and H_chunk, so that it too is TN)
// In the GEMM library's column-major terms a row-major [r, c] matrix with
// pitch p is a c x r matrix with leading dimension p, so the logits GEMM is
// S^T (V x n) = op_T(W^T as d x V) * (H^T as d x n) and the gradient GEMM
// is dH^T (d x n) = op_T(Wt^T as V x d) * (G^T as V x n), with Wt the
// head transposed to [d, V] once per call (a hand-written LDS-tiled copy
// into the workspace): both products then read their two operands along
// the contraction, the layout the library runs fastest (measured: the
// gradient GEMM on W itself, not transposed, was 25-30% slower).
// Algorithm choice: bdvocab_tune times the library's top candidates for
// every GEMM shape a loss call of the same arguments will run (the head GEMM
// on a scratch output, since its runs accumulate) and keeps the fastest per
// shape for the process.  bdvocab_loss itself never times or synchronises:
// a shape nobody tuned takes the library's first candidate.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "bdvocab.h"
#include "vocab_kernels.h"

namespace {

using namespace bdvocab;

constexpr int32_t kDefaultChunk = 8192;
constexpr size_t kBlasWs = size_t(64) << 20;  // GEMM library workspace
constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;
constexpr int kCandidates = 8;  // GEMM algorithms timed on a shape's first use

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// fp32 logit row pitch: V rounded up to 64 floats (256-byte rows).
int64_t logit_pitch(int32_t V) { return ((int64_t)V + 63) / 64 * 64; }

struct Layout {
  int64_t chunk = 0;
  int64_t ld = 0;
  int64_t ldc = 0;  // row pitch of the transposed chunk copies (chunk rounded up to 64)
  size_t s_off = 0, wt_off = 0, hc_off = 0, dhc_off = 0, gt_off = 0, ht_off = 0, blas_off = 0, total = 0;
};

int check_problem(const bdvocab_problem* p) {
  if (!p) return BDVOCAB_EINVAL;
  if (p->n_rows < 0 || p->vocab < 1 || p->hidden < 1 || p->chunk < 0) return BDVOCAB_EINVAL;
  if (p->dh_dtype != BDVOCAB_BF16 && p->dh_dtype != BDVOCAB_F32) return BDVOCAB_ENOTSUP;
  if (p->hidden < 8 || p->hidden % 8 != 0) return BDVOCAB_ENOTSUP;
  return BDVOCAB_OK;
}

Layout layout(const bdvocab_problem& p, bool row_list, bool head_grad) {
  Layout L;
  int64_t c = p.chunk > 0 ? p.chunk : kDefaultChunk;
  c = std::min<int64_t>(c, std::max<int64_t>(p.n_rows, 1));
  L.chunk = c;
  L.ld = logit_pitch(p.vocab);
  const size_t es = p.dh_dtype == BDVOCAB_F32 ? 4 : 2;
  size_t off = 0;
  L.s_off = off;
  off = round_up(off + (size_t)c * (size_t)L.ld * 4, kAlign);
  L.wt_off = off;  // the head transposed, [d, ld] bf16
  off = round_up(off + (size_t)p.hidden * (size_t)L.ld * 2, kAlign);
  if (row_list) {
    L.hc_off = off;
    off = round_up(off + (size_t)c * (size_t)p.hidden * 2, kAlign);
    L.dhc_off = off;
    off = round_up(off + (size_t)c * (size_t)p.hidden * es, kAlign);
  }
  L.ldc = (c + 63) / 64 * 64;
  if (head_grad) {  // G^T [V, ldc] and H^T [d, ldc], bf16
    L.gt_off = off;
    off = round_up(off + (size_t)p.vocab * (size_t)L.ldc * 2, kAlign);
    L.ht_off = off;
    off = round_up(off + (size_t)p.hidden * (size_t)L.ldc * 2, kAlign);
  }
  L.blas_off = off;
  off += kBlasWs;
  L.total = off;
  return L;
}

// ------------------------------------------------------------------ profiling
enum Kind { K_LOGITS, K_ROWS, K_GRAD, K_GATHER, K_SCATTER, K_SUM, K_TRANSPOSE, K_HEAD, K_COUNT };
const char* kKindNames[K_COUNT] = {"logits_gemm", "rows", "grad_gemm", "gather", "scatter", "loss_sum",
                                   "transpose", "head_grad_gemm"};

struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> rec;
} g_prof;

hipEvent_t prof_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs launch() (returning a bdvocab status), bracketed by events when
// profiling is on.
template <typename F>
int timed(int kind, hipStream_t s, F&& launch) {
  std::unique_lock<std::mutex> lk(g_prof.mu);
  if (!g_prof.on) {
    lk.unlock();
    return launch();
  }
  hipEvent_t a = prof_event(), b = prof_event();
  if (!a || !b) return BDVOCAB_EHIP;
  if (hipEventRecord(a, s) != hipSuccess) return BDVOCAB_EHIP;
  const int rc = launch();
  if (rc != BDVOCAB_OK) return rc;
  if (hipEventRecord(b, s) != hipSuccess) return BDVOCAB_EHIP;
  g_prof.rec.push_back({kind, {a, b}});
  return BDVOCAB_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? BDVOCAB_OK : BDVOCAB_EHIP; }

// ------------------------------------------------------------------ GEMMs
struct GemmKey {
  int dev, ta, tb;
  int64_t m, n, k, lda, ldb, ldd;
  int dtype, accumulate;
  bool operator<(const GemmKey& o) const {
    return std::tie(dev, ta, tb, m, n, k, lda, ldb, ldd, dtype, accumulate) <
           std::tie(o.dev, o.ta, o.tb, o.m, o.n, o.k, o.lda, o.ldb, o.ldd, o.dtype, o.accumulate);
  }
};

struct Blas {
  std::mutex mu;
  hipblasLtHandle_t handle[kMaxDevices] = {};
  std::map<GemmKey, hipblasLtMatmulHeuristicResult_t> algos;
} g_blas;

struct GemmDescs {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  ~GemmDescs() {
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (d) hipblasLtMatrixLayoutDestroy(d);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

// D (m x n, column-major, leading dimension ldd, type dt) = op(A) op(B)
// (+ D when accumulate), A and B bf16.
// tune: time the candidates on `s` (synchronising it), keep the fastest
// for the shape and run nothing else; D is scratch then.  Otherwise run with
// the kept algorithm, or the library's first candidate (kept from then on).
int gemm(bool ta, bool tb, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, const void* B,
         int64_t ldb, void* D, hipDataType dt, int64_t ldd, void* ws, hipStream_t s, bool accumulate = false,
         bool tune = false) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BDVOCAB_EHIP;
  hipblasLtHandle_t h;
  {
    std::lock_guard<std::mutex> lk(g_blas.mu);
    if (!g_blas.handle[dev] && hipblasLtCreate(&g_blas.handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
      g_blas.handle[dev] = nullptr;
      return BDVOCAB_EBLAS;
    }
    h = g_blas.handle[dev];
  }
  GemmDescs g;
  const hipblasOperation_t opa = ta ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const hipblasOperation_t opb = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  if (hipblasLtMatmulDescCreate(&g.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) !=
          HIPBLAS_STATUS_SUCCESS)
    return BDVOCAB_EBLAS;
  // stored shapes: A is k x m when transposed, m x k otherwise; B likewise
  if (hipblasLtMatrixLayoutCreate(&g.a, HIP_R_16BF, ta ? k : m, ta ? m : k, lda) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&g.b, HIP_R_16BF, tb ? n : k, tb ? k : n, ldb) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&g.d, dt, m, n, ldd) != HIPBLAS_STATUS_SUCCESS)
    return BDVOCAB_EBLAS;
  const GemmKey key{dev, ta, tb, m, n, k, lda, ldb, ldd, (int)dt, accumulate ? 1 : 0};
  hipblasLtMatmulHeuristicResult_t best{};
  {
    std::lock_guard<std::mutex> lk(g_blas.mu);
    auto it = g_blas.algos.find(key);
    if (it != g_blas.algos.end() && !tune) {
      best = it->second;
    } else {
      hipblasLtMatmulPreference_t pref = nullptr;
      if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return BDVOCAB_EBLAS;
      uint64_t cap = kBlasWs;
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap));
      hipblasLtMatmulHeuristicResult_t cand[kCandidates];
      int found = 0;
      const hipblasStatus_t st =
          hipblasLtMatmulAlgoGetHeuristic(h, g.op, g.a, g.b, g.d, g.d, pref, kCandidates, cand, &found);
      hipblasLtMatmulPreferenceDestroy(pref);
      if (st != HIPBLAS_STATUS_SUCCESS || found < 1) return BDVOCAB_EBLAS;
      int pick = -1;
      if (tune) {
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return BDVOCAB_EHIP;
        float best_ms = 0.f;
        const float one = 1.f, zero = 0.f;
        for (int i = 0; i < found; ++i) {
          if (cand[i].state != HIPBLAS_STATUS_SUCCESS || cand[i].workspaceSize > kBlasWs) continue;
          // one untimed run, then two timed ones (accumulating runs add into the scratch D)
          const float* beta = accumulate ? &one : &zero;
          bool ok = hipblasLtMatmul(h, g.op, &one, A, g.a, B, g.b, beta, D, g.d, D, g.d, &cand[i].algo, ws,
                                    kBlasWs, s) == HIPBLAS_STATUS_SUCCESS;
          ok = ok && hipEventRecord(e0, s) == hipSuccess;
          for (int r = 0; ok && r < 2; ++r)
            ok = hipblasLtMatmul(h, g.op, &one, A, g.a, B, g.b, beta, D, g.d, D, g.d, &cand[i].algo, ws, kBlasWs,
                                 s) == HIPBLAS_STATUS_SUCCESS;
          ok = ok && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
          float ms = 0.f;
          ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
          if (ok && (pick < 0 || ms < best_ms)) {
            pick = i;
            best_ms = ms;
          }
        }
        (void)hipEventDestroy(e0);  // timing only: a failure here changes no result
        (void)hipEventDestroy(e1);
      } else {
        for (int i = 0; i < found && pick < 0; ++i)
          if (cand[i].state == HIPBLAS_STATUS_SUCCESS && cand[i].workspaceSize <= kBlasWs) pick = i;
      }
      if (pick < 0) return BDVOCAB_EBLAS;
      best = cand[pick];
      g_blas.algos[key] = best;
    }
  }
  if (tune) return BDVOCAB_OK;
  const float one = 1.f, zero = 0.f;
  const hipblasStatus_t st = hipblasLtMatmul(h, g.op, &one, A, g.a, B, g.b, accumulate ? &one : &zero, D, g.d, D,
                                             g.d, &best.algo, ws, kBlasWs, s);
  return st == HIPBLAS_STATUS_SUCCESS ? BDVOCAB_OK : BDVOCAB_EBLAS;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

// ===================================================================== ABI
extern "C" {

size_t bdvocab_workspace_bytes(const bdvocab_problem* problem, int flags) {
  if (check_problem(problem) != BDVOCAB_OK) return 0;
  if (flags & ~(BDVOCAB_WS_ROW_LIST | BDVOCAB_WS_HEAD_GRAD)) return 0;
  return layout(*problem, (flags & BDVOCAB_WS_ROW_LIST) != 0, (flags & BDVOCAB_WS_HEAD_GRAD) != 0).total;
}

int bdvocab_loss(const bdvocab_problem* problem, const void* h, int64_t h_stride, const void* w_head,
                 const int32_t* rows, const int32_t* targets, const float* weights, float* lse, float* loss,
                 float* loss_sum, void* dh, int64_t dh_stride, float* dw, void* workspace, size_t ws_bytes,
                 void* hip_stream) {
  const int pc = check_problem(problem);
  if (pc != BDVOCAB_OK) return pc;
  const bdvocab_problem& p = *problem;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int64_t R = p.n_rows;
  const int64_t d = p.hidden;
  const int es = p.dh_dtype == BDVOCAB_F32 ? 4 : 2;
  if (R > 0) {
    if (!h || !w_head || !targets || !loss) return BDVOCAB_EINVAL;
    if (h_stride < d || h_stride % 8 != 0 || !aligned16(h) || !aligned16(w_head)) return BDVOCAB_EINVAL;
    if (dh && (dh_stride < d || (dh_stride * es) % 16 != 0 || !aligned16(dh))) return BDVOCAB_EINVAL;
    if (dw && !aligned16(dw)) return BDVOCAB_EINVAL;
    const Layout L = layout(p, rows != nullptr, dw != nullptr);
    if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0 || ws_bytes < L.total)
      return BDVOCAB_EWORKSPACE;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* S = reinterpret_cast<float*>(ws + L.s_off);
    uint16_t* hc = reinterpret_cast<uint16_t*>(ws + L.hc_off);
    uint8_t* dhc = ws + L.dhc_off;
    uint16_t* wt = reinterpret_cast<uint16_t*>(ws + L.wt_off);
    uint16_t* gt = reinterpret_cast<uint16_t*>(ws + L.gt_off);
    uint16_t* ht = reinterpret_cast<uint16_t*>(ws + L.ht_off);
    void* blas_ws = ws + L.blas_off;
    if (dh) {
      const TransposeArgs ta{static_cast<const uint16_t*>(w_head), p.vocab, (int32_t)d, d, wt, L.ld};
      const int rc = timed(K_TRANSPOSE, s, [&] { return hip_rc(launch_transpose(ta, s)); });
      if (rc != BDVOCAB_OK) return rc;
    }
    const hipDataType dt = p.dh_dtype == BDVOCAB_F32 ? HIP_R_32F : HIP_R_16BF;
    for (int64_t c0 = 0; c0 < R; c0 += L.chunk) {
      const int64_t n = std::min<int64_t>(L.chunk, R - c0);
      const void* Hb = static_cast<const uint16_t*>(h) + c0 * h_stride;
      int64_t ldh = h_stride;
      if (rows) {
        const GatherArgs ga{static_cast<const uint16_t*>(h), h_stride, rows + c0, n, (int32_t)d, hc};
        int rc = timed(K_GATHER, s, [&] { return hip_rc(launch_gather(ga, s)); });
        if (rc != BDVOCAB_OK) return rc;
        Hb = hc;
        ldh = d;
      }
      int rc = timed(K_LOGITS, s, [&] {
        return gemm(true, false, p.vocab, n, d, w_head, d, Hb, ldh, S, HIP_R_32F, L.ld, blas_ws, s);
      });
      if (rc != BDVOCAB_OK) return rc;
      const RowsArgs ra{S, L.ld, n, p.vocab, targets + c0, weights ? weights + c0 : nullptr,
                        lse ? lse + c0 : nullptr, loss + c0};
      rc = timed(K_ROWS, s, [&] { return hip_rc(launch_rows(ra, s)); });
      if (rc != BDVOCAB_OK) return rc;
      if (dh) {
        void* D = rows ? static_cast<void*>(dhc)
                       : static_cast<void*>(static_cast<uint8_t*>(dh) + c0 * dh_stride * es);
        const int64_t ldd = rows ? d : dh_stride;
        rc = timed(K_GRAD, s,
                   [&] { return gemm(true, false, d, n, p.vocab, wt, L.ld, S, 2 * L.ld, D, dt, ldd, blas_ws, s); });
        if (rc != BDVOCAB_OK) return rc;
        if (rows) {
          const ScatterArgs sa{dhc, n, (int32_t)d, es, rows + c0, static_cast<uint8_t*>(dh), dh_stride};
          rc = timed(K_SCATTER, s, [&] { return hip_rc(launch_scatter(sa, s)); });
          if (rc != BDVOCAB_OK) return rc;
        }
      }
      if (dw) {
        // G [n, V] (pitch 2 ld) -> G^T [V, ldc]; H_chunk [n, d] -> H^T [d, ldc]
        const TransposeArgs tg{reinterpret_cast<const uint16_t*>(S), n, p.vocab, 2 * L.ld, gt, L.ldc};
        const TransposeArgs th{static_cast<const uint16_t*>(Hb), n, (int32_t)d, ldh, ht, L.ldc};
        rc = timed(K_TRANSPOSE, s, [&] {
          const int r1 = hip_rc(launch_transpose(tg, s));
          return r1 != BDVOCAB_OK ? r1 : hip_rc(launch_transpose(th, s));
        });
        if (rc != BDVOCAB_OK) return rc;
        // dW^T (d x V) += op_T(H^T^T as n x d) * (G^T^T as n x V): both read along the rows
        rc = timed(K_HEAD, s, [&] {
          return gemm(true, false, d, p.vocab, n, ht, L.ldc, gt, L.ldc, dw, HIP_R_32F, d, blas_ws, s, true);
        });
        if (rc != BDVOCAB_OK) return rc;
      }
    }
  }
  if (loss_sum) return timed(K_SUM, s, [&] { return hip_rc(launch_loss_sum(loss, R, loss_sum, s)); });
  return BDVOCAB_OK;
}

int bdvocab_tune(const bdvocab_problem* problem, int flags, const void* h, int64_t h_stride, const void* w_head,
                 int64_t dh_stride, void* workspace, size_t ws_bytes, void* hip_stream) {
  const int pc = check_problem(problem);
  if (pc != BDVOCAB_OK) return pc;
  if (flags & ~(BDVOCAB_WS_ROW_LIST | BDVOCAB_WS_HEAD_GRAD)) return BDVOCAB_EINVAL;
  const bdvocab_problem& p = *problem;
  const int64_t R = p.n_rows, d = p.hidden;
  if (R == 0) return BDVOCAB_OK;
  const bool rows = (flags & BDVOCAB_WS_ROW_LIST) != 0, head = (flags & BDVOCAB_WS_HEAD_GRAD) != 0;
  const int es = p.dh_dtype == BDVOCAB_F32 ? 4 : 2;
  if (!h || !w_head || h_stride < d || h_stride % 8 != 0 || !aligned16(h) || !aligned16(w_head))
    return BDVOCAB_EINVAL;
  if (dh_stride < 0 || (dh_stride > 0 && (dh_stride < d || (dh_stride * es) % 16 != 0))) return BDVOCAB_EINVAL;
  const Layout L = layout(p, rows, head);
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0 || ws_bytes < L.total)
    return BDVOCAB_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* S = reinterpret_cast<float*>(ws + L.s_off);
  void* blas_ws = ws + L.blas_off;
  const hipDataType dt = p.dh_dtype == BDVOCAB_F32 ? HIP_R_32F : HIP_R_16BF;
  // scratch outputs of the GEMMs whose real outputs are the caller's
  const int64_t nmax = L.chunk;
  const size_t dh_scratch = (dh_stride > 0 && !rows) ? (size_t)nmax * dh_stride * es : 0;
  const size_t dw_scratch = head ? (size_t)p.vocab * d * 4 : 0;
  void* scratch = nullptr;
  if (dh_scratch + dw_scratch > 0 && hipMalloc(&scratch, round_up(dh_scratch, kAlign) + dw_scratch) != hipSuccess)
    return BDVOCAB_EHIP;
  uint8_t* sc = static_cast<uint8_t*>(scratch);
  float* dw_sc = reinterpret_cast<float*>(sc + round_up(dh_scratch, kAlign));
  int rc = BDVOCAB_OK;
  // the chunk sizes a loss call runs: full chunks and the last, shorter one
  int64_t sizes[2] = {std::min<int64_t>(L.chunk, R), R % L.chunk};
  const int nsizes = (R > L.chunk && sizes[1] > 0) ? 2 : 1;
  for (int i = 0; i < nsizes && rc == BDVOCAB_OK; ++i) {
    const int64_t n = sizes[i];
    const void* Hb = rows ? static_cast<const void*>(ws + L.hc_off) : h;
    const int64_t ldh = rows ? d : h_stride;
    rc = gemm(true, false, p.vocab, n, d, w_head, d, Hb, ldh, S, HIP_R_32F, L.ld, blas_ws, s, false, true);
    if (rc == BDVOCAB_OK && dh_stride > 0) {
      void* D = rows ? static_cast<void*>(ws + L.dhc_off) : scratch;
      const int64_t ldd = rows ? d : dh_stride;
      rc = gemm(true, false, d, n, p.vocab, ws + L.wt_off, L.ld, S, 2 * L.ld, D, dt, ldd, blas_ws, s, false, true);
    }
    if (rc == BDVOCAB_OK && head)
      rc = gemm(true, false, d, p.vocab, n, ws + L.ht_off, L.ldc, ws + L.gt_off, L.ldc, dw_sc, HIP_R_32F, d,
                blas_ws, s, true, true);
  }
  if (hipStreamSynchronize(s) != hipSuccess && rc == BDVOCAB_OK) rc = BDVOCAB_EHIP;
  if (scratch && hipFree(scratch) != hipSuccess && rc == BDVOCAB_OK) rc = BDVOCAB_EHIP;
  return rc;
}

const char* bdvocab_status_string(int status) {
  switch (status) {
    case BDVOCAB_OK: return "ok";
    case BDVOCAB_EINVAL: return "invalid argument";
    case BDVOCAB_ENOTSUP: return "unsupported (hidden size must be a multiple of 8; dh dtype bf16 or fp32)";
    case BDVOCAB_EHIP: return "HIP runtime error";
    case BDVOCAB_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case BDVOCAB_EBLAS: return "GEMM library error (hipBLASLt)";
    default: return "unknown status";
  }
}

int bdvocab_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = enable != 0;
  return BDVOCAB_OK;
}

int bdvocab_profile_read(const char** names, int64_t* counts, double* ms, int32_t cap, int32_t* n) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!n || cap < 0) return BDVOCAB_EINVAL;
  int64_t cnt[K_COUNT] = {0};
  double tot[K_COUNT] = {0};
  int rc = BDVOCAB_OK;
  for (auto& r : g_prof.rec) {
    float t = 0.f;
    if (hipEventSynchronize(r.second.second) != hipSuccess ||
        hipEventElapsedTime(&t, r.second.first, r.second.second) != hipSuccess)
      rc = BDVOCAB_EHIP;
    cnt[r.first] += 1;
    tot[r.first] += t;
    g_prof.pool.push_back(r.second.first);
    g_prof.pool.push_back(r.second.second);
  }
  g_prof.rec.clear();
  int32_t k = 0;
  for (int i = 0; i < K_COUNT && k < cap; ++i) {
    if (cnt[i] == 0) continue;
    if (names) names[k] = kKindNames[i];
    if (counts) counts[k] = cnt[i];
    if (ms) ms[k] = tot[i];
    ++k;
  }
  *n = k;
  return rc;
}

}  // extern "C"
