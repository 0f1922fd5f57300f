// bdattn.cpp — the C ABI of libbdattn: argument validation, planning,
// workspace layout and kernel orchestration.  See include/bdattn.h.
#include "bdattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "abi_internal.h"
#include "kernels.h"
#include "plan.h"

using namespace bd;

namespace {

// ------------------------------------------------------------------ validation
bool problem_ok(const bdattn_problem* p) {
  if (!p) return false;
  if (p->batch < 1 || p->L < 1 || p->M < 1 || p->hq < 1 || p->hkv < 1 || p->d < 1) return false;
  if (p->L % p->M != 0 || p->hq % p->hkv != 0) return false;
  if (p->dtype != BDATTN_BF16 && p->dtype != BDATTN_F32) return false;
  if (p->clean_mask != BDATTN_CLEAN_BLOCK_CAUSAL && p->clean_mask != BDATTN_CLEAN_TOKEN_CAUSAL)
    return false;
  if (!std::isfinite(p->scale)) return false;
  if (p->window < 0) return false;
  if ((int64_t)p->batch * p->hq > (1 << 20) || p->L > (1 << 29)) return false;
  return true;
}

bool problem_supported(const bdattn_problem* p) { return p->d == 64 || p->d == 128; }

bool ranges_ok(int32_t n, const int32_t* lo, const int32_t* hi, int32_t limit) {
  if (n < 0 || n > 2) return false;
  for (int32_t r = 0; r < n; ++r) {
    if (lo[r] < 0 || hi[r] <= lo[r] || hi[r] > limit) return false;
    if (r > 0 && lo[r] < hi[r - 1]) return false;
  }
  return true;
}

bool share_ok(const bdattn_problem* p, const bdattn_share* s, int32_t* nruns) {
  if (!s) return false;
  const int32_t B = p->L / p->M;
  if (s->n_blocks < 0 || s->n_blocks > B) return false;
  if (s->n_blocks > 0 && !s->blocks) return false;
  int32_t runs = 0;
  for (int32_t i = 0; i < s->n_blocks; ++i) {
    const int32_t b = s->blocks[i];
    if (b < 0 || b >= B) return false;
    if (i > 0 && b <= s->blocks[i - 1]) return false;
    if (i == 0 || b != s->blocks[i - 1] + 1) ++runs;
  }
  if (runs > BDATTN_MAX_RUNS) return false;
  if (!ranges_ok(s->n_clean, s->clean_lo, s->clean_hi, p->L)) return false;
  if ((int64_t)s->n_blocks * p->M + p->L > (int64_t)1 << 30) return false;
  *nruns = runs;
  return true;
}

bool kv_ok(const bdattn_problem* p, const bdattn_kv* kv) {
  if (!kv) return false;
  if (kv->include_local != 0 && kv->include_local != 1) return false;
  return ranges_ok(kv->n, kv->lo, kv->hi, p->L);
}

int32_t round_up(int32_t x, int32_t m) { return (x + m - 1) / m * m; }

// Builds the plan; arguments already validated.
Plan make_plan(const bdattn_problem* p, const bdattn_share* s, const bdattn_kv* kv) {
  Plan P;
  std::memset(&P, 0, sizeof P);
  P.batch = p->batch;
  P.L = p->L;
  P.M = p->M;
  P.M_log2 = (P.M & (P.M - 1)) == 0 ? __builtin_ctz((unsigned)P.M) : -1;
  P.hq = p->hq;
  P.hkv = p->hkv;
  P.d = p->d;
  P.G = p->hq / p->hkv;
  P.token_causal = p->clean_mask == BDATTN_CLEAN_TOKEN_CAUSAL;
  P.window = p->window;
  P.scale = p->scale > 0.f ? p->scale : 1.f / std::sqrt((float)p->d);
  P.scale_log2 = P.scale * 1.4426950408889634f;
  int32_t row = 0, tile = 0;
  for (int32_t r = 0; r < s->n_clean; ++r) {
    QSeg& q = P.q[P.nq++];
    q.kind = KIND_CLEAN;
    q.row0 = row;
    q.nrows = s->clean_hi[r] - s->clean_lo[r];
    q.src0 = row;
    q.first = s->clean_lo[r];
    q.tile0 = tile;
    q.ntiles = (q.nrows + kBQ - 1) / kBQ;
    row += q.nrows;
    tile += q.ntiles;
  }
  P.n_clean_rows = row;
  P.n_clean_tiles = tile;
  for (int32_t i = 0; i < s->n_blocks;) {
    int32_t j = i + 1;
    while (j < s->n_blocks && s->blocks[j] == s->blocks[j - 1] + 1) ++j;
    QSeg& q = P.q[P.nq++];
    q.kind = KIND_CORR;
    q.row0 = row;
    q.nrows = (j - i) * p->M;
    q.src0 = i * p->M;
    q.first = s->blocks[i];
    q.tile0 = tile;
    q.ntiles = (q.nrows + kBQ - 1) / kBQ;
    row += q.nrows;
    tile += q.ntiles;
    i = j;
  }
  P.R = row;
  P.n_corr_rows = s->n_blocks * p->M;
  P.ntiles = tile;
  P.nqc = tile * kBQ;
  P.npairs = (P.n_clean_tiles + 1) / 2 + (P.ntiles - P.n_clean_tiles + 1) / 2;
  int32_t c = 0;
  for (int32_t r = 0; r < kv->n; ++r) {
    KSeg& k = P.k[P.nk++];
    k.kind = KIND_CLEAN;
    k.t0 = kv->lo[r];
    k.len = kv->hi[r] - kv->lo[r];
    k.c0 = c;
    c += round_up(k.len, kAlign);
  }
  if (kv->include_local && s->n_blocks > 0) {
    KSeg& k = P.k[P.nk++];
    k.kind = KIND_CORR;
    k.t0 = 0;
    k.len = s->n_blocks * p->M;
    k.c0 = c;
    c += round_up(k.len, kAlign);
  }
  P.nkc = c;
  int32_t nkt = 0;
  for (int32_t j = 0; j < P.nk; ++j) nkt += ktiles_of(P.k[j]);
  P.nkt = nkt;
  const int32_t ncl = n_clean_ktiles(P);
  P.nkpairs = (ncl + 1) / 2 + (nkt - ncl);
  P.nwg_q = (int64_t)P.batch * P.hq * P.npairs;
  P.nwg_k = (int64_t)P.batch * P.hkv * P.nkpairs;
  return P;
}

// ------------------------------------------------------------------ workspace
struct Carve {
  char* base;
  size_t off;
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T* r = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return r;
  }
};

// Every bf16 workspace starts with a 4 KB header whose first int32 is
// the call's range flag (cleared by the call, set by the packing kernels
// when a value converted to fp16 lies outside the half range), followed by
// the kernels' work-queue heads (kernels.h).
constexpr size_t kHeaderBytes = 4 * kHeaderWords;

struct FwdWs {
  int32_t* flag;
  uint16_t* kn;
  _Float16* vt;
};
struct BwdWs {
  int32_t* flag;
  _Float16 *kh, *vh;
  _Float16 *qh, *doh;
  float *lse2, *dc;
  int32_t* vis;
};

size_t carve_fwd(const Plan& P, bool f32, char* base, FwdWs* w) {
  Carve cv{base, 0};
  if (f32) return 0;
  const size_t nk = (size_t)P.batch * P.hkv * P.nkc * P.d;
  FwdWs t;
  t.flag = cv.take<int32_t>(kHeaderBytes / 4);
  t.kn = cv.take<uint16_t>(nk);
  t.vt = cv.take<_Float16>(nk);
  if (w) *w = t;
  return cv.off;
}

size_t carve_bwd(const Plan& P, char* base, BwdWs* w) {
  Carve cv{base, 0};
  const size_t nk = (size_t)P.batch * P.hkv * P.nkc * P.d;
  const size_t nq = (size_t)P.batch * P.hq * P.nqc * P.d;
  const size_t nr = (size_t)P.batch * P.hq * P.nqc;
  BwdWs t;
  t.flag = cv.take<int32_t>(kHeaderBytes / 4);
  t.kh = cv.take<_Float16>(nk);
  t.vh = cv.take<_Float16>(nk);
  t.qh = cv.take<_Float16>(nq);
  t.doh = cv.take<_Float16>(nq);
  t.lse2 = cv.take<float>(nr);
  t.dc = cv.take<float>(nr);
  t.vis = cv.take<int32_t>((size_t)4 * P.nqc);
  if (w) *w = t;
  return cv.off;
}

// ------------------------------------------------------------------ tensors
bool tensor_ok(const bdattn_tensor& t, int elem_bytes) {
  if (!t.ptr) return false;
  if (reinterpret_cast<uintptr_t>(t.ptr) % 16 != 0) return false;
  const int64_t vec = 16 / elem_bytes;
  if (t.batch_stride < 0 || t.row_stride < 0 || t.head_stride < 0) return false;
  return t.batch_stride % vec == 0 && t.row_stride % vec == 0 && t.head_stride % vec == 0;
}

TensorArg targ(const bdattn_tensor& t) { return TensorArg{t.ptr, t.batch_stride, t.row_stride, t.head_stride}; }

// ------------------------------------------------------------------ profiling
enum Kind { K_PACK_K, K_PACK_Q, K_FWD, K_FWD_F32, K_DQ, K_DKDV, K_MERGE, K_FLAG, K_COUNT };
const char* kKindNames[K_COUNT] = {"pack_k", "pack_q", "fwd_bf16", "fwd_f32", "dq", "dkdv", "merge", "flag_clear"};

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

template <typename F>
hipError_t timed(int kind, hipStream_t s, F&& launch) {
  std::unique_lock<std::mutex> lk(g_prof.mu);
  if (!g_prof.on) {
    lk.unlock();
    return launch();
  }
  hipEvent_t a = prof_event(), b = prof_event();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  g_prof.rec.push_back({kind, {a, b}});
  return hipSuccess;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BDATTN_OK : BDATTN_EHIP; }

}  // namespace

// ===================================================================== ABI
extern "C" {

const char* bdattn_status_string(int status) {
  switch (status) {
    case BDATTN_OK: return "ok";
    case BDATTN_EINVAL: return "invalid argument";
    case BDATTN_ENOTSUP: return "not supported";
    case BDATTN_EHIP: return "HIP runtime error";
    case BDATTN_EWORKSPACE: return "workspace missing or too small";
    case BDATTN_ERANGE: return "an input value lies outside the fp16 range (clamped)";
    case BDATTN_ESCRATCH: return "problem needs more scratch than the static buffer holds";
    default: return "unknown status";
  }
}

int bdattn_assign_blocks(int32_t B, int32_t P, int32_t r, int32_t* out) {
  if (!out || B <= 0 || P <= 0 || r < 0 || r >= P || B % (2 * P) != 0) return BDATTN_EINVAL;
  const int32_t c = B / (2 * P);
  // rank r owns pairs r*c .. r*c + c-1; pair t = (t, B-1-t): the early
  // members form the ascending run [r*c, r*c + c), the late members the
  // ascending run [B - (r+1)*c, B - r*c).
  for (int32_t t = 0; t < c; ++t) out[t] = r * c + t;
  for (int32_t t = 0; t < c; ++t) out[c + t] = B - (r + 1) * c + t;
  return BDATTN_OK;
}

int bdattn_clean_shard(int32_t L, int32_t P, int32_t s, bdattn_kv* out) {
  if (!out || L <= 0 || P <= 0 || s < 0 || s >= P || L % (2 * P) != 0) return BDATTN_EINVAL;
  const int32_t w = L / (2 * P);
  out->n = 2;
  out->lo[0] = s * w;
  out->hi[0] = (s + 1) * w;
  out->lo[1] = (2 * P - 1 - s) * w;
  out->hi[1] = (2 * P - s) * w;
  out->include_local = 0;
  return BDATTN_OK;
}

int bdattn_plan_order(const bdattn_problem* problem, const bdattn_share* share, const bdattn_kv* kv,
                      int32_t* items, int64_t cap, int64_t* n) {
  int32_t runs = 0;
  if (!n || !problem_ok(problem) || !share_ok(problem, share, &runs) || !kv_ok(problem, kv))
    return BDATTN_EINVAL;
  const Plan P = make_plan(problem, share, kv);
  *n = P.nwg_q;
  if (items) {
    if (cap < 4 * P.nwg_q) return BDATTN_EINVAL;
    for (int64_t w = 0; w < P.nwg_q; ++w) {
      const WgQ wg = decode_wg_q(P, w);
      items[4 * w + 0] = wg.b;
      items[4 * w + 1] = wg.h;
      items[4 * w + 2] = wg.tile_a;
      items[4 * w + 3] = wg.tile_b;
    }
  }
  return BDATTN_OK;
}

int bdattn_plan_order_keys(const bdattn_problem* problem, const bdattn_share* share, const bdattn_kv* kv,
                           int32_t* items, int64_t cap, int64_t* n) {
  int32_t runs = 0;
  if (!n || !problem_ok(problem) || !share_ok(problem, share, &runs) || !kv_ok(problem, kv))
    return BDATTN_EINVAL;
  const Plan P = make_plan(problem, share, kv);
  *n = P.nwg_k;
  if (items) {
    if (cap < 4 * P.nwg_k) return BDATTN_EINVAL;
    for (int64_t w = 0; w < P.nwg_k; ++w) {
      const WgK wg = decode_wg_k(P, w);
      items[4 * w + 0] = wg.b;
      items[4 * w + 1] = wg.g;
      items[4 * w + 2] = wg.tile_a;
      items[4 * w + 3] = wg.tile_b;
    }
  }
  return BDATTN_OK;
}

size_t bdattn_workspace_bytes(const bdattn_problem* problem, const bdattn_share* share,
                              const bdattn_kv* kv, int bwd) {
  int32_t runs = 0;
  if (!problem_ok(problem) || !share_ok(problem, share, &runs) || !kv_ok(problem, kv)) return 0;
  const Plan P = make_plan(problem, share, kv);
  const size_t need = bwd ? carve_bwd(P, nullptr, nullptr) : carve_fwd(P, problem->dtype == BDATTN_F32, nullptr, nullptr);
  return need;
}

}  // extern "C"

namespace bd {

// Body of bdattn_fwd: validation, then the packing and forward kernels on
// the given scratch of `ws_bytes` bytes.
int fwd_impl(const bdattn_problem* problem, const bdattn_share* share, const bdattn_kv* kv,
             bdattn_tensor q_clean, bdattn_tensor q_corr, bdattn_tensor k_clean, bdattn_tensor v_clean,
             bdattn_tensor k_corr, bdattn_tensor v_corr, bdattn_tensor o, int32_t o_dtype, float* lse,
             void* workspace, size_t ws_bytes, void* hip_stream) {
  int32_t runs = 0;
  if (!problem_ok(problem) || !share_ok(problem, share, &runs) || !kv_ok(problem, kv)) return BDATTN_EINVAL;
  if (!problem_supported(problem)) return BDATTN_ENOTSUP;
  if (o_dtype != BDATTN_BF16 && o_dtype != BDATTN_F32) return BDATTN_EINVAL;
  const bool f32 = problem->dtype == BDATTN_F32;
  if (f32 && o_dtype != BDATTN_F32) return BDATTN_ENOTSUP;
  const int eb = f32 ? 4 : 2;
  const Plan P = make_plan(problem, share, kv);
  if (P.R == 0) return BDATTN_OK;
  if (!lse || reinterpret_cast<uintptr_t>(lse) % 4) return BDATTN_EINVAL;
  if (!tensor_ok(o, o_dtype == BDATTN_F32 ? 4 : 2)) return BDATTN_EINVAL;
  if (P.n_clean_rows > 0 && !tensor_ok(q_clean, eb)) return BDATTN_EINVAL;
  if (P.n_corr_rows > 0 && !tensor_ok(q_corr, eb)) return BDATTN_EINVAL;
  if (kv->n > 0 && (!tensor_ok(k_clean, eb) || !tensor_ok(v_clean, eb))) return BDATTN_EINVAL;
  if (kv->include_local && P.n_corr_rows > 0 && (!tensor_ok(k_corr, eb) || !tensor_ok(v_corr, eb)))
    return BDATTN_EINVAL;
  const size_t need = carve_fwd(P, f32, nullptr, nullptr);
  if (need > 0 && (!workspace || ws_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256))
    return BDATTN_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);

  if (f32) {
    FwdF32Args a;
    a.q_clean = targ(q_clean);
    a.q_corr = targ(q_corr);
    a.k_clean = targ(k_clean);
    a.v_clean = targ(v_clean);
    a.k_corr = targ(k_corr);
    a.v_corr = targ(v_corr);
    a.o = static_cast<float*>(o.ptr);
    a.o_bs = o.batch_stride;
    a.o_rs = o.row_stride;
    a.o_hs = o.head_stride;
    a.lse = lse;
    return hip_status(timed(K_FWD_F32, s, [&] { return launch_fwd_f32(P, a, s); }));
  }
  FwdWs ws;
  carve_fwd(P, false, static_cast<char*>(workspace), &ws);
  hipError_t e = timed(K_FLAG, s, [&] { return launch_flag_clear(ws.flag, s); });
  if (e != hipSuccess) return BDATTN_EHIP;
  PackKArgs pk;
  std::memset(&pk, 0, sizeof pk);
  pk.k_clean = targ(k_clean);
  pk.v_clean = targ(v_clean);
  pk.k_corr = targ(k_corr);
  pk.v_corr = targ(v_corr);
  pk.kn = ws.kn;
  pk.vt = ws.vt;
  pk.flag = ws.flag;
  e = timed(K_PACK_K, s, [&] { return launch_pack_k(P, pk, s); });
  if (e != hipSuccess) return BDATTN_EHIP;
  FwdArgs a;
  a.q_clean = targ(q_clean);
  a.q_corr = targ(q_corr);
  a.kn = ws.kn;
  a.vt = ws.vt;
  a.o = o.ptr;
  a.o_bs = o.batch_stride;
  a.o_rs = o.row_stride;
  a.o_hs = o.head_stride;
  a.o_f32 = o_dtype == BDATTN_F32;
  a.lse = lse;
  a.queue = ws.flag + kQueueFwd;
  return hip_status(timed(K_FWD, s, [&] { return launch_fwd_bf16(P, a, s); }));
}

}  // namespace

extern "C" {

int bdattn_fwd(const bdattn_problem* problem, const bdattn_share* share, const bdattn_kv* kv,
               bdattn_tensor q_clean, bdattn_tensor q_corr, bdattn_tensor k_clean, bdattn_tensor v_clean,
               bdattn_tensor k_corr, bdattn_tensor v_corr, bdattn_tensor o, int32_t o_dtype, float* lse,
               void* workspace, size_t ws_bytes, void* hip_stream) {
  return fwd_impl(problem, share, kv, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr, o, o_dtype, lse,
                  workspace, ws_bytes, hip_stream);
}

int bdattn_workspace_status(const void* workspace, void* hip_stream) {
  const void* ws = workspace;
  if (!ws) {  // the static scratch of bdattn_fwd_static on the current device
    ws = static_scratch_ptr();
    if (!ws) return BDATTN_EHIP;
  }
  if (reinterpret_cast<uintptr_t>(ws) % 256) return BDATTN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  int32_t flag = 0;
  if (hipStreamSynchronize(s) != hipSuccess) return BDATTN_EHIP;
  if (hipMemcpy(&flag, ws, sizeof flag, hipMemcpyDeviceToHost) != hipSuccess) return BDATTN_EHIP;
  return flag ? BDATTN_ERANGE : BDATTN_OK;
}

int bdattn_shard_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc, const float* o_part,
                       const float* lse_part, void* o_final_bf16, void* hip_stream) {
  if (rows < 0 || d <= 0 || d % 4 != 0) return BDATTN_EINVAL;
  if (rows == 0) return BDATTN_OK;
  if (!o_acc || !lse_acc || !o_part || !lse_part) return BDATTN_EINVAL;
  if (reinterpret_cast<uintptr_t>(o_acc) % 16 || reinterpret_cast<uintptr_t>(o_part) % 16) return BDATTN_EINVAL;
  if (o_final_bf16 && reinterpret_cast<uintptr_t>(o_final_bf16) % 8) return BDATTN_EINVAL;
  if (64 % (d / 4) != 0 && (d / 4) % 64 != 0) return BDATTN_ENOTSUP;  // a row's lanes share one wave
  MergeArgs a{rows, d, o_acc, lse_acc, o_part, lse_part, static_cast<uint16_t*>(o_final_bf16)};
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  return hip_status(timed(K_MERGE, s, [&] { return launch_merge(a, s); }));
}

int bdattn_bwd(const bdattn_problem* problem, const bdattn_share* share, const bdattn_kv* kv,
               bdattn_tensor q_clean, bdattn_tensor q_corr, bdattn_tensor k_clean, bdattn_tensor v_clean,
               bdattn_tensor k_corr, bdattn_tensor v_corr, bdattn_tensor o_final, int32_t o_dtype,
               const float* lse_final, bdattn_tensor d_o, float* delta, int32_t flags, float* dq_acc,
               float* dk_clean_acc, float* dv_clean_acc, float* dk_corr_acc, float* dv_corr_acc,
               void* workspace, size_t ws_bytes, void* hip_stream) {
  int32_t runs = 0;
  if (!problem_ok(problem) || !share_ok(problem, share, &runs) || !kv_ok(problem, kv)) return BDATTN_EINVAL;
  if (!problem_supported(problem) || problem->dtype != BDATTN_BF16) return BDATTN_ENOTSUP;
  if (o_dtype != BDATTN_BF16 && o_dtype != BDATTN_F32) return BDATTN_EINVAL;
  if (flags & ~(BDATTN_BWD_DELTA_READY | BDATTN_BWD_OVERWRITE)) return BDATTN_EINVAL;
  const bool delta_ready = (flags & BDATTN_BWD_DELTA_READY) != 0;
  const bool overwrite = (flags & BDATTN_BWD_OVERWRITE) != 0;
  // overwrite is exact only where this one call writes every gradient
  // element: the whole mask (every row sees its own block, every key is seen
  // by its own block's rows)
  if (overwrite && !(share->n_blocks == problem->L / problem->M && share->n_clean == 1 &&
                     share->clean_lo[0] == 0 && share->clean_hi[0] == problem->L && kv->n == 1 &&
                     kv->lo[0] == 0 && kv->hi[0] == problem->L && kv->include_local != 0))
    return BDATTN_EINVAL;
  const Plan P = make_plan(problem, share, kv);
  if (P.R == 0) return BDATTN_OK;
  auto al16 = [](const void* p) { return p && reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (!lse_final || !delta || !al16(dq_acc)) return BDATTN_EINVAL;
  if (P.n_clean_rows > 0 && !tensor_ok(q_clean, 2)) return BDATTN_EINVAL;
  if (P.n_corr_rows > 0 && !tensor_ok(q_corr, 2)) return BDATTN_EINVAL;
  if (!tensor_ok(d_o, 2)) return BDATTN_EINVAL;
  if (!delta_ready && !tensor_ok(o_final, o_dtype == BDATTN_F32 ? 4 : 2)) return BDATTN_EINVAL;
  if (kv->n > 0 && (!tensor_ok(k_clean, 2) || !tensor_ok(v_clean, 2) || !al16(dk_clean_acc) ||
                    !al16(dv_clean_acc)))
    return BDATTN_EINVAL;
  const bool local = kv->include_local && P.n_corr_rows > 0;
  if (local && (!tensor_ok(k_corr, 2) || !tensor_ok(v_corr, 2) || !al16(dk_corr_acc) || !al16(dv_corr_acc)))
    return BDATTN_EINVAL;
  const size_t need = carve_bwd(P, nullptr, nullptr);
  if (!workspace || ws_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256) return BDATTN_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  BwdWs ws;
  carve_bwd(P, static_cast<char*>(workspace), &ws);
  hipError_t e = timed(K_FLAG, s, [&] { return launch_flag_clear(ws.flag, s); });
  if (e != hipSuccess) return BDATTN_EHIP;
  // pack_q also forms D = rowsum(dO * O) unless the caller gives it
  PackQArgs pq{targ(q_clean), targ(q_corr), targ(d_o), delta_ready ? TensorArg{} : targ(o_final),
               o_dtype == BDATTN_F32, delta_ready != 0, lse_final, delta, ws.qh, ws.doh,
               ws.lse2, ws.dc, ws.vis, ws.flag};
  e = timed(K_PACK_Q, s, [&] { return launch_pack_q(P, pq, s); });
  if (e != hipSuccess) return BDATTN_EHIP;
  if (P.nkc == 0) return BDATTN_OK;  // no key in this call: nothing to add
  PackKArgs pk;
  std::memset(&pk, 0, sizeof pk);
  pk.k_clean = targ(k_clean);
  pk.v_clean = targ(v_clean);
  pk.k_corr = targ(k_corr);
  pk.v_corr = targ(v_corr);
  pk.kh = ws.kh;
  pk.vh = ws.vh;
  pk.flag = ws.flag;
  e = timed(K_PACK_K, s, [&] { return launch_pack_k(P, pk, s); });
  if (e != hipSuccess) return BDATTN_EHIP;
  DkdvArgs ka{ws.qh, ws.doh, ws.lse2, ws.dc, ws.vis, ws.kh, ws.vh,
              dk_clean_acc, dv_clean_acc, dk_corr_acc, dv_corr_acc, overwrite ? 1 : 0, ws.flag + kQueueDkdv};
  e = timed(K_DKDV, s, [&] { return launch_dkdv(P, ka, s); });
  if (e != hipSuccess) return BDATTN_EHIP;
  DqArgs qa{ws.qh, ws.doh, ws.lse2, ws.dc, ws.kh, ws.vh, dq_acc, overwrite ? 1 : 0, ws.flag + kQueueDq};
  return hip_status(timed(K_DQ, s, [&] { return launch_dq(P, qa, s); }));
}

int bdattn_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = enable != 0;
  return BDATTN_OK;
}

int bdattn_profile_read(const char** names, int64_t* counts, double* ms, int32_t cap, int32_t* n) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!n || cap < 0) return BDATTN_EINVAL;
  int64_t cnt[K_COUNT] = {0};
  double tot[K_COUNT] = {0};
  int rc = BDATTN_OK;
  for (auto& r : g_prof.rec) {
    float t = 0.f;
    if (hipEventSynchronize(r.second.second) != hipSuccess ||
        hipEventElapsedTime(&t, r.second.first, r.second.second) != hipSuccess)
      rc = BDATTN_EHIP;
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
