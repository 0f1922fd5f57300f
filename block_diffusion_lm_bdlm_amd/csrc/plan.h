// plan.h — work decomposition shared by the host planner and the kernels.
//
// Every mapping from a workgroup to its work (query tiles, key tiles, heads)
// and every row's visible key range is computed by the __host__ __device__
// functions below, so the order the host exports (bdattn_plan_order) and the
// order the kernels run are the same code.
//
// Visibility (pages: "CSBP 完全拆解", sections "传统上下文并行为什么会传错东西"
// and "CSBP：BP 管损坏块，CP 管干净上下文"): a corrupted query of block b sees
// clean tokens < b*M and the corrupted tokens of block b; a clean query of
// token t sees clean tokens < (t/M + 1)*M (block-causal) or <= t
// (token-causal).  With a sliding window W over the clean keys, a query at
// token position t (the corrupted token at offset i of block b sits at
// b*M + i) sees clean token j only if t - j < W.  Every row therefore sees
// one interval of clean tokens, and both its ends grow with the row.
//
// Load balance ("CSBP 完全拆解", section "负载均衡：为什么要首尾块配对"): the
// query tiles of each kind are paired early with late (tile t with tile
// n-1-t), so every workgroup carries the same number of key tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

constexpr int kMaxRuns = 8;
constexpr int kMaxQSeg = 2 + kMaxRuns;
constexpr int kMaxKSeg = 3;
constexpr int kBQ = 128;     // query rows per tile (forward, dQ)
constexpr int kBK = 64;      // keys per tile (forward, dQ)
constexpr int kBKB = 128;    // keys per tile (dK/dV)
constexpr int kBQB = 64;     // query rows per step (dK/dV)
constexpr int kAlign = 128;  // compact key segments start at multiples of this
constexpr int kXCD = 8;      // MI355X accelerator complex dies

enum { KIND_CLEAN = 0, KIND_CORR = 1 };

struct QSeg {
  int32_t kind;    // KIND_CLEAN or KIND_CORR
  int32_t row0;    // first share row
  int32_t nrows;
  int32_t src0;    // first row in q_clean (clean) or q_corr / k_corr (corrupted)
  int32_t first;   // clean: first token; corrupted: first block id
  int32_t tile0;   // first query tile of the segment
  int32_t ntiles;  // ceil(nrows / kBQ)
  int32_t pad_;
};

struct KSeg {
  int32_t kind;  // KIND_CLEAN: token rows of k_clean; KIND_CORR: packed rows of k_corr
  int32_t t0;    // first source row
  int32_t len;
  int32_t c0;    // compact start, multiple of kAlign
};

struct Plan {
  int32_t batch, L, M, hq, hkv, d, G, token_causal;
  int32_t M_log2;         // log2(M) when M is a power of two, else -1
  int32_t window;         // clean-key sliding window in tokens (0 = none)
  float scale, scale_log2;
  int32_t R;              // share rows
  int32_t n_clean_rows;   // share clean rows (first in row order)
  int32_t n_corr_rows;    // n_blocks * M
  int32_t nq;             // query segments (clean ones first)
  int32_t ntiles;         // query tiles
  int32_t n_clean_tiles;  // query tiles of the clean segments
  int32_t npairs;         // query-tile pairs per (batch, head)
  int32_t nk;             // key segments (clean ranges first, then local)
  int32_t nkc;            // compact key rows (multiple of kAlign)
  int32_t nkt;            // dK/dV key tiles (kBKB keys each, within one segment)
  int32_t nkpairs;        // dK/dV key-tile pairs per (batch, KV head)
  int32_t nqc;            // compact query rows = ntiles * kBQ
  int64_t nwg_q;          // work items of the query-major kernels
  int64_t nwg_k;          // work items of the key-major kernel
  QSeg q[kMaxQSeg];
  KSeg k[kMaxKSeg];
};

// Dispatch order w -> logical work index.  Workgroups are handed to the
// XCDs round-robin (w % 8); mapping each XCD's workgroups to a contiguous
// block of logical indices keeps one KV head's query heads and neighbouring
// query tiles on one XCD, where they share that die's L2.
__host__ __device__ inline int64_t xcd_logical(int64_t w, int64_t n) {
  const int64_t x = w % kXCD, per = n / kXCD, rem = n % kXCD;
  const int64_t base = x * per + (x < rem ? x : rem);
  return base + w / kXCD;
}

// The kernels take their work items from one queue per XCD: queue x holds
// the XCD's contiguous block of logical indices above (the order
// xcd_logical assigns), so the L2 locality of that order is kept, while a
// workgroup whose own queue is empty takes items from the other queues.
// The dies do not run at one speed (the same work measured up to 10% apart
// between the XCDs of one device), so a fixed split of the items leaves
// the faster dies idle at the end.
__host__ __device__ inline int64_t queue_base(int64_t n, int x) {
  const int64_t per = n / kXCD, rem = n % kXCD;
  return x * per + (x < rem ? x : rem);
}
__host__ __device__ inline int64_t queue_len(int64_t n, int x) { return n / kXCD + (x < n % kXCD ? 1 : 0); }

// Workgroups of a launch over `items` work items: one per item, plus a
// quarter more (rounded up to whole rounds of the eight XCDs).  Workgroups
// go to the XCDs round-robin, so each die runs the same number; the spares
// let a die that finishes its own queue early take items from the others,
// and on the last die to finish they find every queue empty and end.
inline unsigned queue_grid(int64_t items) {
  const int64_t spare = (items / 4 + kXCD - 1) / kXCD * kXCD;
  return (unsigned)(items + spare);
}

// Next work item of a workgroup on XCD x: its own queue first, then the
// others in turn; -1 when all are empty.  heads[q * stride] counts the
// items taken from queue q (zeroed before the launch); *scan counts the
// queues this workgroup has found empty.  Called by one thread of the
// workgroup.
__device__ inline int64_t next_item(int32_t* heads, int stride, int64_t n, int x, int* scan) {
  while (*scan < kXCD) {
    const int q = (x + *scan) % kXCD;
    const int32_t k = atomicAdd(heads + q * stride, 1);
    if (k < queue_len(n, q)) return queue_base(n, q) + k;
    ++*scan;
  }
  return -1;
}

// Pair p of the query tiles -> (heavier tile, lighter tile or -1).
__host__ __device__ inline void pair_tiles(const Plan& P, int32_t p, int32_t* a, int32_t* b) {
  const int32_t nc = P.n_clean_tiles, nx = P.ntiles - P.n_clean_tiles;
  const int32_t pc = (nc + 1) / 2;
  int32_t base, n, t;
  if (p < pc) { base = 0; n = nc; t = p; }
  else { base = nc; n = nx; t = p - pc; }
  const int32_t hi = n - 1 - t;
  *a = base + hi;
  *b = (hi == t) ? -1 : base + t;
}

struct WgQ {
  int32_t b, h, g, tile_a, tile_b;
};

// Query-major workgroup w (dispatch order) -> batch, head, its two tiles.
// Logical order: batch, KV head, pair, query head within the group.
// Logical work item l of the query-major kernels -> (batch, head, tiles).
__host__ __device__ inline WgQ decode_item_q(const Plan& P, int64_t l) {
  WgQ r;
  const int32_t gq = (int32_t)(l % P.G);
  int64_t rest = l / P.G;
  const int32_t pair = (int32_t)(rest % P.npairs);
  rest /= P.npairs;
  r.g = (int32_t)(rest % P.hkv);
  r.b = (int32_t)(rest / P.hkv);
  r.h = r.g * P.G + gq;
  pair_tiles(P, pair, &r.tile_a, &r.tile_b);
  return r;
}
// Item w of the exported order: queue w % 8's (w / 8)-th item.
__host__ __device__ inline WgQ decode_wg_q(const Plan& P, int64_t w) { return decode_item_q(P, xcd_logical(w, P.nwg_q)); }

__host__ __device__ inline int32_t seg_of_tile(const Plan& P, int32_t t) {
  int32_t s = 0;
  while (s + 1 < P.nq && t >= P.q[s + 1].tile0) ++s;
  return s;
}

// Visible key interval(s) of one query row, in source-row coordinates.
struct RowBounds {
  int32_t lo_clean;  // clean tokens [lo_clean, hi_clean) are visible
  int32_t hi_clean;
  int32_t lo_loc;    // packed corrupted rows [lo_loc, hi_loc) are visible
  int32_t hi_loc;
};

// Token position of row 0 of segment s (rows of a segment are consecutive
// tokens: clean tokens, or the tokens of consecutive blocks).
// n / M and n % M for n >= 0: a shift and a mask when M is a power of two
// (every block size the pages use), a division otherwise.
__host__ __device__ inline int32_t div_M(const Plan& P, int32_t n) { return P.M_log2 >= 0 ? n >> P.M_log2 : n / P.M; }
__host__ __device__ inline int32_t mod_M(const Plan& P, int32_t n) {
  return P.M_log2 >= 0 ? n & (P.M - 1) : n % P.M;
}

__host__ __device__ inline int64_t seg_token0(const Plan& P, const QSeg& s) {
  return s.kind == KIND_CLEAN ? (int64_t)s.first : (int64_t)s.first * P.M;
}

__host__ __device__ inline RowBounds row_bounds(const Plan& P, const QSeg& s, int32_t r) {
  RowBounds rb;
  if (s.kind == KIND_CLEAN) {
    const int32_t t = s.first + r;
    rb.hi_clean = P.token_causal ? t + 1 : (div_M(P, t) + 1) * P.M;
    rb.lo_loc = rb.hi_loc = 0;
  } else {
    const int32_t blk = s.first + div_M(P, r);
    rb.hi_clean = blk * P.M;
    rb.lo_loc = s.src0 + r - mod_M(P, r);
    rb.hi_loc = rb.lo_loc + P.M;
  }
  const int64_t lo = P.window > 0 ? seg_token0(P, s) + r - P.window + 1 : 0;
  rb.lo_clean = lo > 0 ? (int32_t)lo : 0;
  return rb;
}

__host__ __device__ inline int32_t clampi(int32_t x, int32_t lo, int32_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Number of keys a row sees in the whole mask (every key of every call):
// its clean interval plus, for a corrupted row, its own block.
__host__ __device__ inline int32_t row_nkeys(const RowBounds& rb) {
  const int32_t nc = rb.hi_clean > rb.lo_clean ? rb.hi_clean - rb.lo_clean : 0;
  return nc + (rb.hi_loc - rb.lo_loc);
}

// Probability scale of a backward row: the kernels form P * 2^c instead of
// P, with dO and D of the row packed as dO * 2^-c and D * 2^-c, so every
// product (P dO, P (dP - D)) keeps its value while P leaves fp16's
// subnormal range.  A row that sees n keys has probabilities of order 1/n;
// c = ceil(log2 n) - 7, within [0, 15], lifts them to about 2^-7, and
// P * 2^c <= 2^15 holds for any row (P <= 1).
constexpr int32_t kPScaleBias = 7;
constexpr int32_t kPScaleMax = 15;
__host__ __device__ inline int32_t row_pscale(int32_t n) {
  const int32_t lg = n <= 1 ? 0 : 32 - __builtin_clz((uint32_t)(n - 1));  // ceil(log2 n)
  return clampi(lg - kPScaleBias, 0, kPScaleMax);
}

// Row's visible compact interval [vlo, vhi) within key segment ks.
__host__ __device__ inline void compact_range(const KSeg& ks, const RowBounds& rb, bool clean_row,
                                              int32_t* vlo, int32_t* vhi) {
  if (ks.kind == KIND_CLEAN) {
    *vlo = ks.c0 + clampi(rb.lo_clean - ks.t0, 0, ks.len);
    *vhi = ks.c0 + clampi(rb.hi_clean - ks.t0, 0, ks.len);
    if (*vhi < *vlo) *vhi = *vlo;
  } else if (clean_row) {
    *vlo = *vhi = ks.c0;
  } else {
    *vlo = ks.c0 + clampi(rb.lo_loc - ks.t0, 0, ks.len);
    *vhi = ks.c0 + clampi(rb.hi_loc - ks.t0, 0, ks.len);
    if (*vhi < *vlo) *vhi = *vlo;
  }
}

// ---------------------------------------------------------------- dK/dV side
// Key tiles of kBKB keys never straddle a key segment; tile index -> segment.
__host__ __device__ inline int32_t ktiles_of(const KSeg& ks) { return (ks.len + kBKB - 1) / kBKB; }

__host__ __device__ inline void ktile_locate(const Plan& P, int32_t t, int32_t* seg, int32_t* off) {
  int32_t s = 0;
  while (s < P.nk - 1 && t >= ktiles_of(P.k[s])) { t -= ktiles_of(P.k[s]); ++s; }
  *seg = s;
  *off = t * kBKB;
}

// Key-major pairs: clean key tiles paired early/late (tile t with n-1-t, the
// same dual-end rule), local tiles (seen by one block each) appended singly.
__host__ __device__ inline int32_t n_clean_ktiles(const Plan& P) {
  int32_t n = 0;
  for (int32_t s = 0; s < P.nk; ++s)
    if (P.k[s].kind == KIND_CLEAN) n += ktiles_of(P.k[s]);
  return n;
}

__host__ __device__ inline void kpair_tiles(const Plan& P, int32_t p, int32_t* a, int32_t* b) {
  const int32_t nc = n_clean_ktiles(P);
  const int32_t pc = (nc + 1) / 2;
  if (p < pc) {
    const int32_t hi = nc - 1 - p;
    *a = p;  // early clean keys are seen by the most queries: heavier first
    *b = (hi == p) ? -1 : hi;
  } else {
    *a = nc + (p - pc);
    *b = -1;
  }
}

struct WgK {
  int32_t b, g, tile_a, tile_b;
};

// The key-major kernel's queues hand out their blocks longest first: the
// k-th claim on queue q takes the block's clean pairs (long walks) in
// order, then its local tiles (a few steps each).  In the logical order the
// local tiles sit between rounds of long items; at 8K (two long items per
// CU) a workgroup of the second round then at times waited a whole item
// for a CU of one shader engine while a CU of another engine stood idle,
// and the launch took 2.6 instead of 1.9 ms.  Items are l = group * np + p,
// pair p < pc a clean pair; nlong(m) counts the clean pairs below item m.
__host__ __device__ inline int64_t ktile_claim(const Plan& P, int q, int64_t k) {
  const int64_t n = P.nwg_k, np = P.nkpairs, pc = (n_clean_ktiles(P) + 1) / 2, ns = np - pc;
  const int64_t b0 = queue_base(n, q), b1 = b0 + queue_len(n, q);
  auto nlong = [&](int64_t m) { return (m / np) * pc + (m % np < pc ? m % np : pc); };
  const int64_t l0 = nlong(b0), nl = nlong(b1) - l0;
  if (k < nl) {
    const int64_t j = l0 + k;
    return (j / pc) * np + j % pc;
  }
  if (ns == 0) return -1;  // not reached: a block without local tiles has only long items
  const int64_t j = (b0 - l0) + (k - nl);  // short items below b0, plus the rank in the block
  return (j / ns) * np + pc + j % ns;
}

// next_item for the key-major kernel, in ktile_claim order.
__device__ inline int64_t next_item_k(const Plan& P, int32_t* heads, int stride, int x, int* scan) {
  const int64_t n = P.nwg_k;
  while (*scan < kXCD) {
    const int q = (x + *scan) % kXCD;
    const int32_t k = atomicAdd(heads + q * stride, 1);
    if (k < queue_len(n, q)) return ktile_claim(P, q, k);
    ++*scan;
  }
  return -1;
}

// Logical work item l of the key-major kernel -> (batch, KV head, tiles).
__host__ __device__ inline WgK decode_item_k(const Plan& P, int64_t l) {
  WgK r;
  const int32_t pair = (int32_t)(l % P.nkpairs);
  const int64_t rest = l / P.nkpairs;
  r.g = (int32_t)(rest % P.hkv);
  r.b = (int32_t)(rest / P.hkv);
  kpair_tiles(P, pair, &r.tile_a, &r.tile_b);
  return r;
}
// Item w of the exported order: the (w / 8)-th item queue w % 8 hands out.
__host__ __device__ inline WgK decode_wg_k(const Plan& P, int64_t w) {
  return decode_item_k(P, ktile_claim(P, (int)(w % kXCD), w / kXCD));
}

// First row of query segment s that sees any key at or after source row
// `k0` of a key segment of kind `kkind` (rows are monotone in visibility).
__host__ __device__ inline int32_t first_seeing_row(const Plan& P, const QSeg& s, int32_t kkind,
                                                    int32_t k0) {
  if (kkind == KIND_CLEAN) {
    if (s.kind == KIND_CLEAN) {
      const int32_t tmin = P.token_causal ? k0 : div_M(P, k0) * P.M;
      return clampi(tmin - s.first, 0, s.nrows);
    }
    const int32_t bmin = div_M(P, k0) + 1;
    const int64_t r = (int64_t)(bmin - s.first) * P.M;
    return (int32_t)(r < 0 ? 0 : (r > s.nrows ? s.nrows : r));
  }
  if (s.kind == KIND_CLEAN) return s.nrows;
  // packed corrupted key rows: the rows of the same packed block
  const int32_t pmin = div_M(P, k0) * P.M;
  return clampi(pmin - s.src0, 0, s.nrows);
}

// One past the last row of segment s that sees any key before source row
// `k1` (exclusive end of the key tile).
__host__ __device__ inline int32_t end_seeing_row(const Plan& P, const QSeg& s, int32_t kkind,
                                                  int32_t k1) {
  if (kkind == KIND_CLEAN) {
    if (P.window <= 0) return s.nrows;
    // rows at token position >= k1 + W - 1 see only clean tokens >= k1
    const int64_t r = (int64_t)k1 + P.window - 1 - seg_token0(P, s);
    return (int32_t)(r < 0 ? 0 : (r > s.nrows ? s.nrows : r));
  }
  if (s.kind == KIND_CLEAN) return 0;
  const int32_t pmax = div_M(P, k1 + P.M - 1) * P.M;
  return clampi(pmax - s.src0, 0, s.nrows);
}

}  // namespace bd
