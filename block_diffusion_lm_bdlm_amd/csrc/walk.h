// walk.h — key-tile walk of a query tile (forward and dQ kernels).
#pragma once

#include "plan.h"

namespace bd {

// Key tiles a query tile visits: one slot per key segment (count 0 when the
// segment holds no key the tile's rows see).  Constant-indexed so it stays
// in registers.
struct KeyWalk {
  int32_t total;
  int32_t start[kMaxKSeg], count[kMaxKSeg];
  int32_t full_lo[kMaxKSeg], full_hi[kMaxKSeg];  // tiles inside [full_lo, full_hi) need no mask
};

__device__ inline void keywalk_build(const Plan& P, const QSeg& S, int32_t r_first, int32_t r_last,
                                     KeyWalk& w) {
  const bool clean = S.kind == KIND_CLEAN;
  const RowBounds rf = row_bounds(P, S, r_first), rl = row_bounds(P, S, r_last);
  w.total = 0;
#pragma unroll
  for (int32_t j = 0; j < kMaxKSeg; ++j) {
    w.start[j] = 0;
    w.count[j] = 0;
    w.full_lo[j] = 0;
    w.full_hi[j] = 0;
    if (j < P.nk) {
      const KSeg K = P.k[j];
      int32_t flo, fhi, llo, lhi;
      compact_range(K, rf, clean, &flo, &fhi);
      compact_range(K, rl, clean, &llo, &lhi);
      if (lhi > flo) {
        const int32_t a = K.c0 + ((flo - K.c0) / kBK) * kBK;
        w.start[j] = a;
        w.count[j] = (lhi - a + kBK - 1) / kBK;
        w.full_lo[j] = llo;
        w.full_hi[j] = fhi;
      }
    }
    w.total += w.count[j];
  }
}

// Tile t of the walk -> compact start c and key segment j.
__device__ inline void keywalk_at(const KeyWalk& w, int32_t t, int32_t* c, int32_t* j) {
  int32_t sel = 0, u = t;
#pragma unroll
  for (int32_t k = 0; k < kMaxKSeg; ++k) {
    if (sel == k && u >= w.count[k] && k + 1 < kMaxKSeg) {
      u -= w.count[k];
      sel = k + 1;
    }
  }
  int32_t st = w.start[0];
#pragma unroll
  for (int32_t k = 1; k < kMaxKSeg; ++k)
    if (sel == k) st = w.start[k];
  *j = sel;
  *c = st + u * kBK;
}

__device__ inline bool keywalk_full(const KeyWalk& w, int32_t j, int32_t c) {
  int32_t lo = w.full_lo[0], hi = w.full_hi[0];
#pragma unroll
  for (int32_t k = 1; k < kMaxKSeg; ++k)
    if (j == k) {
      lo = w.full_lo[k];
      hi = w.full_hi[k];
    }
  return c >= lo && c + kBK <= hi;
}

}  // namespace bd
