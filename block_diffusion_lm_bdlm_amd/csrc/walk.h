// walk.h — key-tile walk of a query tile (forward and dQ kernels).
//
// A query tile visits, per key segment (at most three: two clean ranges and
// the local corrupted keys), the key tiles any of its rows can see.  Fields
// are named scalars so the walk lives in scalar registers.
#pragma once

#include "plan.h"

namespace bd {

static_assert(kMaxKSeg == 3, "KeyWalk holds exactly three segments");

struct KeyWalk {
  int32_t total;
  int32_t s0, s1, s2;     // first tile (compact row) per segment
  int32_t n0, n1, n2;     // tiles per segment
  int32_t fl0, fl1, fl2;  // tiles inside [fl, fh) need no mask
  int32_t fh0, fh1, fh2;
};

__device__ inline void keywalk_seg(const Plan& P, int32_t j, bool clean, const RowBounds& rf,
                                   const RowBounds& rl, int32_t* s, int32_t* n, int32_t* fl,
                                   int32_t* fh) {
  *s = *n = *fl = *fh = 0;
  if (j >= P.nk) return;
  const KSeg K = P.k[j];
  int32_t flo, fhi, llo, lhi;
  compact_range(K, rf, clean, &flo, &fhi);
  compact_range(K, rl, clean, &llo, &lhi);
  if (lhi <= flo) return;
  const int32_t a = K.c0 + ((flo - K.c0) / kBK) * kBK;
  *s = a;
  *n = (lhi - a + kBK - 1) / kBK;
  *fl = llo;
  *fh = fhi;
}

// Rows r_first..r_last of segment S are monotone in what they see, so the
// first and last rows bound the walk.
__device__ inline KeyWalk keywalk_build(const Plan& P, const QSeg& S, int32_t r_first, int32_t r_last) {
  const bool clean = S.kind == KIND_CLEAN;
  const RowBounds rf = row_bounds(P, S, r_first), rl = row_bounds(P, S, r_last);
  KeyWalk w;
  keywalk_seg(P, 0, clean, rf, rl, &w.s0, &w.n0, &w.fl0, &w.fh0);
  keywalk_seg(P, 1, clean, rf, rl, &w.s1, &w.n1, &w.fl1, &w.fh1);
  keywalk_seg(P, 2, clean, rf, rl, &w.s2, &w.n2, &w.fl2, &w.fh2);
  w.total = w.n0 + w.n1 + w.n2;
  return w;
}

// Tile t of the walk -> compact start c, segment j and whether it needs a mask.
__device__ inline void keywalk_at(const KeyWalk& w, int32_t t, int32_t* c, int32_t* j, bool* full) {
  int32_t start, lo, hi;
  if (t < w.n0) {
    *j = 0;
    start = w.s0;
    lo = w.fl0;
    hi = w.fh0;
  } else if (t < w.n0 + w.n1) {
    t -= w.n0;
    *j = 1;
    start = w.s1;
    lo = w.fl1;
    hi = w.fh1;
  } else {
    t -= w.n0 + w.n1;
    *j = 2;
    start = w.s2;
    lo = w.fl2;
    hi = w.fh2;
  }
  *c = start + t * kBK;
  *full = *c >= lo && *c + kBK <= hi;
}

// Whether a row with compact visible range [vlo, vhi) sees any of the 32
// keys from compact position k0 on.
__device__ __forceinline__ bool sees_block32(int32_t vlo, int32_t vhi, int32_t k0) {
  return max(vlo, k0) < min(vhi, k0 + 32);
}

}  // namespace bd
