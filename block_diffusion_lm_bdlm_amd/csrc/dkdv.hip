// dkdv.hip — dK and dV of BDLM attention, key-major.
//
// For every visible pair, with the final LSE and D_i = dO_i . O_i:
//   P = exp(s - LSE),  dS = P (dO_i . v_j - D_i),
//   dV_j += P dO_i,  dK_j += scale dS q_i
// (chain rule of the attention equation in "CSBP 完全拆解"; clean keys collect
// contributions from every later block, section "CSBP：BP 管损坏块，CP 管干净
// 上下文").
//
// A workgroup owns 128 keys of one KV head and runs 8 waves, two per SIMD,
// in pairs that own the same 32 keys:
//   S-wave: K in registers; S = Q K^T, P = exp(S - LSE) (masked), writes P
//           to LDS, accumulates dV^T += dO^T P.
//   P-wave: V in registers; dP = dO V^T, reads P, dS = P (dP - D),
//           accumulates dK^T += Q^T dS.
// Each key has exactly one writer per gradient, so no atomics are needed,
// and the two waves of a SIMD overlap one's vector work with the other's
// matrix work.  The workgroup walks every query row (of every query head of
// the group) that sees its keys, in steps of 64 rows staged through LDS
// (natural Q, dO for S and dP; transposed fp16 Q^T, dO^T for the
// contractions over rows).
// The walk runs back to front by position (all heads of the group at each
// position): the last rows are seen by every key tile, so the workgroups
// resident on one XCD stay on the same rows and share them through L2.  Each step stages per-row visibility bounds next to LSE and D,
// so a step that straddles the mask boundary needs no division per element.
#include <climits>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace bd {

namespace {

constexpr int kNB = kBQB / 32;     // 32-row MFMA blocks per step
constexpr int kPairs = kBKB / 32;  // S-wave / P-wave pairs per workgroup, 32 keys each
static_assert(kBQB % 32 == 0 && 64 % kBQB == 0, "steps are whole MFMA blocks inside one 64-row tile");

template <int D>
struct __attribute__((aligned(16))) DkdvSmem {
  static constexpr int NS = D + 8;     // natural row stride (bf16)
  static constexpr int TS = kBQB + 8;  // transposed row stride (fp16)
  uint16_t q[2][kBQB * NS];
  uint16_t dO[2][kBQB * NS];
  _Float16 qt[2][D * TS];
  _Float16 dot[2][D * TS];
  float lse2[2][kBQB];
  float dc[2][kBQB];
  int32_t vlo[2][kBQB];  // row sees key sources [vlo, vhi) of this key tile's segment
  int32_t vhi[2][kBQB];
  // P from each S-wave to its P-wave, in the MFMA C-tile order of each lane
  _Float16 xchg[kPairs][kNB][64][16];
  // steps of the walk: segment s contributes wcount[s] steps from row wfirst[s]
  int32_t wseg[kMaxQSeg], wfirst[kMaxQSeg], wcount[kMaxQSeg];
  int32_t wn, wper;
};

// Position of the walk: k-th step from the end of walk segment j, query head
// hs within the group.
struct StepPos {
  int32_t k, j, hs;
};

constexpr int kThreads = 128 * kPairs;  // two waves per pair

// Prefetch of one step, in two halves so each is live for half a step:
// A = natural Q, dO and the per-row data; B = transposed Q^T, dO^T.
template <int D>
struct StageA {
  static constexpr int NCH = (kBQB * D / 8 + kThreads - 1) / kThreads;  // 16-byte chunks per thread per tensor
  u32x4 r[2 * NCH];
  float l2, dd;
  int32_t lo, hi;
};
template <int D>
struct StageB {
  static constexpr int NCH = (kBQB * D / 8 + kThreads - 1) / kThreads;
  u32x4 r[2 * NCH];
};

template <int D>
__device__ inline void stage_load_a(const DkdvArgs& A, const Plan& P, const KSeg& K, const QSeg& S, int64_t hb,
                                    int32_t r0, int tid, StageA<D>& st) {
  constexpr int NCH = StageA<D>::NCH;
  const int32_t cq = S.tile0 * kBQ + r0;  // compact row of the step's first row
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = tid + kThreads * j;
    if (ch >= kBQB * D / 8) break;
    const int row = ch / (D / 8), dcol = ch % (D / 8);
    st.r[j] = ldg16(A.qn + (hb * P.nqc + cq + row) * D + dcol * 8);
    st.r[NCH + j] = ldg16(A.don + (hb * P.nqc + cq + row) * D + dcol * 8);
  }
  if (tid < kBQB) {
    st.l2 = A.lse2[hb * P.nqc + cq + tid];
    st.dd = A.dc[hb * P.nqc + cq + tid];
    const int32_t rr = r0 + tid;
    st.lo = 0;
    st.hi = 0;
    if (rr < S.nrows) {
      const RowBounds rb = row_bounds(P, S, rr);
      if (K.kind == KIND_CLEAN) {
        st.hi = rb.hi_clean;
      } else if (S.kind == KIND_CORR) {
        st.lo = rb.lo_loc;
        st.hi = rb.hi_loc;
      }
    }
  }
}

template <int D>
__device__ inline void stage_load_b(const DkdvArgs& A, const Plan& P, const QSeg& S, int64_t hb, int32_t r0,
                                    int tid, StageB<D>& st) {
  constexpr int NCH = StageB<D>::NCH;
  const int32_t cq = S.tile0 * kBQ + r0;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = tid + kThreads * j;
    if (ch >= kBQB * D / 8) break;
    const int d = ch / (kBQB / 8), sc = ch % (kBQB / 8);
    // row cq lies in the 64-row tile cq / 64, stored [D][64]
    const int64_t t = hb * D * P.nqc + (int64_t)(cq & ~63) * D + d * 64 + (cq & 63) + sc * 8;
    st.r[j] = ldg16(A.qt + t);
    st.r[NCH + j] = ldg16(A.dot + t);
  }
}

template <int D>
__device__ inline void stage_store_a(DkdvSmem<D>& sm, int buf, int tid, const StageA<D>& st) {
  constexpr int NCH = StageA<D>::NCH;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = tid + kThreads * j;
    if (ch >= kBQB * D / 8) break;
    const int row = ch / (D / 8), dcol = ch % (D / 8);
    *reinterpret_cast<u32x4*>(&sm.q[buf][row * DkdvSmem<D>::NS + dcol * 8]) = st.r[j];
    *reinterpret_cast<u32x4*>(&sm.dO[buf][row * DkdvSmem<D>::NS + dcol * 8]) = st.r[NCH + j];
  }
  if (tid < kBQB) {
    sm.lse2[buf][tid] = st.l2;
    sm.dc[buf][tid] = st.dd;
    sm.vlo[buf][tid] = st.lo;
    sm.vhi[buf][tid] = st.hi;
  }
}

template <int D>
__device__ inline void stage_store_b(DkdvSmem<D>& sm, int buf, int tid, const StageB<D>& st) {
  constexpr int NCH = StageB<D>::NCH;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = tid + kThreads * j;
    if (ch >= kBQB * D / 8) break;
    const int d = ch / (kBQB / 8), sc = ch % (kBQB / 8);
    *reinterpret_cast<u32x4*>(&sm.qt[buf][d * DkdvSmem<D>::TS + sc * 8]) = st.r[j];
    *reinterpret_cast<u32x4*>(&sm.dot[buf][d * DkdvSmem<D>::TS + sc * 8]) = st.r[NCH + j];
  }
}

// S-wave, one 32-row block: P = exp2(S c2 - LSE2) on visible pairs, in fp16,
// packed as the two B operands (k-steps) of the contraction over rows.
__device__ __forceinline__ void block_p(bool full, const f32x16& sacc, const float* lse2, const int32_t* vlo,
                                        const int32_t* vhi, int hh, int32_t mysrc, float c2,
                                        f16x8 (&pf)[2]) {
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int rb = i4 * 8 + hh * 4;  // C rows rb .. rb+3 of the block
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + rb);
    // full steps: every row sees every key, [INT_MIN, INT_MAX) admits all
    int4 lo4 = {INT_MIN, INT_MIN, INT_MIN, INT_MIN}, hi4 = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
    if (!full) {
      lo4 = *reinterpret_cast<const int4*>(vlo + rb);
      hi4 = *reinterpret_cast<const int4*>(vhi + rb);
    }
    const int32_t los[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
    const int32_t his[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i4 * 4 + e;
      const float x = (mysrc >= los[e] && mysrc < his[e]) ? fmaf(sacc[i], c2, -l4[e]) : -INFINITY;
      pf[i >> 3][i & 7] = (_Float16)__builtin_amdgcn_exp2f(x);
    }
  }
}

// S-wave, first half of a step: S = Q K^T and P (kept in pf, copied to LDS).
template <int D>
__device__ __forceinline__ void s_phase_a(DkdvSmem<D>& sm, bool full, int BUF, int kw, int lane, int ql, int hh,
                                          int32_t mysrc, float c2, const bf16x8 (&kreg)[D / 16],
                                          f16x8 (&pf)[kNB][2]) {
  constexpr int NS = DkdvSmem<D>::NS;
  const uint16_t* qb = &sm.q[BUF][ql * NS + hh * 8];
  f32x16 sacc[kNB];
#pragma unroll
  for (int blk = 0; blk < kNB; ++blk) sacc[blk] = f32x16{};
  // consecutive products feed different accumulators (independent chains)
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk)
      sacc[blk] = mfma_bf16(ld16<bf16x8>(qb + blk * 32 * NS + ks * 16), kreg[ks], sacc[blk]);
#pragma unroll
  for (int blk = 0; blk < kNB; ++blk) {
    block_p(full, sacc[blk], &sm.lse2[BUF][blk * 32], &sm.vlo[BUF][blk * 32], &sm.vhi[BUF][blk * 32], hh,
            mysrc, c2, pf[blk]);
    *reinterpret_cast<f16x8*>(&sm.xchg[kw][blk][lane][0]) = pf[blk][0];
    *reinterpret_cast<f16x8*>(&sm.xchg[kw][blk][lane][8]) = pf[blk][1];
  }
}

// S-wave, second half: dV^T += dO^T P.
template <int D>
__device__ __forceinline__ void s_phase_b(DkdvSmem<D>& sm, int BUF, int ql, int hh, const f16x8 (&pf)[kNB][2],
                                          f32x16 (&dvacc)[D / 32]) {
  constexpr int TS = DkdvSmem<D>::TS;
  const _Float16* otb = &sm.dot[BUF][ql * TS + hh * 8];
#pragma unroll
  for (int blk = 0; blk < kNB; ++blk)
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dvacc[db] = mfma_f16(ld16<f16x8>(otb + db * 32 * TS + blk * 32 + ss * 16), pf[blk][ss], dvacc[db]);
}

// P-wave, first half of a step: dP = dO V^T.
template <int D>
__device__ __forceinline__ void p_phase_a(DkdvSmem<D>& sm, int BUF, int ql, int hh, const bf16x8 (&vreg)[D / 16],
                                          f32x16 (&pacc)[kNB]) {
  constexpr int NS = DkdvSmem<D>::NS;
  const uint16_t* ob = &sm.dO[BUF][ql * NS + hh * 8];
#pragma unroll
  for (int blk = 0; blk < kNB; ++blk) pacc[blk] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk)
      pacc[blk] = mfma_bf16(ld16<bf16x8>(ob + blk * 32 * NS + ks * 16), vreg[ks], pacc[blk]);
}

// P-wave, second half: dS = P (dP - D) with P from its S-wave, dK^T += Q^T dS.
template <int D>
__device__ __forceinline__ void p_phase_b(DkdvSmem<D>& sm, int BUF, int kw, int lane, int ql, int hh,
                                          const f32x16 (&pacc)[kNB], f32x16 (&dkacc)[D / 32]) {
  constexpr int TS = DkdvSmem<D>::TS;
  const _Float16* qtb = &sm.qt[BUF][ql * TS + hh * 8];
#pragma unroll
  for (int blk = 0; blk < kNB; ++blk) {
    const f16x8 p0 = ld16<f16x8>(&sm.xchg[kw][blk][lane][0]);
    const f16x8 p1 = ld16<f16x8>(&sm.xchg[kw][blk][lane][8]);
    f16x8 dsf[2];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dc[BUF][blk * 32 + i4 * 8 + hh * 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i4 * 4 + e;
        const float p = (float)((i < 8) ? p0[i & 7] : p1[i & 7]);
        dsf[i >> 3][i & 7] = (_Float16)(p * (pacc[blk][i] - d4[e]));
      }
    }
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dkacc[db] = mfma_f16(ld16<f16x8>(qtb + db * 32 * TS + blk * 32 + ss * 16), dsf[ss], dkacc[db]);
  }
}

// The query walk of one role.  S-waves and P-waves run the same sequence of
// barriers: two per step (after P is exchanged, after the prefetch lands).
template <int D, bool S_WAVE>
__device__ __forceinline__ void dkdv_walk(const Plan& P, const DkdvArgs& A, DkdvSmem<D>& sm, const KSeg& K, int b,
                                          int g, int32_t kvalid, int32_t kt1, int tid, int kw, int lane, int ql,
                                          int hh, int32_t mysrc, int32_t nseg, int32_t total,
                                          const bf16x8 (&kvreg)[D / 16], f32x16 (&acc)[D / 32]) {
  const float c2 = P.scale_log2;
  // Walk back to front by position: the k-th step from the end of every
  // segment, for every query head, then step k+1.  Every key tile's rows
  // run to the end of each segment, so the workgroups resident together on
  // an XCD visit the same rows at the same time and share them through L2.
  StepPos cur{0, nseg - 1, P.G - 1};
  auto advance = [&](StepPos p) {
    if (--p.hs >= 0) return p;
    p.hs = P.G - 1;
    do {
      if (--p.j < 0) {
        p.j = nseg - 1;
        ++p.k;
      }
    } while (p.k >= sm.wcount[p.j]);
    return p;
  };
  auto row_of = [&](const StepPos& p) { return sm.wfirst[p.j] + (sm.wcount[p.j] - 1 - p.k) * kBQB; };
  auto hb_of = [&](const StepPos& p) { return (int64_t)(b * P.hq + g * P.G + p.hs); };
  StageA<D> sa;
  StageB<D> sb;
  {
    const int32_t r0 = row_of(cur);
    stage_load_a<D>(A, P, K, P.q[sm.wseg[cur.j]], hb_of(cur), r0, tid, sa);
    stage_load_b<D>(A, P, P.q[sm.wseg[cur.j]], hb_of(cur), r0, tid, sb);
    stage_store_a<D>(sm, 0, tid, sa);
    stage_store_b<D>(sm, 0, tid, sb);
  }
  __syncthreads();
  for (int32_t t = 0; t < total; ++t) {
    const int BUF = t & 1;
    const int32_t si = sm.wseg[cur.j];
    const int32_t r0 = row_of(cur);
    const bool more = t + 1 < total;
    StepPos nxt = cur;
    int32_t sn = si, rn = 0;
    if (more) {
      nxt = advance(cur);
      sn = sm.wseg[nxt.j];
      rn = row_of(nxt);
      stage_load_a<D>(A, P, K, P.q[sn], hb_of(nxt), rn, tid, sa);
    }
    if constexpr (S_WAVE) {
      // no mask when every row of the step exists and sees every key of the tile
      bool full = false;
      if (K.kind == KIND_CLEAN && kvalid == kBKB && r0 + kBQB <= P.q[si].nrows)
        full = row_bounds(P, P.q[si], r0).hi_clean >= kt1;
      f16x8 pf[kNB][2];
      s_phase_a<D>(sm, full, BUF, kw, lane, ql, hh, mysrc, c2, kvreg, pf);
      if (more) stage_store_a<D>(sm, BUF ^ 1, tid, sa);
      __syncthreads();  // P visible to the P-waves
      if (more) stage_load_b<D>(A, P, P.q[sn], hb_of(nxt), rn, tid, sb);
      s_phase_b<D>(sm, BUF, ql, hh, pf, acc);
    } else {
      f32x16 pacc[kNB];
      p_phase_a<D>(sm, BUF, ql, hh, kvreg, pacc);
      if (more) stage_store_a<D>(sm, BUF ^ 1, tid, sa);
      __syncthreads();  // P from the S-waves
      if (more) stage_load_b<D>(A, P, P.q[sn], hb_of(nxt), rn, tid, sb);
      p_phase_b<D>(sm, BUF, kw, lane, ql, hh, pacc, acc);
    }
    if (more) stage_store_b<D>(sm, BUF ^ 1, tid, sb);
    __syncthreads();
    cur = nxt;
  }
}

template <int D>
__device__ void dkdv_tile(const Plan& P, const DkdvArgs& A, DkdvSmem<D>& sm, int b, int g, int32_t ktile) {
  static_assert(kThreads >= kBQB, "one thread per row stages the per-row data");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int kw = wave % kPairs;       // which 32 keys of the tile
  const bool s_wave = wave < kPairs;  // S-wave (dV) or P-wave (dK)
  int32_t kseg, koff;
  ktile_locate(P, ktile, &kseg, &koff);
  const KSeg K = P.k[kseg];
  const int32_t kvalid = min(kBKB, K.len - koff);  // valid keys in the tile
  const int32_t kt0 = K.t0 + koff;                 // first source row
  const int32_t kt1 = kt0 + kvalid;
  const int32_t c = K.c0 + koff;                   // compact start
  const int32_t mykey = kw * 32 + ql;
  const bool key_ok = mykey < kvalid;
  const int32_t mysrc = key_ok ? kt0 + mykey : INT_MIN;

  // this wave's 32 keys as B operands: K (S-wave) or V (P-wave)
  bf16x8 kvreg[D / 16];
  {
    const uint16_t* src = s_wave ? A.kn : A.vn;
    const int64_t nb = ((int64_t)(b * P.hkv + g) * P.nkc + c + kw * 32 + ql) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kvreg[ks] = ld16<bf16x8>(src + nb + ks * 16 + hh * 8);
  }
  f32x16 acc[D / 32];  // dV^T (S-wave) or dK^T (P-wave)
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  if (tid == 0) {
    int32_t nseg = 0, per = 0;
    for (int32_t s = 0; s < P.nq; ++s) {
      const QSeg& S = P.q[s];
      const int32_t rf = first_seeing_row(P, S, K.kind, kt0);
      const int32_t re = end_seeing_row(P, S, K.kind, kt1);
      if (re <= rf) continue;
      const int32_t a = (rf / kBQB) * kBQB;
      sm.wseg[nseg] = s;
      sm.wfirst[nseg] = a;
      sm.wcount[nseg] = (re - a + kBQB - 1) / kBQB;
      per += sm.wcount[nseg];
      ++nseg;
    }
    sm.wn = nseg;
    sm.wper = per;
  }
  __syncthreads();
  const int32_t nseg = sm.wn;
  const int32_t total = sm.wper * P.G;

  if (total > 0) {
    if (s_wave)
      dkdv_walk<D, true>(P, A, sm, K, b, g, kvalid, kt1, tid, kw, lane, ql, hh, mysrc, nseg, total, kvreg, acc);
    else
      dkdv_walk<D, false>(P, A, sm, K, b, g, kvalid, kt1, tid, kw, lane, ql, hh, mysrc, nseg, total, kvreg, acc);
  }
  if (key_ok) {
    float* dst;
    int64_t rowoff;
    if (K.kind == KIND_CLEAN) {
      dst = s_wave ? A.dv_clean : A.dk_clean;
      rowoff = (((int64_t)b * P.L + mysrc) * P.hkv + g) * D;
    } else {
      dst = s_wave ? A.dv_corr : A.dk_corr;
      rowoff = (((int64_t)b * P.n_corr_rows + mysrc) * P.hkv + g) * D;
    }
    const float f = s_wave ? 1.f : P.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        f32x4* pd = reinterpret_cast<f32x4*>(dst + rowoff + db * 32 + crow(i, hh));
        f32x4 cur4 = *pd;
#pragma unroll
        for (int e = 0; e < 4; ++e) cur4[e] += f * acc[db][i + e];
        *pd = cur4;
      }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(const Plan P, const DkdvArgs A) {
  __shared__ DkdvSmem<D> sm;
  const WgK wg = decode_wg_k(P, blockIdx.x);
  dkdv_tile<D>(P, A, sm, wg.b, wg.g, wg.tile_a);
  if (wg.tile_b >= 0) {
    __syncthreads();
    dkdv_tile<D>(P, A, sm, wg.b, wg.g, wg.tile_b);
  }
}

}  // namespace

hipError_t launch_dkdv(const Plan& P, const DkdvArgs& a, hipStream_t s) {
  if (P.nwg_k == 0) return hipSuccess;
  if (P.d == 128)
    hipLaunchKernelGGL(dkdv_kernel<128>, dim3((unsigned)P.nwg_k), dim3(kThreads), 0, s, P, a);
  else
    hipLaunchKernelGGL(dkdv_kernel<64>, dim3((unsigned)P.nwg_k), dim3(kThreads), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace bd
