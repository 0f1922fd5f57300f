// dkdv.hip — dK and dV of BDLM attention, key-major.
//
// For every visible pair, with the final LSE and D_i = dO_i . O_i:
//   P = exp(s - LSE),  dS = P (dO_i . v_j - D_i),
//   dV_j += P dO_i,  dK_j += scale dS q_i
// (chain rule of the attention equation in "CSBP 完全拆解"; clean keys collect
// contributions from every later block, section "CSBP：BP 管损坏块，CP 管干净
// 上下文").
//
// A workgroup owns 128 keys of one KV head, 32 per wave: K and V sit in
// registers as B operands, dK^T and dV^T accumulate in registers, so every
// key has exactly one writer and no atomics are needed.  The workgroup walks
// every query row (of every query head of the group) that sees its keys, in
// steps of 64 rows staged through LDS (natural Q, dO for S = Q K^T and
// dP = dO V^T; transposed fp16 Q^T, dO^T for the contractions over rows).
// The walk runs back to front: the last rows are seen by every key tile, so
// the workgroups resident on one XCD start on the same rows and share them
// through L2.  Each step stages per-row visibility bounds next to LSE and D,
// so a step that straddles the mask boundary needs no division per element.
#include <climits>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace bd {

namespace {

constexpr int kNB = kBQB / 32;  // 32-row MFMA blocks per step

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
  // steps of the walk: segment s contributes wcount[s] steps from row wfirst[s]
  int32_t wseg[kMaxQSeg], wfirst[kMaxQSeg], wcount[kMaxQSeg];
  int32_t wn, wper;
};

// Position of the walk: query head (within the group), walk segment, step.
struct StepPos {
  int32_t hs, j, u;
};

template <int D>
struct Stage {
  static constexpr int NCH = kBQB * D / 8 / 256;  // 16-byte chunks per thread per tensor
  u32x4 r[4 * NCH];
  float l2, dd;
  int32_t lo, hi;
};

template <int D>
__device__ inline void stage_load(const DkdvArgs& A, const Plan& P, const KSeg& K, const QSeg& S, int64_t hb,
                                  int32_t r0, int tid, Stage<D>& st) {
  constexpr int NCH = Stage<D>::NCH;
  const int32_t cq = S.tile0 * kBQ + r0;  // compact row of the step's first row
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = tid + 256 * j;
    const int row = ch / (D / 8), dcol = ch % (D / 8);
    st.r[j] = ldg16(A.qn + (hb * P.nqc + cq + row) * D + dcol * 8);
    st.r[NCH + j] = ldg16(A.don + (hb * P.nqc + cq + row) * D + dcol * 8);
    const int d = ch / (kBQB / 8), sc = ch % (kBQB / 8);
    st.r[2 * NCH + j] = ldg16(A.qt + (hb * D + d) * P.nqc + cq + sc * 8);
    st.r[3 * NCH + j] = ldg16(A.dot + (hb * D + d) * P.nqc + cq + sc * 8);
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
__device__ inline void stage_store(DkdvSmem<D>& sm, int buf, int tid, const Stage<D>& st) {
  constexpr int NCH = Stage<D>::NCH;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = tid + 256 * j;
    const int row = ch / (D / 8), dcol = ch % (D / 8);
    *reinterpret_cast<u32x4*>(&sm.q[buf][row * DkdvSmem<D>::NS + dcol * 8]) = st.r[j];
    *reinterpret_cast<u32x4*>(&sm.dO[buf][row * DkdvSmem<D>::NS + dcol * 8]) = st.r[NCH + j];
    const int d = ch / (kBQB / 8), sc = ch % (kBQB / 8);
    *reinterpret_cast<u32x4*>(&sm.qt[buf][d * DkdvSmem<D>::TS + sc * 8]) = st.r[2 * NCH + j];
    *reinterpret_cast<u32x4*>(&sm.dot[buf][d * DkdvSmem<D>::TS + sc * 8]) = st.r[3 * NCH + j];
  }
  if (tid < kBQB) {
    sm.lse2[buf][tid] = st.l2;
    sm.dc[buf][tid] = st.dd;
    sm.vlo[buf][tid] = st.lo;
    sm.vhi[buf][tid] = st.hi;
  }
}

// One 32-row block's probabilities and dS in fp16, packed as the two B
// operands (k-steps) of the contraction over rows.
__device__ __forceinline__ void block_softmax(bool full, const f32x16& sacc, const f32x16& pacc,
                                              const float* lse2, const float* dc, const int32_t* vlo,
                                              const int32_t* vhi, int hh, int32_t mysrc, float c2,
                                              f16x8 (&pf)[2], f16x8 (&dsf)[2]) {
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int rb = i4 * 8 + hh * 4;  // C rows rb .. rb+3 of the block
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + rb);
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dc + rb);
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
      const float p = __builtin_amdgcn_exp2f(x);
      pf[i >> 3][i & 7] = (_Float16)p;
      dsf[i >> 3][i & 7] = (_Float16)(p * (pacc[i] - d4[e]));
    }
  }
}

// One step: 64 query rows staged in LDS buffer BUF against this wave's 32 keys.
template <int D>
__device__ __forceinline__ void dkdv_step(DkdvSmem<D>& sm, bool full, int BUF, int ql, int hh, int32_t mysrc, float c2,
                                          const bf16x8 (&kreg)[D / 16], const bf16x8 (&vreg)[D / 16],
                                          f32x16 (&dkacc)[D / 32], f32x16 (&dvacc)[D / 32]) {
  constexpr int NS = DkdvSmem<D>::NS, TS = DkdvSmem<D>::TS;
  const uint16_t* qb = &sm.q[BUF][ql * NS + hh * 8];
  const uint16_t* ob = &sm.dO[BUF][ql * NS + hh * 8];
  const _Float16* qtb = &sm.qt[BUF][ql * TS + hh * 8];
  const _Float16* otb = &sm.dot[BUF][ql * TS + hh * 8];
#pragma unroll
  for (int blk = 0; blk < kNB; ++blk) {
    // S = Q K^T, dP = dO V^T for the block's 32 rows
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      sacc = mfma_bf16(ld16<bf16x8>(qb + blk * 32 * NS + ks * 16), kreg[ks], sacc);
      pacc = mfma_bf16(ld16<bf16x8>(ob + blk * 32 * NS + ks * 16), vreg[ks], pacc);
    }
    f16x8 pf[2], dsf[2];
    block_softmax(full, sacc, pacc, &sm.lse2[BUF][blk * 32], &sm.dc[BUF][blk * 32], &sm.vlo[BUF][blk * 32],
                        &sm.vhi[BUF][blk * 32], hh, mysrc, c2, pf, dsf);
    // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over the block's 32 rows)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const int off = db * 32 * TS + blk * 32 + ss * 16;
        dvacc[db] = mfma_f16(ld16<f16x8>(otb + off), pf[ss], dvacc[db]);
        dkacc[db] = mfma_f16(ld16<f16x8>(qtb + off), dsf[ss], dkacc[db]);
      }
  }
}

template <int D>
__device__ void dkdv_tile(const Plan& P, const DkdvArgs& A, DkdvSmem<D>& sm, int b, int g, int32_t ktile) {
  static_assert(kBQB * D / 8 >= 256 && (kBQB * D / 8) % 256 == 0, "chunking");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  int32_t kseg, koff;
  ktile_locate(P, ktile, &kseg, &koff);
  const KSeg K = P.k[kseg];
  const int32_t kvalid = min(kBKB, K.len - koff);  // valid keys in the tile
  const int32_t kt0 = K.t0 + koff;                 // first source row
  const int32_t kt1 = kt0 + kvalid;
  const int32_t c = K.c0 + koff;                   // compact start
  const int32_t mykey = wave * 32 + ql;
  const bool key_ok = mykey < kvalid;
  const int32_t mysrc = key_ok ? kt0 + mykey : INT_MIN;

  bf16x8 kreg[D / 16], vreg[D / 16];
  {
    const int64_t nb = ((int64_t)(b * P.hkv + g) * P.nkc + c + wave * 32 + ql) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kreg[ks] = ld16<bf16x8>(A.kn + nb + ks * 16 + hh * 8);
      vreg[ks] = ld16<bf16x8>(A.vn + nb + ks * 16 + hh * 8);
    }
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

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
  const float c2 = P.scale_log2;

  if (total > 0) {
    // walk back to front: last head, last segment, last step first
    StepPos cur{P.G - 1, nseg - 1, sm.wcount[nseg - 1] - 1};
    auto advance = [&](StepPos p) {
      if (--p.u < 0) {
        if (--p.j < 0) {
          p.j = nseg - 1;
          --p.hs;
        }
        p.u = sm.wcount[p.j] - 1;
      }
      return p;
    };
    auto hb_of = [&](const StepPos& p) { return (int64_t)(b * P.hq + g * P.G + p.hs); };
    Stage<D> st;
    {
      const QSeg& S = P.q[sm.wseg[cur.j]];
      stage_load<D>(A, P, K, S, hb_of(cur), sm.wfirst[cur.j] + cur.u * kBQB, tid, st);
      stage_store<D>(sm, 0, tid, st);
    }
    __syncthreads();
    // each step: prefetch the next one into registers, compute from LDS
    // buffer t & 1, then move the prefetch into the other buffer
    for (int32_t t = 0; t < total; ++t) {
      const int BUF = t & 1;
      const QSeg S = P.q[sm.wseg[cur.j]];
      const int32_t r0 = sm.wfirst[cur.j] + cur.u * kBQB;
      StepPos nxt = cur;
      if (t + 1 < total) {
        nxt = advance(cur);
        const QSeg& Sn = P.q[sm.wseg[nxt.j]];
        stage_load<D>(A, P, K, Sn, hb_of(nxt), sm.wfirst[nxt.j] + nxt.u * kBQB, tid, st);
      }
      // no mask when every row of the step exists and sees every key of the tile
      bool full = false;
      if (K.kind == KIND_CLEAN && kvalid == kBKB && r0 + kBQB <= S.nrows)
        full = row_bounds(P, S, r0).hi_clean >= kt1;
      dkdv_step<D>(sm, full, BUF, ql, hh, mysrc, c2, kreg, vreg, dkacc, dvacc);
      if (t + 1 < total) stage_store<D>(sm, BUF ^ 1, tid, st);
      __syncthreads();
      cur = nxt;
    }
  }
  if (key_ok) {
    float *dk, *dv;
    int64_t rowoff;
    if (K.kind == KIND_CLEAN) {
      dk = A.dk_clean;
      dv = A.dv_clean;
      rowoff = (((int64_t)b * P.L + mysrc) * P.hkv + g) * D;
    } else {
      dk = A.dk_corr;
      dv = A.dv_corr;
      rowoff = (((int64_t)b * P.n_corr_rows + mysrc) * P.hkv + g) * D;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const int d = db * 32 + crow(i, hh);
        f32x4* pk = reinterpret_cast<f32x4*>(dk + rowoff + d);
        f32x4* pv = reinterpret_cast<f32x4*>(dv + rowoff + d);
        f32x4 ck = *pk, cv = *pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ck[e] += P.scale * dkacc[db][i + e];
          cv[e] += dvacc[db][i + e];
        }
        *pk = ck;
        *pv = cv;
      }
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(const Plan P, const DkdvArgs A) {
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
    hipLaunchKernelGGL(dkdv_kernel<128>, dim3((unsigned)P.nwg_k), dim3(256), 0, s, P, a);
  else
    hipLaunchKernelGGL(dkdv_kernel<64>, dim3((unsigned)P.nwg_k), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace bd
