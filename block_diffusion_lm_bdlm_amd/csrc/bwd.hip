// bwd.hip — backward of BDLM attention for the loss sum(O * dO).
//
// With the final softmax (LSE over every key the row sees) and
// D_i = dO_i . O_i, every visible pair contributes
//   P = exp(s - LSE),  dP = dO_i . v_j,  dS = P (dP - D_i),
//   dV_j += P dO_i,  dK_j += scale dS q_i,  dQ_i += scale dS k_j
// (the chain rule of the attention equation in "CSBP 完全拆解"; the
// "exact fused backward" of the Turbo-dLLM page).  Restricting j to one
// call's keys gives that call's share; the shares of a split key set sum to
// the full gradient.
//
// This file holds the dQ kernel (dkdv.hip holds dK/dV): query-major, in the
// forward's work order, recomputing S^T and dP^T per key tile.
#include "device.h"
#include "kernels.h"
#include "walk.h"

namespace bd {

namespace {

// ----------------------------------------------------------------- dQ
// A workgroup owns a 128-row query tile of one head and runs 8 waves, two
// per SIMD, in pairs that own the same 32 query rows:
//   S-wave: Q in registers; S^T = K Q^T, P^T = exp(S^T - LSE) (masked),
//           hands P^T to its partner through LDS.
//   P-wave: dO in registers; dP^T = V dO^T, dS^T = P^T (dP^T - D),
//           accumulates dQ^T += K^T dS^T; one writer per row.
constexpr int kDqThreads = 512;

template <int D>
struct __attribute__((aligned(16))) DqSmem {
  static constexpr int KS = D + 8;
  static constexpr int TS = kBK + 8;
  uint16_t k[2][kBK * KS];
  uint16_t v[2][kBK * KS];
  _Float16 kt[2][D * TS];
  _Float16 xchg[4][2][64][16];  // P^T from each S-wave, per 32-key block, per lane
};

template <int D>
struct DqStage {
  static constexpr int NCH = kBK * D / 8 / kDqThreads;  // chunks per thread per tensor
  u32x4 kr[NCH], vr[NCH], tr[NCH];
};

template <int D>
__device__ inline void dq_load(const DqArgs& A, const Plan& P, int b, int g, int c, int tid, DqStage<D>& st) {
  constexpr int NCH = DqStage<D>::NCH;
  const int64_t nb = ((int64_t)(b * P.hkv + g) * P.nkc + c) * D;
  const _Float16* tb = A.kt + (int64_t)(b * P.hkv + g) * D * P.nkc + (int64_t)c * D;  // [D][64] tile
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = tid + kDqThreads * j;
    const int key = ch / (D / 8), dc = ch % (D / 8);
    st.kr[j] = ldg16(A.kn + nb + key * D + dc * 8);
    st.vr[j] = ldg16(A.vn + nb + key * D + dc * 8);
    const int d = ch / (kBK / 8), kc = ch % (kBK / 8);
    st.tr[j] = ldg16(tb + d * kBK + kc * 8);
  }
}

template <int D>
__device__ inline void dq_store(DqSmem<D>& sm, int buf, int tid, const DqStage<D>& st) {
  constexpr int NCH = DqStage<D>::NCH;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = tid + kDqThreads * j;
    const int key = ch / (D / 8), dc = ch % (D / 8);
    *reinterpret_cast<u32x4*>(&sm.k[buf][key * DqSmem<D>::KS + dc * 8]) = st.kr[j];
    *reinterpret_cast<u32x4*>(&sm.v[buf][key * DqSmem<D>::KS + dc * 8]) = st.vr[j];
    const int d = ch / (kBK / 8), kc = ch % (kBK / 8);
    *reinterpret_cast<u32x4*>(&sm.kt[buf][d * DqSmem<D>::TS + kc * 8]) = st.tr[j];
  }
}

// One role's walk over the key tiles; both roles run the same barriers.
template <int D, bool S_WAVE>
__device__ __forceinline__ void dq_walk(const Plan& P, const DqArgs& A, DqSmem<D>& sm, const KeyWalk& w,
                                        const RowBounds& rb, bool clean, int b, int g, int tid, int pw, int lane,
                                        int ql, int hh, const bf16x8 (&qreg)[D / 16], float rowval,
                                        f32x16 (&dqacc)[D / 32]) {
  const float c2 = P.scale_log2;
  DqStage<D> st;
  {
    int32_t c, ri;
    bool fu;
    keywalk_at(w, 0, &c, &ri, &fu);
    dq_load<D>(A, P, b, g, c, tid, st);
    dq_store<D>(sm, 0, tid, st);
  }
  __syncthreads();
  for (int32_t t = 0; t < w.total; ++t) {
    const int buf = t & 1;
    int32_t c, ri;
    bool full;
    keywalk_at(w, t, &c, &ri, &full);
    const bool more = t + 1 < w.total;
    if (more) {
      int32_t cn, rn;
      bool fn;
      keywalk_at(w, t + 1, &cn, &rn, &fn);
      dq_load<D>(A, P, b, g, cn, tid, st);
    }
    if constexpr (S_WAVE) {
      // S^T = K Q^T for two blocks of 32 keys; P^T = exp2(S^T c2 - LSE2)
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int off = (kb * 32 + ql) * DqSmem<D>::KS + ks * 16 + hh * 8;
          sacc[kb] = mfma_bf16(ld16<bf16x8>(&sm.k[buf][off]), qreg[ks], sacc[kb]);
        }
      int32_t vlo = c, vhi = c + kBK;
      if (!full) compact_range(P.k[ri], rb, clean, &vlo, &vhi);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f16x8 pf[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t key = c + kb * 32 + crow(i, hh);
          const float x = (key >= vlo && key < vhi) ? fmaf(sacc[kb][i], c2, -rowval) : -INFINITY;
          pf[i >> 3][i & 7] = (_Float16)__builtin_amdgcn_exp2f(x);
        }
        *reinterpret_cast<f16x8*>(&sm.xchg[pw][kb][lane][0]) = pf[0];
        *reinterpret_cast<f16x8*>(&sm.xchg[pw][kb][lane][8]) = pf[1];
      }
      if (more) dq_store<D>(sm, buf ^ 1, tid, st);
      __syncthreads();  // P^T visible to the P-waves
    } else {
      // dP^T = V dO^T, then dS^T = P^T (dP^T - D) and dQ^T += K^T dS^T
      f32x16 pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int off = (kb * 32 + ql) * DqSmem<D>::KS + ks * 16 + hh * 8;
          pacc[kb] = mfma_bf16(ld16<bf16x8>(&sm.v[buf][off]), qreg[ks], pacc[kb]);
        }
      if (more) dq_store<D>(sm, buf ^ 1, tid, st);
      __syncthreads();  // P^T from the S-waves
      f16x8 dsf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f16x8 p0 = ld16<f16x8>(&sm.xchg[pw][kb][lane][0]);
        const f16x8 p1 = ld16<f16x8>(&sm.xchg[pw][kb][lane][8]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = (float)((i < 8) ? p0[i & 7] : p1[i & 7]);
          dsf[kb][i >> 3][i & 7] = (_Float16)(pv * (pacc[kb][i] - rowval));
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const f16x8 a =
                ld16<f16x8>(&sm.kt[buf][(db * 32 + ql) * DqSmem<D>::TS + kb * 32 + ss * 16 + hh * 8]);
            dqacc[db] = mfma_f16(a, dsf[kb][ss], dqacc[db]);
          }
    }
    __syncthreads();
  }
}

template <int D>
__device__ void dq_tile(const Plan& P, const DqArgs& A, DqSmem<D>& sm, int b, int h, int g, int32_t tile) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int pw = wave & 3;           // which 32 rows of the tile
  const bool s_wave = wave < 4;
  const QSeg S = P.q[seg_of_tile(P, tile)];
  const int32_t r0 = (tile - S.tile0) * kBQ;
  const int32_t n = min(kBQ, S.nrows - r0);
  const int32_t rq = pw * 32 + ql;
  const int32_t rc = min(rq, n - 1);
  const bool clean = S.kind == KIND_CLEAN;
  const int64_t hb = (int64_t)(b * P.hq + h);
  const int64_t crow_q = hb * P.nqc + (int64_t)tile * kBQ + rq;  // compact (zero-padded) row

  // Q (S-wave) or dO (P-wave) of this lane's row as B operands
  bf16x8 qreg[D / 16];
  {
    const uint16_t* src = s_wave ? A.qn : A.don;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = ld16<bf16x8>(src + crow_q * D + ks * 16 + hh * 8);
  }
  const float rowval = s_wave ? A.lse2[crow_q] : A.dc[crow_q];  // LSE2 (S-wave) or D (P-wave)
  const RowBounds rb = row_bounds(P, S, r0 + rc);
  const KeyWalk w = keywalk_build(P, S, r0, r0 + n - 1);

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};
  if (w.total > 0) {
    if (s_wave)
      dq_walk<D, true>(P, A, sm, w, rb, clean, b, g, tid, pw, lane, ql, hh, qreg, rowval, dqacc);
    else
      dq_walk<D, false>(P, A, sm, w, rb, clean, b, g, tid, pw, lane, ql, hh, qreg, rowval, dqacc);
  }
  if (!s_wave && rq < n) {
    const int32_t row = S.row0 + r0 + rq;
    float* dp = A.dq + (((int64_t)b * P.R + row) * P.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        f32x4* p4 = reinterpret_cast<f32x4*>(dp + db * 32 + crow(i, hh));
        f32x4 cur = *p4;
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[e] += P.scale * dqacc[db][i + e];
        *p4 = cur;
      }
  }
}

template <int D>
__global__ __launch_bounds__(kDqThreads, 1) void dq_kernel(const Plan P, const DqArgs A) {
  __shared__ DqSmem<D> sm;
  const WgQ wg = decode_wg_q(P, blockIdx.x);
  dq_tile<D>(P, A, sm, wg.b, wg.h, wg.g, wg.tile_a);
  if (wg.tile_b >= 0) dq_tile<D>(P, A, sm, wg.b, wg.h, wg.g, wg.tile_b);
}

}  // namespace

hipError_t launch_dq(const Plan& P, const DqArgs& a, hipStream_t s) {
  if (P.nwg_q == 0) return hipSuccess;
  if (P.d == 128)
    hipLaunchKernelGGL(dq_kernel<128>, dim3((unsigned)P.nwg_q), dim3(kDqThreads), 0, s, P, a);
  else
    hipLaunchKernelGGL(dq_kernel<64>, dim3((unsigned)P.nwg_q), dim3(kDqThreads), 0, s, P, a);
  return hipGetLastError();
}


}  // namespace bd
