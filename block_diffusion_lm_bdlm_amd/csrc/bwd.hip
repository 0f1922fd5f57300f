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
#include "stage.h"
#include "walk.h"

namespace bd {

namespace {

// ----------------------------------------------------------------- dQ
// A workgroup owns a 128-row query tile of one head and runs 8 waves, two
// per SIMD, in pairs that own the same 32 query rows:
//   S-wave: Q in registers; S^T = K Q^T, P^T = exp(S^T - LSE) (masked),
//           hands P^T to its partner through LDS.
//   P-wave: dO in registers; dP^T = V dO^T, dS^T = P^T (dP^T - D),
//           accumulates dQ^T += K^T dS^T in AGPRs; one writer per row.
// Each key tile's K, V (natural bf16) and K^T (fp16) go from global memory
// straight into LDS (global_load_lds), double buffered, as swizzled tiles.
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
static_assert(kBK == kTileRows, "key tiles are staged as 64-row tiles");

template <int D>
struct __attribute__((aligned(16))) DqSmem {
  static constexpr int TILE = kBK * D;  // elements per staged tile
  uint16_t k[2][TILE];                  // natural bf16 [key][d]
  uint16_t v[2][TILE];
  _Float16 kt[2][TILE];                 // transposed fp16 [d][key], perm16 keys
  _Float16 xchg[4][2][2][64][8];        // P^T per pair, 32-key block, k-step, lane
};

// Issues the copies of key tile c (compact start) into buffer B.
template <int D>
__device__ __forceinline__ void dq_stage(const DqArgs& A, const Plan& P, int b, int g, int32_t c, int wave,
                                         const LaneOff<D>& o, DqSmem<D>& sm, int B) {
  constexpr int PER = kBK * D / 512 / kDqWaves;  // 1 KB blocks per wave per tile
  const int64_t base = uniform64(((int64_t)(b * P.hkv + g) * P.nkc + c) * D);  // natural and transposed alike
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int blk = (wave + kDqWaves * j) * 512;  // elements
    const int64_t e = base + (int64_t)j * kDqWaves * 512;
    copy16(A.kn + e, o.dn, &sm.k[B][blk]);
    copy16(A.vn + e, o.dn, &sm.v[B][blk]);
    copy16(A.kt + e, o.dt, &sm.kt[B][blk]);
  }
}

// S-wave: S^T, then P^T = exp2(S^T c2 - LSE2) on visible pairs, to LDS.
template <int D, bool FULL>
__device__ __forceinline__ void dq_s_phase(DqSmem<D>& sm, int B, int pw, int lane, int ql, int hh, int32_t c,
                                           int32_t vlo, int32_t vhi, float c2, float lse2,
                                           const bf16x8 (&qreg)[D / 16], const LaneOff<D>& o) {
  f32x16 sacc[2];
  scores_2kb<D>(sm.k[B], ql, qreg, o, sacc);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f16x8 pf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = fmaf(sacc[kb][i], c2, -lse2);
      if constexpr (!FULL) {
        const int32_t key = c + kb * 32 + crow(i, hh);
        x = (key >= vlo && key < vhi) ? x : -INFINITY;
      }
      pf[i >> 3][i & 7] = (_Float16)__builtin_amdgcn_exp2f(x);
    }
    *reinterpret_cast<f16x8*>(&sm.xchg[pw][kb][0][lane][0]) = pf[0];
    *reinterpret_cast<f16x8*>(&sm.xchg[pw][kb][1][lane][0]) = pf[1];
  }
}

// P-wave, after the exchange: dS^T = P^T (dP^T - D) (dP - D rounded to fp16
// before the product) and dQ^T += K^T dS^T; fragment f = (s, db).
template <int D>
__device__ __forceinline__ void dq_p_phase(DqSmem<D>& sm, int B, int pw, int lane, int ql, float dval,
                                           const f32x16 (&pacc)[2], const LaneOff<D>& o,
                                           f32x16 (&dqacc)[D / 32]) {
  f16x8 dsf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const f16x8 p = ld16<f16x8>(&sm.xchg[pw][kb][ss][lane][0]);
      f16x8 t;
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = (_Float16)(pacc[kb][ss * 8 + e] - dval);
      dsf[kb][ss] = p * t;
    }
  constexpr int NDB = D / 32, NF = (kBK / 16) * NDB;
  const _Float16* tb = sm.kt[B] + ql * kBK;
  f16x8 fr[NF];
#pragma unroll
  for (int f = 0; f < kAhead; ++f) fr[f] = ld16<f16x8>(tb + (f % NDB) * 32 * kBK + o.tr[f / NDB]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + kAhead < NF) {
      const int h = f + kAhead;
      fr[h] = ld16<f16x8>(tb + (h % NDB) * 32 * kBK + o.tr[h / NDB]);
    }
    const int s = f / NDB, db = f % NDB;
    mfma_f16_agpr(dqacc[db], fr[f], dsf[s >> 1][s & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One role's walk over the key tiles; both roles run the same barriers.
template <int D, bool S_WAVE>
__device__ __forceinline__ void dq_walk(const Plan& P, const DqArgs& A, DqSmem<D>& sm, const KeyWalk& w,
                                        const RowBounds& rb, bool clean, int b, int g, int wave, int pw, int lane,
                                        int ql, int hh, const bf16x8 (&qreg)[D / 16], float rowval,
                                        const LaneOff<D>& o, f32x16 (&dqacc)[D / 32]) {
  const float c2 = P.scale_log2;
  {
    int32_t c, ri;
    bool fu;
    keywalk_at(w, 0, &c, &ri, &fu);
    dq_stage<D>(A, P, b, g, c, wave, o, sm, 0);
  }
  wait_copies();
  __syncthreads();
  for (int32_t t = 0; t < w.total; ++t) {
    const int B = t & 1;
    int32_t c, ri;
    bool full;
    keywalk_at(w, t, &c, &ri, &full);
    if (t + 1 < w.total) {
      int32_t cn, rn;
      bool fn;
      keywalk_at(w, t + 1, &cn, &rn, &fn);
      dq_stage<D>(A, P, b, g, cn, wave, o, sm, B ^ 1);
    }
    if constexpr (S_WAVE) {
      if (full) {
        dq_s_phase<D, true>(sm, B, pw, lane, ql, hh, c, 0, 0, c2, rowval, qreg, o);
      } else {
        int32_t vlo, vhi;
        compact_range(P.k[ri], rb, clean, &vlo, &vhi);
        dq_s_phase<D, false>(sm, B, pw, lane, ql, hh, c, vlo, vhi, c2, rowval, qreg, o);
      }
      barrier_lds();  // P^T visible to the P-waves
    } else {
      f32x16 pacc[2];
      scores_2kb<D>(sm.v[B], ql, qreg, o, pacc);  // dP^T = V dO^T
      barrier_lds();  // P^T from the S-waves
      dq_p_phase<D>(sm, B, pw, lane, ql, rowval, pacc, o, dqacc);
    }
    wait_copies();
    __syncthreads();  // the next tile's copies have landed; this tile's reads are done
  }
}

template <int D, bool S_WAVE>
__device__ __forceinline__ void dq_role(const Plan& P, const DqArgs& A, DqSmem<D>& sm, int b, int h, int g,
                                        int wave, int pw, int lane, int ql, int hh, const QSeg& S, int32_t r0,
                                        int32_t n, int32_t rq, int64_t crow_q) {
  bf16x8 qreg[D / 16];  // Q (S-wave) or dO (P-wave) of this lane's row as B operands
  {
    const uint16_t* src = S_WAVE ? A.qn : A.don;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = ld16<bf16x8>(src + crow_q * D + ks * 16 + hh * 8);
  }
  const float rowval = S_WAVE ? A.lse2[crow_q] : A.dc[crow_q];  // LSE2 (S-wave) or D (P-wave)
  const RowBounds rb = row_bounds(P, S, r0 + min(rq, n - 1));
  const KeyWalk w = keywalk_build(P, S, r0, r0 + n - 1);
  const LaneOff<D> o = lane_offsets<D, kDqWaves>(wave, lane);
  f32x16 dqacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};
  if (w.total > 0)
    dq_walk<D, S_WAVE>(P, A, sm, w, rb, S.kind == KIND_CLEAN, b, g, wave, pw, lane, ql, hh, qreg, rowval, o,
                       dqacc);
  if constexpr (!S_WAVE) {
    agpr_settle();
    if (rq < n) {
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
}

template <int D>
__device__ void dq_tile(const Plan& P, const DqArgs& A, DqSmem<D>& sm, int b, int h, int g, int32_t tile) {
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = uniform(tid >> 6);
  const int pw = wave & 3;  // which 32 rows of the tile
  const QSeg S = P.q[seg_of_tile(P, tile)];
  const int32_t r0 = (tile - S.tile0) * kBQ;
  const int32_t n = min(kBQ, S.nrows - r0);
  const int32_t rq = pw * 32 + ql;
  const int64_t hb = (int64_t)(b * P.hq + h);
  const int64_t crow_q = hb * P.nqc + (int64_t)tile * kBQ + rq;  // compact (zero-padded) row
  if (wave < 4)
    dq_role<D, true>(P, A, sm, b, h, g, wave, pw, lane, ql, hh, S, r0, n, rq, crow_q);
  else
    dq_role<D, false>(P, A, sm, b, h, g, wave, pw, lane, ql, hh, S, r0, n, rq, crow_q);
}

template <int D>
__global__ __launch_bounds__(kDqThreads, 1) void dq_kernel(const Plan P, const DqArgs A) {
  __shared__ DqSmem<D> sm;
  const WgQ wg = decode_wg_q(P, blockIdx.x);
  dq_tile<D>(P, A, sm, wg.b, wg.h, wg.g, wg.tile_a);
  if (wg.tile_b >= 0) {
    __syncthreads();
    dq_tile<D>(P, A, sm, wg.b, wg.h, wg.g, wg.tile_b);
  }
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
