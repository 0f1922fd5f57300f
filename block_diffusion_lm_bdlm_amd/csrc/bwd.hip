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
// dkdv: key-major.  A workgroup owns 128 keys of one KV head (32 per wave,
//       K and V held in registers as B operands), walks every query row of
//       the group's query heads that sees them in steps of 32 rows staged in
//       LDS, and accumulates dK^T, dV^T in registers: clean keys collect
//       contributions from every later block without atomics.
// dq:   query-major, the forward's work order: recomputes S^T and dP^T per
//       key tile and accumulates dQ^T in registers.
#include "device.h"
#include "kernels.h"
#include "walk.h"

namespace bd {

namespace {

// ----------------------------------------------------------------- dQ
template <int D>
struct __attribute__((aligned(16))) DqSmem {
  static constexpr int KS = D + 8;
  static constexpr int TS = kBK + 8;
  uint16_t k[2][kBK * KS];
  uint16_t v[2][kBK * KS];
  _Float16 kt[2][D * TS];
};

template <int D>
__device__ inline void dq_load(const DqArgs& A, const Plan& P, int b, int g, int c, int tid,
                               u32x4 (&kr)[D / 32], u32x4 (&vr)[D / 32], u32x4 (&tr)[D / 32]) {
  const int64_t nb = ((int64_t)(b * P.hkv + g) * P.nkc + c) * D;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const int ch = tid + 256 * j;
    const int key = ch / (D / 8), dc = ch % (D / 8);
    kr[j] = ldg16(A.kn + nb + key * D + dc * 8);
    vr[j] = ldg16(A.vn + nb + key * D + dc * 8);
  }
  const _Float16* tb = A.kt + (int64_t)(b * P.hkv + g) * D * P.nkc + c;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const int ch = tid + 256 * j;
    const int d = ch / (kBK / 8), kc = ch % (kBK / 8);
    tr[j] = ldg16(tb + (int64_t)d * P.nkc + kc * 8);
  }
}

template <int D>
__device__ inline void dq_store(DqSmem<D>& sm, int buf, int tid, const u32x4 (&kr)[D / 32],
                                const u32x4 (&vr)[D / 32], const u32x4 (&tr)[D / 32]) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const int ch = tid + 256 * j;
    const int key = ch / (D / 8), dc = ch % (D / 8);
    *reinterpret_cast<u32x4*>(&sm.k[buf][key * DqSmem<D>::KS + dc * 8]) = kr[j];
    *reinterpret_cast<u32x4*>(&sm.v[buf][key * DqSmem<D>::KS + dc * 8]) = vr[j];
    const int d = ch / (kBK / 8), kc = ch % (kBK / 8);
    *reinterpret_cast<u32x4*>(&sm.kt[buf][d * DqSmem<D>::TS + kc * 8]) = tr[j];
  }
}

template <int D>
__device__ void dq_tile(const Plan& P, const DqArgs& A, DqSmem<D>& sm, int b, int h, int g, int32_t tile) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const QSeg S = P.q[seg_of_tile(P, tile)];
  const int32_t r0 = (tile - S.tile0) * kBQ;
  const int32_t n = min(kBQ, S.nrows - r0);
  const int32_t rq = wave * 32 + ql;
  const int32_t rc = min(rq, n - 1);
  const bool clean = S.kind == KIND_CLEAN;
  const int64_t hb = (int64_t)(b * P.hq + h);
  const int64_t crow_q = hb * P.nqc + (int64_t)tile * kBQ + rq;  // compact (zero-padded) row

  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qreg[ks] = ld16<bf16x8>(A.qn + crow_q * D + ks * 16 + hh * 8);
    doreg[ks] = ld16<bf16x8>(A.don + crow_q * D + ks * 16 + hh * 8);
  }
  const float lse2 = A.lse2[crow_q];
  const float Dr = A.dc[crow_q];
  const RowBounds rb = row_bounds(P, S, r0 + rc);
  const KeyWalk w = keywalk_build(P, S, r0, r0 + n - 1);
  const float c2 = P.scale_log2;

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};

  if (w.total > 0) {
    u32x4 kr[D / 32], vr[D / 32], tr[D / 32];
    {
      int32_t c, ri;
      bool fu;
      keywalk_at(w, 0, &c, &ri, &fu);
      dq_load<D>(A, P, b, g, c, tid, kr, vr, tr);
      dq_store<D>(sm, 0, tid, kr, vr, tr);
    }
    __syncthreads();
    for (int32_t t = 0; t < w.total; ++t) {
      const int buf = t & 1;
      int32_t c, ri;
      bool full;
      keywalk_at(w, t, &c, &ri, &full);
      if (t + 1 < w.total) {
        int32_t cn, rn;
        bool fn;
        keywalk_at(w, t + 1, &cn, &rn, &fn);
        dq_load<D>(A, P, b, g, cn, tid, kr, vr, tr);
      }
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        pacc[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int off = (kb * 32 + ql) * DqSmem<D>::KS + ks * 16 + hh * 8;
          sacc[kb] = mfma_bf16(ld16<bf16x8>(&sm.k[buf][off]), qreg[ks], sacc[kb]);
          pacc[kb] = mfma_bf16(ld16<bf16x8>(&sm.v[buf][off]), doreg[ks], pacc[kb]);
        }
      }
      int32_t vlo = c, vhi = c + kBK;
      if (!full) compact_range(P.k[ri], rb, clean, &vlo, &vhi);
      f16x8 dsf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t key = c + kb * 32 + crow(i, hh);
          const float x = (key >= vlo && key < vhi) ? fmaf(sacc[kb][i], c2, -lse2) : -INFINITY;
          const float p = __builtin_amdgcn_exp2f(x);
          dsf[kb][i >> 3][i & 7] = (_Float16)(p * (pacc[kb][i] - Dr));
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ss = 0; ss < 2; ++ss) {
            const f16x8 a =
                ld16<f16x8>(&sm.kt[buf][(db * 32 + ql) * DqSmem<D>::TS + kb * 32 + ss * 16 + hh * 8]);
            dqacc[db] = mfma_f16(a, dsf[kb][ss], dqacc[db]);
          }
      if (t + 1 < w.total) dq_store<D>(sm, buf ^ 1, tid, kr, vr, tr);
      __syncthreads();
    }
  }
  if (rq < n) {
    const int32_t row = S.row0 + r0 + rq;
    float* dp = A.dq + (((int64_t)b * P.R + row) * P.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        f32x4* p4 = reinterpret_cast<f32x4*>(dp + db * 32 + crow(i, hh));
        f32x4 cur = *p4;
        cur[0] += P.scale * dqacc[db][i];
        cur[1] += P.scale * dqacc[db][i + 1];
        cur[2] += P.scale * dqacc[db][i + 2];
        cur[3] += P.scale * dqacc[db][i + 3];
        *p4 = cur;
      }
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void dq_kernel(const Plan P, const DqArgs A) {
  __shared__ DqSmem<D> sm;
  const WgQ wg = decode_wg_q(P, blockIdx.x);
  dq_tile<D>(P, A, sm, wg.b, wg.h, wg.g, wg.tile_a);
  if (wg.tile_b >= 0) dq_tile<D>(P, A, sm, wg.b, wg.h, wg.g, wg.tile_b);
}

// ----------------------------------------------------------------- dK / dV
template <int D>
struct __attribute__((aligned(16))) DkdvSmem {
  static constexpr int NS = D + 8;      // natural row stride
  static constexpr int TS = kBQB + 8;   // transposed row stride
  uint16_t q[2][kBQB * NS];
  uint16_t dO[2][kBQB * NS];
  _Float16 qt[2][D * TS];
  _Float16 dot[2][D * TS];
  float lse2[2][kBQB];
  float dc[2][kBQB];
  // query steps of kBQB rows that see the key tile, per query head:
  // segment s contributes count[s] steps starting at row first[s]
  int32_t wseg[kMaxQSeg], wfirst[kMaxQSeg], wcount[kMaxQSeg];
  int32_t wn, wper;
};

template <int D>
__device__ inline void dkdv_load(const DkdvArgs& A, const Plan& P, int64_t hb, int32_t cq, int tid,
                                 u32x4 (&r)[D / 16], float& l2, float& dd) {
  // natural Q, dO: kBQB rows x D -> kBQB*D/8 chunks; transposed: D rows x kBQB
  constexpr int NCH = kBQB * D / 8;  // chunks per tensor
#pragma unroll
  for (int j = 0; j < NCH / 256; ++j) {
    const int ch = tid + 256 * j;
    const int row = ch / (D / 8), dc = ch % (D / 8);
    r[j] = ldg16(A.qn + (hb * P.nqc + cq + row) * D + dc * 8);
    r[NCH / 256 + j] = ldg16(A.don + (hb * P.nqc + cq + row) * D + dc * 8);
    const int d = ch / (kBQB / 8), sc = ch % (kBQB / 8);
    r[2 * (NCH / 256) + j] = ldg16(A.qt + (hb * D + d) * P.nqc + cq + sc * 8);
    r[3 * (NCH / 256) + j] = ldg16(A.dot + (hb * D + d) * P.nqc + cq + sc * 8);
  }
  if (tid < kBQB) {
    l2 = A.lse2[hb * P.nqc + cq + tid];
    dd = A.dc[hb * P.nqc + cq + tid];
  }
}

template <int D>
__device__ inline void dkdv_store(DkdvSmem<D>& sm, int buf, int tid, const u32x4 (&r)[D / 16], float l2,
                                  float dd) {
  constexpr int NCH = kBQB * D / 8;
#pragma unroll
  for (int j = 0; j < NCH / 256; ++j) {
    const int ch = tid + 256 * j;
    const int row = ch / (D / 8), dc = ch % (D / 8);
    *reinterpret_cast<u32x4*>(&sm.q[buf][row * DkdvSmem<D>::NS + dc * 8]) = r[j];
    *reinterpret_cast<u32x4*>(&sm.dO[buf][row * DkdvSmem<D>::NS + dc * 8]) = r[NCH / 256 + j];
    const int d = ch / (kBQB / 8), sc = ch % (kBQB / 8);
    *reinterpret_cast<u32x4*>(&sm.qt[buf][d * DkdvSmem<D>::TS + sc * 8]) = r[2 * (NCH / 256) + j];
    *reinterpret_cast<u32x4*>(&sm.dot[buf][d * DkdvSmem<D>::TS + sc * 8]) = r[3 * (NCH / 256) + j];
  }
  if (tid < kBQB) {
    sm.lse2[buf][tid] = l2;
    sm.dc[buf][tid] = dd;
  }
}

template <int D>
__device__ void dkdv_tile(const Plan& P, const DkdvArgs& A, DkdvSmem<D>& sm, int b, int g, int32_t ktile) {
  static_assert(kBQB * D / 8 >= 256 && (kBQB * D / 8) % 256 == 0, "chunking");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  int32_t kseg, koff;
  ktile_locate(P, ktile, &kseg, &koff);
  const KSeg K = P.k[kseg];
  const int32_t kvalid = min(kBKB, K.len - koff);  // valid keys in this tile
  const int32_t kt0 = K.t0 + koff;                 // first source row
  const int32_t kt1 = kt0 + kvalid;
  const int32_t c = K.c0 + koff;                   // compact start
  const int32_t mykey = wave * 32 + ql;            // key within the tile (this lane's column)
  const bool key_ok = mykey < kvalid;
  const int32_t mysrc = kt0 + mykey;

  // this wave's 32 keys as B operands: K[key][ks*16 + hh*8 ..]
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

  // query steps that see this key tile, per head (workgroup-uniform, in LDS)
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
  const int32_t per_head = sm.wper, nseg = sm.wn;
  const int32_t total = per_head * P.G;
  const float c2 = P.scale_log2;

  // walked back to front: the last rows are seen by every key tile, so the
  // workgroups resident together start on the same rows and share them in L2
  auto locate = [&](int32_t t, int32_t* hsel, int32_t* sidx, int32_t* r0) {
    t = total - 1 - t;
    *hsel = t / per_head;
    int32_t u = t - *hsel * per_head, j = 0;
    while (j + 1 < nseg && u >= sm.wcount[j]) { u -= sm.wcount[j]; ++j; }
    *sidx = sm.wseg[j];
    *r0 = sm.wfirst[j] + u * kBQB;
  };

  if (total > 0) {
    u32x4 r[D / 16];
    float l2 = 0.f, dd = 0.f;
    {
      int32_t hs, sj, r0;
      locate(0, &hs, &sj, &r0);
      const QSeg& S = P.q[sj];
      dkdv_load<D>(A, P, (int64_t)(b * P.hq + g * P.G + hs), S.tile0 * kBQ + r0, tid, r, l2, dd);
      dkdv_store<D>(sm, 0, tid, r, l2, dd);
    }
    __syncthreads();
    for (int32_t t = 0; t < total; ++t) {
      const int buf = t & 1;
      int32_t hs, sj, r0;
      locate(t, &hs, &sj, &r0);
      const QSeg S = P.q[sj];
      if (t + 1 < total) {
        int32_t hn, sn, rn;
        locate(t + 1, &hn, &sn, &rn);
        const QSeg& Sn = P.q[sn];
        dkdv_load<D>(A, P, (int64_t)(b * P.hq + g * P.G + hn), Sn.tile0 * kBQ + rn, tid, r, l2, dd);
      }
      // S = Q K^T and dP = dO V^T for 32 query rows x this wave's 32 keys
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int off = ql * DkdvSmem<D>::NS + ks * 16 + hh * 8;
        sacc = mfma_bf16(ld16<bf16x8>(&sm.q[buf][off]), kreg[ks], sacc);
        pacc = mfma_bf16(ld16<bf16x8>(&sm.dO[buf][off]), vreg[ks], pacc);
      }
      // full: every row of the step sees every key of the tile
      const RowBounds rfirst = row_bounds(P, S, min(r0, S.nrows - 1));
      bool full = key_ok && (r0 + kBQB <= S.nrows) && (kvalid == kBKB);
      if (K.kind == KIND_CLEAN) full = full && rfirst.hi_clean >= kt1;
      else full = false;
      f16x8 pf[2], dsf[2];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][i4 * 8 + hh * 4]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dc[buf][i4 * 8 + hh * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i4 * 4 + e;
          bool vis = true;
          if (!full) {
            const int32_t rr = r0 + crow(i, hh);
            vis = key_ok && rr < S.nrows;
            if (vis) {
              const RowBounds rb = row_bounds(P, S, rr);
              vis = (K.kind == KIND_CLEAN) ? (mysrc < rb.hi_clean)
                                           : (S.kind == KIND_CORR && mysrc >= rb.lo_loc && mysrc < rb.hi_loc);
            }
          }
          const float x = vis ? fmaf(sacc[i], c2, -l4[e]) : -INFINITY;
          const float p = __builtin_amdgcn_exp2f(x);
          pf[i >> 3][i & 7] = (_Float16)p;
          dsf[i >> 3][i & 7] = (_Float16)(p * (pacc[i] - d4[e]));
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over the 32 query rows)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const int off = (db * 32 + ql) * DkdvSmem<D>::TS + ss * 16 + hh * 8;
          dvacc[db] = mfma_f16(ld16<f16x8>(&sm.dot[buf][off]), pf[ss], dvacc[db]);
          dkacc[db] = mfma_f16(ld16<f16x8>(&sm.qt[buf][off]), dsf[ss], dkacc[db]);
        }
      if (t + 1 < total) dkdv_store<D>(sm, buf ^ 1, tid, r, l2, dd);
      __syncthreads();
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

hipError_t launch_dq(const Plan& P, const DqArgs& a, hipStream_t s) {
  if (P.nwg_q == 0) return hipSuccess;
  if (P.d == 128)
    hipLaunchKernelGGL(dq_kernel<128>, dim3((unsigned)P.nwg_q), dim3(256), 0, s, P, a);
  else
    hipLaunchKernelGGL(dq_kernel<64>, dim3((unsigned)P.nwg_q), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

hipError_t launch_dkdv(const Plan& P, const DkdvArgs& a, hipStream_t s) {
  if (P.nwg_k == 0) return hipSuccess;
  if (P.d == 128)
    hipLaunchKernelGGL(dkdv_kernel<128>, dim3((unsigned)P.nwg_k), dim3(256), 0, s, P, a);
  else
    hipLaunchKernelGGL(dkdv_kernel<64>, dim3((unsigned)P.nwg_k), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace bd
