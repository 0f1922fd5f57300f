// dq.hip — dQ of BDLM attention, query-major, 32 query rows per wave.
//
// For every visible pair, with the final LSE and D_i = dO_i . O_i:
//   P = exp(s - LSE),  dS = P (dO_i . v_j - D_i),  dQ_i += scale dS k_j
// (chain rule of the attention equation in "CSBP 完全拆解").  The packing
// hands over each row's dO and D times 2^-c and log2 LSE minus c, so P comes
// out as P * 2^c and dS unchanged.
//
// A workgroup owns a 128-row query tile of one head, in the forward's work
// order, and runs 4 waves of 32 rows each (two workgroups per CU, so two
// waves per SIMD: one wave's exponentials and dS run under the other's
// matrix products).  A wave holds its rows' Q and dO as B operands and its
// dQ^T accumulators, and per key tile of 64 keys computes
//   S^T = K Q^T and dP^T = V dO^T (interleaved),
//   P^T = exp2(S^T c2 - LSE2) (masked),  dS^T = P^T (dP^T - D),  dQ^T += K^T dS^T,
// with K and V (fp16 rows) staged double buffered in LDS (global_load_lds)
// and K^T fragments read across the rows of the staged K tile.  All products
// are compiler builtins, so the compiler places every wait state.  (One
// 64-row wave per SIMD with its operands and accumulators in AGPRs through
// inline-assembly products ran the same 64K walk no faster and the 8K and
// windowed workloads' short walks 10-15% slower.)
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "stage.h"
#include "walk.h"

namespace bd {

namespace {

constexpr int kDqWaves = 4;
static_assert(kBQ == 32 * kDqWaves, "32 rows per wave");
static_assert(kBK == kTileRows, "key tiles are staged as 64-row tiles");

template <int D>
struct __attribute__((aligned(16))) DqSmem {
  static constexpr int TILE = kBK * D;
  _Float16 k[2][TILE];  // fp16 [key][d]
  _Float16 v[2][TILE];
};

template <int D>
__device__ __forceinline__ void dq_stage(const DqArgs& A, const Plan& P, int b, int g, int32_t c, int wave,
                                           const LaneOff<D>& o, DqSmem<D>& sm, int B) {
  constexpr int PER = kBK * D / 512 / kDqWaves;  // 1 KB blocks per wave per tile
  const int64_t base = uniform64(((int64_t)(b * P.hkv + g) * P.nkc + c) * D);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int blk = (wave + kDqWaves * j) * 512;
    const int64_t e = base + (int64_t)j * kDqWaves * 512;
    copy16(A.kh + e, o.dn[j & 1], &sm.k[B][blk]);
    copy16(A.vh + e, o.dn[j & 1], &sm.v[B][blk]);
  }
}

template <int D>
__device__ void dq_tile(const Plan& P, const DqArgs& A, DqSmem<D>& sm, int b, int h, int g, int32_t tile) {
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = uniform(tid >> 6);
  const QSeg S = P.q[seg_of_tile(P, tile)];
  const int32_t r0 = (tile - S.tile0) * kBQ;
  const int32_t n = min(kBQ, S.nrows - r0);
  const bool clean = S.kind == KIND_CLEAN;
  const int64_t hb = (int64_t)(b * P.hq + h);
  const int32_t rq = wave * 32 + ql;
  const int64_t cr = hb * P.nqc + (int64_t)tile * kBQ + rq;  // compact (zero-padded) row

  f16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qreg[ks] = ld16<f16x8>(A.qh + cr * D + ks * 16 + hh * 8);
    doreg[ks] = ld16<f16x8>(A.doh + cr * D + ks * 16 + hh * 8);
  }
  const float lse2 = A.lse2[cr];
  const float dval = A.dc[cr];
  const RowBounds rb = row_bounds(P, S, r0 + min(rq, n - 1));
  const KeyWalk w = keywalk_build(P, S, r0, r0 + n - 1);
  const LaneOff<D> o = lane_offsets<D, kDqWaves>(wave, lane);
  const float c2 = P.scale_log2;
  constexpr int NDB = D / 32;
  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

  if (w.total > 0) {
    {
      int32_t c, ri;
      bool fu;
      keywalk_at(w, 0, &c, &ri, &fu);
      dq_stage<D>(A, P, b, g, c, wave, o, sm, 0);
    }
    wait_copies();
    __syncthreads();
    auto tile_step = [&](int32_t t, auto buf_c) {
      constexpr int buf = decltype(buf_c)::value;
      int32_t c, ri;
      bool full;
      keywalk_at(w, t, &c, &ri, &full);
      if (t + 1 < w.total) {
        int32_t cn, rn;
        bool fn;
        keywalk_at(w, t + 1, &cn, &rn, &fn);
        dq_stage<D>(A, P, b, g, cn, wave, o, sm, buf ^ 1);
      }
      // one 32-key block at a time: S^T, P^T, dP^T and dS^T of a block live
      // together, so the wave fits two to a SIMD
      const _Float16* kt = sm.k[buf];
      int32_t vlo = 0, vhi = 0;
      bool see[2] = {true, true};
      if (!full) {
        compact_range(P.k[ri], rb, clean, &vlo, &vhi);
        see[0] = __any(sees_block32(vlo, vhi, c));
        see[1] = __any(sees_block32(vlo, vhi, c + 32));
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // a block none of the wave's rows sees (a masked tile's window edge
        // or another corrupted block's keys) has P = 0: nothing to add
        if (!see[kb]) continue;
        // S^T = K Q^T and dP^T = V dO^T, as two interleaved chains; the other
        // wave of the SIMD runs its vector work meanwhile
        f32x16 sacc, pacc;
        __builtin_amdgcn_s_setprio(2);
        scores_1kb_pair_f16<D>(kt + kb * 32 * D, qreg, sm.v[buf] + kb * 32 * D, doreg, ql, o, sacc, pacc);
        __builtin_amdgcn_s_setprio(0);
        if (!full) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int32_t key = c + kb * 32 + crow(i, hh);
            if (key < vlo || key >= vhi) sacc[i] = -INFINITY;
          }
        }
        f16x8 pf[2];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pf[i >> 3][i & 7] = (_Float16)__builtin_amdgcn_exp2f(fmaf(sacc[i], c2, -lse2));
        // dS^T = P^T (dP^T - D), with dP - D rounded to fp16 before the product
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          f16x8 tt;
#pragma unroll
          for (int e = 0; e < 8; ++e) tt[e] = (_Float16)(pacc[ss * 8 + e] - dval);
          pf[ss] = pf[ss] * tt;
        }
        // dQ^T += K^T dS^T over the block's two 16-key steps: fragment f = (step, d block)
        constexpr int NT = 2 * NDB;
        f16x8 fr[NT];
#pragma unroll
        for (int f = 0; f < kAhead && f < NT; ++f)
          fr[f] = tr_frag<D>(kt + (2 * kb + f / NDB) * 16 * D, o, f % NDB);
        __builtin_amdgcn_s_setprio(2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < NT; ++f) {
          if (f + kAhead < NT) {
            const int hf = f + kAhead;
            fr[hf] = tr_frag<D>(kt + (2 * kb + hf / NDB) * 16 * D, o, hf % NDB);
          }
          dqacc[f % NDB] = mfma_f16(fr[f], pf[f / NDB], dqacc[f % NDB]);
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      wait_copies();
      __syncthreads();  // the next tile's K, V have landed; this tile's reads are done
    };
    int32_t t = 0;
    for (; t + 1 < w.total; t += 2) {
      tile_step(t, std::integral_constant<int, 0>{});
      tile_step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < w.total) tile_step(t, std::integral_constant<int, 0>{});
  }
  if (rq < n) {
    const int32_t row = S.row0 + r0 + rq;
    float* dp = A.dq + (((int64_t)b * P.R + row) * P.hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        f32x4* p4 = reinterpret_cast<f32x4*>(dp + db * 32 + crow(i, hh));
        f32x4 cur = A.overwrite ? f32x4{0.f, 0.f, 0.f, 0.f} : *p4;
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[e] += P.scale * dqacc[db][i + e];
        *p4 = cur;
      }
  }
}

template <int D>
__global__ __launch_bounds__(64 * kDqWaves, 2) void dq_kernel(const Plan P, const DqArgs A) {
  __shared__ DqSmem<D> sm;
  __shared__ int64_t item;
  // one work item from the XCD queues (plan.h); a spare workgroup that
  // finds every queue empty ends here
  if (threadIdx.x == 0) {
    int scan = 0;
    item = next_item(A.queue, kQueueStride, P.nwg_q, (int)(blockIdx.x % kXCD), &scan);
  }
  __syncthreads();
  const int64_t l = item;
  if (l < 0) return;
  const WgQ wg = decode_item_q(P, l);
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
    hipLaunchKernelGGL(dq_kernel<128>, dim3(queue_grid(P.nwg_q)), dim3(64 * kDqWaves), 0, s, P, a);
  else
    hipLaunchKernelGGL(dq_kernel<64>, dim3(queue_grid(P.nwg_q)), dim3(64 * kDqWaves), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace bd
