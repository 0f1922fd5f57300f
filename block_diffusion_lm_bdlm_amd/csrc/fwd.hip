// fwd.hip — forward of BDLM attention over one call's key set.
//
// O_i = sum_j softmax_j(s_ij) v_j with s_ij = scale q_i . k_j over the keys j
// the mask lets row i see ("CSBP 完全拆解", CP attention equation and the
// key/value set [K_b; K^clean_<b] of a corrupted block), plus
// LSE_i = ln sum_j exp(s_ij).  The softmax is taken online over key tiles
// in fp32 (running max and normaliser), with scores in base 2.
//
// bf16 kernel: a workgroup of 4 waves owns a 128-row query tile (32 rows
// per wave, the rows held as the B operand of S^T = K Q^T) and walks the
// key tiles of 64 keys that any of its rows can see.  K tiles (natural) and
// V^T tiles (fp16) go from global memory straight into LDS
// (global_load_lds), double buffered, as swizzled tiles.  A key tile that
// no row sees is never visited; a tile every row sees fully skips the mask.
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "stage.h"
#include "walk.h"

namespace bd {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;

constexpr int kFwdWaves = 4;
static_assert(kBK == kTileRows, "key tiles are staged as 64-row tiles");

template <int D>
struct __attribute__((aligned(16))) FwdSmem {
  static constexpr int TILE = kBK * D;  // elements per staged tile
  uint16_t k[2][TILE];                  // natural bf16 [key][d]
  _Float16 vt[2][TILE];                 // transposed fp16 [d][key], perm16 keys
};

// One C^T block of 32 rows of a staged natural tile (starting at `block`)
// times the lane's row held in registers: acc = block row^T, kAhead reads
// in flight (scores_2kb for a single 32-key block).
template <int D>
__device__ __forceinline__ void scores_1kb(const uint16_t* block, int ql, const bf16x8 (&row)[D / 16],
                                           const LaneOff<D>& o, f32x16& acc) {
  constexpr int NF = D / 16;
  const uint16_t* tb = block + ql * D;
  bf16x8 fr[NF];
#pragma unroll
  for (int f = 0; f < kAhead && f < NF; ++f) fr[f] = ld16<bf16x8>(tb + o.nat[f]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + kAhead < NF) fr[f + kAhead] = ld16<bf16x8>(tb + o.nat[f + kAhead]);
    acc = mfma_bf16(fr[f], row[f], f ? acc : f32x16{});
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Issues the copies of key tile c (compact start) into buffer B.
template <int D>
__device__ __forceinline__ void fwd_stage(const FwdArgs& A, const Plan& P, int b, int g, int32_t c, int wave,
                                          const LaneOff<D>& o, FwdSmem<D>& sm, int B) {
  constexpr int PER = kBK * D / 512 / kFwdWaves;  // 1 KB blocks per wave per tile
  const int64_t base = uniform64(((int64_t)(b * P.hkv + g) * P.nkc + c) * D);  // natural and transposed alike
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int blk = (wave + kFwdWaves * j) * 512;  // elements
    const int64_t e = base + (int64_t)j * kFwdWaves * 512;
    copy16(A.kn + e, o.dn[j & 1], &sm.k[B][blk]);
    copy16(A.vt + e, o.dt, &sm.vt[B][blk]);
  }
}

template <int D>
__device__ void fwd_tile(const Plan& P, const FwdArgs& A, FwdSmem<D>& sm, int b, int h, int g,
                         int32_t tile) {
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = uniform(tid >> 6);
  const QSeg S = P.q[seg_of_tile(P, tile)];
  const int32_t r0 = (tile - S.tile0) * kBQ;
  const int32_t n = min(kBQ, S.nrows - r0);
  const int32_t rq = wave * 32 + ql;
  const int32_t rc = min(rq, n - 1);
  const bool clean = S.kind == KIND_CLEAN;

  // this lane's query row (B operand: Q[row][ks*16 + hh*8 .. +8])
  const TensorArg& QT = clean ? A.q_clean : A.q_corr;
  const uint16_t* qp = static_cast<const uint16_t*>(QT.p) + b * QT.bs +
                       (int64_t)(S.src0 + r0 + rc) * QT.rs + (int64_t)h * QT.hs;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = ld16<bf16x8>(qp + ks * 16 + hh * 8);

  const RowBounds rb = row_bounds(P, S, r0 + rc);
  const KeyWalk w = keywalk_build(P, S, r0, r0 + n - 1);
  const LaneOff<D> o = lane_offsets<D, kFwdWaves>(wave, lane);

  const float c2 = P.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  if (w.total > 0) {
    {
      int32_t c, ri;
      bool fu;
      keywalk_at(w, 0, &c, &ri, &fu);
      fwd_stage<D>(A, P, b, g, c, wave, o, sm, 0);
    }
    wait_copies();
    __syncthreads();
    // one tile of the walk; the buffer index is a constant in each of the
    // two unrolled copies, so it folds into the LDS instructions' offsets
    auto tile_step = [&](int32_t t, auto buf_c) {
      constexpr int buf = decltype(buf_c)::value;
      int32_t c, ri;
      bool full;
      keywalk_at(w, t, &c, &ri, &full);
      if (t + 1 < w.total) {
        int32_t cn, rn;
        bool fn;
        keywalk_at(w, t + 1, &cn, &rn, &fn);
        fwd_stage<D>(A, P, b, g, cn, wave, o, sm, buf ^ 1);
      }
      // In a masked tile the wave forms scores only for the 32-key blocks
      // one of its rows sees; the other block's scores are -inf, so its P is
      // zero and its O products add nothing.  (The window's edges and a
      // corrupted tile's own-block keys put about an eighth of the products
      // of the 1,024-token windowed 64K walk in such blocks.  Skipping the
      // O products too, with a test per product, cost 6% on whole masks.)
      // The lane's visible range is formed again for the mask rather than
      // held across the score products, where the registers are all in use.
      bool see0 = true, see1 = true;
      if (!full) {
        int32_t vlo, vhi;
        compact_range(P.k[ri], rb, clean, &vlo, &vhi);
        see0 = __any(sees_block32(vlo, vhi, c));
        see1 = __any(sees_block32(vlo, vhi, c + 32));
        if (!see0 && !see1) {
          wait_copies();
          __syncthreads();
          return;
        }
      }
      // S^T = K Q^T for two blocks of 32 keys.  The two waves sharing a SIMD
      // belong to different workgroups; a wave raises its priority while it
      // issues matrix products and drops it for the softmax, so the other
      // wave's vector work fills the matrix core's shadow instead of
      // competing with it.
      f32x16 sacc[2];
      __builtin_amdgcn_s_setprio(2);
      if (see0 && see1) {
        scores_2kb<D>(sm.k[buf], ql, qreg, o, sacc);
      } else if (see0) {
        scores_1kb<D>(sm.k[buf], ql, qreg, o, sacc[0]);
        sacc[1] = f32x16{} - INFINITY;
      } else {
        scores_1kb<D>(sm.k[buf] + 32 * D, ql, qreg, o, sacc[1]);
        sacc[0] = f32x16{} - INFINITY;
      }
      __builtin_amdgcn_s_setprio(0);
      // the first V^T fragments of the O products, read under the softmax;
      // fragment f = (s, db), s = 16-key step
      constexpr int NDB = D / 32, NFO = (kBK / 16) * NDB;
      const _Float16* vtb = sm.vt[buf] + ql * kBK;
      f16x8 vfr[NFO];
#pragma unroll
      for (int f = 0; f < kAhead; ++f) vfr[f] = ld16<f16x8>(vtb + (f % NDB) * 32 * kBK + o.tr[f / NDB]);
      if (!full) {
        int32_t vlo, vhi;
        compact_range(P.k[ri], rb, clean, &vlo, &vhi);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int32_t key = c + kb * 32 + crow(i, hh);
            if (key < vlo || key >= vhi) sacc[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = wave_max32(mx);
      // The running max moves only when the tile's max exceeds it by more
      // than 8 (base 2, after scaling): probabilities then stay <= 2^8, which
      // fp16 P and the fp32 sums hold as well as values <= 1, and O is
      // rescaled only on such jumps instead of on every increase.  LSE uses
      // whichever max was kept, so it is unchanged.
      const bool grow = mx * c2 > m_run * c2 + 8.f;
      const float m_new = grow ? mx : m_run;
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float mc = m_use * c2;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run * c2 - mc) : 1.f;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      }
      m_run = m_new;
      // P of 16-key step s (8 values per lane, kb = s / 2) and its share of
      // the normaliser, which sums the fp16 probabilities the O product uses,
      // two per instruction (fp32 accumulation).  Step s + 1's exponentials
      // are issued after step s's O products, so they run while those
      // products occupy the matrix core (-1% at 64K, -2% at 8K against all
      // exponentials first).
      f16x8 pf[2][2];
      float lsum = 0.f;
      auto p_step = [&](int s) {
        const int kb = s >> 1, hf = s & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[kb][hf][e] = (_Float16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][hf * 8 + e], c2, -mc));
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f16x2 pp = {pf[kb][hf][e], pf[kb][hf][e + 1]};
          lsum = __builtin_amdgcn_fdot2(pp, f16x2{(_Float16)1.f, (_Float16)1.f}, lsum, false);
        }
      };
      p_step(0);
      // O^T += V^T P^T
      __builtin_amdgcn_s_setprio(2);
      {
        constexpr int NF = NFO;
        const _Float16* tb = vtb;
        f16x8 (&fr)[NF] = vfr;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f + kAhead < NF) {
            const int hf = f + kAhead;
            fr[hf] = ld16<f16x8>(tb + (hf % NDB) * 32 * kBK + o.tr[hf / NDB]);
          }
          const int s = f / NDB, db = f % NDB;
          oacc[db] = mfma_f16(fr[f], pf[s >> 1][s & 1], oacc[db]);
          __builtin_amdgcn_sched_barrier(0);
          if (db == NDB - 1 && s + 1 < kBK / 16) {
            p_step(s + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      l_run = l_run * alpha + lsum;
      __builtin_amdgcn_s_setprio(0);
      wait_copies();
      __syncthreads();  // the next tile's copies have landed; this tile's reads are done
    };
    int32_t t = 0;
    for (; t + 1 < w.total; t += 2) {
      tile_step(t, std::integral_constant<int, 0>{});
      tile_step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < w.total) tile_step(t, std::integral_constant<int, 0>{});
  }

  // epilogue: O = acc / l, LSE = (m * c2 + log2 l) * ln 2
  const float l = wave_sum32(l_run);
  if (rq < n) {
    const int32_t row = S.row0 + r0 + rq;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t obase = b * A.o_bs + (int64_t)row * A.o_rs + (int64_t)h * A.o_hs;
    if (A.o_f32) {
      float* op = static_cast<float*>(A.o) + obase;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          f32x4 v = {oacc[db][i] * inv, oacc[db][i + 1] * inv, oacc[db][i + 2] * inv,
                     oacc[db][i + 3] * inv};
          *reinterpret_cast<f32x4*>(op + db * 32 + crow(i, hh)) = v;
        }
    } else {
      uint16_t* op = static_cast<uint16_t*>(A.o) + obase;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          const uint32_t lo = bf16_bits(oacc[db][i] * inv) | ((uint32_t)bf16_bits(oacc[db][i + 1] * inv) << 16);
          const uint32_t hi = bf16_bits(oacc[db][i + 2] * inv) | ((uint32_t)bf16_bits(oacc[db][i + 3] * inv) << 16);
          *reinterpret_cast<uint2*>(op + db * 32 + crow(i, hh)) = make_uint2(lo, hi);
        }
    }
    if (hh == 0) {
      const float m_fin = (m_run == -INFINITY) ? 0.f : m_run;
      A.lse[((int64_t)b * P.R + row) * P.hq + h] =
          l > 0.f ? (m_fin * c2 + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(const Plan P, const FwdArgs A) {
  __shared__ FwdSmem<D> sm;
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
  fwd_tile<D>(P, A, sm, wg.b, wg.h, wg.g, wg.tile_a);
  if (wg.tile_b >= 0) {
    __syncthreads();
    fwd_tile<D>(P, A, sm, wg.b, wg.h, wg.g, wg.tile_b);
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const Plan& P, const FwdArgs& a, hipStream_t s) {
  if (P.nwg_q == 0) return hipSuccess;
  if (P.d == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3(queue_grid(P.nwg_q)), dim3(256), 0, s, P, a);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(queue_grid(P.nwg_q)), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace bd
