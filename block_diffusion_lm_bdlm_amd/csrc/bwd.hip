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
// A workgroup owns a 128-row query tile of one head and runs 2 waves, one
// per SIMD (two workgroups per CU), each owning 64 rows (two 32-row
// blocks).  A wave holds its rows' Q and dO (B operands) and its dQ^T
// accumulators in AGPRs and, per key tile of 64 keys,
//   S^T = K Q^T,  P^T = exp(S^T - LSE) (masked),  dP^T = V dO^T,
//   dS^T = P^T (dP^T - D),  dQ^T += K^T dS^T,
// reading each K, V and K^T fragment from LDS once for both row blocks.
// K and V (fp16 rows) go from global memory straight into LDS
// (global_load_lds), double buffered; K^T fragments are read across the
// rows of the staged K tile with the transposing LDS read.  Every product
// runs in fp16 on Q, dO, K and V as converted by the packing (the values of
// the bf16 inputs).
constexpr int kDqWaves = 2;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRows = kBQ / kDqWaves;  // query rows per wave
static_assert(kDqRows == 64, "two 32-row blocks per wave");
static_assert(kBK == kTileRows, "key tiles are staged as 64-row tiles");

template <int D>
struct __attribute__((aligned(16))) DqSmem {
  static constexpr int TILE = kBK * D;  // elements per staged tile
  _Float16 k[2][TILE];                  // fp16 [key][d]
  _Float16 v[2][TILE];
};

template <int D>
constexpr int kDqPer = kBK * D / 512 / kDqWaves;  // 1 KB blocks per wave per tile

template <int D>
__device__ __forceinline__ int64_t dq_tile_base(const Plan& P, int b, int g, int32_t c) {
  return uniform64(((int64_t)(b * P.hkv + g) * P.nkc + c) * D);
}

// Copies of key tile c: K and V into buffer B.
template <int D>
__device__ __forceinline__ void dq_stage_kv(const DqArgs& A, const Plan& P, int b, int g, int32_t c, int wave,
                                            const LaneOff<D>& o, DqSmem<D>& sm, int B) {
  const int64_t base = dq_tile_base<D>(P, b, g, c);
#pragma unroll
  for (int j = 0; j < kDqPer<D>; ++j) {
    const int blk = (wave + kDqWaves * j) * 512;
    const int64_t e = base + (int64_t)j * kDqWaves * 512;
    copy16(A.kh + e, o.dn[j & 1], &sm.k[B][blk]);
    copy16(A.vh + e, o.dn[j & 1], &sm.v[B][blk]);
  }
}

// acc[rb][kb] = tile[kb*32 .. +32][:] times row block rb's registers (AGPR
// B operands), for both key and row blocks; each fragment (ks, kb) is read
// once and feeds both row blocks.
template <int D>
__device__ __forceinline__ void dq_products(const _Float16* tile, int ql, const f16x8 (&rows)[2][D / 16],
                                            const LaneOff<D>& o, f32x16 (&acc)[2][2]) {
  constexpr int NF = 2 * (D / 16);
  const _Float16* tb = tile + ql * D;
  f16x8 fr[NF];
#pragma unroll
  for (int f = 0; f < kAhead; ++f) fr[f] = ld16<f16x8>(tb + (f & 1) * 32 * D + o.nat[f >> 1]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + kAhead < NF) {
      const int h = f + kAhead;
      fr[h] = ld16<f16x8>(tb + (h & 1) * 32 * D + o.nat[h >> 1]);
    }
    const int kb = f & 1, ks = f >> 1;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if (ks == 0)
        acc[rb][kb] = mfma_f16_bagpr0(fr[f], rows[rb][ks]);
      else
        mfma_f16_bagpr(acc[rb][kb], fr[f], rows[rb][ks]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct DqRows {
  float lse2[2], dval[2];
  int32_t vlo[2], vhi[2];  // visible compact keys of this tile (masked tiles)
};

// dS^T chunk (kb, ss) of both row blocks: P^T (dP^T - D), with dP - D
// rounded to fp16 before the product; written over P^T.
__device__ __forceinline__ void dq_ds_chunk(int kb, int ss, const f32x16 (&pc)[2][2], const float (&dval)[2],
                                            f16x8 (&pf)[2][2][2]) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    f16x8 t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = (_Float16)(pc[rb][kb][ss * 8 + e] - dval[rb]);
    pf[rb][kb][ss] = pf[rb][kb][ss] * t;
  }
}

// Piece q of NP of the dS^T chunk (kb, ss) of both row blocks: row block
// q / (NP / 2), elements of the 8 in slice q % (NP / 2).
template <int NP>
__device__ __forceinline__ void dq_ds_piece(int q, int kb, int ss, const f32x16 (&pc)[2][2], const float (&dval)[2],
                                            f16x8 (&pf)[2][2][2]) {
  constexpr int H = NP / 2, W = 8 / H;  // pieces per row block, elements per piece
  static_assert(8 % H == 0 && W % 2 == 0, "pieces of whole fp16 pairs");
  const int rb = q / H, e0 = (q % H) * W;
#pragma unroll
  for (int e = e0; e < e0 + W; e += 2) {
    f16x2 t = {(_Float16)(pc[rb][kb][ss * 8 + e] - dval[rb]), (_Float16)(pc[rb][kb][ss * 8 + e + 1] - dval[rb])};
    f16x2 p = {pf[rb][kb][ss][e], pf[rb][kb][ss][e + 1]};
    const f16x2 r = p * t;
    pf[rb][kb][ss][e] = r[0];
    pf[rb][kb][ss][e + 1] = r[1];
  }
}

// One key tile of the wave's walk (buffers B).  The vector work of each stage runs between the matrix products of the next:
// the exponentials between the dP^T products, each dS^T chunk between the
// dQ^T products of the previous chunk.
template <int D>
__device__ __forceinline__ void dq_step(DqSmem<D>& sm, int B, bool full, int32_t c, const DqRows& rw, float c2,
                                        int ql, int hh, const f16x8 (&qreg)[2][D / 16],
                                        const f16x8 (&doreg)[2][D / 16], const LaneOff<D>& o,
                                        f32x16 (&dqacc)[2][D / 32]) {
  constexpr int NF = 2 * (D / 16);  // K or V fragments (ks, kb)
  // S^T
  f32x16 sc[2][2];
  dq_products<D>(sm.k[B], ql, qreg, o, sc);
  mfma_settle();
  if (!full) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t key = c + kb * 32 + crow(i, hh);
          if (key < rw.vlo[rb] || key >= rw.vhi[rb]) sc[rb][kb][i] = -INFINITY;
        }
  }
  // dP^T = V dO^T, with P^T = exp2(S^T c2 - LSE2) between the products
  f16x8 pf[2][2][2];
  f32x16 pc[2][2];
  {
    constexpr int PE = 64 / NF;  // probabilities per fragment
    const _Float16* tb = sm.v[B] + ql * D;
    f16x8 fr[NF];
#pragma unroll
    for (int f = 0; f < kAhead; ++f) fr[f] = ld16<f16x8>(tb + (f & 1) * 32 * D + o.nat[f >> 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f + kAhead < NF) {
        const int h = f + kAhead;
        fr[h] = ld16<f16x8>(tb + (h & 1) * 32 * D + o.nat[h >> 1]);
      }
      const int kb = f & 1, ks = f >> 1;
      // each product is followed by half of this fragment's probabilities
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if (ks == 0)
          pc[rb][kb] = mfma_f16_bagpr0(fr[f], doreg[rb][ks]);
        else
          mfma_f16_bagpr(pc[rb][kb], fr[f], doreg[rb][ks]);
#pragma unroll
        for (int e = rb * (PE / 2); e < (rb + 1) * (PE / 2); ++e) {
          const int x = f * PE + e, prb = x >> 5, pkb = (x >> 4) & 1, i = x & 15;
          pf[prb][pkb][i >> 3][i & 7] =
              (_Float16)__builtin_amdgcn_exp2f(fmaf(sc[prb][pkb][i], c2, -rw.lse2[prb]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // dQ^T += K^T dS^T; fragment f = (s, db) feeds both row blocks, chunk s + 1
  // of dS^T is formed during group s
  constexpr int NDB = D / 32, NT = (kBK / 16) * NDB;
  const _Float16* kb16 = sm.k[B];
  f16x8 fr[NT];
#pragma unroll
  for (int f = 0; f < kAhead; ++f) fr[f] = tr_frag<D>(kb16 + (f / NDB) * 16 * D, o, f % NDB);
  mfma_settle();
  dq_ds_chunk(0, 0, pc, rw.dval, pf);
  mfma_settle_short();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < NT; ++f) {
    if (f + kAhead < NT) {
      const int h = f + kAhead;
      fr[h] = tr_frag<D>(kb16 + (h / NDB) * 16 * D, o, h % NDB);
    }
    const int sk = f / NDB, db = f % NDB;
    if (db == 0 && sk > 0) mfma_settle_short();
    // each product is followed by a quarter of the next chunk's dS^T (one
    // row block, four of its eight elements)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      mfma_f16_agpr(dqacc[rb][db], fr[f], pf[rb][sk >> 1][sk & 1]);
      if (sk + 1 < kBK / 16) {
        const int nk = sk + 1, q = db * 2 + rb;  // quarter q of 2 * NDB pieces
        dq_ds_piece<2 * NDB>(q, nk >> 1, nk & 1, pc, rw.dval, pf);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
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

  // Q and dO of this lane's two rows (B operands, kept in AGPRs)
  f16x8 qreg[2][D / 16];
  f16x8 doreg[2][D / 16];
  DqRows rw;
  RowBounds rbd[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int32_t rq = wave * kDqRows + rb * 32 + ql;
    const int64_t cr = hb * P.nqc + (int64_t)tile * kBQ + rq;  // compact (zero-padded) row
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qreg[rb][ks] = ld16<f16x8>(A.qh + cr * D + ks * 16 + hh * 8);
      doreg[rb][ks] = ld16<f16x8>(A.doh + cr * D + ks * 16 + hh * 8);
      keep_in_agpr(qreg[rb][ks]);
      keep_in_agpr(doreg[rb][ks]);
    }
    rw.lse2[rb] = A.lse2[cr];
    rw.dval[rb] = A.dc[cr];
    rbd[rb] = row_bounds(P, S, r0 + min(rq, n - 1));
  }
  const KeyWalk w = keywalk_build(P, S, r0, r0 + n - 1);
  const LaneOff<D> o = lane_offsets<D, kDqWaves>(wave, lane);
  const float c2 = P.scale_log2;
  f32x16 dqacc[2][D / 32];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqacc[rb][db] = f32x16{};

  if (w.total > 0) {
    {
      int32_t c, ri;
      bool fu;
      keywalk_at(w, 0, &c, &ri, &fu);
      dq_stage_kv<D>(A, P, b, g, c, wave, o, sm, 0);
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
        dq_stage_kv<D>(A, P, b, g, cn, wave, o, sm, B ^ 1);
      }
      if (!full) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) compact_range(P.k[ri], rbd[rb], clean, &rw.vlo[rb], &rw.vhi[rb]);
      }
      dq_step<D>(sm, B, full, c, rw, c2, ql, hh, qreg, doreg, o, dqacc);
      wait_copies();
      __syncthreads();  // the next tile's K, V have landed; this tile's reads are done
    }
  }
  agpr_settle();
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int32_t rq = wave * kDqRows + rb * 32 + ql;
    if (rq < n) {
      const int32_t row = S.row0 + r0 + rq;
      float* dp = A.dq + (((int64_t)b * P.R + row) * P.hq + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          f32x4* p4 = reinterpret_cast<f32x4*>(dp + db * 32 + crow(i, hh));
          f32x4 cur = A.overwrite ? f32x4{0.f, 0.f, 0.f, 0.f} : *p4;
#pragma unroll
          for (int e = 0; e < 4; ++e) cur[e] += P.scale * dqacc[rb][db][i + e];
          *p4 = cur;
        }
    }
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kDqThreads, kDqThreads), amdgpu_waves_per_eu(1, 1)))
void dq_kernel(const Plan P, const DqArgs A) {
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
