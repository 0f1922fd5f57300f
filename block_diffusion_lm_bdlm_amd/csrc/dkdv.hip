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
//   S-wave: K in registers; S = Q K^T, P = exp(S - LSE) (masked), hands P
//           to its partner through LDS, accumulates dV^T += dO^T P.
//   P-wave: V in registers; dP = dO V^T, reads P, dS = P (dP - D),
//           accumulates dK^T += Q^T dS.
// Each key has exactly one writer per gradient, so no atomics are needed,
// and the two waves of a SIMD overlap one's vector work with the other's
// matrix work.  (The keys per wave are a parameter: 64 keys per wave make
// each LDS fragment feed two products but need one wave per SIMD, which
// measured slower.)
// The workgroup walks every query row (of every query head of the group)
// that sees its keys, in steps of 64 rows.  Each step's operands (Q and dO
// as fp16 rows; per-row log2 LSE, D and visible key interval) go from
// global memory straight into LDS through the load units (global_load_lds),
// double buffered, into unpadded tiles whose 16-byte chunks are
// XOR-swizzled by row; the P-waves issue these copies (see kCopyWaves).  S and dP read the tiles along their rows; the
// contractions over rows (dV, dK) read the same tiles across their rows
// with the transposing LDS read, so each operand is staged once.  All
// products run in fp16 (Q, dO, K and V come converted by the packing): the
// values are those of the bf16 inputs.
// The walk runs back to front by position (all heads of the group at each
// position): the last rows are seen by every key tile, so the workgroups
// resident on one XCD stay on the same rows and share them through L2.
#include <climits>
#include <cstddef>
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "stage.h"

namespace bd {

namespace {

constexpr int kKW = 32;               // keys per wave
constexpr int kPairs = kBKB / kKW;    // S-wave / P-wave pairs per workgroup
constexpr int kWaves = 2 * kPairs;    // two waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kRB = kBQB / 32;        // 32-row MFMA blocks per step
constexpr int kKB = kKW / 32;         // 32-key MFMA blocks per wave
static_assert(kBKB % kKW == 0 && kKW % 32 == 0, "whole 32-key blocks per wave");
static_assert(kBQB == kTileRows, "one lane per row stages the per-row data; 64-row tiles");
// The P-waves issue every copy: the step's global -> LDS copies (32 KB)
// take the CU's load path about 500 cycles, and a wave stalls while its
// copies are accepted.  The S-waves' scores and exponentials lead to the
// mid-step barrier, where the P-waves otherwise wait, so the stall belongs
// on the P-waves.
constexpr int kCopyWaves = kPairs;
static_assert(kCopyWaves >= 4, "the four per-row arrays are staged one per copying wave");

template <int D>
struct __attribute__((aligned(16))) DkdvSmem {
  static constexpr int TILE = kBQB * D;  // elements per staged tile
  _Float16 q[2][TILE];                   // fp16 [row][d]
  _Float16 dO[2][TILE];
  float lse2[2][kBQB];
  float dc[2][kBQB];
  int32_t vlo[2][kBQB];  // row sees key sources [vlo, vhi) of the tile's kind
  int32_t vhi[2][kBQB];
  // P from each S-wave to its P-wave, in the MFMA C-tile order of each lane
  _Float16 xchg[kPairs][kRB][kKB][2][64][8];
  // steps of the walk: segment s contributes wcount[s] steps from row wfirst[s]
  int32_t wseg[kMaxQSeg], wfirst[kMaxQSeg], wcount[kMaxQSeg];
  int32_t wn, wper;
};

typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const i32x4 lds_i32x4;

// The lane's per-row values of a step (log2 LSE, D, visible interval; rows
// hh * 4 + 8 i4 + 32 rb + 0..3) are read at one base address plus constant
// offsets.  The base is formed in every step behind an empty asm: left to
// itself the compiler forms one address per read, as the arrays lie beyond
// the 16-bit offset field of the LDS instructions, hoists them out of the
// walk and spills them, and every reload then stalls its read.
template <int D>
__device__ __forceinline__ uint32_t row_vals_base(const DkdvSmem<D>& sm, int hh) {
  uint32_t a = (uint32_t)(uintptr_t)(lds_void*)&sm.lse2[0][hh * 4];
  asm volatile("" : "+v"(a));
  return a;
}
// Byte offset of row r of buffer B of a per-row array (its offset in the
// shared block given) from that base.
template <int D>
__device__ __forceinline__ constexpr uint32_t row_vals_off(size_t array_off, int B, int r) {
  return (uint32_t)(array_off - offsetof(DkdvSmem<D>, lse2)) + (uint32_t)(B * kBQB + r) * 4u;
}

// Issues the copies of one step (64 rows from compact row cq of head hb)
// into buffer B: copying wave cw (of kCopyWaves, lane offsets oc) copies
// its share of each tile.
template <int D>
__device__ __forceinline__ void stage(const DkdvArgs& A, const Plan& P, int kkind, int64_t hb, int64_t cq,
                                      int cw, int lane, const LaneOff<D>& oc, DkdvSmem<D>& sm, int B) {
  constexpr int PER = kBQB * D / 512 / kCopyWaves;  // 1 KB blocks per copying wave per tile
  const int64_t base = uniform64((hb * P.nqc + cq) * D);  // natural and transposed tiles alike
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int blk = (cw + kCopyWaves * j) * 512;  // elements
    const int64_t e = base + (int64_t)j * kCopyWaves * 512;
    copy16(A.qh + e, oc.dn[j & 1], &sm.q[B][blk]);
    copy16(A.doh + e, oc.dn[j & 1], &sm.dO[B][blk]);
  }
  const uint32_t lo = (uint32_t)lane * 4;
  switch (cw) {
    case 0: copy4(A.lse2 + hb * P.nqc + cq, lo, &sm.lse2[B][0]); break;
    case 1: copy4(A.dc + hb * P.nqc + cq, lo, &sm.dc[B][0]); break;
    case 2: copy4(A.vis + (int64_t)(2 * kkind) * P.nqc + cq, lo, &sm.vlo[B][0]); break;
    case 3: copy4(A.vis + (int64_t)(2 * kkind + 1) * P.nqc + cq, lo, &sm.vhi[B][0]); break;
    default: break;
  }
}

// S-wave, first half of a step: S = Q K^T, then P = exp2(S c2 - LSE2) on
// visible pairs (every pair when FULL), in fp16, as the B operands of the
// contraction over rows.
template <int D, bool FULL>
__device__ __forceinline__ void s_phase_a(DkdvSmem<D>& sm, int B, int kw, int lane, int ql, int hh,
                                          const int32_t (&mysrc)[kKB], float c2, const f16x8 (&kreg)[kKB][D / 16],
                                          const LaneOff<D>& o, f16x8 (&pf)[kRB][kKB][2]) {
  constexpr int NKS = D / 16;
  const _Float16* qb = &sm.q[B][ql * D];
  f32x16 sacc[kRB][kKB];
  // fragment f = (rb, ks); kAhead reads stay in flight ahead of the products
  constexpr int NF = kRB * NKS;
  f16x8 fr[NF];
  f32x4 l4s[kRB][4];  // log2 LSE of this lane's rows, read while the last products run
  const uint32_t rv = row_vals_base<D>(sm, hh);
#pragma unroll
  for (int f = 0; f < kAhead; ++f) fr[f] = ld16<f16x8>(qb + (f / NKS) * 32 * D + o.nat[f % NKS]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + kAhead < NF) {
      const int g = f + kAhead;
      fr[g] = ld16<f16x8>(qb + (g / NKS) * 32 * D + o.nat[g % NKS]);
    }
    if (f == NF - kAhead) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          l4s[rb][i4] = *(lds_f32x4*)(rv + row_vals_off<D>(offsetof(DkdvSmem<D>, lse2), B, rb * 32 + i4 * 8));
    }
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
      sacc[f / NKS][kb] = mfma_f16(fr[f], kreg[kb][f % NKS], f % NKS ? sacc[f / NKS][kb] : f32x16{});
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int r = rb * 32 + i4 * 8;
      const f32x4 l4 = l4s[rb][i4];
      i32x4 los = {INT_MIN, INT_MIN, INT_MIN, INT_MIN}, his = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
      if constexpr (!FULL) {
        los = *(lds_i32x4*)(rv + row_vals_off<D>(offsetof(DkdvSmem<D>, vlo), B, r));
        his = *(lds_i32x4*)(rv + row_vals_off<D>(offsetof(DkdvSmem<D>, vhi), B, r));
      }
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i4 * 4 + e;
          float x = fmaf(sacc[rb][kb][i], c2, -l4[e]);
          // both bounds tested (no short circuit, which the compiler turns into a branch per value)
          if constexpr (!FULL) x = ((mysrc[kb] >= los[e]) & (mysrc[kb] < his[e])) ? x : -INFINITY;
          pf[rb][kb][i >> 3][i & 7] = (_Float16)__builtin_amdgcn_exp2f(x);
        }
    }
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) *reinterpret_cast<f16x8*>(&sm.xchg[kw][rb][kb][ss][lane][0]) = pf[rb][kb][ss];
  }
}

// Fragments f = (s, db) of the contraction over rows.  The first kAhead
// are read by rows_contract_head ahead of the mid-step barrier (the tile is
// already in LDS), so the barrier's wait covers their latency.
template <int D>
constexpr int kRcFrags = (kBQB / 16) * (D / 32);
template <int D>
__device__ __forceinline__ void rows_contract_head(const _Float16* tile, const LaneOff<D>& o,
                                                   f16x8 (&fr)[kRcFrags<D>]) {
  constexpr int NDB = D / 32;
#pragma unroll
  for (int f = 0; f < kAhead; ++f) fr[f] = tr_frag<D>(tile + (f / NDB) * 16 * D, o, f % NDB);
}

// Contraction over the step's rows: acc^T[d][key] += T^T[d][row] X[row][key]
// with T a staged row tile (read across its rows) and X (P or dS) in
// registers, continuing from rows_contract_head.  The products are compiler
// builtins (accumulators in VGPRs), so the compiler inserts every wait state
// around them; a schedule with these products as inline assembly (AGPR
// accumulators) gave wrong dK once they ran one step behind the
// exponentials.
template <int D>
__device__ __forceinline__ void rows_contract(const _Float16* tile, const LaneOff<D>& o,
                                              const f16x8 (&x)[kRB][kKB][2], f32x16 (&acc)[D / 32][kKB],
                                              f16x8 (&fr)[kRcFrags<D>]) {
  // kAhead reads stay in flight ahead of the products
  constexpr int NDB = D / 32, NF = kRcFrags<D>;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + kAhead < NF) {
      const int g = f + kAhead;
      fr[g] = tr_frag<D>(tile + (g / NDB) * 16 * D, o, g % NDB);
    }
    const int s = f / NDB, db = f % NDB;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) acc[db][kb] = mfma_f16(fr[f], x[s >> 1][kb][s & 1], acc[db][kb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// P-wave, first half of a step: dP = dO V^T; D of this lane's rows is read
// while the last products run.
template <int D>
__device__ __forceinline__ void p_phase_a(DkdvSmem<D>& sm, int B, int ql, int hh, const f16x8 (&vreg)[kKB][D / 16],
                                          const LaneOff<D>& o, f32x16 (&pacc)[kRB][kKB], f32x4 (&dcs)[kRB][4]) {
  const _Float16* ob = &sm.dO[B][ql * D];
  const uint32_t rv = row_vals_base<D>(sm, hh);
  constexpr int NKS = D / 16, NF = kRB * NKS;
  f16x8 fr[NF];
#pragma unroll
  for (int f = 0; f < kAhead; ++f) fr[f] = ld16<f16x8>(ob + (f / NKS) * 32 * D + o.nat[f % NKS]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + kAhead < NF) {
      const int g = f + kAhead;
      fr[g] = ld16<f16x8>(ob + (g / NKS) * 32 * D + o.nat[g % NKS]);
    }
    if (f == NF - kAhead) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          dcs[rb][i4] = *(lds_f32x4*)(rv + row_vals_off<D>(offsetof(DkdvSmem<D>, dc), B, rb * 32 + i4 * 8));
    }
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
      pacc[f / NKS][kb] = mfma_f16(fr[f], vreg[kb][f % NKS], f % NKS ? pacc[f / NKS][kb] : f32x16{});
    __builtin_amdgcn_sched_barrier(0);
  }
}

// P-wave, second half: dS = P (dP - D) with P from its S-wave (dP - D is
// rounded to fp16 before the product; dS is an fp16 operand either way).
template <int D>
__device__ __forceinline__ void p_phase_ds(DkdvSmem<D>& sm, int kw, int lane, const f32x4 (&dcs)[kRB][4],
                                           const f32x16 (&pacc)[kRB][kKB], f16x8 (&dsf)[kRB][kKB][2]) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const f32x4 d0 = dcs[rb][2 * ss];
      const f32x4 d1 = dcs[rb][2 * ss + 1];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        const f16x8 p = ld16<f16x8>(&sm.xchg[kw][rb][kb][ss][lane][0]);
        // dP - D in fp32, then the product with P in packed fp16
        f16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (_Float16)(pacc[rb][kb][ss * 8 + e] - (e < 4 ? d0[e & 3] : d1[e & 3]));
        dsf[rb][kb][ss] = p * t;
      }
    }
}

// Position of the walk: k-th step from the end of walk segment j, query head
// hs within the group.
struct StepPos {
  int32_t k, j, hs;
};

// The query walk of one role.  S-waves and P-waves run the same sequence of
// barriers: two per step (after P is exchanged, after the next step lands).
template <int D, bool S_WAVE>
__device__ __forceinline__ void dkdv_walk(const Plan& P, const DkdvArgs& A, DkdvSmem<D>& sm, const KSeg& K, int b,
                                          int g, int32_t kvalid, int32_t kt1, int wave, int kw, int lane, int ql,
                                          int hh, const int32_t (&mysrc)[kKB], int32_t nseg, int32_t total,
                                          const LaneOff<D>& o, const f16x8 (&kvreg)[kKB][D / 16],
                                          f32x16 (&acc)[D / 32][kKB]) {
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
    } while (p.k >= uniform(sm.wcount[p.j]));
    return p;
  };
  auto row_of = [&](const StepPos& p) {
    return uniform(sm.wfirst[p.j]) + (uniform(sm.wcount[p.j]) - 1 - p.k) * kBQB;
  };
  auto hb_of = [&](const StepPos& p) { return (int64_t)(b * P.hq + g * P.G + p.hs); };
  auto cq_of = [&](const StepPos& p) { return (int64_t)P.q[uniform(sm.wseg[p.j])].tile0 * kBQ + row_of(p); };
  // copy offsets of the P-waves (copying wave wave - kPairs)
  const LaneOff<D> oc = lane_offsets<D, kCopyWaves>(S_WAVE ? 0 : wave - kPairs, lane);
  if constexpr (!S_WAVE) stage<D>(A, P, K.kind, hb_of(cur), cq_of(cur), wave - kPairs, lane, oc, sm, 0);
  // S-waves: no mask when every row of the step exists and sees every key of
  // the tile.  Formed for the next step at the end of the current one, so
  // its dependent reads (walk metadata, segment table) wait under the copy
  // wait instead of delaying the scores.
  auto full_of = [&](const StepPos& p) {
    const QSeg& S = P.q[uniform(sm.wseg[p.j])];
    const int32_t r0 = row_of(p);
    bool f = false;
    if (K.kind == KIND_CLEAN && kvalid == kBKB && r0 + kBQB <= S.nrows)
      f = row_bounds(P, S, r0).hi_clean >= kt1 && row_bounds(P, S, r0 + kBQB - 1).lo_clean <= kt1 - kvalid;
    return f;
  };
  bool full_next = S_WAVE ? full_of(cur) : false;
  wait_copies();
  __syncthreads();
  // one step of the walk; the buffer index is a constant in each of the two
  // unrolled copies, so it folds into the LDS instructions' offsets
  auto step = [&](int32_t t, auto b_c) {
    constexpr int B = decltype(b_c)::value;
    const bool more = t + 1 < total;
    StepPos nxt = cur;
    if constexpr (!S_WAVE) {
      if (more) {
        nxt = advance(cur);
        stage<D>(A, P, K.kind, hb_of(nxt), cq_of(nxt), wave - kPairs, lane, oc, sm, B ^ 1);
      }
    }
    if constexpr (S_WAVE) {
      const bool full = full_next;
      f16x8 pf[kRB][kKB][2];
      if (full)
        s_phase_a<D, true>(sm, B, kw, lane, ql, hh, mysrc, c2, kvreg, o, pf);
      else
        s_phase_a<D, false>(sm, B, kw, lane, ql, hh, mysrc, c2, kvreg, o, pf);
      __builtin_amdgcn_sched_barrier(0);  // the P writes stay ahead of the reads below
      f16x8 fr[kRcFrags<D>];
      rows_contract_head<D>(sm.dO[B], o, fr);
      // P visible to the P-waves; the 2 kAhead transposed reads just issued stay in flight
      barrier_lds_behind<2 * kAhead>();
      rows_contract<D>(sm.dO[B], o, pf, acc, fr);  // dV^T += dO^T P
    } else {
      f32x16 pacc[kRB][kKB];
      f32x4 dcs[kRB][4];
      p_phase_a<D>(sm, B, ql, hh, kvreg, o, pacc, dcs);
      f16x8 fr[kRcFrags<D>];
      rows_contract_head<D>(sm.q[B], o, fr);
      barrier_reads_in_flight();  // P from the S-waves
      f16x8 dsf[kRB][kKB][2];
      p_phase_ds<D>(sm, kw, lane, dcs, pacc, dsf);
      rows_contract<D>(sm.q[B], o, dsf, acc, fr);  // dK^T += Q^T dS
    }
    if constexpr (S_WAVE) {
      if (more) {
        nxt = advance(cur);
        full_next = full_of(nxt);
      }
    }
    wait_copies();
    __syncthreads();  // the next step's copies have landed; this step's reads are done
    cur = nxt;
  };
  int32_t t = 0;
  for (; t + 1 < total; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < total) step(t, std::integral_constant<int, 0>{});
}

// One role of the workgroup on its key tile: this wave's 64 keys in
// registers (K for the S-wave, V for the P-wave), the query walk, and the
// write-out of its gradient (dV or dK).  Each role keeps its accumulators
// in one place for the whole walk.
template <int D, bool S_WAVE>
__device__ __forceinline__ void dkdv_role(const Plan& P, const DkdvArgs& A, DkdvSmem<D>& sm, const KSeg& K, int b,
                                          int g, int32_t c, int32_t kvalid, int32_t kt1, int wave, int kw, int lane,
                                          int ql, int hh, const int32_t (&mysrc)[kKB], const bool (&key_ok)[kKB],
                                          int32_t nseg, int32_t total, const LaneOff<D>& o) {
  f16x8 kvreg[kKB][D / 16];
  {
    const int64_t nb = ((int64_t)(b * P.hkv + g) * P.nkc + c + kw * kKW + ql) * D + hh * 8;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int64_t e = nb + kb * 32 * D + ks * 16;
        if constexpr (S_WAVE)
          kvreg[kb][ks] = ld16<f16x8>(A.kh + e);
        else
          kvreg[kb][ks] = ld16<f16x8>(A.vh + e);
      }
  }
  f32x16 acc[D / 32][kKB];  // dV^T (S-wave) or dK^T (P-wave)
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) acc[db][kb] = f32x16{};
  if (total > 0)
    dkdv_walk<D, S_WAVE>(P, A, sm, K, b, g, kvalid, kt1, wave, kw, lane, ql, hh, mysrc, nseg, total, o, kvreg, acc);
  const float f = S_WAVE ? 1.f : P.scale;
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) {
    if (!key_ok[kb]) continue;
    float* dst;
    int64_t rowoff;
    if (K.kind == KIND_CLEAN) {
      dst = S_WAVE ? A.dv_clean : A.dk_clean;
      rowoff = (((int64_t)b * P.L + mysrc[kb]) * P.hkv + g) * D;
    } else {
      dst = S_WAVE ? A.dv_corr : A.dk_corr;
      rowoff = (((int64_t)b * P.n_corr_rows + mysrc[kb]) * P.hkv + g) * D;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        f32x4* pd = reinterpret_cast<f32x4*>(dst + rowoff + db * 32 + crow(i, hh));
        f32x4 cur4 = A.overwrite ? f32x4{0.f, 0.f, 0.f, 0.f} : *pd;
#pragma unroll
        for (int e = 0; e < 4; ++e) cur4[e] += f * acc[db][kb][i + e];
        *pd = cur4;
      }
  }
}

template <int D>
__device__ void dkdv_tile(const Plan& P, const DkdvArgs& A, DkdvSmem<D>& sm, int b, int g, int32_t ktile) {
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave % kPairs;  // which 64 keys of the tile
  int32_t kseg, koff;
  ktile_locate(P, ktile, &kseg, &koff);
  const KSeg K = P.k[kseg];
  const int32_t kvalid = min(kBKB, K.len - koff);  // valid keys in the tile
  const int32_t kt0 = K.t0 + koff;                 // first source row
  const int32_t kt1 = kt0 + kvalid;
  const int32_t c = K.c0 + koff;                   // compact start
  int32_t mysrc[kKB];
  bool key_ok[kKB];
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) {
    const int32_t key = kw * kKW + kb * 32 + ql;
    key_ok[kb] = key < kvalid;
    mysrc[kb] = key_ok[kb] ? kt0 + key : INT_MIN;
  }
  const LaneOff<D> o = lane_offsets<D, kWaves>(wave, lane);

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
  if (wave < kPairs)
    dkdv_role<D, true>(P, A, sm, K, b, g, c, kvalid, kt1, wave, kw, lane, ql, hh, mysrc, key_ok, nseg, total, o);
  else
    dkdv_role<D, false>(P, A, sm, K, b, g, c, kvalid, kt1, wave, kw, lane, ql, hh, mysrc, key_ok, nseg, total, o);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(const Plan P, const DkdvArgs A) {
  __shared__ DkdvSmem<D> sm;
  __shared__ int64_t item;
  // one work item from the XCD queues, longest first (plan.h); a spare
  // workgroup that finds every queue empty ends here
  if (threadIdx.x == 0) {
    int scan = 0;
    item = next_item_k(P, A.queue, kQueueStride, (int)(blockIdx.x % kXCD), &scan);
  }
  __syncthreads();
  const int64_t l = item;
  if (l < 0) return;
  const WgK wg = decode_item_k(P, l);
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
    hipLaunchKernelGGL(dkdv_kernel<128>, dim3(queue_grid(P.nwg_k)), dim3(kThreads), 0, s, P, a);
  else
    hipLaunchKernelGGL(dkdv_kernel<64>, dim3(queue_grid(P.nwg_k)), dim3(kThreads), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace bd
