// pack.hip — layout kernels that feed the matrix-core kernels.
//
//  pack_k: gathers the call's key rows (clean token ranges, then the share's
//          packed corrupted rows) into one compact, zero-padded key space;
//          writes the layouts its consumer asks for: natural bf16 K,
//          natural fp16 K and V, transposed fp16 V^T.  The transposed copy is tiled: each tile of 64 rows is one contiguous [d][64] block
//          (so a consumer's tile is a single 16 KB read), and every aligned
//          group of 16 rows is in perm16 order, the order in which an MFMA C
//          tile delivers its rows as a B operand.
//  pack_q: the same for the share's query side of the backward (Q and dO,
//          natural fp16), plus log2-scaled LSE and D per row and each
//          row's visible key interval per key kind.  Unless the caller
//          gives D, it is formed here from the dO row being packed and the
//          final O: D_i = sum_t dO_i[t] O_i[t], the softmax backward's row
//          term, and stored for later calls.
// Both are bandwidth-bound copies.  The bf16 -> fp16 conversions are exact
// for values in the half range above its subnormals; a value outside the
// half range is clamped to it and raises the call's range flag.  pack_q
// also applies each row's probability scale 2^-c (row_pscale): dO and D are
// stored times 2^-c and log2 LSE minus c, so the backward kernels form
// P * 2^c, which stays out of fp16's subnormal range on long rows, while
// every product they accumulate keeps its value.
#include "device.h"
#include "kernels.h"

namespace bd {

namespace {

constexpr int kPT = 64;  // rows per packing block = rows per transposed tile
static_assert(kPT == kBK, "consumers read whole transposed key tiles");

template <int D>
struct __attribute__((aligned(16))) PackSmem {
  uint16_t b[kPT][D + 8];  // bf16 rows of V (16-byte aligned)
};

// bf16 -> fp16, clamped to the half range; `bad` records a value outside it.
__device__ inline _Float16 bf16_to_f16(uint16_t u, bool& bad) {
  float x = bf16_to_f32(u);
  bad |= !(fabsf(x) <= kHalfMax);
  if (fabsf(x) > kHalfMax) x = copysignf(kHalfMax, x);
  return (_Float16)x;
}

// Records an out-of-range conversion in the call's flag word (a plain
// vector store; every writer stores the same value).
__device__ inline void raise_flag(int32_t* flag, bool bad) {
  if (bad) *reinterpret_cast<volatile int32_t*>(flag) = 1;
}


// Writes the transposed, perm16-ordered fp16 tile [D][kPT] (contiguous) from LDS rows.
template <int D>
__device__ inline void store_transposed(const uint16_t (*rows)[D + 8], _Float16* out, int tid, bool& bad) {
  constexpr int ld = kPT;
  // each thread writes 8 consecutive slots (16 bytes) of one output row
  for (int ch = tid; ch < D * (kPT / 8); ch += 256) {
    const int d = ch / (kPT / 8), s0 = (ch % (kPT / 8)) * 8;
    f16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int slot = s0 + e;
      const int key = (slot & ~15) + perm16(slot & 15);
      v[e] = bf16_to_f16(rows[key][d], bad);
    }
    *reinterpret_cast<f16x8*>(out + (int64_t)d * ld + s0) = v;
  }
}

template <int D>
__global__ __launch_bounds__(256) void pack_k_kernel(const Plan P, const PackKArgs A) {
  __shared__ PackSmem<D> sm;
  const int tid = threadIdx.x;
  const int32_t c = blockIdx.x * kPT;
  const int g = blockIdx.y, b = blockIdx.z;
  // segment holding compact rows [c, c + kPT) (segments are kAlign-aligned)
  int32_t j = 0;
  while (j + 1 < P.nk && c >= P.k[j + 1].c0) ++j;
  const KSeg K = P.k[j];
  const TensorArg& KT = K.kind == KIND_CLEAN ? A.k_clean : A.k_corr;
  const TensorArg& VT = K.kind == KIND_CLEAN ? A.v_clean : A.v_corr;
  bool bad = false;
  for (int ch = tid; ch < kPT * (D / 8); ch += 256) {
    const int r = ch / (D / 8), dc = (ch % (D / 8)) * 8;
    const int32_t cc = c + r;
    u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (cc >= K.c0 && cc < K.c0 + K.len) {
      const int64_t src = K.t0 + (cc - K.c0);
      kv = ldg16(static_cast<const uint16_t*>(KT.p) + b * KT.bs + src * KT.rs + (int64_t)g * KT.hs + dc);
      vv = ldg16(static_cast<const uint16_t*>(VT.p) + b * VT.bs + src * VT.rs + (int64_t)g * VT.hs + dc);
    }
    const int64_t nat = ((int64_t)(b * P.hkv + g) * P.nkc + cc) * D + dc;
    if (A.kn) *reinterpret_cast<u32x4*>(A.kn + nat) = kv;
    if (A.kh) *reinterpret_cast<f16x8*>(A.kh + nat) = bf16x8_to_f16x8(kv, 1.f, bad);
    if (A.vh) *reinterpret_cast<f16x8*>(A.vh + nat) = bf16x8_to_f16x8(vv, 1.f, bad);
    *reinterpret_cast<u32x4*>(&sm.b[r][dc]) = vv;
  }
  if (A.vt) {
    __syncthreads();
    const int64_t tb = (int64_t)(b * P.hkv + g) * D * P.nkc + (int64_t)c * D;  // tile c / kPT
    store_transposed<D>(sm.b, A.vt + tb, tid, bad);
  }
  raise_flag(A.flag, bad);
}

// OM: how D = rowsum(dO * O) is obtained: kDeltaGiven (read from A.delta),
// kOBf16 / kOF32 (formed here from the final O in that dtype).  A template
// parameter, so the load phase has no branch.
enum { kDeltaGiven = 0, kOBf16 = 1, kOF32 = 2 };
template <int D, int OM>
__global__ __launch_bounds__(256) void pack_q_kernel(const Plan P, const PackQArgs A) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row: consecutive lanes of one wave
  static_assert(kPT * CPR % 256 == 0 && 64 % CPR == 0, "every lane runs every chunk loop; rows within a wave");
  __shared__ float dsum[kPT];
  const int tid = threadIdx.x;
  // the head is the fastest grid index: workgroups running together read
  // the heads of the same rows, whole row spans of the [rows, heads, d] inputs
  // (1.58 -> 1.35 ms at 64K, against row tiles of one head first).  Row
  // tiles stride by gridDim.y (capped at 65535 by the launch).
  const int h = blockIdx.x, b = blockIdx.z;
  for (int64_t ty = blockIdx.y; ty < P.nqc / kPT; ty += gridDim.y) {
    const int32_t c = (int32_t)(ty * kPT);  // compact query row
    const int32_t tile = c / kBQ;
    const QSeg S = P.q[seg_of_tile(P, tile)];
    const int32_t rbase = c - S.tile0 * kBQ;  // row within segment of compact row c
    const TensorArg& QT = S.kind == KIND_CLEAN ? A.q_clean : A.q_corr;
    const int64_t hb = (int64_t)(b * P.hq + h);
    // All loads of the thread's chunks are issued first, with the row index
    // clamped into the segment (it holds at least one row) and the values of
    // rows past its end zeroed afterwards: loads under a branch would each be
    // waited for before the next.
    constexpr int kIter = kPT * CPR / 256;
    const int32_t last = S.nrows - 1;
    u32x4 qv[kIter], dv[kIter];
    u32x4 ob[OM == kOBf16 ? kIter : 1];
    f32x4 o0[OM == kOF32 ? kIter : 1], o1[OM == kOF32 ? kIter : 1];
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int ch = tid + 256 * it;
      const int r = ch / CPR, dc = (ch % CPR) * 8;
      const int32_t rr = min(rbase + r, last);
      qv[it] = ldg16(static_cast<const uint16_t*>(QT.p) + b * QT.bs + (int64_t)(S.src0 + rr) * QT.rs +
                     (int64_t)h * QT.hs + dc);
      dv[it] = ldg16(static_cast<const uint16_t*>(A.d_o.p) + b * A.d_o.bs + (int64_t)(S.row0 + rr) * A.d_o.rs +
                     (int64_t)h * A.d_o.hs + dc);
      if constexpr (OM != kDeltaGiven) {
        const int64_t oo = b * A.o.bs + (int64_t)(S.row0 + rr) * A.o.rs + (int64_t)h * A.o.hs + dc;
        if constexpr (OM == kOF32) {
          o0[it] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(A.o.p) + oo);
          o1[it] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(A.o.p) + oo + 4);
        } else {
          ob[it] = ldg16(static_cast<const uint16_t*>(A.o.p) + oo);
        }
      }
    }
    bool bad = false;
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int ch = tid + 256 * it;
      const int r = ch / CPR, dc = (ch % CPR) * 8;
      if (rbase + r > last) {
        qv[it] = u32x4{0, 0, 0, 0};
        dv[it] = u32x4{0, 0, 0, 0};
      }
      // this row's probability scale: dO is stored times 2^-c
      const int32_t cs = row_pscale(row_nkeys(row_bounds(P, S, min(rbase + r, last))));
      const float dscale = __int_as_float((127 - cs) << 23);
      float dd = 0.f;  // this chunk's part of D
      if constexpr (OM != kDeltaGiven) {
        float ov[8];
        if constexpr (OM == kOF32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ov[e] = o0[it][e];
            ov[e + 4] = o1[it][e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) ov[e] = bf16_to_f32((uint16_t)(ob[it][e >> 1] >> (16 * (e & 1))));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dd = fmaf(bf16_to_f32((uint16_t)(dv[it][e >> 1] >> (16 * (e & 1)))), ov[e], dd);
        // sum over the row's CPR lanes
#pragma unroll
        for (int m = CPR / 2; m >= 1; m >>= 1) dd += __shfl_xor(dd, m, CPR);
        if (dc == 0) dsum[r] = dd;
      }
      const int64_t nat = (hb * P.nqc + c + r) * D + dc;
      *reinterpret_cast<f16x8*>(A.qh + nat) = bf16x8_to_f16x8(qv[it], 1.f, bad);
      *reinterpret_cast<f16x8*>(A.doh + nat) = bf16x8_to_f16x8(dv[it], dscale, bad);
    }
    raise_flag(A.flag, bad);
    __syncthreads();  // dsum
    if (tid < kPT) {
      const int32_t rr = rbase + tid;
      float l2 = INFINITY, dd = 0.f;
      if (rr < S.nrows) {
        const int64_t idx = ((int64_t)b * P.R + S.row0 + rr) * P.hq + h;
        const float lse = A.lse[idx];
        const int32_t cs = row_pscale(row_nkeys(row_bounds(P, S, rr)));
        // a row that sees no key (LSE = -inf) has O = 0 and no gradient: +inf
        // makes every recomputed probability exp2(s - inf) vanish.  Otherwise
        // log2 LSE - c, so the kernels' exp2(s log2 e - lse2) is P * 2^c.
        l2 = lse == -INFINITY ? INFINITY : lse * 1.4426950408889634f - (float)cs;
        if constexpr (OM == kDeltaGiven) {
          dd = A.delta[idx];
        } else {
          dd = dsum[tid];
          A.delta[idx] = dd;
        }
        dd *= __int_as_float((127 - cs) << 23);  // D * 2^-c, like the row's dO
      }
      A.lse2[hb * P.nqc + c + tid] = l2;
      A.dc[hb * P.nqc + c + tid] = dd;
      if (h == 0 && b == 0) {  // per compact row, the same for every head and batch
        int32_t v[4] = {0, 0, 0, 0};
        if (rr < S.nrows) {
          const RowBounds rb = row_bounds(P, S, rr);
          v[0] = rb.lo_clean;
          v[1] = rb.hi_clean;
          if (S.kind == KIND_CORR) {
            v[2] = rb.lo_loc;
            v[3] = rb.hi_loc;
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) A.vis[(int64_t)k * P.nqc + c + tid] = v[k];
      }
    }
    __syncthreads();  // the next row tile reuses dsum
  }
}

// Zeroes the range flag and the work-queue heads of a workspace header.
__global__ void flag_clear_kernel(int32_t* header) {
  const int t = threadIdx.x;
  volatile int32_t* h = header;
  if (t == 0) h[0] = 0;
  if (t < 3 * kXCD) h[kQueueFwd + (t / kXCD) * (kQueueDq - kQueueFwd) + (t % kXCD) * kQueueStride] = 0;
}

}  // namespace

hipError_t launch_flag_clear(int32_t* header, hipStream_t s) {
  static_assert(kQueueDq - kQueueFwd == kQueueDkdv - kQueueDq && kQueueDkdv + kXCD * kQueueStride <= kHeaderWords,
                "three equally spaced queue-head blocks inside the header");
  hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(64), 0, s, header);
  return hipGetLastError();
}

hipError_t launch_pack_k(const Plan& P, const PackKArgs& a, hipStream_t s) {
  if (P.nkc == 0) return hipSuccess;
  dim3 grid(P.nkc / kPT, P.hkv, P.batch);
  if (P.d == 128)
    hipLaunchKernelGGL(pack_k_kernel<128>, grid, dim3(256), 0, s, P, a);
  else
    hipLaunchKernelGGL(pack_k_kernel<64>, grid, dim3(256), 0, s, P, a);
  return hipGetLastError();
}

hipError_t launch_pack_q(const Plan& P, const PackQArgs& a, hipStream_t s) {
  if (P.nqc == 0) return hipSuccess;
  const int64_t tiles = P.nqc / kPT;
  dim3 grid(P.hq, (unsigned)(tiles < 65535 ? tiles : 65535), P.batch);
  const int om = a.delta_ready ? kDeltaGiven : (a.o_f32 ? kOF32 : kOBf16);
#define BD_PACK_Q(DD, OMV) hipLaunchKernelGGL((pack_q_kernel<DD, OMV>), grid, dim3(256), 0, s, P, a)
  if (P.d == 128) {
    if (om == kDeltaGiven) BD_PACK_Q(128, kDeltaGiven);
    else if (om == kOF32) BD_PACK_Q(128, kOF32);
    else BD_PACK_Q(128, kOBf16);
  } else {
    if (om == kDeltaGiven) BD_PACK_Q(64, kDeltaGiven);
    else if (om == kOF32) BD_PACK_Q(64, kOF32);
    else BD_PACK_Q(64, kOBf16);
  }
#undef BD_PACK_Q
  return hipGetLastError();
}

}  // namespace bd
