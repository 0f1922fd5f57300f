// pack.hip — layout kernels that feed the matrix-core kernels.
//
//  pack_k: gathers the call's key rows (clean token ranges, then the share's
//          packed corrupted rows) into one compact, zero-padded key space;
//          writes the layouts its consumer asks for: natural bf16 K/V,
//          natural fp16 K, transposed fp16 V^T.  The transposed copy is tiled: each tile of 64 rows is one contiguous [d][64] block
//          (so a consumer's tile is a single 16 KB read), and every aligned
//          group of 16 rows is in perm16 order, the order in which an MFMA C
//          tile delivers its rows as a B operand.
//  pack_q: the same for the share's query side of the backward (Q, dO,
//          natural bf16 and natural fp16), plus log2-scaled LSE and delta
//          per row and each row's visible key interval per key kind.
//  delta:  D_i = sum_t dO_i[t] O_i[t], the softmax backward's row term.
// All three are bandwidth-bound copies; none changes a value except the
// bf16 -> fp16 conversions (exact for values in the half range and above
// its subnormals).
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

__device__ inline _Float16 bf16_to_f16(uint16_t u) { return (_Float16)bf16_to_f32(u); }


// Writes the transposed, perm16-ordered fp16 tile [D][kPT] (contiguous) from LDS rows.
template <int D>
__device__ inline void store_transposed(const uint16_t (*rows)[D + 8], _Float16* out, int tid) {
  constexpr int ld = kPT;
  // each thread writes 8 consecutive slots (16 bytes) of one output row
  for (int ch = tid; ch < D * (kPT / 8); ch += 256) {
    const int d = ch / (kPT / 8), s0 = (ch % (kPT / 8)) * 8;
    f16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int slot = s0 + e;
      const int key = (slot & ~15) + perm16(slot & 15);
      v[e] = bf16_to_f16(rows[key][d]);
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
    if (A.vn) *reinterpret_cast<u32x4*>(A.vn + nat) = vv;
    if (A.kh) *reinterpret_cast<f16x8*>(A.kh + nat) = bf16x8_to_f16x8(kv);
    *reinterpret_cast<u32x4*>(&sm.b[r][dc]) = vv;
  }
  if (A.vt) {
    __syncthreads();
    const int64_t tb = (int64_t)(b * P.hkv + g) * D * P.nkc + (int64_t)c * D;  // tile c / kPT
    store_transposed<D>(sm.b, A.vt + tb, tid);
  }
}

template <int D>
__global__ __launch_bounds__(256) void pack_q_kernel(const Plan P, const PackQArgs A) {
  const int tid = threadIdx.x;
  const int32_t c = blockIdx.x * kPT;  // compact query row
  const int h = blockIdx.y, b = blockIdx.z;
  const int32_t tile = c / kBQ;
  const QSeg S = P.q[seg_of_tile(P, tile)];
  const int32_t rbase = c - S.tile0 * kBQ;  // row within segment of compact row c
  const TensorArg& QT = S.kind == KIND_CLEAN ? A.q_clean : A.q_corr;
  const int64_t hb = (int64_t)(b * P.hq + h);
  for (int ch = tid; ch < kPT * (D / 8); ch += 256) {
    const int r = ch / (D / 8), dc = (ch % (D / 8)) * 8;
    const int32_t rr = rbase + r;
    u32x4 qv = {0, 0, 0, 0}, dv = {0, 0, 0, 0};
    if (rr < S.nrows) {
      qv = ldg16(static_cast<const uint16_t*>(QT.p) + b * QT.bs + (int64_t)(S.src0 + rr) * QT.rs +
                 (int64_t)h * QT.hs + dc);
      dv = ldg16(static_cast<const uint16_t*>(A.d_o.p) + b * A.d_o.bs + (int64_t)(S.row0 + rr) * A.d_o.rs +
                 (int64_t)h * A.d_o.hs + dc);
    }
    const int64_t nat = (hb * P.nqc + c + r) * D + dc;
    *reinterpret_cast<u32x4*>(A.qn + nat) = qv;
    *reinterpret_cast<u32x4*>(A.don + nat) = dv;
    *reinterpret_cast<f16x8*>(A.qh + nat) = bf16x8_to_f16x8(qv);
    *reinterpret_cast<f16x8*>(A.doh + nat) = bf16x8_to_f16x8(dv);
  }
  if (tid < kPT) {
    const int32_t rr = rbase + tid;
    float l2 = INFINITY, dd = 0.f;
    if (rr < S.nrows) {
      const int64_t idx = ((int64_t)b * P.R + S.row0 + rr) * P.hq + h;
      const float lse = A.lse[idx];
      // a row that sees no key (LSE = -inf) has O = 0 and no gradient: +inf
      // makes every recomputed probability exp2(s - inf) vanish.
      l2 = lse == -INFINITY ? INFINITY : lse * 1.4426950408889634f;
      dd = A.delta[idx];
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
}

// D_i = dO_i . O_i: 16 lanes per (batch, row, head), 8 elements per lane.
__global__ __launch_bounds__(256) void delta_kernel(const Plan P, const DeltaArgs A, int64_t nrows) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int sub = threadIdx.x & 15;
  const int64_t r = gid >> 4;
  float acc = 0.f;
  const int per = P.d / 16;
  if (r < nrows) {
    const int h = (int)(r % P.hq);
    const int64_t rest = r / P.hq;
    const int64_t row = rest % P.R, b = rest / P.R;
    const uint16_t* dop = static_cast<const uint16_t*>(A.d_o.p) + b * A.d_o.bs + row * A.d_o.rs +
                          (int64_t)h * A.d_o.hs + sub * per;
    if (A.o_f32) {
      const float* op = static_cast<const float*>(A.o.p) + b * A.o.bs + row * A.o.rs + (int64_t)h * A.o.hs +
                        sub * per;
      for (int t = 0; t < per; ++t) acc = fmaf(bf16_to_f32(dop[t]), op[t], acc);
    } else {
      const uint16_t* op = static_cast<const uint16_t*>(A.o.p) + b * A.o.bs + row * A.o.rs +
                           (int64_t)h * A.o.hs + sub * per;
      for (int t = 0; t < per; ++t) acc = fmaf(bf16_to_f32(dop[t]), bf16_to_f32(op[t]), acc);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (r < nrows && sub == 0) A.delta[r] = acc;
}

}  // namespace

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
  dim3 grid(P.nqc / kPT, P.hq, P.batch);
  if (P.d == 128)
    hipLaunchKernelGGL(pack_q_kernel<128>, grid, dim3(256), 0, s, P, a);
  else
    hipLaunchKernelGGL(pack_q_kernel<64>, grid, dim3(256), 0, s, P, a);
  return hipGetLastError();
}

hipError_t launch_delta(const Plan& P, const DeltaArgs& a, hipStream_t s) {
  const int64_t nrows = (int64_t)P.batch * P.R * P.hq;
  if (nrows == 0) return hipSuccess;
  const int64_t blocks = (nrows * 16 + 255) / 256;
  hipLaunchKernelGGL(delta_kernel, dim3((unsigned)blocks), dim3(256), 0, s, P, a, nrows);
  return hipGetLastError();
}

}  // namespace bd
