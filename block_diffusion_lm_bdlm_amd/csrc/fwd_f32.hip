// fwd_f32.hip — forward of BDLM attention for fp32 inputs, on the fp32
// matrix cores.
//
// Same result as the bf16 forward (O_i = sum_j softmax_j(s_ij) v_j and
// LSE_i over the visible keys of the call; "CSBP 完全拆解", CP attention
// equation and the key/value set [K_b; K^clean_<b]), with every product in
// fp32: v_mfma_f32_32x32x2_f32 for S^T = K Q^T and O^T += V^T P^T, the
// softmax in fp32.
//
// A workgroup owns 32 query rows of one head and runs NW waves (8 at
// d = 64, 4 at d = 128) that split the rows' key walk (tiles of 64 keys)
// between them, wave w taking tiles w, w + NW, ...; each keeps its own
// running max, normaliser and O^T, and the partial results are merged
// exactly through LDS at the end (the same log-sum-exp rule the sharded form
// uses between calls).  The fp32 workload is small (a few thousand query
// rows), so rows are cut into 32-row workgroups and the walk into NW parts
// to fill the device.
//
// Operands come straight from the caller's tensors (L2-resident at these
// sizes): for a 32x32x2 product lane l supplies A[m = l % 32][k = l / 32]
// and B[k = l / 32][n = l % 32].  The contraction over d pairs d = s with
// d = s + D/2 (k = 0, 1), so a lane reads one half of a key row or query row
// contiguously; the contraction over keys pairs, in step s, key crow(s, 0)
// with key crow(s, 1) of a 32-key block -- the keys whose scores the lane
// already holds in register s of the S^T tile -- so P^T feeds the product as
// it comes out of the softmax.
#include "device.h"
#include "kernels.h"
#include "walk.h"

namespace bd {

namespace {

constexpr float kLn2f = 0.69314718055994530942f;
constexpr int kF32Rows = 32;   // query rows per workgroup
// waves sharing one workgroup's key walk: 8 at d = 64 (two per SIMD), 4 at
// d = 128, whose registers allow one wave per SIMD
template <int D>
constexpr int kF32Waves = D == 64 ? 8 : 4;

__device__ __forceinline__ f32x16 mfma_f32x2(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
struct F32MergeSmem {
  float m[kF32Waves<D>][kF32Rows];         // running max (raw scores) per wave and row
  float l[kF32Waves<D>][kF32Rows];         // normaliser relative to that max
  float o[kF32Waves<D>][D][kF32Rows + 1];  // O^T partial, unnormalised
};

// Source row of compact key cc of key segment K (clamped into the segment:
// keys past its end are masked by the caller).
__device__ __forceinline__ int64_t key_src(const KSeg& K, int32_t cc) {
  const int32_t last = K.c0 + K.len - 1;
  return (int64_t)K.t0 + ((cc < last ? cc : last) - K.c0);
}

template <int D>
__global__ __launch_bounds__(64 * kF32Waves<D>, 1) void fwd_f32_kernel(const Plan P, const FwdF32Args A) {
  constexpr int NW = kF32Waves<D>;
  static_assert(D % 32 == 0, "whole 32-column blocks of d");
  __shared__ F32MergeSmem<D> sm;
  constexpr int HD = D / 2;
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (batch, head, 128-row plan tile, 32-row quarter)
  int64_t idx = blockIdx.x;
  const int sub = (int)(idx % (kBQ / kF32Rows));
  idx /= kBQ / kF32Rows;
  const int32_t tile = (int32_t)(idx % P.ntiles);
  idx /= P.ntiles;
  const int h = (int)(idx % P.hq);
  const int b = (int)(idx / P.hq);
  const int g = h / P.G;
  const QSeg S = P.q[seg_of_tile(P, tile)];
  const int32_t r0 = (tile - S.tile0) * kBQ + sub * kF32Rows;
  const int32_t n = min(kF32Rows, S.nrows - r0);
  if (n <= 0) return;  // the whole workgroup: past the segment's last row
  const bool clean = S.kind == KIND_CLEAN;
  const int32_t rc = r0 + min(ql, n - 1);

  // this lane's half of its query row: B operands of S^T = K Q^T
  const TensorArg& QT = clean ? A.q_clean : A.q_corr;
  const float* qp = static_cast<const float*>(QT.p) + b * QT.bs + (int64_t)(S.src0 + rc) * QT.rs +
                    (int64_t)h * QT.hs + hh * HD;
  float qreg[HD];
#pragma unroll
  for (int s = 0; s < HD; s += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(qp + s);
    qreg[s] = x[0];
    qreg[s + 1] = x[1];
    qreg[s + 2] = x[2];
    qreg[s + 3] = x[3];
  }
  const RowBounds rb = row_bounds(P, S, rc);
  const KeyWalk w = keywalk_build(P, S, r0, r0 + n - 1);
  const float c2 = P.scale_log2;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  for (int32_t t = wave; t < w.total; t += NW) {
    int32_t c, ri;
    bool full;
    keywalk_at(w, t, &c, &ri, &full);
    const KSeg K = P.k[ri];
    const TensorArg& KT = K.kind == KIND_CLEAN ? A.k_clean : A.k_corr;
    const TensorArg& VT = K.kind == KIND_CLEAN ? A.v_clean : A.v_corr;
    const float* kbase = static_cast<const float*>(KT.p) + b * KT.bs + (int64_t)g * KT.hs;
    const float* vbase = static_cast<const float*>(VT.p) + b * VT.bs + (int64_t)g * VT.hs;
    // S^T for the two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float* kp = kbase + key_src(K, c + kb * 32 + ql) * KT.rs + hh * HD;
      float kfr[HD];
#pragma unroll
      for (int s = 0; s < HD; s += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(kp + s);
        kfr[s] = x[0];
        kfr[s + 1] = x[1];
        kfr[s + 2] = x[2];
        kfr[s + 3] = x[3];
      }
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < HD; ++s) acc = mfma_f32x2(kfr[s], qreg[s], acc);
      sacc[kb] = acc;
    }
    if (!full) {
      int32_t vlo, vhi;
      compact_range(K, rb, clean, &vlo, &vhi);
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
    const float m_new = fmaxf(m_run, mx);
    const float mc = (m_new == -INFINITY ? 0.f : m_new) * c2;
    const float alpha = m_run == m_new ? 1.f : __builtin_amdgcn_exp2f(m_run * c2 - mc);
    float pv[2][16];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[kb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c2, -mc));
        lsum += pv[kb][i];
      }
    l_run = l_run * alpha + lsum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    m_run = m_new;
    // O^T += V^T P^T: step s of block kb pairs keys crow(s, 0) and crow(s, 1)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const float* vp = vbase + key_src(K, c + kb * 32 + crow(s, hh)) * VT.rs + ql;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] = mfma_f32x2(vp[db * 32], pv[kb][s], oacc[db]);
      }
  }

  // merge the waves' partial results: the same log-sum-exp rule as
  // between the calls of the sharded form
  const float l_row = wave_sum32(l_run);
  if (hh == 0) {
    sm.m[wave][ql] = m_run;
    sm.l[wave][ql] = l_row;
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.o[wave][db * 32 + crow(i, hh)][ql] = oacc[db][i];
  __syncthreads();
  for (int e = tid; e < kF32Rows * D; e += 64 * NW) {
    const int r = e / D, dd = e % D;
    if (r >= n) continue;
    float m = -INFINITY;
#pragma unroll
    for (int x = 0; x < NW; ++x) m = fmaxf(m, sm.m[x][r]);
    float L = 0.f, o = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        const float a = sm.m[x][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((sm.m[x][r] - m) * c2);
        L += a * sm.l[x][r];
        o += a * sm.o[x][dd][r];
      }
    }
    const int32_t row = S.row0 + r0 + r;
    A.o[b * A.o_bs + (int64_t)row * A.o_rs + (int64_t)h * A.o_hs + dd] = L > 0.f ? o / L : 0.f;
    if (dd == 0)
      A.lse[((int64_t)b * P.R + row) * P.hq + h] = L > 0.f ? (m * c2 + __log2f(L)) * kLn2f : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const Plan& P, const FwdF32Args& a, hipStream_t s) {
  const int64_t nwg = (int64_t)P.batch * P.hq * P.ntiles * (kBQ / kF32Rows);
  if (nwg == 0) return hipSuccess;
  if (P.d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)nwg), dim3(64 * kF32Waves<128>), 0, s, P, a);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)nwg), dim3(64 * kF32Waves<64>), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace bd
