// merge.hip — exact log-sum-exp merge of a partial attention result into an
// accumulator, in fp32 ("CSBP 完全拆解", section "在线 softmax 合并：为什么分两段
// 算仍是同一个注意力", equations for m, w1, w2, O and z):
//   m = max(z_acc, z_part),  w = exp(z - m),
//   O = (w_acc O_acc + w_part O_part) / (w_acc + w_part),  z = m + log(w_acc + w_part).
// The empty result (O = 0, z = -inf) is the identity; two empty parts stay
// empty.  Bandwidth-bound: each lane moves 4 columns of one row.
#include "device.h"
#include "kernels.h"

namespace bd {

namespace {

__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs A) {
  const int per_row = A.d / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / per_row;
  if (row >= A.rows) return;
  const int col = (int)(gid % per_row) * 4;
  const float za = A.lse_acc[row], zp = A.lse_part[row];
  const float m = fmaxf(za, zp);
  f32x4 out = {0.f, 0.f, 0.f, 0.f};
  float z = -INFINITY;
  if (m != -INFINITY) {
    const float wa = __expf(za - m), wp = __expf(zp - m);
    const float inv = 1.f / (wa + wp);
    const f32x4 oa = *reinterpret_cast<const f32x4*>(A.o_acc + row * A.d + col);
    const f32x4 op = *reinterpret_cast<const f32x4*>(A.o_part + row * A.d + col);
    // an empty side has weight exactly 0, so its O (which is 0) is never read as NaN
    out = (oa * wa + op * wp) * inv;
    z = m + __logf(wa + wp);
  }
  *reinterpret_cast<f32x4*>(A.o_acc + row * A.d + col) = out;
  if (A.o_bf16) {
    const uint32_t lo = bf16_bits(out[0]) | ((uint32_t)bf16_bits(out[1]) << 16);
    const uint32_t hi = bf16_bits(out[2]) | ((uint32_t)bf16_bits(out[3]) << 16);
    *reinterpret_cast<uint2*>(A.o_bf16 + row * A.d + col) = make_uint2(lo, hi);
  }
  if (col == 0) A.lse_acc[row] = z;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const int64_t threads = a.rows * (a.d / 4);
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bd
