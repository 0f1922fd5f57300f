// vocab_rows.hip — the hand-written kernels of the streaming vocabulary loss
// ([P3] Turbo-dLLM project page, "Library" section, "Vocabulary loss" rows):
// the fused per-row pass over one chunk of fp32 logits, the gather of
// listed hidden rows into a packed chunk, the scatter of the chunk's dh
// rows back, the transposed copy of the head and the fixed-order sum of
// the per-row losses.
//
// Per-row pass: rows_onchip_kernel (below) reads each row once and serves
// vocabularies up to kOnChipSubMax sub-blocks; larger ones take the
// two-pass kernel (one workgroup per row at a time, rows strided over a
// grid sized to keep the rows in flight within the chip's caches):
//   pass 1  one read of the row: running (max, sum of exp) per thread in
//           the base-2 domain, one rescale per group of loads, then a
//           workgroup merge of the (max, sum) pairs into lse;
//   pass 2  a second read of the row: g_v = w (exp(s_v - lse) - [v == y]),
//           rounded to bf16 and written over the first half of the same
//           row, so the gradient GEMM reads it with twice the fp32 pitch.
// The in-place write is safe because each group's writes land in bytes
// that every thread of the workgroup has already read: group k reads the
// float4 indices [kUT, (k+1)UT) and writes bf16 over the float4 indices
// [kUT/2, (k+1)UT/2); one barrier between a group's loads and its stores
// orders them.  The logit at the target is read before pass 2 begins.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vocab_kernels.h"

namespace bdvocab {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x with the hardware's v_exp_f32: results below 2^-126 flush to zero
// (they are far below what the fp32 sums and the bf16 gradient keep), and
// exp2(-inf) = 0.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a;  // round to nearest even
  const __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Merge (m, s) with (m2, s2): base-2 log-sum-exp pairs; m = -inf means empty.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * ex2(m - mn) + s2 * ex2(m2 - mn);
  m = mn;
}

template <int T, int U>
__global__ __launch_bounds__(T) void rows_kernel(RowsArgs a) {
  static_assert(T % 64 == 0 && T <= 1024, "workgroup size");
  constexpr int kWaves = T / 64;
  __shared__ float red_m[kWaves], red_s[kWaves];
  __shared__ float row_lse2, row_sy;
  const int tid = threadIdx.x;
  const int64_t n4 = a.ld / 4;  // float4 per row (ld is a multiple of 4)
  const int64_t per_group = (int64_t)U * T;
  const int64_t groups = (n4 + per_group - 1) / per_group;

  for (int64_t r = blockIdx.x; r < a.n; r += gridDim.x) {
    float* srow = a.s + r * a.ld;
    const int32_t y = a.targets[r];
    const bool valid = y >= 0 && y < a.V;
    const float w = valid ? (a.weights ? a.weights[r] : 1.f) : 0.f;
    if (tid == 0) row_sy = valid ? srow[y] : 0.f;

    // pass 1: running base-2 max and sum of exp per thread
    float m = -INFINITY, sum = 0.f;
    for (int64_t g = 0; g < groups; ++g) {
      float4 x[U];
      float gm = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = g * per_group + (int64_t)u * T + tid;
        const float4 v = reinterpret_cast<const float4*>(srow)[j < n4 ? j : n4 - 1];  // clamped, unconditional
        const int64_t e = 4 * j;
        x[u].x = e + 0 < a.V ? v.x * kLog2e : -INFINITY;
        x[u].y = e + 1 < a.V ? v.y * kLog2e : -INFINITY;
        x[u].z = e + 2 < a.V ? v.z * kLog2e : -INFINITY;
        x[u].w = e + 3 < a.V ? v.w * kLog2e : -INFINITY;
        gm = fmaxf(gm, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
      }
      if (gm == -INFINITY) continue;
      const float mn = fmaxf(m, gm);
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u)
        acc += ex2(x[u].x - mn) + ex2(x[u].y - mn) + ex2(x[u].z - mn) + ex2(x[u].w - mn);
      sum = sum * ex2(m - mn) + acc;  // exp2(-inf) = 0 on the first group
      m = mn;
    }
    // workgroup merge of (m, sum)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float m2 = __shfl_xor(m, off);
      const float s2 = __shfl_xor(sum, off);
      lse_merge(m, sum, m2, s2);
    }
    if ((tid & 63) == 0) {
      red_m[tid >> 6] = m;
      red_s[tid >> 6] = sum;
    }
    __syncthreads();
    if (tid == 0) {
      float mm = red_m[0], ss = red_s[0];
      for (int i = 1; i < kWaves; ++i) lse_merge(mm, ss, red_m[i], red_s[i]);
      const float lse2 = mm + log2f(ss);
      row_lse2 = lse2;
      const float lse = lse2 * kLn2;
      if (a.lse) a.lse[r] = lse;
      a.loss[r] = valid ? w * (lse - row_sy) : 0.f;
    }
    __syncthreads();
    const float lse2 = row_lse2;

    // pass 2: g = w (p - onehot) in bf16 over the first half of the row
    uint2* grow = reinterpret_cast<uint2*>(srow);
    for (int64_t g = 0; g < groups; ++g) {
      float4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = g * per_group + (int64_t)u * T + tid;
        x[u] = reinterpret_cast<const float4*>(srow)[j < n4 ? j : n4 - 1];  // clamped, unconditional
      }
      __syncthreads();  // every read of this group is done before any write
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = g * per_group + (int64_t)u * T + tid;
        if (j >= n4) continue;
        const int64_t e = 4 * j;
        float gv[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = e + i < a.V ? ex2(fmaf(gv[i], kLog2e, -lse2)) : 0.f;
          if (e + i == y) p -= 1.f;
          gv[i] = w * p;
        }
        grow[j] = make_uint2(pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]));
      }
    }
    __syncthreads();  // the next row reuses the shared slots
  }
}

// Single-read per-row pass for rows of up to kOnChipMax logits: each thread
// keeps its share of the row on chip while the row's lse is formed, so the
// fp32 row is read once.  Thread t owns NSUB sub-blocks of Q float4 loads
// (float4 index (k Q + q) T + t for sub-block k, load q: every load
// instruction of the workgroup reads consecutive 16-byte pieces).  Per
// sub-block it keeps e = exp2(x - m_k) in fp16 (x the base-2 logit, m_k the
// sub-block's own max, so every e lies in [0, 1]) and adds the fp32 e to
// its running sum.  After the workgroup merge gives lse2, the gradient is
// g = w (e exp2(m_k - lse2) - [v == y]), written in bf16 over the first
// half of the row: every read of the row has completed before the barrier
// that precedes the writes.  fp16 keeps 11 bits of e (bf16 would keep 8);
// values below 2^-24 of their sub-block's max flush to zero, far below the
// bf16 rounding of the result.
// Sub-blocks 0 .. NREG-1 stay in registers, NREG .. NREG+NLDS-1 in LDS
// (the register file alone holds four sub-blocks of eight loads without
// spilling at 512 threads).
template <int T, int Q, int NREG, int NLDS>
__global__ __launch_bounds__(T) void rows_onchip_kernel(RowsArgs a) {
  static_assert(T % 64 == 0 && T <= 1024, "workgroup size");
  constexpr int kWaves = T / 64;
  constexpr int NSUB = NREG + NLDS;
  __shared__ float red_m[kWaves], red_s[kWaves];
  __shared__ float row_lse2, row_sy;
  __shared__ uint2 spill[NLDS > 0 ? NLDS : 1][Q][T];  // packed fp16 quads of the LDS sub-blocks
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const int tid = threadIdx.x;
  const int n4 = (int)(a.ld / 4);  // float4 per row; ld < 2^31 for this kernel
  const int V = a.V;

  for (int64_t r = blockIdx.x; r < a.n; r += gridDim.x) {
    float* srow = a.s + r * a.ld;
    const float4* row4 = reinterpret_cast<const float4*>(srow);
    const int32_t y = a.targets[r];
    const bool valid = y >= 0 && y < V;
    const float w = valid ? (a.weights ? a.weights[r] : 1.f) : 0.f;
    if (tid == 0) row_sy = valid ? srow[y] : 0.f;

    uint32_t e16[NREG > 0 ? NREG : 1][Q][2];  // packed fp16 pairs of the register sub-blocks
    float mk[NSUB];
    float m = -INFINITY, sum = 0.f;
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
      float4 x[Q];
      float gm = -INFINITY;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int j = (k * Q + q) * T + tid;
        // unconditional load of a clamped index (a branch around the load
        // would make the compiler wait for each load before the next)
        const float4 v = row4[j < n4 ? j : n4 - 1];
        const int e = 4 * j;
        x[q].x = e + 0 < V ? v.x * kLog2e : -INFINITY;
        x[q].y = e + 1 < V ? v.y * kLog2e : -INFINITY;
        x[q].z = e + 2 < V ? v.z * kLog2e : -INFINITY;
        x[q].w = e + 3 < V ? v.w * kLog2e : -INFINITY;
        gm = fmaxf(gm, fmaxf(fmaxf(x[q].x, x[q].y), fmaxf(x[q].z, x[q].w)));
      }
      const float sh = gm == -INFINITY ? 0.f : gm;  // an all-pad sub-block keeps e = 0
      mk[k] = sh;
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float ex = ex2(x[q].x - sh), ey = ex2(x[q].y - sh);
        const float ez = ex2(x[q].z - sh), ew = ex2(x[q].w - sh);
        acc += (ex + ey) + (ez + ew);
        uint32_t p0 = __builtin_bit_cast(uint32_t, h2{(_Float16)ex, (_Float16)ey});
        uint32_t p1 = __builtin_bit_cast(uint32_t, h2{(_Float16)ez, (_Float16)ew});
        // pin the packed words here: otherwise the compiler keeps the fp32
        // values alive across the reduction and converts them later
        asm volatile("" : "+v"(p0), "+v"(p1));
        if constexpr (NREG > 0) {
          if (k < NREG) {
            e16[k < NREG ? k : 0][q][0] = p0;
            e16[k < NREG ? k : 0][q][1] = p1;
          }
        }
        if (k >= NREG) spill[k >= NREG ? k - NREG : 0][q][tid] = make_uint2(p0, p1);
      }
      if (gm != -INFINITY) lse_merge(m, sum, gm, acc);
      // keep the next sub-block's loads below this one: only one
      // sub-block of fp32 values is live, the rest stay as fp16
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float m2 = __shfl_xor(m, off);
      const float s2 = __shfl_xor(sum, off);
      lse_merge(m, sum, m2, s2);
    }
    if ((tid & 63) == 0) {
      red_m[tid >> 6] = m;
      red_s[tid >> 6] = sum;
    }
    __syncthreads();
    if (tid == 0) {
      float mm = red_m[0], ss = red_s[0];
      for (int i = 1; i < kWaves; ++i) lse_merge(mm, ss, red_m[i], red_s[i]);
      const float lse2 = mm + log2f(ss);
      row_lse2 = lse2;
      const float lse = lse2 * kLn2;
      if (a.lse) a.lse[r] = lse;
      a.loss[r] = valid ? w * (lse - row_sy) : 0.f;
    }
    __syncthreads();  // also: every read of this row has completed
    const float lse2 = row_lse2;

    // the write phase recomputes its indices from an opaque copy of the
    // thread index, so nothing index-shaped stays live across the pass
    int tw = tid;
    asm volatile("" : "+v"(tw));
    uint2* grow = reinterpret_cast<uint2*>(a.s + r * a.ld);
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
      const float c = w * ex2(mk[k] - lse2);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int j = (k * Q + q) * T + tw;
        if (j >= n4) continue;
        const int e = 4 * j;
        uint32_t w0, w1;
        if (k < NREG) {
          w0 = e16[k < NREG ? k : 0][q][0];
          w1 = e16[k < NREG ? k : 0][q][1];
        } else {
          const uint2 u = spill[k >= NREG ? k - NREG : 0][q][tw];
          w0 = u.x;
          w1 = u.y;
        }
        const h2 p01 = __builtin_bit_cast(h2, w0);
        const h2 p23 = __builtin_bit_cast(h2, w1);
        float g0 = (float)p01.x * c, g1 = (float)p01.y * c;
        float g2 = (float)p23.x * c, g3 = (float)p23.y * c;
        if (e + 0 == y) g0 -= w;
        if (e + 1 == y) g1 -= w;
        if (e + 2 == y) g2 -= w;
        if (e + 3 == y) g3 -= w;
        grow[j] = make_uint2(pack_bf16x2(g0, g1), pack_bf16x2(g2, g3));
      }
    }
    __syncthreads();  // the next row reuses the shared slots
  }
}

// Copy rows idx[r] of h (bf16, pitch h_stride) into a packed [n, d] chunk;
// 16-byte pieces, d % 8 == 0.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int pieces = a.d / 8;
  const int64_t total = a.n * pieces;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / pieces;
    const int c = (int)(i - r * pieces);
    const int64_t src = (int64_t)a.rows[r] * a.h_stride + 8 * c;
    reinterpret_cast<uint4*>(a.out + r * a.d)[c] = *reinterpret_cast<const uint4*>(a.h + src);
  }
}

// Copy the packed [n, d] dh chunk (element size es = 2 or 4) to rows idx[r]
// of dh (pitch dh_stride elements).
__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
  const int pieces = a.d * a.es / 16;
  const int64_t total = a.n * pieces;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / pieces;
    const int c = (int)(i - r * pieces);
    const int64_t dst = ((int64_t)a.rows[r] * a.dh_stride) * a.es + 16 * (int64_t)c;
    *reinterpret_cast<uint4*>(a.dh + dst) = reinterpret_cast<const uint4*>(a.in + r * (int64_t)a.d * a.es)[c];
  }
}

// Transposed copy of a 16-bit matrix: src [rows, cols] -> dst [cols, rows]
// (the head W [V, d] -> [d, V] for the gradient GEMM; a chunk's bf16 logit
// gradient and hidden rows for the head GEMM).  One 64 x 64 tile per
// workgroup through LDS: 16-byte loads along the source rows, 16-byte
// stores along the destination rows; the LDS tile's row pitch is padded by
// two elements so that the column reads of the store phase spread over the
// banks.  Pad columns of dst past `rows` receive values that no reader uses.
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
  __shared__ uint16_t tile[64][66];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
  // column tiles stride by gridDim.y, which the launch caps at 65535
  for (int64_t c0 = (int64_t)blockIdx.y * 64; c0 < a.cols; c0 += (int64_t)gridDim.y * 64) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int piece = tid + 256 * k;  // 64 source rows x 8 pieces of 8
      const int r = piece >> 3, c = (piece & 7) * 8;
      const int64_t row = r0 + r;
      if (row < a.rows && c0 + c < a.cols) {
        const uint4 x = *reinterpret_cast<const uint4*>(a.src + row * a.src_pitch + c0 + c);
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&x);
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[r][c + i] = e[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int piece = tid + 256 * k;  // 64 destination rows (source columns) x 8 pieces of 8
      const int r = piece >> 3, c = (piece & 7) * 8;
      const int64_t col = c0 + r;
      const int64_t row = r0 + c;
      if (col < a.cols && row < a.rows) {
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = tile[c + i][r];
        *reinterpret_cast<uint4*>(a.dst + col * a.dst_pitch + row) = *reinterpret_cast<const uint4*>(e);
      }
    }
    __syncthreads();  // the next column tile reuses the LDS tile
  }
}

// Sum of n per-row losses in a fixed order: thread t adds rows t, t + 1024,
// ... in double, then a fixed tree over the threads.
__global__ __launch_bounds__(1024) void loss_sum_kernel(const float* loss, int64_t n, float* out) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) acc += (double)loss[i];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = (float)part[0];
}

}  // namespace

hipError_t launch_rows(const RowsArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  constexpr int64_t kSub = (int64_t)kOnChipThreads * kOnChipLoads * 4;  // logits per sub-block of the workgroup
  const int64_t nsub = (a.ld + kSub - 1) / kSub;
  if (nsub <= kOnChipSubMax) {
    const int grid = (int)(a.n < kOnChipInFlight ? a.n : kOnChipInFlight);
    switch (nsub) {
#define BDV_ONCHIP(NS, NR, NL)                                                                              \
  case NS:                                                                                                  \
    hipLaunchKernelGGL((rows_onchip_kernel<kOnChipThreads, kOnChipLoads, NR, NL>), dim3(grid),               \
                       dim3(kOnChipThreads), 0, s, a);                                                      \
    return hipGetLastError();
      BDV_ONCHIP(1, 1, 0) BDV_ONCHIP(2, 2, 0) BDV_ONCHIP(3, 3, 0) BDV_ONCHIP(4, 4, 0)
      BDV_ONCHIP(5, 4, 1) BDV_ONCHIP(6, 4, 2) BDV_ONCHIP(7, 4, 3) BDV_ONCHIP(8, 4, 4)
#undef BDV_ONCHIP
      default: break;
    }
  }
  const int grid = (int)(a.n < kRowsInFlight ? a.n : kRowsInFlight);
  hipLaunchKernelGGL((rows_kernel<kRowThreads, kRowGroup>), dim3(grid), dim3(kRowThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const int64_t total = a.n * (a.d / 8);
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const int64_t total = a.n * (a.d * a.es / 16);
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(scatter_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s) {
  if (a.rows <= 0 || a.cols <= 0) return hipSuccess;
  const int64_t ct = (a.cols + 63) / 64;
  const dim3 grid((unsigned)((a.rows + 63) / 64), (unsigned)(ct < 65535 ? ct : 65535));
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_loss_sum(const float* loss, int64_t n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(loss_sum_kernel, dim3(1), dim3(1024), 0, s, loss, n, out);
  return hipGetLastError();
}

}  // namespace bdvocab
