// kernels.h — argument blocks and launchers of the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace bd {

struct TensorArg {
  const void* p;
  int64_t bs, rs, hs;  // strides in elements; head dim contiguous
};

// ---------------------------------------------------------------- packing
// Compact key space: the call's key segments back to back, each starting at
// a multiple of kAlign, zero padded.  Natural layouts are [batch][hkv][nkc][d]
// (bf16, or fp16 for kh); transposed ones fp16 [batch][hkv][nkc/64][d][64]
// (tiles of 64 rows, each contiguous) with perm16 groups.
struct PackKArgs {
  TensorArg k_clean, v_clean, k_corr, v_corr;  // bf16
  uint16_t* kn;   // natural K (nullable)
  uint16_t* vn;   // natural V (nullable)
  _Float16* kh;   // natural K in fp16 (nullable)
  _Float16* vt;   // transposed V (nullable)
};

// Compact query space: the share's query segments back to back, segment s
// at rows [tile0 * kBQ, (tile0 + ntiles) * kBQ), zero padded.
struct PackQArgs {
  TensorArg q_clean, q_corr, d_o;  // bf16
  const float* lse;    // [batch][R][hq]
  const float* delta;  // [batch][R][hq]
  uint16_t* qn;        // [batch][hq][nqc][d] bf16
  uint16_t* don;
  _Float16* qh;        // [batch][hq][nqc][d] fp16: the same values in half precision
  _Float16* doh;
  float* lse2;         // [batch][hq][nqc] log2-scaled LSE; +inf on padding rows
  float* dc;           // [batch][hq][nqc] delta; 0 on padding rows
  int32_t* vis;        // [4][nqc] visible source rows per compact row: [lo, hi) of the
                       // clean keys, then [lo, hi) of the packed corrupted keys; 0 on padding
};

struct FwdArgs {
  TensorArg q_clean, q_corr;  // bf16
  const uint16_t* kn;         // compact natural K
  const _Float16* vt;         // compact transposed V
  void* o;
  int64_t o_bs, o_rs, o_hs;
  int32_t o_f32;
  float* lse;  // [batch][R][hq]
};

struct FwdF32Args {
  TensorArg q_clean, q_corr, k_clean, v_clean, k_corr, v_corr;  // fp32
  float* o;
  int64_t o_bs, o_rs, o_hs;
  float* lse;
};

struct DeltaArgs {
  TensorArg o;  // bf16 or fp32 (o_f32)
  int32_t o_f32;
  TensorArg d_o;  // bf16
  float* delta;   // [batch][R][hq]
};

struct DqArgs {
  const _Float16* qh;  // compact query side (Q fp16, dO bf16)
  const uint16_t* don;
  const float* lse2;
  const float* dc;
  const _Float16* kh;  // compact key side (K fp16, V bf16)
  const uint16_t* vn;
  float* dq;  // [batch][R][hq][d], +=
};

struct DkdvArgs {
  const _Float16* qh;  // compact query side, fp16 natural
  const _Float16* doh;
  const float* lse2;
  const float* dc;
  const int32_t* vis;
  const _Float16* kh;
  const uint16_t* vn;
  float* dk_clean;  // [batch][L][hkv][d], +=
  float* dv_clean;
  float* dk_corr;   // [batch][n_corr_rows][hkv][d], +=
  float* dv_corr;
};

struct MergeArgs {
  int64_t rows;
  int32_t d;
  float* o_acc;
  float* lse_acc;
  const float* o_part;
  const float* lse_part;
  uint16_t* o_bf16;
};

hipError_t launch_pack_k(const Plan& P, const PackKArgs& a, hipStream_t s);
hipError_t launch_pack_q(const Plan& P, const PackQArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16(const Plan& P, const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const Plan& P, const FwdF32Args& a, hipStream_t s);
hipError_t launch_delta(const Plan& P, const DeltaArgs& a, hipStream_t s);
hipError_t launch_dq(const Plan& P, const DqArgs& a, hipStream_t s);
hipError_t launch_dkdv(const Plan& P, const DkdvArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);

}  // namespace bd
