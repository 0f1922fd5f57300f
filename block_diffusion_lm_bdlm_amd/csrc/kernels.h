// kernels.h — argument blocks and launchers of the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace bd {

// The header of every bf16 workspace (kHeaderWords int32): word 0 is the
// call's range flag; words kQueueFwd, kQueueDq and kQueueDkdv start the
// eight per-XCD work-queue heads of those kernels (plan.h), kQueueStride
// words apart so each head has a 128-byte line of its own (claims on one
// queue do not contend with the others).  The clear kernel zeroes the flag
// and the heads at the start of each call.
constexpr int kQueueStride = 32;
constexpr int kQueueFwd = 256, kQueueDq = 512, kQueueDkdv = 768, kHeaderWords = 1024;

struct TensorArg {
  const void* p;
  int64_t bs, rs, hs;  // strides in elements; head dim contiguous
};

// ---------------------------------------------------------------- packing
// Compact key space: the call's key segments back to back, each starting at
// a multiple of kAlign, zero padded.  Natural layouts are [batch][hkv][nkc][d]
// (bf16 for kn, fp16 for kh and vh); transposed ones fp16
// [batch][hkv][nkc/64][d][64] (tiles of 64 rows, each contiguous) with
// perm16 groups.
struct PackKArgs {
  TensorArg k_clean, v_clean, k_corr, v_corr;  // bf16
  uint16_t* kn;   // natural K (nullable)
  _Float16* kh;   // natural K in fp16 (nullable)
  _Float16* vh;   // natural V in fp16 (nullable)
  _Float16* vt;   // transposed V (nullable)
  int32_t* flag;  // set to 1 when a value converted to fp16 lies outside its range
};

// Compact query space: the share's query segments back to back, segment s
// at rows [tile0 * kBQ, (tile0 + ntiles) * kBQ), zero padded.
struct PackQArgs {
  TensorArg q_clean, q_corr, d_o;  // bf16
  TensorArg o;                     // final O (read when !delta_ready)
  int32_t o_f32;                   // O is fp32 (else bf16)
  int32_t delta_ready;             // delta given; else D = dO . O is computed and stored
  const float* lse;    // [batch][R][hq]
  float* delta;        // [batch][R][hq]
  _Float16* qh;        // [batch][hq][nqc][d] fp16: the bf16 values in half precision
  _Float16* doh;
  float* lse2;         // [batch][hq][nqc] log2 LSE - c (row_pscale); +inf on padding rows
  float* dc;           // [batch][hq][nqc] D * 2^-c; 0 on padding rows
  // qh: Q in fp16; doh: dO * 2^-c in fp16 (c = the row's row_pscale)
  int32_t* vis;        // [4][nqc] visible source rows per compact row: [lo, hi) of the
                       // clean keys, then [lo, hi) of the packed corrupted keys; 0 on padding
  int32_t* flag;       // set to 1 when a value converted to fp16 lies outside its range
};

struct FwdArgs {
  TensorArg q_clean, q_corr;  // bf16
  const uint16_t* kn;         // compact natural K
  const _Float16* vt;         // compact transposed V
  void* o;
  int64_t o_bs, o_rs, o_hs;
  int32_t o_f32;
  float* lse;  // [batch][R][hq]
  int32_t* queue;  // per-XCD work-queue heads, zero at launch
};

struct FwdF32Args {
  TensorArg q_clean, q_corr, k_clean, v_clean, k_corr, v_corr;  // fp32
  float* o;
  int64_t o_bs, o_rs, o_hs;
  float* lse;
};

struct DqArgs {
  const _Float16* qh;  // compact query side, fp16 natural
  const _Float16* doh;
  const float* lse2;
  const float* dc;
  const _Float16* kh;  // compact key side, fp16 natural
  const _Float16* vh;
  float* dq;  // [batch][R][hq][d], += (= when overwrite)
  int32_t overwrite;
  int32_t* queue;  // per-XCD work-queue heads, zero at launch
};

struct DkdvArgs {
  const _Float16* qh;  // compact query side, fp16 natural
  const _Float16* doh;
  const float* lse2;
  const float* dc;
  const int32_t* vis;
  const _Float16* kh;
  const _Float16* vh;
  float* dk_clean;  // [batch][L][hkv][d], += (= when overwrite)
  float* dv_clean;
  float* dk_corr;   // [batch][n_corr_rows][hkv][d], += (= when overwrite)
  float* dv_corr;
  int32_t overwrite;
  int32_t* queue;  // per-XCD work-queue heads, zero at launch
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

hipError_t launch_flag_clear(int32_t* header, hipStream_t s);  // zeroes the workspace header's first kHeaderWords
hipError_t launch_pack_k(const Plan& P, const PackKArgs& a, hipStream_t s);
hipError_t launch_pack_q(const Plan& P, const PackQArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16(const Plan& P, const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const Plan& P, const FwdF32Args& a, hipStream_t s);
hipError_t launch_dq(const Plan& P, const DqArgs& a, hipStream_t s);
hipError_t launch_dkdv(const Plan& P, const DkdvArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);

}  // namespace bd
