// vocab_kernels.h — argument blocks and launchers of the vocabulary-loss
// kernels (vocab_rows.hip), called by the host library (bdvocab.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdvocab {

// Per-row pass: workgroup size, float4 loads per thread between barriers,
// and the grid cap (rows in flight at once, strided loop beyond).  The
// macros only serve launch-shape sweeps.
#ifndef BDVOCAB_ROW_THREADS
#define BDVOCAB_ROW_THREADS 1024
#endif
#ifndef BDVOCAB_ROW_GROUP
#define BDVOCAB_ROW_GROUP 4
#endif
#ifndef BDVOCAB_ROWS_IN_FLIGHT
#define BDVOCAB_ROWS_IN_FLIGHT 256
#endif
// Single-read pass: workgroup size, float4 loads per thread per sub-block,
// the largest sub-block count (logits per row up to threads x loads x 4 x
// that count) and the grid cap; one workgroup per CU fits its registers.
constexpr int kOnChipThreads = 512;
constexpr int kOnChipLoads = 8;
constexpr int kOnChipSubMax = 8;
constexpr int kOnChipInFlight = 256;
constexpr int kRowThreads = BDVOCAB_ROW_THREADS;
constexpr int kRowGroup = BDVOCAB_ROW_GROUP;
constexpr int kRowsInFlight = BDVOCAB_ROWS_IN_FLIGHT;

struct RowsArgs {
  float* s;               // [n, ld] fp32 logits in; bf16 gradient out (pitch 2*ld bf16)
  int64_t ld;             // row pitch in floats, multiple of 4, >= V
  int64_t n;              // rows in the chunk
  int32_t V;              // vocabulary size
  const int32_t* targets; // [n]
  const float* weights;   // [n] or nullptr (1)
  float* lse;             // [n] or nullptr
  float* loss;            // [n]
};

struct GatherArgs {
  const uint16_t* h;      // bf16 rows, pitch h_stride elements
  int64_t h_stride;
  const int32_t* rows;    // [n]
  int64_t n;
  int32_t d;              // multiple of 8
  uint16_t* out;          // [n, d] packed
};

struct ScatterArgs {
  const uint8_t* in;      // [n, d] packed, element size es
  int64_t n;
  int32_t d;
  int32_t es;             // 2 (bf16) or 4 (fp32)
  const int32_t* rows;    // [n]
  uint8_t* dh;            // rows at rows[r] * dh_stride elements
  int64_t dh_stride;
};

struct TransposeArgs {
  const uint16_t* src;    // [rows, cols] 16-bit, row pitch src_pitch (a multiple of 8,
                          // >= cols rounded up to 8: the last piece of a row may read pad)
  int64_t rows;
  int32_t cols;
  int64_t src_pitch;
  uint16_t* dst;          // [cols, rows] 16-bit, row pitch dst_pitch (a multiple of 8,
                          // >= rows rounded up to 8; columns past rows get pad values)
  int64_t dst_pitch;
};

hipError_t launch_rows(const RowsArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s);
hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s);
hipError_t launch_loss_sum(const float* loss, int64_t n, float* out, hipStream_t s);

}  // namespace bdvocab
