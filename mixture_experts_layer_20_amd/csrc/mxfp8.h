// MXFP8 launchers and arguments shared by csrc/mxfp8.hip and the C-ABI (gfx950 only).
#pragma once

#include "common.h"

namespace moe {

// ----------------------------------------------------------------------------------------------
// MXFP8: E4M3 elements with one E8M0 scale per 32 consecutive elements of the contraction axis.

// Quantize a bf16 matrix [R, K] (row stride ldx elements) along its rows: codes [R, K], scales
// [R, K/32].
hipError_t launch_mx_quant_rows(const void* x, long long R, int K, long long ldx, uint8_t* codes,
                                uint8_t* scales, hipStream_t s);
// Quantize a bf16 matrix [R, N] along its columns, one row range per group (offsets, or groups of
// group_rows rows when offsets is null), each range padded with zeros to a multiple of kpad; the
// result is transposed: codes [N, ldc], scales [N, ldc/32]; group g's columns start at kbase[g].
hipError_t launch_mx_quant_cols(const void* x, long long R, int N, long long ldx, const int32_t* offsets,
                                int G, long long group_rows, int kpad, uint8_t* codes, uint8_t* scales,
                                long long ldc, int32_t* kbase, hipStream_t s);

enum MxEpilogue { MX_EPI_STORE = 0, MX_EPI_SWIGLU = 1, MX_EPI_SWIGLU_BWD = 2 };

struct MxGemmArgs {
  const uint8_t* a;       // A codes, row stride lda bytes; scales as, row stride lda/32
  const uint8_t* as;
  long long lda;
  const uint8_t* b;       // B codes (group g at b + g*b_gstride), row stride ldb; scales alike /32
  const uint8_t* bs;
  long long ldb, b_gstride;
  const uint8_t* b2;      // second B source (same strides): SwiGLU up rows; else K columns >= ksplit
  const uint8_t* bs2;
  int ksplit;
  const int32_t* offsets; // ragged rows: [G+1] row offsets; ragged K: [G+1] column offsets (kbase)
  int32_t* tile_prefix;   // ragged rows: [G+1] workspace
  int G, M, N, K;         // ragged rows: M rows, K fixed; ragged K: M rows of A (per group output rows)
  void* out0;
  void* out1;
  void* out2;
  const void* aux0;
  const void* aux1;
  int split;              // ragged K: output rows [0, split) -> out0, [split, M) -> out1
  int tiles;              // tile indices of the launch (set by the launcher)
  uint8_t* qc;            // SwiGLU / SwiGLU backward: MXFP8 of the bf16 output rows (codes, scales), or null
  uint8_t* qs;
  int kparts;             // ragged K: splits of each group's K range (fp32 partials, then a reduction)
  float* partial;         // [kparts, G, M, N] fp32 when kparts > 1
};
hipError_t launch_mx_gemm(int epi, bool ragged_k, const MxGemmArgs& a, hipStream_t s);
// Ragged K: the K split the launcher uses for G groups of M x N outputs, and its workspace bytes.
int mx_k_parts(int G, int M, int N);
size_t mx_k_workspace_bytes(int G, int M, int N);

}  // namespace moe
