// Helpers shared by the grouped-GEMM kernels: mode geometry, operand addressing and the
// per-element epilogues of the six GEMM stages of the SwiGLU expert MLP.
#pragma once

#include "common.h"

namespace moe {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int MODE> struct Traits {
  static constexpr bool raggedK = (MODE == GEMM_DOWN_WGRAD || MODE == GEMM_UP_WGRAD);
  static constexpr bool a_kcontig = !raggedK;
  static constexpr bool b_kcontig = (MODE == GEMM_UP_FWD || MODE == GEMM_DOWN_FWD);
};

// Reduction length of the ragged-M modes.
__host__ __device__ inline int mode_K(int mode, int d, int f) {
  switch (mode) {
    case GEMM_UP_FWD: return d;
    case GEMM_DOWN_FWD: return f;
    case GEMM_DOWN_BWD: return d;
    case GEMM_UP_DGRAD: return 2 * f;
    default: return 0;
  }
}
// Output columns (in tile space: the gate/up GEMM packs W1 and W3 columns side by side).
__host__ __device__ inline int mode_N(int mode, int d, int f) {
  switch (mode) {
    case GEMM_UP_FWD: return 2 * f;
    case GEMM_DOWN_FWD: return d;
    case GEMM_DOWN_BWD: return f;
    case GEMM_UP_DGRAD: return d;
    case GEMM_DOWN_WGRAD: return f;
    case GEMM_UP_WGRAD: return d;
    default: return 0;
  }
}
// Output rows of the weight-gradient modes.
__host__ __device__ inline int mode_Mw(int mode, int d, int f) {
  return mode == GEMM_DOWN_WGRAD ? d : 2 * f;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Group row range, clamped into [0, M] (the same clamping the tile-prefix kernel uses).
__device__ __forceinline__ void group_rows(const int32_t* offsets, int g, int M, int& lo, int& hi) {
  lo = clampi(offsets[g], 0, M);
  hi = clampi(offsets[g + 1], lo, M);
}

// --------------------------------------------------------------------------------------------
// Operand addressing.  "A" rows are output rows (tokens, or weight-gradient rows), "B" rows are
// output columns.  K-contiguous operands are addressed by (row, k); K-strided ones by (k, col)
// with the 8 consecutive columns read together.

// Pointer to A(row m, k) for the ragged-M modes: A is [M, K] row-major.
template <int MODE, typename T>
__device__ __forceinline__ const T* a_ptr_kc(const GemmArgs& p, int m, int k) {
  const int K = mode_K(MODE, p.d, p.f);
  return reinterpret_cast<const T*>(p.a) + (size_t)m * K + k;
}

// Pointer to B(row r of the tile, k) for the K-contiguous weight operands.
template <int MODE, typename T, int BNv>
__device__ __forceinline__ const T* b_ptr_kc(const GemmArgs& p, int g, int nt, int r, int k) {
  if constexpr (MODE == GEMM_UP_FWD) {
    constexpr int H = BNv / 2;
    const int n = nt * H + (r < H ? r : r - H);
    const T* w = reinterpret_cast<const T*>(r < H ? p.b0 : p.b1);
    return w + ((size_t)g * p.f + n) * p.d + k;
  } else {  // GEMM_DOWN_FWD: W2[g] is [d, f]
    const int n = nt * BNv + r;
    return reinterpret_cast<const T*>(p.b0) + ((size_t)g * p.d + n) * p.f + k;
  }
}

// Pointer to B(k, column n) for the K-strided operands (column n contiguous).
template <int MODE, typename T>
__device__ __forceinline__ const T* b_ptr_mc(const GemmArgs& p, int g, int k, int n) {
  if constexpr (MODE == GEMM_DOWN_BWD) {  // W2[g] viewed as [d(k), f(n)]
    return reinterpret_cast<const T*>(p.b0) + ((size_t)g * p.d + k) * p.f + n;
  } else if constexpr (MODE == GEMM_UP_DGRAD) {  // [W1[g]; W3[g]] viewed as [2f(k), d(n)]
    const T* w = reinterpret_cast<const T*>(k < p.f ? p.b0 : p.b1);
    const int kk = k < p.f ? k : k - p.f;
    return w + ((size_t)g * p.f + kk) * p.d + n;
  } else if constexpr (MODE == GEMM_DOWN_WGRAD) {  // h rows
    return reinterpret_cast<const T*>(p.b0) + (size_t)k * p.f + n;
  } else {  // GEMM_UP_WGRAD: x rows
    return reinterpret_cast<const T*>(p.b0) + (size_t)k * p.d + n;
  }
}

// Pointer to A(k, row m) for the weight-gradient modes (row m contiguous).
template <int MODE, typename T>
__device__ __forceinline__ const T* a_ptr_mc(const GemmArgs& p, int k, int m) {
  if constexpr (MODE == GEMM_DOWN_WGRAD) {  // dy rows [M, d]
    return reinterpret_cast<const T*>(p.a) + (size_t)k * p.d + m;
  } else {  // dAB rows [M, 2f]
    return reinterpret_cast<const T*>(p.a) + (size_t)k * (2 * p.f) + m;
  }
}

// --------------------------------------------------------------------------------------------
// Epilogue: one output element (v1 is the up-projection value of the gate/up GEMM).
template <int MODE, typename T>
__device__ __forceinline__ void epilogue(const GemmArgs& p, int g, int m, int n, float v0, float v1) {
  if constexpr (MODE == GEMM_UP_FWD) {
    const size_t i = (size_t)m * p.f + n;
    const float h = v0 * sigmoid_f32(v0) * v1;
    if (p.out0) reinterpret_cast<T*>(p.out0)[i] = from_f32<T>(v0);
    if (p.out1) reinterpret_cast<T*>(p.out1)[i] = from_f32<T>(v1);
    reinterpret_cast<T*>(p.out2)[i] = from_f32<T>(h);
  } else if constexpr (MODE == GEMM_DOWN_FWD || MODE == GEMM_UP_DGRAD) {
    reinterpret_cast<T*>(p.out0)[(size_t)m * p.d + n] = from_f32<T>(v0);
  } else if constexpr (MODE == GEMM_DOWN_BWD) {
    const size_t i = (size_t)m * p.f + n;
    const float a = to_f32<T>(reinterpret_cast<const T*>(p.aux0)[i]);
    const float b = to_f32<T>(reinterpret_cast<const T*>(p.aux1)[i]);
    const float s = sigmoid_f32(a);
    const float da = v0 * b * s * (1.0f + a * (1.0f - s));
    const float db = v0 * a * s;
    T* dab = reinterpret_cast<T*>(p.out0) + (size_t)m * (2 * p.f);
    dab[n] = from_f32<T>(da);
    dab[p.f + n] = from_f32<T>(db);
  } else if constexpr (MODE == GEMM_DOWN_WGRAD) {
    reinterpret_cast<T*>(p.out0)[((size_t)g * p.d + m) * p.f + n] = from_f32<T>(v0);
  } else {  // GEMM_UP_WGRAD: rows [0, f) -> dW1, [f, 2f) -> dW3
    T* out = reinterpret_cast<T*>(m < p.f ? p.out0 : p.out1);
    const int mm = m < p.f ? m : m - p.f;
    out[((size_t)g * p.f + mm) * p.d + n] = from_f32<T>(v0);
  }
}


}  // namespace gemm
}  // namespace moe
