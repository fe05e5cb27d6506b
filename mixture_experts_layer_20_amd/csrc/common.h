// Internal helpers and launcher declarations shared by the HIP sources of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ float sigmoid_f32(float a) { return 1.0f / (1.0f + expf(-a)); }

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// ----------------------------------------------------------------------------------------------
// Launchers (host side).  All enqueue on `s` and return the launch status.

// Router
hipError_t launch_router_logits(const void* x, const void* w, const float* bias, float* logits,
                                int T, int d, int E, bool bf16, hipStream_t s);
hipError_t launch_topk_gate(const float* logits, int T, int E, int k, int renormalize,
                            int32_t* topk_idx, float* topk_gate, hipStream_t s);
size_t route_bwd_ws_bytes(long long T, long long d, int E, int k);
hipError_t launch_route_bwd(const float* dgate, const float* gate, const int32_t* topk_idx,
                            const int32_t* offsets, const int32_t* src_row, const void* x,
                            const void* w, int T, int d, int E, int k, bool bf16, float* dw,
                            void* dx_router, void* ws, hipStream_t s);

// Router statistics and the load-balancing loss
size_t router_aux_ws_bytes(long long T, int E);
hipError_t launch_router_aux(const float* logits, const int32_t* counts, int T, int E, int k, float weight,
                             float* loss, float* prob_mean, float* load_frac, void* ws, hipStream_t s);
size_t router_aux_bwd_ws_bytes(long long T, long long d, int E);
hipError_t launch_router_aux_bwd(const float* logits, const float* load_frac, const void* x, const void* w,
                                 int T, int d, int E, float weight, bool bf16, float* dw, void* dx, void* ws,
                                 hipStream_t s);

// Dispatch
size_t permute_ws_bytes(long long T, int E, int k);
hipError_t launch_permute(const void* x, const int32_t* topk_idx, int T, int d, int E, int k,
                          bool bf16, int32_t* counts, int32_t* offsets, int32_t* dest_pos,
                          int32_t* src_row, void* x_perm, void* ws, hipStream_t s);
hipError_t launch_permute_bwd(const void* dx_perm, const int32_t* dest_pos, const void* add0,
                              const void* add1, int T, int d, int k, bool bf16, void* dx,
                              hipStream_t s);

// Combine
hipError_t launch_combine(const void* y_perm, const float* gate, const int32_t* dest_pos,
                          const void* shared_out, int T, int d, int k, bool bf16, void* out,
                          hipStream_t s);
hipError_t launch_combine_bwd(const void* dout, const void* y_perm, const float* gate,
                              const int32_t* dest_pos, int T, int d, int k, bool bf16,
                              void* dy_perm, float* dgate, hipStream_t s);

// Grouped expert GEMMs
enum GemmMode {
  GEMM_UP_FWD = 0,     // h = silu(X W1^T) * (X W3^T), optional A/B stash
  GEMM_DOWN_FWD = 1,   // y = h W2^T
  GEMM_DOWN_BWD = 2,   // dH = dy W2 -> dA, dB (SwiGLU backward)
  GEMM_UP_DGRAD = 3,   // dx = dA W1 + dB W3
  GEMM_DOWN_WGRAD = 4, // dW2 = dy^T h
  GEMM_UP_WGRAD = 5,   // dW1 = dA^T x, dW3 = dB^T x
};

// A second set of groups of the same stage (the shared expert next to the routed experts): its own
// tensors, group offsets, group count, rows and hidden width; d is common.
struct GemmSeg {
  const void* a;
  const void* b0;
  const void* b1;
  const void* aux0;
  const void* aux1;
  void* out0;
  void* out1;
  void* out2;
  const int32_t* offsets;
  int G, M, f;
  int ksplit;   // weight gradients: row-reduction split of this set (fp32 partials; 0 or 1: none)
};

struct GemmArgs {
  const void* a;      // activation operand
  const void* b0;     // weight (or second activation operand for wgrad)
  const void* b1;     // second weight (W3) where needed
  const void* aux0;   // A stash (down bwd)
  const void* aux1;   // B stash (down bwd)
  void* out0;
  void* out1;
  void* out2;
  const int32_t* offsets;     // [G+1] row offsets of the groups
  int32_t* tile_prefix;       // workspace start: [G+1] M-tiles before each group, then split-K partials
  size_t ws_bytes;            // bytes of that workspace
  int G, M, d, f;
  int nseg;                   // 2: s1 is a second set of groups in the same launch (pipelined kernel only)
  GemmSeg s1;
};

size_t gemm_ws_bytes(int G);
// Workspace bytes for the fp32 partial sums of the split weight-gradient reductions.
size_t gemm_partial_bytes(int G, long long M, int d, int f);
// The same for the second set of a two-set weight-gradient launch (its split reduction).
size_t gemm_sets_partial_bytes(int G0, long long M0, int G1, long long M1, int d, int f1);
hipError_t launch_grouped_gemm(int mode, const GemmArgs& args, bool bf16, hipStream_t s);
// Pipelined bf16 kernel (256x256 tiles, direct-to-LDS ring): whether it covers this problem (both
// sets when nseg == 2), and its launcher (ksplit/partial: split weight-gradient reduction, as in
// launch_grouped_gemm; one set only).
bool pipe_supports(int mode, const GemmArgs& args);
hipError_t launch_grouped_gemm_pipe(int mode, const GemmArgs& args, int ksplit, float* partial, hipStream_t s,
                                    int num_cus);

}  // namespace moe
