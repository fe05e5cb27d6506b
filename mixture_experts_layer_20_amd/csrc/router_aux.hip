// Router statistics and the auxiliary load-balancing loss, forward and backward.
//
// The pages run their load-balancing experiments at loss weights 0.02 to 0.50 ("Olmo-core DDP MoE
// examples", "Other experiments in the report") without stating the loss.  The reading built here:
//   loss = weight * E * sum_e f_e P_e,
//   f_e  = count_e / (T k)      fraction of the T k (token, slot) assignments routed to expert e,
//   P_e  = (1/T) sum_t p[t, e]  mean of the softmax over all E router logits.
// The selection, and so f, is piecewise constant: only P carries a gradient.  With
// c = weight E / T the logit gradient is G[t, j] = c p[t, j] (f_j - sum_e f_e p[t, e]), dense over
// all tokens and experts; the backward adds G^T x to the router weight gradient and G w_router to
// the router's input gradient.  Every sum runs in a fixed order: results are bitwise reproducible.
#include "common.h"

namespace moe {
namespace {

constexpr int EV = 4;          // experts per lane: E <= 256 over a 64-lane wave
constexpr int AUX_TPW = 4;     // tokens per wave of the probability sums
constexpr int AUX_TPB = 4 * AUX_TPW;
constexpr int DX_TPB = 8;      // tokens per block of the input gradient
constexpr int DW_ET = 32;      // experts per block of the weight gradient
constexpr int DW_TSPLIT = 256; // tokens per block of the weight gradient
constexpr int DW_TU = 32;      // tokens whose activations are loaded together

// One token's logits over the wave: lane l holds experts l, l + 64, l + 128, l + 192 (0 past E).
__device__ __forceinline__ void wave_row(const float* row, int E, int lane, float (&p)[EV]) {
#pragma unroll
  for (int j = 0; j < EV; ++j) {
    const int e = lane + 64 * j;
    p[j] = e < E ? row[e] : 0.0f;
  }
}
// Softmax over the wave, in place on wave_row's layout.  Butterfly reductions give every lane the
// same maximum and sum.
__device__ __forceinline__ void wave_softmax_inplace(int E, int lane, float (&p)[EV]) {
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EV; ++j)
    if (lane + 64 * j < E) m = fmaxf(m, p[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < EV; ++j) {
    const int e = lane + 64 * j;
    p[j] = e < E ? expf(p[j] - m) : 0.0f;
    s += p[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  const float inv = 1.0f / s;
#pragma unroll
  for (int j = 0; j < EV; ++j) p[j] *= inv;
}
__device__ __forceinline__ void wave_softmax(const float* row, int E, int lane, float (&p)[EV]) {
  wave_row(row, E, lane, p);
  wave_softmax_inplace(E, lane, p);
}

// partial[b][e] = sum of p[t, e] over the AUX_TPB tokens of block b (tokens of a wave in order,
// then the waves in order).  A wave loads its tokens' logits before the first softmax.
__global__ __launch_bounds__(256) void aux_prob_partial_kernel(const float* logits, int T, int E, float* partial) {
  __shared__ float red[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float acc[EV] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int t0 = blockIdx.x * AUX_TPB + w * AUX_TPW;
  float p[AUX_TPW][EV];
#pragma unroll
  for (int i = 0; i < AUX_TPW; ++i)
    if (t0 + i < T) wave_row(logits + (size_t)(t0 + i) * E, E, lane, p[i]);
#pragma unroll
  for (int i = 0; i < AUX_TPW; ++i) {
    if (t0 + i >= T) break;
    wave_softmax_inplace(E, lane, p[i]);
#pragma unroll
    for (int j = 0; j < EV; ++j) acc[j] += p[i][j];
  }
#pragma unroll
  for (int j = 0; j < EV; ++j) red[w][lane + 64 * j] = acc[j];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    partial[(size_t)blockIdx.x * E + e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

// P_e and f_e, one block per expert: thread i sums the block partials i, i + 256, ... in order,
// then a fixed tree over the threads.  stat[e] = f_e P_e for the loss.
__global__ __launch_bounds__(256) void aux_expert_kernel(const float* partial, int nblk, const int32_t* counts, int T,
                                                         int E, int k, float* prob_mean, float* load_frac,
                                                         float* stat) {
  __shared__ float red[256];
  const int e = blockIdx.x, i = threadIdx.x;
  float s = 0.0f;
  for (int b = i; b < nblk; b += 256) s += partial[(size_t)b * E + e];
  red[i] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (i < off) red[i] += red[i + off];
    __syncthreads();
  }
  if (i == 0) {
    const float P = T > 0 ? red[0] / (float)T : 0.0f;
    const float f = T > 0 ? (float)counts[e] / ((float)T * (float)k) : 0.0f;
    prob_mean[e] = P;
    load_frac[e] = f;
    stat[e] = f * P;
  }
}

// loss = weight E sum_e stat[e] (a fixed tree over the experts).
__global__ __launch_bounds__(256) void aux_loss_kernel(const float* stat, int E, float weight, float* loss) {
  __shared__ float red[256];
  const int e = threadIdx.x;
  red[e] = e < E ? stat[e] : 0.0f;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (e < off) red[e] += red[e + off];
    __syncthreads();
  }
  if (e == 0) *loss = weight * (float)E * red[0];
}

// G[t, :] for one token per wave.
__global__ __launch_bounds__(256) void aux_grad_kernel(const float* logits, const float* load_frac, int T, int E,
                                                       float c, float* G) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float p[EV], f[EV];
  wave_softmax(logits + (size_t)t * E, E, lane, p);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < EV; ++j) {
    const int e = lane + 64 * j;
    f[j] = e < E ? load_frac[e] : 0.0f;
    s += f[j] * p[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
#pragma unroll
  for (int j = 0; j < EV; ++j) {
    const int e = lane + 64 * j;
    if (e < E) G[(size_t)t * E + e] = c * p[j] * (f[j] - s);
  }
}

// 8 consecutive elements (16-byte aligned) as fp32, and back.
__device__ __forceinline__ void ld8(const bf16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void st8(bf16_t* p, const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void st8(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// dx[t, :] += sum_e G[t, e] w[e, :]  (DX_TPB tokens per block, 8 columns per thread, experts in
// order; the sum is rounded once to the element type on the way back).
template <typename T>
__global__ __launch_bounds__(256) void aux_dx_kernel(const float* G, const T* w, int ntok, int d, int E, T* dx) {
  __shared__ float gs[DX_TPB][256];
  const int t0 = blockIdx.x * DX_TPB;
  const int nt = min(DX_TPB, ntok - t0);
  for (int q = threadIdx.x; q < DX_TPB * E; q += 256) {
    const int i = q / E, e = q % E;
    gs[i][e] = i < nt ? G[(size_t)(t0 + i) * E + e] : 0.0f;
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[DX_TPB][8];
#pragma unroll
    for (int i = 0; i < DX_TPB; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;
#pragma unroll 4
    for (int e = 0; e < E; ++e) {
      float wv[8];
      ld8(w + (size_t)e * d + c, wv);
#pragma unroll
      for (int i = 0; i < DX_TPB; ++i) {
        const float g = gs[i][e];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][q] += g * wv[q];
      }
    }
#pragma unroll
    for (int i = 0; i < DX_TPB; ++i) {
      if (i >= nt) break;
      float v[8];
      T* out = dx + (size_t)(t0 + i) * d + c;
      ld8(out, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += acc[i][q];
      st8(out, v);
    }
  }
}

// partial[s][e][col] = sum over the tokens of split s of G[t, e] x[t, col].  The split's block of
// G (DW_TSPLIT tokens x DW_ET experts) is staged in LDS and read as broadcasts.
template <typename T>
__global__ __launch_bounds__(256) void aux_dw_partial_kernel(const float* G, const T* x, int ntok, int d, int E,
                                                             float* partial) {
  __shared__ float gs[DW_TSPLIT][DW_ET];
  const int col = blockIdx.x * 256 + threadIdx.x;
  const int e0 = blockIdx.y * DW_ET, s = blockIdx.z;
  const int tb = s * DW_TSPLIT, te = min(ntok, tb + DW_TSPLIT);
  for (int q = threadIdx.x; q < DW_TSPLIT * DW_ET; q += 256) {
    const int t = tb + q / DW_ET, e = e0 + q % DW_ET;
    gs[q / DW_ET][q % DW_ET] = (t < te && e < E) ? G[(size_t)t * E + e] : 0.0f;
  }
  __syncthreads();
  if (col >= d) return;
  float acc[DW_ET];
#pragma unroll
  for (int i = 0; i < DW_ET; ++i) acc[i] = 0.0f;
  // DW_TU tokens' activations in flight at once, then their products in token order
  for (int t = tb; t < te; t += DW_TU) {
    float xv[DW_TU];
#pragma unroll
    for (int u = 0; u < DW_TU; ++u) xv[u] = t + u < te ? to_f32<T>(x[(size_t)(t + u) * d + col]) : 0.0f;
#pragma unroll
    for (int u = 0; u < DW_TU; ++u) {
      if (t + u >= te) break;
      const float* g = gs[t + u - tb];
#pragma unroll
      for (int i = 0; i < DW_ET; ++i) acc[i] += g[i] * xv[u];
    }
  }
#pragma unroll
  for (int i = 0; i < DW_ET; ++i)
    if (e0 + i < E) partial[((size_t)s * E + e0 + i) * d + col] = acc[i];
}

// dw[e, col] += sum over the splits in order.
__global__ __launch_bounds__(256) void aux_dw_reduce_kernel(const float* partial, int nsplit, int E, int d, float* dw) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x, n = (size_t)E * d;
  if (i >= n) return;
  float s = 0.0f;
#pragma unroll 16
  for (int q = 0; q < nsplit; ++q) s += partial[(size_t)q * n + i];   // in order; loads overlap
  dw[i] += s;
}

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t router_aux_ws_bytes(long long T, int E) {
  return align256((size_t)ceil_div(T, AUX_TPB) * E * sizeof(float)) + align256((size_t)E * sizeof(float));
}

hipError_t launch_router_aux(const float* logits, const int32_t* counts, int T, int E, int k, float weight,
                             float* loss, float* prob_mean, float* load_frac, void* ws, hipStream_t s) {
  const int nblk = ceil_div(T, AUX_TPB);
  float* partial = reinterpret_cast<float*>(ws);
  float* stat = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256((size_t)nblk * E * sizeof(float)));
  if (nblk > 0) hipLaunchKernelGGL(aux_prob_partial_kernel, dim3(nblk), dim3(256), 0, s, logits, T, E, partial);
  hipLaunchKernelGGL(aux_expert_kernel, dim3(E), dim3(256), 0, s, partial, nblk, counts, T, E, k, prob_mean,
                     load_frac, stat);
  hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(256), 0, s, stat, E, weight, loss);
  return hipGetLastError();
}

size_t router_aux_bwd_ws_bytes(long long T, long long d, int E) {
  const long long nsplit = (T + DW_TSPLIT - 1) / DW_TSPLIT;
  return align256((size_t)T * E * sizeof(float)) + align256((size_t)nsplit * E * d * sizeof(float));
}

hipError_t launch_router_aux_bwd(const float* logits, const float* load_frac, const void* x, const void* w,
                                 int T, int d, int E, float weight, bool bf16, float* dw, void* dx, void* ws,
                                 hipStream_t s) {
  if (T == 0) return hipSuccess;
  char* p = reinterpret_cast<char*>(ws);
  float* G = reinterpret_cast<float*>(p);
  p += align256((size_t)T * E * sizeof(float));
  float* partial = reinterpret_cast<float*>(p);
  const int nsplit = ceil_div(T, DW_TSPLIT);
  const float c = weight * (float)E / (float)T;
  hipLaunchKernelGGL(aux_grad_kernel, dim3(ceil_div(T, 4)), dim3(256), 0, s, logits, load_frac, T, E, c, G);
  const dim3 gdw(ceil_div(d, 256), ceil_div(E, DW_ET), nsplit);
  if (bf16) {
    hipLaunchKernelGGL(aux_dx_kernel<bf16_t>, dim3(ceil_div(T, DX_TPB)), dim3(256), 0, s, G,
                       reinterpret_cast<const bf16_t*>(w), T, d, E, reinterpret_cast<bf16_t*>(dx));
    hipLaunchKernelGGL(aux_dw_partial_kernel<bf16_t>, gdw, dim3(256), 0, s, G, reinterpret_cast<const bf16_t*>(x),
                       T, d, E, partial);
  } else {
    hipLaunchKernelGGL(aux_dx_kernel<float>, dim3(ceil_div(T, DX_TPB)), dim3(256), 0, s, G,
                       reinterpret_cast<const float*>(w), T, d, E, reinterpret_cast<float*>(dx));
    hipLaunchKernelGGL(aux_dw_partial_kernel<float>, gdw, dim3(256), 0, s, G, reinterpret_cast<const float*>(x),
                       T, d, E, partial);
  }
  hipLaunchKernelGGL(aux_dw_reduce_kernel, dim3(ceil_div((long long)E * d, 256)), dim3(256), 0, s, partial, nsplit,
                     E, d, dw);
  return hipGetLastError();
}

}  // namespace moe
