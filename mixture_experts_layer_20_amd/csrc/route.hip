// Router of the MoE layer: fp32 logits in a fixed summation order, top-k selection, gate softmax,
// and the router backward.
//
// Top-k routing with learned or random scores is the pages' routing step ("Olmo-core DDP MoE
// examples", "Production throughput runs": top-4, learned vs random routing; "Scaling
// Trillion-Parameter Models: The Architecture of Olmo-core 3", "Code Snippet": one expert choice
// per token).  The selection turns floats into integers, so the logits are computed bit-exactly
// in a fixed order: for each (token, expert), products are added in increasing feature index,
// each product and each sum rounded to fp32, the bias added last.  MFMA accumulation order is not
// specified bitwise, so this runs on the vector ALUs.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int RT = 64;   // tokens per block
constexpr int RE = 64;   // experts per block
constexpr int RK = 32;   // features per LDS step

// Logits: one thread owns 4 tokens x 4 experts and walks the features in increasing order.
// bf16 inputs: the product of two bf16 values is exact in fp32, so a fused multiply-add rounds
// exactly like the separate product and sum.  fp32 inputs: separate multiply and add.
template <bool BF16>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* xv, const void* wv,
                                                            const float* bias, float* logits,
                                                            int T, int d, int E) {
  __shared__ float xs[RK][RT + 1];
  __shared__ float ws[RK][RE + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * RT, e0 = blockIdx.y * RE;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < d; k0 += RK) {
#pragma unroll
    for (int i = 0; i < (RT * RK) / 256; ++i) {
      const int e = tid + i * 256;
      const int r = e / RK, kk = e % RK;
      const int t = t0 + r, ex = e0 + r, k = k0 + kk;
      float xval = 0.0f, wval = 0.0f;
      if (t < T && k < d) {
        xval = BF16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(xv)[(size_t)t * d + k])
                    : reinterpret_cast<const float*>(xv)[(size_t)t * d + k];
      }
      if (ex < E && k < d) {
        wval = BF16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(wv)[(size_t)ex * d + k])
                    : reinterpret_cast<const float*>(wv)[(size_t)ex * d + k];
      }
      xs[kk][r] = xval;
      ws[kk][r] = wval;
    }
    __syncthreads();
    const int kn = d - k0 < RK ? d - k0 : RK;
    for (int kk = 0; kk < kn; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (BF16) {
            acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
          } else {
            const float prod = a[i] * b[j];
            acc[i][j] = acc[i][j] + prod;
          }
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e >= E) continue;
      float v = acc[i][j];
      if (bias) v = v + bias[e];
      logits[(size_t)t * E + e] = v;
    }
  }
}

// Top-k and gates: one wavefront per token, each lane holding up to 4 logits (E <= 256).
// k rounds of a wave-wide arg-max under the order (larger logit first, then lower index).
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* logits, int T, int E, int k,
                                                        int renormalize, int32_t* topk_idx,
                                                        float* topk_gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[4];
  bool taken[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    taken[i] = e >= E;
    v[i] = taken[i] ? 0.0f : logits[(size_t)t * E + e];
  }
  float selv[8];
  int seli[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (!taken[i] && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    selv[j] = bv;
    seli[j] = bi;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == bi) taken[i] = true;
  }
  // Gates.  selv[0] is the largest logit of the token.
  float denom = 0.0f;
  if (renormalize) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) denom += expf(selv[j] - selv[0]);
  } else {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) part += expf(v[i] - selv[0]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    denom = part;
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        topk_idx[(size_t)t * k + j] = seli[j];
        topk_gate[(size_t)t * k + j] = expf(selv[j] - selv[0]) / denom;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Router backward (gates = softmax over the chosen logits).

// dl[t*k+j] = g_j (dg_j - sum_i g_i dg_i): the logit gradient of the chosen experts.  Evaluated
// as g_j * sum_i g_i (dg_j - dg_i), equal because the gates sum to one; this form has no
// cancellation between large terms when one gate is close to 1 and the others are tiny.
__global__ void route_dl_kernel(const float* dgate, const float* gate, int T, int k, float* dl) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float g[8], dg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    g[j] = j < k ? gate[(size_t)t * k + j] : 0.0f;
    dg[j] = j < k ? dgate[(size_t)t * k + j] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < k) s += g[i] * (dg[j] - dg[i]);
    dl[(size_t)t * k + j] = g[j] * s;
  }
}

// dx_router[t] = sum_j dl[t,j] * w_router[idx[t,j]], one block per token.
template <typename T>
__global__ __launch_bounds__(256) void route_dx_kernel(const float* dl, const int32_t* idx,
                                                       const T* w, int d, int k, T* dx) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      const size_t a = (size_t)t * k + j;
      acc += dl[a] * to_f32<T>(w[(size_t)idx[a] * d + c]);
    }
    dx[(size_t)t * d + c] = from_f32<T>(acc);
  }
}

constexpr int SEG = 256;     // permuted rows per partial sum of the router weight gradient
constexpr int DWCOLS = 1024; // columns per block

// Segment prefix: number of SEG-row segments before each expert.
__global__ void seg_prefix_kernel(const int32_t* offsets, int E, int Tk, int32_t* prefix) {
  __shared__ int s[256];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < E; base += 256) {
    const int e = base + tid;
    int c = 0;
    if (e < E) {
      int lo = offsets[e], hi = offsets[e + 1];
      lo = lo < 0 ? 0 : (lo > Tk ? Tk : lo);
      hi = hi < lo ? lo : (hi > Tk ? Tk : hi);
      c = (hi - lo + SEG - 1) / SEG;
    }
    s[tid] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? s[tid - off] : 0;
      __syncthreads();
      s[tid] += v;
      __syncthreads();
    }
    const int carry = carry_s;
    if (e < E) prefix[e] = carry + s[tid] - c;
    __syncthreads();
    if (tid == 255) carry_s = carry + s[255];
    __syncthreads();
  }
  if (tid == 0) prefix[E] = carry_s;
}

// Partial dW_router rows: segment s of expert e sums dl(a) * x[a / k] over its rows in order.
template <typename T>
__global__ __launch_bounds__(256) void route_dw_partial_kernel(const float* dl, const int32_t* src_row,
                                                               const int32_t* offsets,
                                                               const int32_t* seg_prefix,
                                                               const T* x, int E, int Tk, int d,
                                                               int k, float* partial) {
  const int seg = blockIdx.x;
  if (seg >= seg_prefix[E]) return;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_prefix[mid] <= seg) lo = mid; else hi = mid;
  }
  const int e = lo;
  int r0 = offsets[e], r1 = offsets[e + 1];
  r0 = r0 < 0 ? 0 : (r0 > Tk ? Tk : r0);
  r1 = r1 < r0 ? r0 : (r1 > Tk ? Tk : r1);
  const int p0 = r0 + (seg - seg_prefix[e]) * SEG;
  const int p1 = p0 + SEG < r1 ? p0 + SEG : r1;
  const int cbase = blockIdx.y * DWCOLS;
  // Stage the segment's token rows and weights, then stream the rows in order.
  __shared__ int tok_s[SEG];
  __shared__ float w_s[SEG];
  const int n = p1 - p0;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int a = src_row[p0 + i];
    tok_s[i] = a / k;
    w_s[i] = dl[a];
  }
  __syncthreads();
  constexpr int NC = DWCOLS / 256;
  float acc[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) acc[i] = 0.0f;
  for (int r0 = 0; r0 < n; r0 += 8) {
    float xv[8][NC];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = r0 + u < n;
      const T* xr = x + (size_t)(ok ? tok_s[r0 + u] : 0) * d;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = cbase + threadIdx.x + i * 256;
        xv[u][i] = (ok && c < d) ? to_f32<T>(xr[c]) : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r0 + u < n) {
        const float w = w_s[r0 + u];
#pragma unroll
        for (int i = 0; i < NC; ++i) acc[i] += w * xv[u][i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = cbase + threadIdx.x + i * 256;
    if (c < d) partial[(size_t)seg * d + c] = acc[i];
  }
}

// dW_router[e] = sum of the expert's segment partials, in segment order (zeros if none).
__global__ __launch_bounds__(256) void route_dw_reduce_kernel(const float* partial,
                                                              const int32_t* seg_prefix, int d,
                                                              float* dw) {
  const int e = blockIdx.x;
  const int s0 = seg_prefix[e], s1 = seg_prefix[e + 1];
  for (int c = blockIdx.y * DWCOLS + threadIdx.x; c < d && c < (blockIdx.y + 1) * DWCOLS; c += 256) {
    float acc = 0.0f;
    for (int s = s0; s < s1; ++s) acc += partial[(size_t)s * d + c];
    dw[(size_t)e * d + c] = acc;
  }
}

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

hipError_t launch_router_logits(const void* x, const void* w, const float* bias, float* logits,
                                int T, int d, int E, bool bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid(ceil_div(T, RT), ceil_div(E, RE));
  if (bf16) hipLaunchKernelGGL(router_logits_kernel<true>, grid, dim3(256), 0, s, x, w, bias, logits, T, d, E);
  else hipLaunchKernelGGL(router_logits_kernel<false>, grid, dim3(256), 0, s, x, w, bias, logits, T, d, E);
  return hipGetLastError();
}

hipError_t launch_topk_gate(const float* logits, int T, int E, int k, int renormalize,
                            int32_t* topk_idx, float* topk_gate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_gate_kernel, dim3(ceil_div(T, 4)), dim3(256), 0, s, logits, T, E, k,
                     renormalize, topk_idx, topk_gate);
  return hipGetLastError();
}

static inline long long max_segments(long long Tk, int E) { return (Tk + SEG - 1) / SEG + E; }

size_t route_bwd_ws_bytes(long long T, long long d, int E, int k) {
  const long long Tk = T * k;
  return align256((size_t)Tk * sizeof(float)) + align256((size_t)(E + 1) * sizeof(int32_t)) +
         align256((size_t)max_segments(Tk, E) * d * sizeof(float));
}

hipError_t launch_route_bwd(const float* dgate, const float* gate, const int32_t* topk_idx,
                            const int32_t* offsets, const int32_t* src_row, const void* x,
                            const void* w, int T, int d, int E, int k, bool bf16, float* dw,
                            void* dx_router, void* ws, hipStream_t s) {
  const int Tk = T * k;
  char* p = reinterpret_cast<char*>(ws);
  float* dl = reinterpret_cast<float*>(p);
  p += align256((size_t)Tk * sizeof(float));
  int32_t* seg_prefix = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)(E + 1) * sizeof(int32_t));
  float* partial = reinterpret_cast<float*>(p);

  if (T > 0) {
    hipLaunchKernelGGL(route_dl_kernel, dim3(ceil_div(T, 256)), dim3(256), 0, s, dgate, gate, T, k, dl);
    if (bf16)
      hipLaunchKernelGGL(route_dx_kernel<bf16_t>, dim3(T), dim3(256), 0, s, dl, topk_idx,
                         reinterpret_cast<const bf16_t*>(w), d, k, reinterpret_cast<bf16_t*>(dx_router));
    else
      hipLaunchKernelGGL(route_dx_kernel<float>, dim3(T), dim3(256), 0, s, dl, topk_idx,
                         reinterpret_cast<const float*>(w), d, k, reinterpret_cast<float*>(dx_router));
  }
  hipLaunchKernelGGL(seg_prefix_kernel, dim3(1), dim3(256), 0, s, offsets, E, Tk, seg_prefix);
  const int ncb = ceil_div(d, DWCOLS);
  const long long nseg = max_segments(Tk, E);
  if (bf16)
    hipLaunchKernelGGL(route_dw_partial_kernel<bf16_t>, dim3((unsigned)nseg, ncb), dim3(256), 0, s, dl,
                       src_row, offsets, seg_prefix, reinterpret_cast<const bf16_t*>(x), E, Tk, d, k,
                       partial);
  else
    hipLaunchKernelGGL(route_dw_partial_kernel<float>, dim3((unsigned)nseg, ncb), dim3(256), 0, s, dl,
                       src_row, offsets, seg_prefix, reinterpret_cast<const float*>(x), E, Tk, d, k,
                       partial);
  hipLaunchKernelGGL(route_dw_reduce_kernel, dim3(E, ncb), dim3(256), 0, s, partial, seg_prefix, d, dw);
  return hipGetLastError();
}

}  // namespace moe
