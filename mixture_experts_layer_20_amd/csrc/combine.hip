// Weighted combine of the MoE layer and its backward.
//
// The output of a token is the gate-weighted sum of its k routed experts' outputs plus the shared
// expert's output ("Olmo-core DDP MoE examples", "Production throughput runs": top-4 routing with
// one shared expert).  Row gathers are 16-byte vector loads; sums are fp32; one block per token.
#include "common.h"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 8-element row segments.  NT: a stream nothing later in the layer pass reads again (a
// nontemporal access, which does not displace reused data from the caches).
template <typename T> struct V8;
template <> struct V8<bf16_t> {
  typedef u32x4_t Raw;
  template <bool NT = false>
  __device__ static Raw load_raw(const bf16_t* p) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
    return NT ? __builtin_nontemporal_load(q) : *q;
  }
  __device__ static void unpack(const Raw& w, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  template <bool NT = false>
  __device__ static void load(const bf16_t* p, float (&v)[8]) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
    const u32x4_t w = NT ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  template <bool NT = false>
  __device__ static void store(bf16_t* p, const float (&v)[8]) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    if (NT) __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
    else *reinterpret_cast<u32x4_t*>(p) = w;
  }
};
template <> struct V8<float> {
  struct Raw {
    float4 a, b;
  };
  template <bool NT = false>
  __device__ static Raw load_raw(const float* p) {
    Raw r;
    r.a = reinterpret_cast<const float4*>(p)[0];
    r.b = reinterpret_cast<const float4*>(p)[1];
    return r;
  }
  __device__ static void unpack(const Raw& r, float (&v)[8]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
  template <bool NT = false>
  __device__ static void load(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  template <bool NT = false>
  __device__ static void store(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// out[t] = shared[t] + sum_j g[t,j] y_perm[dest_pos[t*k+j]]
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* y_perm, const float* gate,
                                                      const int32_t* dest_pos, const T* shared,
                                                      int d, int k, T* out) {
  const int t = blockIdx.x;
  int rows[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? dest_pos[(size_t)t * k + j] : 0;
    g[j] = j < k ? gate[(size_t)t * k + j] : 0.0f;
  }
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        V8<T>::template load<true>(y_perm + (size_t)rows[j] * d + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += g[j] * v[i];
      }
    }
    if (shared) {
      V8<T>::template load<true>(shared + (size_t)t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    V8<T>::template store<true>(out + (size_t)t * d + c, acc);
  }
}

// dy_perm[dest_pos[t*k+j]] = g[t,j] dout[t];  dgate[t,j] = <dout[t], y_perm[dest_pos[t*k+j]]>.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* dout, const T* y_perm,
                                                          const float* gate,
                                                          const int32_t* dest_pos, int d, int k,
                                                          T* dy_perm, float* dgate) {
  __shared__ float red[4][8];
  const int t = blockIdx.x;
  int rows[8];
  float g[8], dot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? dest_pos[(size_t)t * k + j] : 0;
    g[j] = j < k ? gate[(size_t)t * k + j] : 0.0f;
    dot[j] = 0.0f;
  }
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float go[8], v[8], o[8];
    V8<T>::load(dout + (size_t)t * d + c, go);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = g[j] * go[i];
        V8<T>::store(dy_perm + (size_t)rows[j] * d + c, o);
        if (dgate) {
          V8<T>::template load<true>(y_perm + (size_t)rows[j] * d + c, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) dot[j] += go[i] * v[i];
        }
      }
    }
  }
  if (!dgate) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float s = dot[j];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) red[w][j] = s;
  }
  __syncthreads();
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    dgate[(size_t)t * k + j] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
  }
}

// The same two passes for a fixed k: every row segment a thread needs in an iteration is requested
// before any is used, so its k + 1 loads are in flight together (with k a run-time bound each load
// sat behind its own guard and the thread waited for one row at a time).  Same arithmetic, in the
// same order, as the kernels above.
template <typename T, int K>
__global__ __launch_bounds__(256) void combine_k_kernel(const T* y_perm, const float* gate, const int32_t* dest_pos,
                                                        const T* shared, int d, T* out) {
  const int t = blockIdx.x;
  int rows[K];
  float g[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = dest_pos[(size_t)t * K + j];
    g[j] = gate[(size_t)t * K + j];
  }
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    typename V8<T>::Raw raw[K], rs;
#pragma unroll
    for (int j = 0; j < K; ++j) raw[j] = V8<T>::template load_raw<true>(y_perm + (size_t)rows[j] * d + c);
    if (shared) rs = V8<T>::template load_raw<true>(shared + (size_t)t * d + c);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float v[8];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      V8<T>::unpack(raw[j], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += g[j] * v[i];
    }
    if (shared) {
      V8<T>::unpack(rs, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    V8<T>::template store<true>(out + (size_t)t * d + c, acc);
  }
}

template <typename T, int K>
__global__ __launch_bounds__(256) void combine_bwd_k_kernel(const T* dout, const T* y_perm, const float* gate,
                                                            const int32_t* dest_pos, int d, T* dy_perm,
                                                            float* dgate) {
  __shared__ float red[4][K];
  const int t = blockIdx.x;
  int rows[K];
  float g[K], dot[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = dest_pos[(size_t)t * K + j];
    g[j] = gate[(size_t)t * K + j];
    dot[j] = 0.0f;
  }
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    const typename V8<T>::Raw graw = V8<T>::load_raw(dout + (size_t)t * d + c);
    typename V8<T>::Raw yraw[K];
    if (dgate) {
#pragma unroll
      for (int j = 0; j < K; ++j) yraw[j] = V8<T>::template load_raw<true>(y_perm + (size_t)rows[j] * d + c);
    }
    float go[8], v[8], o[8];
    V8<T>::unpack(graw, go);
#pragma unroll
    for (int j = 0; j < K; ++j) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = g[j] * go[i];
      V8<T>::store(dy_perm + (size_t)rows[j] * d + c, o);
      if (dgate) {
        V8<T>::unpack(yraw[j], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) dot[j] += go[i] * v[i];
      }
    }
  }
  if (!dgate) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float s = dot[j];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) red[w][j] = s;
  }
  __syncthreads();
  if (threadIdx.x < K) {
    const int j = threadIdx.x;
    dgate[(size_t)t * K + j] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
  }
}

template <typename T>
hipError_t launch_combine_t(const T* y, const float* gate, const int32_t* dest_pos, const T* shared, int T_, int d,
                            int k, T* out, hipStream_t s) {
  switch (k) {
    case 1: hipLaunchKernelGGL((combine_k_kernel<T, 1>), dim3(T_), dim3(256), 0, s, y, gate, dest_pos, shared, d, out); break;
    case 2: hipLaunchKernelGGL((combine_k_kernel<T, 2>), dim3(T_), dim3(256), 0, s, y, gate, dest_pos, shared, d, out); break;
    case 4: hipLaunchKernelGGL((combine_k_kernel<T, 4>), dim3(T_), dim3(256), 0, s, y, gate, dest_pos, shared, d, out); break;
    case 8: hipLaunchKernelGGL((combine_k_kernel<T, 8>), dim3(T_), dim3(256), 0, s, y, gate, dest_pos, shared, d, out); break;
    default: hipLaunchKernelGGL(combine_kernel<T>, dim3(T_), dim3(256), 0, s, y, gate, dest_pos, shared, d, k, out);
  }
  return hipGetLastError();
}
template <typename T>
hipError_t launch_combine_bwd_t(const T* dout, const T* y, const float* gate, const int32_t* dest_pos, int T_, int d,
                                int k, T* dy, float* dgate, hipStream_t s) {
  switch (k) {
    case 1: hipLaunchKernelGGL((combine_bwd_k_kernel<T, 1>), dim3(T_), dim3(256), 0, s, dout, y, gate, dest_pos, d, dy, dgate); break;
    case 2: hipLaunchKernelGGL((combine_bwd_k_kernel<T, 2>), dim3(T_), dim3(256), 0, s, dout, y, gate, dest_pos, d, dy, dgate); break;
    case 4: hipLaunchKernelGGL((combine_bwd_k_kernel<T, 4>), dim3(T_), dim3(256), 0, s, dout, y, gate, dest_pos, d, dy, dgate); break;
    case 8: hipLaunchKernelGGL((combine_bwd_k_kernel<T, 8>), dim3(T_), dim3(256), 0, s, dout, y, gate, dest_pos, d, dy, dgate); break;
    default: hipLaunchKernelGGL(combine_bwd_kernel<T>, dim3(T_), dim3(256), 0, s, dout, y, gate, dest_pos, d, k, dy, dgate);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* y_perm, const float* gate, const int32_t* dest_pos,
                          const void* shared_out, int T, int d, int k, bool bf16, void* out,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    return launch_combine_t<bf16_t>(reinterpret_cast<const bf16_t*>(y_perm), gate, dest_pos,
                                    reinterpret_cast<const bf16_t*>(shared_out), T, d, k,
                                    reinterpret_cast<bf16_t*>(out), s);
  return launch_combine_t<float>(reinterpret_cast<const float*>(y_perm), gate, dest_pos,
                                 reinterpret_cast<const float*>(shared_out), T, d, k, reinterpret_cast<float*>(out), s);
}

hipError_t launch_combine_bwd(const void* dout, const void* y_perm, const float* gate,
                              const int32_t* dest_pos, int T, int d, int k, bool bf16,
                              void* dy_perm, float* dgate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    return launch_combine_bwd_t<bf16_t>(reinterpret_cast<const bf16_t*>(dout), reinterpret_cast<const bf16_t*>(y_perm),
                                        gate, dest_pos, T, d, k, reinterpret_cast<bf16_t*>(dy_perm), dgate, s);
  return launch_combine_bwd_t<float>(reinterpret_cast<const float*>(dout), reinterpret_cast<const float*>(y_perm), gate,
                                     dest_pos, T, d, k, reinterpret_cast<float*>(dy_perm), dgate, s);
}

}  // namespace moe
