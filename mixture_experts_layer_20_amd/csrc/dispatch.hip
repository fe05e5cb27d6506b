// Token dispatch of the MoE layer: per-expert histogram, exclusive prefix sum, stable
// permutation to an expert-major layout and the row gather; plus the gather's backward.
//
// Tokens are moved to experts that stay in place ("Olmo-core 3 Opens Large MoE Training",
// "Enhanced Key Takeaways" and "Technical Deep Dive").  The permutation is a stable counting sort
// of the (token, slot) assignments by expert, so within an expert rows keep ascending token
// order.  Ranks come from wavefront ballots and a scan, never from atomic slot claims, so every
// output is deterministic.
#include "common.h"

namespace moe {
namespace {

constexpr int CH_THREADS = 256;
constexpr int CH_PER_THREAD = 4;
constexpr int CHUNK = CH_THREADS * CH_PER_THREAD;  // assignments per chunk (1024)

// Pass 1.  Each block ranks the assignments of one chunk among equal experts, in assignment
// order.  Wave w takes the contiguous quarter [w*256, (w+1)*256) of the chunk in 4 steps of 64; inside a step the rank of a lane is the number of lower lanes with the same expert, found
// from ballots of the expert id's bits.  Afterwards the per-wave counts are prefix-summed so the
// rank is the chunk-local stable rank.  Writes local_rank[a] and chunk_counts[chunk][E].
__global__ __launch_bounds__(CH_THREADS) void local_rank_kernel(const int32_t* topk_idx, int Tk,
                                                                int E, int nbits,
                                                                int32_t* local_rank,
                                                                int32_t* chunk_counts) {
  __shared__ int cnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 4 * 256; i += CH_THREADS) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int base = blockIdx.x * CHUNK + w * (CHUNK / 4);
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int ev[CH_PER_THREAD], rk[CH_PER_THREAD], ld[CH_PER_THREAD];
  // All of the thread's expert ids first: the wave barriers below would otherwise keep each step's
  // load behind the previous step's counter update (one memory latency per step).
#pragma unroll
  for (int it = 0; it < CH_PER_THREAD; ++it) {
    const int a = base + it * 64 + lane;
    ld[it] = topk_idx[min(a, Tk - 1)];   // unconditional (clamped), so the loads stay in flight together
  }
#pragma unroll
  for (int it = 0; it < CH_PER_THREAD; ++it) {
    const int a = base + it * 64 + lane;
    const bool valid = a < Tk;
    const int e = ld[it];
    unsigned long long peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int before = __popcll(peers & lt);
    int r = 0;
    if (valid) r = cnt[w][e] + before;
    // The highest lane of each group of equal experts advances the wave's counter.
    const bool leader = valid && ((peers >> lane) == 1ull);
    __builtin_amdgcn_wave_barrier();
    if (leader) cnt[w][e] = r + 1;
    __builtin_amdgcn_wave_barrier();
    ev[it] = valid ? e : -1;
    rk[it] = r;
  }
  __syncthreads();
  // Exclusive prefix over the four waves, per expert; chunk totals.
  for (int e = tid; e < E; e += CH_THREADS) {
    int run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = cnt[q][e];
      cnt[q][e] = run;
      run += c;
    }
    chunk_counts[(size_t)blockIdx.x * E + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < CH_PER_THREAD; ++it) {
    const int a = base + it * 64 + lane;
    if (ev[it] >= 0) local_rank[a] = rk[it] + cnt[w][ev[it]];
  }
}

// Pass 2.  One block: counts, offsets, and the first row of every (chunk, expert) pair.  The
// chunk counts are staged in LDS ([chunk][expert]), each expert's column is prefix-summed by one
// thread, the expert totals by the block, and the results go back out in one coalesced pass.
constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_LDS = 12288;   // staged counts (ints); larger problems take the plain scan
__global__ __launch_bounds__(SCAN_THREADS) void scan_lds_kernel(const int32_t* chunk_counts, int nch, int E,
                                                                 int Tk, int32_t* counts, int32_t* offsets,
                                                                 int32_t* chunk_base) {
  __shared__ int cc[SCAN_LDS];
  __shared__ int tot[SCAN_THREADS];
  const int tid = threadIdx.x, n = nch * E;
  for (int i = tid; i < n; i += SCAN_THREADS) cc[i] = chunk_counts[i];
  __syncthreads();
  int total = 0;
  if (tid < E) {
    for (int c = 0; c < nch; ++c) {
      const int v = cc[c * E + tid];
      cc[c * E + tid] = total;
      total += v;
    }
  }
  tot[tid] = total;
  __syncthreads();
  for (int off = 1; off < SCAN_THREADS; off <<= 1) {
    const int v = tid >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    counts[tid] = total;
    offsets[tid] = tot[tid] - total;
  }
  if (tid == 0) offsets[E] = Tk;
  for (int i = tid; i < n; i += SCAN_THREADS) {
    const int e = i % E;
    chunk_base[i] = cc[i] + (e > 0 ? tot[e - 1] : 0);
  }
}

// The same for any size, with the counts left in global memory.
__global__ __launch_bounds__(256) void scan_kernel(const int32_t* chunk_counts, int nch, int E,
                                                   int Tk, int32_t* counts, int32_t* offsets,
                                                   int32_t* chunk_base) {
  __shared__ int s[256];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
#pragma unroll 8
    for (int c = 0; c < nch; ++c) {
      const int v = chunk_counts[(size_t)c * E + e];
      chunk_base[(size_t)c * E + e] = total;
      total += v;
    }
  }
  s[e] = total;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  const int excl = s[e] - total;
  if (e < E) {
    counts[e] = total;
    offsets[e] = excl;
    for (int c = 0; c < nch; ++c) chunk_base[(size_t)c * E + e] += excl;
  }
  if (e == 0) offsets[E] = Tk;
}

// Pass 3.  dest_pos, src_row, and (optionally) the row copy x_perm[dest] = x[a / k].
// One block per token: its k destinations first, then the row is read once (16 bytes per thread)
// and written to each destination.
template <typename T>
__global__ __launch_bounds__(256) void scatter_gather_kernel(const T* x, const int32_t* topk_idx,
                                                             const int32_t* local_rank,
                                                             const int32_t* chunk_base, int Tk,
                                                             int d, int E, int k,
                                                             int32_t* dest_pos, int32_t* src_row,
                                                             T* x_perm) {
  __shared__ int dst_s[8];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    const int a = t * k + threadIdx.x;
    const int e = topk_idx[a];
    const int dst = chunk_base[(size_t)(a / CHUNK) * E + e] + local_rank[a];
    dest_pos[a] = dst;
    src_row[dst] = a;
    dst_s[threadIdx.x] = dst;
  }
  if (x_perm == nullptr) return;
  __syncthreads();
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte vector
  const int nv = d / V;
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * d);
  for (int c = threadIdx.x; c < nv; c += 256) {
    const uint4 v = src[c];
    for (int j = 0; j < k; ++j) reinterpret_cast<uint4*>(x_perm + (size_t)dst_s[j] * d)[c] = v;
  }
}

// Passes 2 and 3 in one launch, for problems whose chunk counts fit in LDS (nch * E <= FUSED_LDS).
// Each block takes GT consecutive tokens: it issues the loads of their rows first, then derives
// from all chunk counts the first row of each (chunk, expert) pair for the (at most two) chunks
// its assignments fall in (the scan of pass 2, recomputed per block from 32 KiB of counts), writes
// dest_pos and src_row, and stores each row at its k destinations.  Block 0 also writes counts and
// offsets.
typedef uint32_t v4u32_t __attribute__((ext_vector_type(4)));   // native vector: stays in registers
constexpr int GT = 8;              // tokens per block of the fused pass
constexpr int FUSED_LDS = 8192;    // chunk counts (ints) staged per block
constexpr int FUSED_MAXV = 2;      // 16-byte row pieces per thread and token (d * esize <= 8 KiB)
template <typename T>
__global__ __launch_bounds__(256) void scan_gather_kernel(const T* x, const int32_t* topk_idx,
                                                          const int32_t* local_rank,
                                                          const int32_t* chunk_counts, int nch, int T_, int d,
                                                          int E, int k, int32_t* counts, int32_t* offsets,
                                                          int32_t* dest_pos, int32_t* src_row, T* x_perm) {
  __shared__ __attribute__((aligned(16))) int cc[FUSED_LDS];
  __shared__ int tot[256];
  __shared__ int base_s[2][256];
  __shared__ int dst_s[GT * 8];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * GT, nt = min(GT, T_ - t0);
  const int Tk = T_ * k;
  constexpr int V = 16 / sizeof(T);
  const int nv = x_perm ? d / V : 0;
  // 1. the block's rows into registers (independent of everything below).  Loads are unconditional
  // (token and piece indices clamped) so the row array stays in registers.
  v4u32_t row[GT][FUSED_MAXV];
  const int nvl = max(nv, 1);
#pragma unroll
  for (int i = 0; i < GT; ++i)
#pragma unroll
    for (int q = 0; q < FUSED_MAXV; ++q) {
      const v4u32_t* src = reinterpret_cast<const v4u32_t*>(x + (size_t)(t0 + min(i, nt - 1)) * d);
      row[i][q] = src[min(tid + q * 256, nvl - 1)];
    }
  // 2. counts -> per-expert totals -> offsets; first rows of the block's chunks
  // counts: 16-byte loads, all of a round issued before any is stored (one wait per round)
  const int n = nch * E, n4 = n / 4;
  const int4* cc4 = reinterpret_cast<const int4*>(chunk_counts);
  for (int b = 0; b < n4; b += 4 * 256) {
    int4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = cc4[min(b + u * 256 + tid, n4 - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (b + u * 256 + tid < n4) reinterpret_cast<int4*>(cc)[b + u * 256 + tid] = v[u];
  }
  for (int i = 4 * n4 + tid; i < n; i += 256) cc[i] = chunk_counts[i];
  __syncthreads();
  const int c0 = (t0 * k) / CHUNK;
  int total = 0, below0 = 0, below1 = 0;
  if (tid < E) {
    for (int c = 0; c < nch; ++c) {
      const int v = cc[c * E + tid];
      if (c < c0) below0 += v;
      if (c < c0 + 1) below1 += v;
      total += v;
    }
  }
  tot[tid] = total;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    const int excl = tot[tid] - total;
    base_s[0][tid] = excl + below0;
    base_s[1][tid] = excl + below1;
    if (blockIdx.x == 0) {
      counts[tid] = total;
      offsets[tid] = excl;
    }
  }
  if (blockIdx.x == 0 && tid == 0) offsets[E] = Tk;
  __syncthreads();
  // 3. destinations of the block's assignments
  if (tid < nt * k) {
    // An expert index outside [0, E) (not produced by moe_route) gives an unspecified permutation,
    // but every access stays inside the buffers.
    const int a = t0 * k + tid;
    const int e = min(max(topk_idx[a], 0), E - 1);
    const int dst = min(max(base_s[a / CHUNK - c0][e] + local_rank[a], 0), Tk - 1);
    dest_pos[a] = dst;
    src_row[dst] = a;
    dst_s[tid] = dst;
  }
  if (x_perm == nullptr) return;
  __syncthreads();
  // 4. each row to its k destinations
  for (int j = 0; j < k; ++j) {   // slot-major: the row array is indexed at compile time
#pragma unroll
    for (int i = 0; i < GT; ++i) {
      if (i < nt) {
        v4u32_t* dst = reinterpret_cast<v4u32_t*>(x_perm + (size_t)dst_s[i * k + j] * d);
#pragma unroll
        for (int q = 0; q < FUSED_MAXV; ++q)
          if (tid + q * 256 < nv) dst[tid + q * 256] = row[i][q];
      }
    }
  }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 8 consecutive elements as fp32.  NT: a stream nothing later in the layer pass reads again (a
// nontemporal access, which does not displace reused data from the caches).
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
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
template <> struct Vec8<float> {
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

// dx[t] = sum_j dx_perm[dest_pos[t*k+j]] + add0[t] + add1[t], fp32 sums, one block per token.
template <typename T>
__global__ __launch_bounds__(256) void permute_bwd_kernel(const T* dx_perm, const int32_t* dest_pos,
                                                          const T* add0, const T* add1, int d,
                                                          int k, T* dx) {
  const int t = blockIdx.x;
  int rows[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rows[j] = j < k ? dest_pos[(size_t)t * k + j] : 0;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        Vec8<T>::template load<true>(dx_perm + (size_t)rows[j] * d + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    }
    if (add0) {
      Vec8<T>::template load<true>(add0 + (size_t)t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (add1) {
      Vec8<T>::template load<true>(add1 + (size_t)t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    Vec8<T>::template store<true>(dx + (size_t)t * d + c, acc);
  }
}

// The same for a fixed k: the k gathered segments and the addends of an iteration are all requested
// before any is used (k + 2 loads in flight together); same sums in the same order.
template <typename T, int K>
__global__ __launch_bounds__(256) void permute_bwd_k_kernel(const T* dx_perm, const int32_t* dest_pos,
                                                            const T* add0, const T* add1, int d, T* dx) {
  const int t = blockIdx.x;
  int rows[K];
#pragma unroll
  for (int j = 0; j < K; ++j) rows[j] = dest_pos[(size_t)t * K + j];
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    typename Vec8<T>::Raw raw[K], r0, r1;
#pragma unroll
    for (int j = 0; j < K; ++j) raw[j] = Vec8<T>::template load_raw<true>(dx_perm + (size_t)rows[j] * d + c);
    if (add0) r0 = Vec8<T>::template load_raw<true>(add0 + (size_t)t * d + c);
    if (add1) r1 = Vec8<T>::template load_raw<true>(add1 + (size_t)t * d + c);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float v[8];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      Vec8<T>::unpack(raw[j], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (add0) {
      Vec8<T>::unpack(r0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (add1) {
      Vec8<T>::unpack(r1, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    Vec8<T>::template store<true>(dx + (size_t)t * d + c, acc);
  }
}

template <typename T>
void launch_permute_bwd_t(const T* dx_perm, const int32_t* dest_pos, const T* add0, const T* add1, int T_, int d,
                          int k, T* dx, hipStream_t s) {
  switch (k) {
    case 1: hipLaunchKernelGGL((permute_bwd_k_kernel<T, 1>), dim3(T_), dim3(256), 0, s, dx_perm, dest_pos, add0, add1, d, dx); break;
    case 2: hipLaunchKernelGGL((permute_bwd_k_kernel<T, 2>), dim3(T_), dim3(256), 0, s, dx_perm, dest_pos, add0, add1, d, dx); break;
    case 4: hipLaunchKernelGGL((permute_bwd_k_kernel<T, 4>), dim3(T_), dim3(256), 0, s, dx_perm, dest_pos, add0, add1, d, dx); break;
    case 8: hipLaunchKernelGGL((permute_bwd_k_kernel<T, 8>), dim3(T_), dim3(256), 0, s, dx_perm, dest_pos, add0, add1, d, dx); break;
    default: hipLaunchKernelGGL(permute_bwd_kernel<T>, dim3(T_), dim3(256), 0, s, dx_perm, dest_pos, add0, add1, d, k, dx);
  }
}

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t permute_ws_bytes(long long T, int E, int k) {
  const long long Tk = T * k;
  const long long nch = (Tk + CHUNK - 1) / CHUNK;
  return 2 * align256((size_t)nch * E * sizeof(int32_t)) + align256((size_t)Tk * sizeof(int32_t));
}

hipError_t launch_permute(const void* x, const int32_t* topk_idx, int T, int d, int E, int k,
                          bool bf16, int32_t* counts, int32_t* offsets, int32_t* dest_pos,
                          int32_t* src_row, void* x_perm, void* ws, hipStream_t s) {
  const int Tk = T * k;
  const int nch = ceil_div(Tk, CHUNK);
  char* p = reinterpret_cast<char*>(ws);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)nch * E * sizeof(int32_t));
  int32_t* chunk_base = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)nch * E * sizeof(int32_t));
  int32_t* local_rank = reinterpret_cast<int32_t*>(p);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (Tk > 0)
    hipLaunchKernelGGL(local_rank_kernel, dim3(nch), dim3(CH_THREADS), 0, s, topk_idx, Tk, E, nbits,
                       local_rank, chunk_counts);
  const size_t esz = bf16 ? 2 : 4;
  if (Tk > 0 && (long long)nch * E <= FUSED_LDS && E <= 256 && k <= 8 && (d * esz) % 16 == 0 &&
      d * esz <= (size_t)FUSED_MAXV * 256 * 16) {
    if (bf16)
      hipLaunchKernelGGL(scan_gather_kernel<bf16_t>, dim3(ceil_div(T, GT)), dim3(256), 0, s,
                         reinterpret_cast<const bf16_t*>(x), topk_idx, local_rank, chunk_counts, nch, T, d, E, k,
                         counts, offsets, dest_pos, src_row, reinterpret_cast<bf16_t*>(x_perm));
    else
      hipLaunchKernelGGL(scan_gather_kernel<float>, dim3(ceil_div(T, GT)), dim3(256), 0, s,
                         reinterpret_cast<const float*>(x), topk_idx, local_rank, chunk_counts, nch, T, d, E, k,
                         counts, offsets, dest_pos, src_row, reinterpret_cast<float*>(x_perm));
    return hipGetLastError();
  }
  if ((long long)nch * E <= SCAN_LDS && E <= SCAN_THREADS)
    hipLaunchKernelGGL(scan_lds_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, chunk_counts, nch, E, Tk, counts,
                       offsets, chunk_base);
  else
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, chunk_counts, nch, E, Tk, counts, offsets,
                       chunk_base);
  if (Tk > 0) {
    if (bf16)
      hipLaunchKernelGGL(scatter_gather_kernel<bf16_t>, dim3(T), dim3(256), 0, s,
                         reinterpret_cast<const bf16_t*>(x), topk_idx, local_rank, chunk_base, Tk, d,
                         E, k, dest_pos, src_row, reinterpret_cast<bf16_t*>(x_perm));
    else
      hipLaunchKernelGGL(scatter_gather_kernel<float>, dim3(T), dim3(256), 0, s,
                         reinterpret_cast<const float*>(x), topk_idx, local_rank, chunk_base, Tk, d,
                         E, k, dest_pos, src_row, reinterpret_cast<float*>(x_perm));
  }
  return hipGetLastError();
}

hipError_t launch_permute_bwd(const void* dx_perm, const int32_t* dest_pos, const void* add0,
                              const void* add1, int T, int d, int k, bool bf16, void* dx,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    launch_permute_bwd_t<bf16_t>(reinterpret_cast<const bf16_t*>(dx_perm), dest_pos,
                                 reinterpret_cast<const bf16_t*>(add0), reinterpret_cast<const bf16_t*>(add1), T, d, k,
                                 reinterpret_cast<bf16_t*>(dx), s);
  else
    launch_permute_bwd_t<float>(reinterpret_cast<const float*>(dx_perm), dest_pos,
                                reinterpret_cast<const float*>(add0), reinterpret_cast<const float*>(add1), T, d, k,
                                reinterpret_cast<float*>(dx), s);
  return hipGetLastError();
}

}  // namespace moe
