// Grouped expert GEMMs of the MoE layer for gfx950: the SwiGLU expert MLP forward and its
// dgrad/wgrad backward over expert-ragged row groups.
//
// Each routed expert owns a contiguous, ragged range of rows of the expert-major token buffer
// (tokens are moved to stationary experts: "Olmo-core 3 Opens Large MoE Training", "Technical
// Deep Dive").  Forward and dgrad GEMMs are ragged in M (rows), weight gradients are ragged in K
// (the reduction runs over the expert's rows; an expert with no rows gets zeros).
//
// bf16 path: 128x128x64 workgroup tiles, 4 waves of 64x64, v_mfma_f32_32x32x16_bf16 with fp32
// accumulation, double-buffered LDS with one barrier per K step.  LDS tiles are always stored
// K-contiguous ([row][k], 128-byte rows, 16-byte chunks XOR-swizzled by row) so the MFMA operand
// reads are single 16-byte loads; operands that are K-strided in memory (weights in dgrad,
// activations in wgrad) are transposed in registers on their way into LDS.
// fp32 path: a plain LDS-tiled FMA kernel with the same tile schedule and epilogues.
#include "common.h"

namespace moe {
namespace {

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

// M-tiles per group, exclusive prefix over groups, one block.
__global__ void tile_prefix_kernel(const int32_t* offsets, int G, int M, int bm, int32_t* prefix) {
  __shared__ int s[256];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < G; base += 256) {
    const int g = base + tid;
    int c = 0;
    if (g < G) {
      int lo, hi;
      group_rows(offsets, g, M, lo, hi);
      c = (hi - lo + bm - 1) / bm;
    }
    s[tid] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive scan
      const int v = tid >= off ? s[tid - off] : 0;
      __syncthreads();
      s[tid] += v;
      __syncthreads();
    }
    const int carry = carry_s;
    if (g < G) prefix[g] = carry + s[tid] - c;
    __syncthreads();
    if (tid == 255) carry_s = carry + s[255];
    __syncthreads();
  }
  if (tid == 0) prefix[G] = carry_s;
}

// Tile decode for the ragged-M modes.  Workgroups are dealt round-robin to the 8 XCDs
// (workgroup i runs on XCD i % 8), so the logical tile order is remapped to give every XCD one
// contiguous run of tiles: neighbouring tiles (same rows, next columns; then the next rows of the
// same expert) share operands through that XCD's L2.  Returns false for workgroups without work.
template <int BMv>
__device__ __forceinline__ bool decode_ragged_m(const GemmArgs& p, int NT, bool xcd_remap, int& g,
                                                int& m0, int& m_end, int& nt) {
  const int TM = p.tile_prefix[p.G];
  const int real = TM * NT;
  int L;
  if (xcd_remap) {
    const int per = (real + 7) >> 3;
    const int i = blockIdx.x, x = i & 7, j = i >> 3;
    if (j >= per) return false;
    L = x * per + j;
  } else {
    L = blockIdx.x;
  }
  if (L >= real) return false;
  const int mt = L / NT;
  nt = L - mt * NT;
  int lo = 0, hi = p.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_prefix[mid] <= mt) lo = mid; else hi = mid;
  }
  g = lo;
  int r0, r1;
  group_rows(p.offsets, g, p.M, r0, r1);
  m0 = r0 + (mt - p.tile_prefix[g]) * BMv;
  m_end = r1;
  return true;
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

// --------------------------------------------------------------------------------------------
// bf16 MFMA kernel

constexpr int BM = 128, BN = 128, BK = 64, NTHREADS = 256;

// LDS element offset of (row, 16-byte chunk) in a [rows][64] bf16 tile, chunk XOR-swizzled by row.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

__device__ __forceinline__ uint2 pack_lo(uint32_t a, uint32_t b, uint32_t c, uint32_t e) {
  return make_uint2((a & 0xffffu) | (b << 16), (c & 0xffffu) | (e << 16));
}
__device__ __forceinline__ uint2 pack_hi(uint32_t a, uint32_t b, uint32_t c, uint32_t e) {
  return make_uint2((a >> 16) | (b & 0xffff0000u), (c >> 16) | (e & 0xffff0000u));
}

// Write 4 k-rows x 8 columns (r[0..3], each 8 consecutive columns) into a K-contiguous LDS tile
// as 8 rows x 4 k: tile row = col0 + i, k offset = kq*4.
__device__ __forceinline__ void store_transposed(bf16_t* tile, const uint4 (&r)[4], int col0, int kq) {
  const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
  const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
  const uint32_t w2[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
  const uint32_t w3[4] = {r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = col0 + 2 * w + h;
      const uint2 v = h == 0 ? pack_lo(w0[w], w1[w], w2[w], w3[w]) : pack_hi(w0[w], w1[w], w2[w], w3[w]);
      const int off = row * BK + ((((kq >> 1) ^ (row & 7))) << 3) + ((kq & 1) << 2);
      *reinterpret_cast<uint2*>(tile + off) = v;
    }
  }
}

// 16-byte load through the global address space.
__device__ __forceinline__ uint4 gload16(const void* ptr) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef const __attribute__((address_space(1))) uint4* gptr_t;
  return *(gptr_t)(ptr);
#else
  return *reinterpret_cast<const uint4*>(ptr);
#endif
}

// Global -> registers for the K step starting at k0.
template <int MODE>
__device__ __forceinline__ void load_tiles(const GemmArgs& p, int g, int m0, int m_end, int nt, int k0,
                                           int k_end, int tid, uint4 (&ra)[4], uint4 (&rb)[4]) {
  typedef Traits<MODE> TR;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  if constexpr (TR::a_kcontig) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + i * 32 + (tid >> 3);
      ra[i] = m < m_end ? gload16(a_ptr_kc<MODE, bf16_t>(p, m, k0 + c * 8)) : zero4;
    }
  } else {
    const int q = tid & 15, c = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + q * 4 + i;
      ra[i] = k < k_end ? gload16(a_ptr_mc<MODE, bf16_t>(p, k, m0 + c * 8)) : zero4;
    }
  }
  if constexpr (TR::b_kcontig) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 32 + (tid >> 3);
      rb[i] = gload16(b_ptr_kc<MODE, bf16_t, BN>(p, g, nt, r, k0 + c * 8));
    }
  } else {
    const int q = tid & 15, c = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + q * 4 + i;
      rb[i] = k < k_end ? gload16(b_ptr_mc<MODE, bf16_t>(p, g, k, nt * BN + c * 8)) : zero4;
    }
  }
}

// Registers -> one LDS buffer (A tile, B tile).
template <int MODE>
__device__ __forceinline__ void store_tiles(bf16_t* As, bf16_t* Bs, int tid, const uint4 (&ra)[4],
                                            const uint4 (&rb)[4]) {
  typedef Traits<MODE> TR;
  if constexpr (TR::a_kcontig) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(As + lds_off(i * 32 + (tid >> 3), c)) = ra[i];
  } else {
    store_transposed(As, ra, (tid >> 4) * 8, tid & 15);
  }
  if constexpr (TR::b_kcontig) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(Bs + lds_off(i * 32 + (tid >> 3), c)) = rb[i];
  } else {
    store_transposed(Bs, rb, (tid >> 4) * 8, tid & 15);
  }
}

template <int MODE>
__global__ __launch_bounds__(NTHREADS) void grouped_gemm_bf16(GemmArgs p, int NT, int MT) {
  typedef Traits<MODE> TR;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][2][BM * BK];

  const int tid = threadIdx.x;
  int g, m0, m_end, nt, k_begin, k_end;
  if constexpr (!TR::raggedK) {
    if (!decode_ragged_m<BM>(p, NT, true, g, m0, m_end, nt)) return;
    k_begin = 0;
    k_end = mode_K(MODE, p.d, p.f);
  } else {
    const int L = blockIdx.x;
    nt = L % NT;
    const int r = L / NT;
    const int mt = r % MT;
    g = r / MT;
    m0 = mt * BM;
    m_end = m0 + BM;
    group_rows(p.offsets, g, p.M, k_begin, k_end);
  }
  const int nk = (k_end - k_begin + BK - 1) / BK;

  uint4 ra[4], rb[4];
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  // Tile rows of the wave's two 32-column blocks.  The gate/up GEMM pairs W1 column block
  // (rows [0, 64) of the B tile) with the same W3 block (rows [64, 128)), so one lane holds
  // A and B of the same output element.
  const int nb0 = MODE == GEMM_UP_FWD ? wn * 32 : wn * 64;
  const int nb1 = MODE == GEMM_UP_FWD ? 64 + wn * 32 : wn * 64 + 32;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  if (nk > 0) {
    load_tiles<MODE>(p, g, m0, m_end, nt, k_begin, k_end, tid, ra, rb);
    store_tiles<MODE>(lds[0][0], lds[0][1], tid, ra, rb);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles<MODE>(p, g, m0, m_end, nt, k_begin + (kt + 1) * BK, k_end, tid, ra, rb);
    const bf16_t* As = lds[buf][0];
    const bf16_t* Bs = lds[buf][1];
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int chunk = s * 2 + (lane >> 5);
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int row = wm * 64 + mi * 32 + (lane & 31);
        af[mi] = *reinterpret_cast<const bf16x8_t*>(As + lds_off(row, chunk));
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = (ni == 0 ? nb0 : nb1) + (lane & 31);
        bfr[ni] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(row, chunk));
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles<MODE>(lds[buf ^ 1][0], lds[buf ^ 1][1], tid, ra, rb);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31) and, for element v,
  // row 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (m >= m_end) continue;
      if constexpr (MODE == GEMM_UP_FWD) {
        const int n = nt * (BN / 2) + wn * 32 + (lane & 31);
        epilogue<MODE, bf16_t>(p, g, m, n, acc[mi][0][v], acc[mi][1][v]);
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int n = nt * BN + (ni == 0 ? nb0 : nb1) + (lane & 31);
          epilogue<MODE, bf16_t>(p, g, m, n, acc[mi][ni][v], 0.0f);
        }
      }
    }
  }
}

// --------------------------------------------------------------------------------------------
// fp32 kernel: 64x64x16 tiles, 256 threads, 4x4 outputs per thread, plain FMAs.

constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int MODE>
__device__ __forceinline__ float load_a_f32(const GemmArgs& p, int m, int k, bool ok) {
  if (!ok) return 0.0f;
  if constexpr (Traits<MODE>::a_kcontig) return *a_ptr_kc<MODE, float>(p, m, k);
  else return *a_ptr_mc<MODE, float>(p, k, m);
}
template <int MODE>
__device__ __forceinline__ float load_b_f32(const GemmArgs& p, int g, int nt, int r, int k, bool ok) {
  if (!ok) return 0.0f;
  if constexpr (Traits<MODE>::b_kcontig) return *b_ptr_kc<MODE, float, FBN>(p, g, nt, r, k);
  else return *b_ptr_mc<MODE, float>(p, g, k, nt * FBN + r);
}

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(GemmArgs p, int NT, int MT) {
  typedef Traits<MODE> TR;
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  const int tid = threadIdx.x;
  int g, m0, m_end, nt, k_begin, k_end;
  if constexpr (!TR::raggedK) {
    if (!decode_ragged_m<FBM>(p, NT, false, g, m0, m_end, nt)) return;
    k_begin = 0;
    k_end = mode_K(MODE, p.d, p.f);
  } else {
    const int L = blockIdx.x;
    nt = L % NT;
    const int r = L / NT;
    const int mt = r % MT;
    g = r / MT;
    m0 = mt * FBM;
    m_end = m0 + FBM;
    group_rows(p.offsets, g, p.M, k_begin, k_end);
  }
  const int tx = tid & 15, ty = tid >> 4;
  // Tile column of the thread's j-th output.  Gate/up: columns j and j+2 are the W1 and W3
  // values of the same output element.
  auto col_of = [&](int j) {
    if constexpr (MODE == GEMM_UP_FWD) return (j < 2 ? 0 : FBN / 2) + tx * 2 + (j & 1);
    else return tx * 4 + j;
  };
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = k_begin; k0 < k_end; k0 += FBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      // A tile: K-contiguous sources walk k fastest, K-strided ones walk rows fastest.
      int r, kk;
      if constexpr (TR::a_kcontig) { r = e / FBK; kk = e % FBK; } else { r = e % FBM; kk = e / FBM; }
      const int m = m0 + r, k = k0 + kk;
      As[kk][r] = load_a_f32<MODE>(p, m, k, m < m_end && k < k_end);
      int rb, kb;
      if constexpr (TR::b_kcontig) { rb = e / FBK; kb = e % FBK; } else { rb = e % FBN; kb = e / FBN; }
      Bs[kb][rb] = load_b_f32<MODE>(p, g, nt, rb, k0 + kb, k0 + kb < k_end);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][col_of(j)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= m_end) continue;
    if constexpr (MODE == GEMM_UP_FWD) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = nt * (FBN / 2) + tx * 2 + j;
        epilogue<MODE, float>(p, g, m, n, acc[i][j], acc[i][j + 2]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) epilogue<MODE, float>(p, g, m, nt * FBN + tx * 4 + j, acc[i][j], 0.0f);
    }
  }
}

template <int MODE>
hipError_t launch_mode(const GemmArgs& p, bool bf16, hipStream_t s) {
  typedef Traits<MODE> TR;
  const int bm = bf16 ? BM : FBM, bn = bf16 ? BN : FBN;
  const int NT = mode_N(MODE, p.d, p.f) / bn;
  int grid, MT = 0;
  if constexpr (!TR::raggedK) {
    if (p.M == 0) return hipSuccess;
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(256), 0, s, p.offsets, p.G, p.M, bm,
                       p.tile_prefix);
    long long tiles = ((long long)ceil_div(p.M, bm) + p.G) * NT;
    tiles = (tiles + 7) / 8 * 8;
    grid = (int)tiles;
  } else {
    MT = mode_Mw(MODE, p.d, p.f) / bm;
    grid = p.G * MT * NT;
  }
  if (grid <= 0) return hipSuccess;
  if (bf16) hipLaunchKernelGGL(grouped_gemm_bf16<MODE>, dim3(grid), dim3(NTHREADS), 0, s, p, NT, MT);
  else hipLaunchKernelGGL(grouped_gemm_f32<MODE>, dim3(grid), dim3(256), 0, s, p, NT, MT);
  return hipGetLastError();
}

}  // namespace

size_t gemm_ws_bytes(int G) { return ((size_t)(G + 1) * sizeof(int32_t) + 255) / 256 * 256; }

hipError_t launch_grouped_gemm(int mode, const GemmArgs& p, bool bf16, hipStream_t s) {
  switch (mode) {
    case GEMM_UP_FWD: return launch_mode<GEMM_UP_FWD>(p, bf16, s);
    case GEMM_DOWN_FWD: return launch_mode<GEMM_DOWN_FWD>(p, bf16, s);
    case GEMM_DOWN_BWD: return launch_mode<GEMM_DOWN_BWD>(p, bf16, s);
    case GEMM_UP_DGRAD: return launch_mode<GEMM_UP_DGRAD>(p, bf16, s);
    case GEMM_DOWN_WGRAD: return launch_mode<GEMM_DOWN_WGRAD>(p, bf16, s);
    case GEMM_UP_WGRAD: return launch_mode<GEMM_UP_WGRAD>(p, bf16, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
