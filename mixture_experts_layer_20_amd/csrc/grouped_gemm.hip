// Grouped expert GEMMs of the MoE layer for gfx950: the SwiGLU expert MLP forward and its
// dgrad/wgrad backward over expert-ragged row groups.
//
// Each routed expert owns a contiguous, ragged range of rows of the expert-major token buffer
// (tokens are moved to stationary experts: "Olmo-core 3 Opens Large MoE Training", "Technical
// Deep Dive").  Forward and dgrad GEMMs are ragged in M (rows), weight gradients are ragged in K
// (the reduction runs over the expert's rows; an expert with no rows gets zeros).
//
// bf16 path: the pipelined 256x256 kernel (grouped_gemm_pipe.hip) for every problem whose output
// columns are a multiple of 256; otherwise (d or f an odd multiple of 128) the kernel here:
// 128x128x64 workgroup tiles, 4 waves of 64x64, v_mfma_f32_32x32x16_bf16 with fp32 accumulation,
// double-buffered LDS with one barrier per K step.  Its LDS tiles are always stored K-contiguous
// ([row][k], 128-byte rows, 16-byte chunks XOR-swizzled by row) so the MFMA operand reads are
// single 16-byte loads; operands that are K-strided in memory (weights in dgrad, activations in
// wgrad) are transposed in registers on their way into LDS.
// fp32 path: a plain LDS-tiled FMA kernel with the same tile schedule and epilogues.
#include "common.h"
#include "gemm_common.h"

#include <algorithm>

namespace moe {
namespace {

using namespace gemm;

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
// bf16 MFMA kernel

constexpr int BK = 64, NTHREADS = 256, MAXG = 1024;

// LDS element offset of (row, 16-byte chunk) in a [rows][64] bf16 tile (128-byte rows).  The
// chunk is XOR-swizzled with (row & 7) ^ ((row >> 3) & 1): 16 consecutive rows read at the same
// logical chunk (one MFMA operand load of 16 lanes) then hit 16 distinct 16-byte bank groups of
// gfx950's 64-bank LDS, and any 8 consecutive rows hit 8 distinct chunks.
__host__ __device__ __forceinline__ int lds_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__host__ __device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ lds_swz(row)) << 3); }

__device__ __forceinline__ uint2 pack_lo(uint32_t a, uint32_t b, uint32_t c, uint32_t e) {
  return make_uint2((a & 0xffffu) | (b << 16), (c & 0xffffu) | (e << 16));
}
__device__ __forceinline__ uint2 pack_hi(uint32_t a, uint32_t b, uint32_t c, uint32_t e) {
  return make_uint2((a >> 16) | (b & 0xffff0000u), (c >> 16) | (e & 0xffff0000u));
}

// Write 4 k-rows x 8 columns (r[0..3], each 8 consecutive columns) into a K-contiguous LDS tile
// as 8 rows x 4 k: tile row = col0 + i, k offset = kq*4.
__device__ __forceinline__ void store_transposed(bf16_t* tile, const uint4* r, int col0, int kq) {
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
      const int off = lds_off(row, kq >> 1) + ((kq & 1) << 2);
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

// Tile configuration: BM x BN output tile, 64-deep K steps, a WGM x WGN grid of waves, each wave
// owning a (BM/WGM) x (BN/WGN) block built from 32x32x16 MFMAs.
template <int BM_, int BN_, int WGM_, int WGN_> struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int NTH = 64 * WGM * WGN;           // threads
  static constexpr int MI = BM / (32 * WGM);           // 32-row MFMA blocks per wave
  static constexpr int NI = BN / (32 * WGN);           // 32-column MFMA blocks per wave
  static constexpr int KC_ROWS = NTH / 8;              // rows per pass of a K-contiguous load
  static constexpr int MC_COLS = NTH / 2;              // columns per pass of a K-strided load
  static constexpr int LDS = 2 * (BM + BN) * BK * 2;   // double-buffered stages, bytes
  // 16-byte staging registers per thread for an R-row operand: K-contiguous loads spread the
  // R*64 elements over all threads; K-strided loads give each thread 4 k-rows x 8 columns per
  // pass of MC_COLS columns (a tile narrower than one pass leaves the remaining threads idle).
  static constexpr int nregs(bool kcontig, int R) {
    return kcontig ? R * BK / 8 / NTH : 4 * (R >= MC_COLS ? R / MC_COLS : 1);
  }
  static_assert(BM * BK / 8 % NTH == 0 && BN * BK / 8 % NTH == 0, "tile too small for the thread count");
};

// Global -> registers for one K step starting at k0.  K-contiguous operands: 8 threads per
// 128-byte row segment.  K-strided operands: each thread reads 4 consecutive k-rows x 8 columns.
template <int MODE, class C>
__device__ __forceinline__ void load_tiles(const GemmArgs& p, int g, int m0, int m_end, int nt, int k0,
                                           int k_end, int tid,
                                           uint4 (&ra)[C::nregs(Traits<MODE>::a_kcontig, C::BM)],
                                           uint4 (&rb)[C::nregs(Traits<MODE>::b_kcontig, C::BN)]) {
  typedef Traits<MODE> TR;
  constexpr int NA = C::nregs(TR::a_kcontig, C::BM), NB = C::nregs(TR::b_kcontig, C::BN);
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  if constexpr (TR::a_kcontig) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int m = m0 + i * C::KC_ROWS + (tid >> 3);
      ra[i] = m < m_end ? gload16(a_ptr_kc<MODE, bf16_t>(p, m, k0 + c * 8)) : zero4;
    }
  } else {
    const int q = tid & 15, c = tid >> 4;
#pragma unroll
    for (int ps = 0; ps < NA / 4; ++ps)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k0 + q * 4 + i;
        const int col = ps * C::MC_COLS + c * 8;
        ra[ps * 4 + i] = (k < k_end && col < C::BM) ? gload16(a_ptr_mc<MODE, bf16_t>(p, k, m0 + col)) : zero4;
      }
  }
  if constexpr (TR::b_kcontig) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = i * C::KC_ROWS + (tid >> 3);
      rb[i] = gload16(b_ptr_kc<MODE, bf16_t, C::BN>(p, g, nt, r, k0 + c * 8));
    }
  } else {
    const int q = tid & 15, c = tid >> 4;
#pragma unroll
    for (int ps = 0; ps < NB / 4; ++ps)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k0 + q * 4 + i;
        const int col = ps * C::MC_COLS + c * 8;
        rb[ps * 4 + i] = (k < k_end && col < C::BN) ? gload16(b_ptr_mc<MODE, bf16_t>(p, g, k, nt * C::BN + col)) : zero4;
      }
  }
}

// Registers -> one LDS stage (A tile [BM][64], then B tile [BN][64]).
template <int MODE, class C>
__device__ __forceinline__ void store_tiles(bf16_t* As, bf16_t* Bs, int tid,
                                            const uint4 (&ra)[C::nregs(Traits<MODE>::a_kcontig, C::BM)],
                                            const uint4 (&rb)[C::nregs(Traits<MODE>::b_kcontig, C::BN)]) {
  typedef Traits<MODE> TR;
  constexpr int NA = C::nregs(TR::a_kcontig, C::BM), NB = C::nregs(TR::b_kcontig, C::BN);
  if constexpr (TR::a_kcontig) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<uint4*>(As + lds_off(i * C::KC_ROWS + (tid >> 3), c)) = ra[i];
  } else {
#pragma unroll
    for (int ps = 0; ps < NA / 4; ++ps) {
      const int col = ps * C::MC_COLS + (tid >> 4) * 8;
      if (col < C::BM) store_transposed(As, &ra[ps * 4], col, tid & 15);
    }
  }
  if constexpr (TR::b_kcontig) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<uint4*>(Bs + lds_off(i * C::KC_ROWS + (tid >> 3), c)) = rb[i];
  } else {
#pragma unroll
    for (int ps = 0; ps < NB / 4; ++ps) {
      const int col = ps * C::MC_COLS + (tid >> 4) * 8;
      if (col < C::BN) store_transposed(Bs, &rb[ps * 4], col, tid & 15);
    }
  }
}

// Tile row of the wave's ni-th 32-column block.  The gate/up GEMM's B tile holds BN/2 W1 rows
// then the same BN/2 W3 rows; blocks ni and ni + NI/2 cover the same output columns, so a lane
// holds the gate and the up value of one output element.
template <int MODE, class C>
__device__ __forceinline__ int wave_nrow(int wn, int ni) {
  if constexpr (MODE == GEMM_UP_FWD) {
    constexpr int H = C::BN / (2 * C::WGN);   // W1 columns per wave
    return (ni < C::NI / 2) ? wn * H + 32 * ni : C::BN / 2 + wn * H + 32 * (ni - C::NI / 2);
  } else {
    return wn * (C::BN / C::WGN) + 32 * ni;
  }
}

// Per-group tile prefix in LDS (ragged-M modes): pref[g] = M-tiles of the groups before g.
template <int BMv, int NTH>
__device__ void block_tile_prefix(const GemmArgs& p, int* pref, int* scratch) {
  const int tid = threadIdx.x;
  if (tid == 0) scratch[NTH] = 0;
  __syncthreads();
  for (int base = 0; base < p.G; base += NTH) {
    const int g = base + tid;
    int c = 0;
    if (g < p.G) {
      int lo, hi;
      group_rows(p.offsets, g, p.M, lo, hi);
      c = (hi - lo + BMv - 1) / BMv;
    }
    scratch[tid] = c;
    __syncthreads();
    for (int off = 1; off < NTH; off <<= 1) {
      const int v = tid >= off ? scratch[tid - off] : 0;
      __syncthreads();
      scratch[tid] += v;
      __syncthreads();
    }
    const int carry = scratch[NTH];
    if (g < p.G) pref[g] = carry + scratch[tid] - c;
    __syncthreads();
    if (tid == NTH - 1) scratch[NTH] = carry + scratch[NTH - 1];
    __syncthreads();
  }
  if (tid == 0) pref[p.G] = scratch[NTH];
  __syncthreads();
}

// Persistent grouped GEMM.  Workgroups are dealt round-robin to the 8 XCDs (workgroup b runs on
// XCD b % 8); each XCD gets one contiguous run of logical tiles so that neighbouring tiles (same
// expert rows, next columns; then the next rows of the same expert) share operands in that XCD's
// L2.  Weight-gradient modes may split the reduction over the expert's rows into `ksplit` parts
// written as fp32 partials (summed in order afterwards).
template <int MODE, class C>
__global__ __launch_bounds__(C::NTH, 1) void grouped_gemm_bf16(GemmArgs p, int NT, int MT, int ksplit,
                                                               float* partial) {
  typedef Traits<MODE> TR;
  constexpr int BMv = C::BM, BNv = C::BN, MI = C::MI, NI = C::NI;
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  __shared__ int pref[MAXG + 1];
  __shared__ int scan_scratch[C::NTH + 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave % C::WGM, wn = wave / C::WGM;

  int total;
  if constexpr (!TR::raggedK) {
    block_tile_prefix<BMv, C::NTH>(p, pref, scan_scratch);
    total = pref[p.G] * NT;
  } else {
    total = p.G * ksplit * MT * NT;
  }
  const int per = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int nbx = gridDim.x >> 3;
  const int L_end = min(total, (xcd + 1) * per);

  for (int L = xcd * per + (blockIdx.x >> 3); L < L_end; L += nbx) {
    int g, m0, m_end, nt, k_begin, k_end, split = 0;
    if constexpr (!TR::raggedK) {
      const int mt = L / NT;
      nt = L - mt * NT;
      int lo = 0, hi = p.G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] <= mt) lo = mid; else hi = mid;
      }
      g = lo;
      int r0, r1;
      group_rows(p.offsets, g, p.M, r0, r1);
      m0 = r0 + (mt - pref[g]) * BMv;
      m_end = r1;
      k_begin = 0;
      k_end = mode_K(MODE, p.d, p.f);
    } else {
      nt = L % NT;
      int r = L / NT;
      const int mt = r % MT;
      r /= MT;
      split = r % ksplit;
      g = r / ksplit;
      m0 = mt * BMv;
      m_end = m0 + BMv;
      int r0, r1;
      group_rows(p.offsets, g, p.M, r0, r1);
      // Split s covers a contiguous, BK-aligned share of the expert's rows.
      const int chunk = ((r1 - r0 + ksplit - 1) / ksplit + BK - 1) / BK * BK;
      k_begin = min(r1, r0 + split * chunk);
      k_end = min(r1, k_begin + chunk);
    }
    const int nk = (k_end - k_begin + BK - 1) / BK;

    uint4 ra[C::nregs(TR::a_kcontig, BMv)], rb[C::nregs(TR::b_kcontig, BNv)];
    f32x16_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    if (nk > 0) {
      load_tiles<MODE, C>(p, g, m0, m_end, nt, k_begin, k_end, tid, ra, rb);
      store_tiles<MODE, C>(lds, lds + BMv * BK, tid, ra, rb);
      __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load_tiles<MODE, C>(p, g, m0, m_end, nt, k_begin + (kt + 1) * BK, k_end, tid, ra, rb);
      const bf16_t* As = lds + buf * (BMv + BNv) * BK;
      const bf16_t* Bs = As + BMv * BK;
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const int chunk = s * 2 + (lane >> 5);
        bf16x8_t af[MI], bfr[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          af[mi] = *reinterpret_cast<const bf16x8_t*>(As + lds_off(wm * (BMv / C::WGM) + mi * 32 + (lane & 31), chunk));
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          bfr[ni] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(wave_nrow<MODE, C>(wn, ni) + (lane & 31), chunk));
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
      }
      if (kt + 1 < nk) {
        bf16_t* Ns = lds + (buf ^ 1) * (BMv + BNv) * BK;
        store_tiles<MODE, C>(Ns, Ns + BMv * BK, tid, ra, rb);
      }
      __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31) and, for element v,
    // row 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * (BMv / C::WGM) + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m >= m_end) continue;
        if constexpr (MODE == GEMM_UP_FWD) {
#pragma unroll
          for (int ni = 0; ni < NI / 2; ++ni) {
            const int n = nt * (BNv / 2) + wave_nrow<MODE, C>(wn, ni) + (lane & 31);
            epilogue<MODE, bf16_t>(p, g, m, n, acc[mi][ni][v], acc[mi][ni + NI / 2][v]);
          }
        } else {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int n = nt * BNv + wave_nrow<MODE, C>(wn, ni) + (lane & 31);
            if constexpr (TR::raggedK) {
              if (ksplit > 1) {
                const int Mw = mode_Mw(MODE, p.d, p.f), Nw = mode_N(MODE, p.d, p.f);
                partial[(((size_t)split * p.G + g) * Mw + m) * Nw + n] = acc[mi][ni][v];
                continue;
              }
            }
            epilogue<MODE, bf16_t>(p, g, m, n, acc[mi][ni][v], 0.0f);
          }
        }
      }
    }
  }
}

// Sum of the split-K partials in split order, written as bf16 weight gradients (dW2, or dW1/dW3
// by gradient row).  Each thread sums 8 consecutive columns (16-byte loads, one 16-byte store).
template <int MODE>
__global__ __launch_bounds__(256) void splitk_reduce(GemmArgs p, const float* partial, int ksplit) {
  const int Mw = mode_Mw(MODE, p.d, p.f), Nw = mode_N(MODE, p.d, p.f);
  const size_t per_split = (size_t)p.G * Mw * Nw;
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8; i < per_split; i += (size_t)gridDim.x * 256 * 8) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < ksplit; ++k) {
      const float4* src = reinterpret_cast<const float4*>(partial + (size_t)k * per_split + i);
      const float4 a = src[0], b = src[1];
      s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
      s[4] += b.x; s[5] += b.y; s[6] += b.z; s[7] += b.w;
    }
    const int n = (int)(i % Nw);
    const size_t r = i / Nw;
    const int m = (int)(r % Mw);
    const int g = (int)(r / Mw);
    bf16_t* dst;
    if constexpr (MODE == GEMM_DOWN_WGRAD) {
      dst = reinterpret_cast<bf16_t*>(p.out0) + ((size_t)g * p.d + m) * p.f + n;
    } else {
      const bool up = m >= p.f;
      dst = reinterpret_cast<bf16_t*>(up ? p.out1 : p.out0) + ((size_t)g * p.f + (up ? m - p.f : m)) * p.d + n;
    }
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f32_to_bf16(s[2 * j]) | ((uint32_t)f32_to_bf16(s[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
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

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Split of the weight-gradient reduction: only when there are too few output tiles to fill the
// chip, and only as far as the workspace holds the fp32 partials.
int choose_ksplit(int tiles, int G, int M, int Mw, int Nw, size_t partial_bytes) {
  const int cus = num_cus();
  if (tiles >= 2 * cus) return 1;
  int ks = (2 * cus + tiles - 1) / tiles;
  const int rows_per_group = G > 0 ? M / G : 0;
  ks = std::min(ks, std::max(1, rows_per_group / 512));
  ks = std::min(ks, 8);
  while (ks > 1 && (size_t)ks * G * Mw * Nw * sizeof(float) > partial_bytes) --ks;
  return std::max(ks, 1);
}

template <int MODE, class C>
hipError_t launch_bf16(const GemmArgs& p, size_t partial_bytes, float* partial, hipStream_t s) {
  typedef Traits<MODE> TR;
  auto kern = grouped_gemm_bf16<MODE, C>;
  static int blocks_per_cu = 0;
  if (blocks_per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, C::NTH, C::LDS);
    if (e != hipSuccess) return e;
    blocks_per_cu = nb > 0 ? nb : 1;
  }
  const int NT = mode_N(MODE, p.d, p.f) / C::BN;
  int MT = 0, ksplit = 1;
  long long tiles;
  if constexpr (!TR::raggedK) {
    if (p.M == 0) return hipSuccess;
    if (p.G > MAXG) return hipErrorInvalidValue;
    tiles = ((long long)ceil_div(p.M, C::BM) + p.G) * NT;
  } else {
    MT = mode_Mw(MODE, p.d, p.f) / C::BM;
    tiles = (long long)p.G * MT * NT;
    ksplit = choose_ksplit((int)tiles, p.G, p.M, mode_Mw(MODE, p.d, p.f), NT * C::BN, partial_bytes);
    tiles *= ksplit;
  }
  long long grid = std::min<long long>(tiles, (long long)num_cus() * blocks_per_cu);
  grid = (grid + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NTH), C::LDS, s, p, NT, MT, ksplit, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (TR::raggedK) {
    if (ksplit > 1) {
      const size_t n = (size_t)p.G * mode_Mw(MODE, p.d, p.f) * mode_N(MODE, p.d, p.f);
      const unsigned blocks = (unsigned)std::min<size_t>((n / 8 + 255) / 256, 4096);
      hipLaunchKernelGGL(splitk_reduce<MODE>, dim3(blocks), dim3(256), 0, s, p, partial, ksplit);
      e = hipGetLastError();
    }
  }
  return e;
}

typedef Cfg<128, 128, 2, 2> T128x128;   // 4 waves of 64x64

template <int MODE>
hipError_t launch_mode(const GemmArgs& p, bool bf16, size_t partial_bytes, float* partial, hipStream_t s) {
  typedef Traits<MODE> TR;
  if (bf16) {
    // The pipelined 256x256 kernel wherever its shape rules hold (output columns a multiple of 256),
    // else the 128x128 register-staged kernel (d and f are multiples of 128).
    if (pipe_supports(MODE, p)) {
      int ksplit = 1;
      if constexpr (TR::raggedK) {
        const int Mw = mode_Mw(MODE, p.d, p.f), N = mode_N(MODE, p.d, p.f);
        ksplit = choose_ksplit(p.G * (Mw / 256) * (N / 256), p.G, p.M, Mw, N, partial_bytes);
      }
      hipError_t e = launch_grouped_gemm_pipe(MODE, p, ksplit, partial, s, num_cus());
      if (e != hipSuccess || ksplit <= 1) return e;
      const size_t n = (size_t)p.G * mode_Mw(MODE, p.d, p.f) * mode_N(MODE, p.d, p.f);
      hipLaunchKernelGGL(splitk_reduce<MODE>, dim3((unsigned)std::min<size_t>((n / 8 + 255) / 256, 4096)), dim3(256), 0,
                         s, p, partial, ksplit);
      return hipGetLastError();
    }
    return launch_bf16<MODE, T128x128>(p, partial_bytes, partial, s);
  }
  const int NT = mode_N(MODE, p.d, p.f) / FBN;
  int grid, MT = 0;
  if constexpr (!TR::raggedK) {
    if (p.M == 0) return hipSuccess;
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(256), 0, s, p.offsets, p.G, p.M, FBM, p.tile_prefix);
    grid = (int)(((long long)ceil_div(p.M, FBM) + p.G) * NT);
  } else {
    MT = mode_Mw(MODE, p.d, p.f) / FBM;
    grid = p.G * MT * NT;
  }
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_f32<MODE>, dim3(grid), dim3(256), 0, s, p, NT, MT);
  return hipGetLastError();
}

}  // namespace

size_t gemm_ws_bytes(int G) { return ((size_t)(G + 1) * sizeof(int32_t) + 255) / 256 * 256; }

// Split of the second set's row reduction in a two-set weight-gradient launch: enough chunks for
// its tiles to give every CU one (they are dealt first), chunks of at least 512 rows, at most 8.
static int sets_split(int mode, int G1, long long M1, int d, int f1) {
  const long long tiles = (long long)G1 * (mode_Mw(mode, d, f1) / 256) * (mode_N(mode, d, f1) / 256);
  if (tiles <= 0) return 1;
  long long ks = (num_cus() + tiles - 1) / tiles;
  ks = std::min<long long>(ks, M1 / std::max(1, G1) / 512);
  return (int)std::max<long long>(1, std::min<long long>(ks, 8));
}

size_t gemm_sets_partial_bytes(int G0, long long M0, int G1, long long M1, int d, int f1) {
  (void)G0; (void)M0;
  size_t best = 0;
  for (int mode : {GEMM_DOWN_WGRAD, GEMM_UP_WGRAD}) {
    const int ks = sets_split(mode, G1, M1, d, f1);
    if (ks > 1) best = std::max(best, (size_t)ks * G1 * mode_Mw(mode, d, f1) * mode_N(mode, d, f1) * sizeof(float));
  }
  return best;
}

size_t gemm_partial_bytes(int G, long long M, int d, int f) {
  size_t best = 0;
  for (int mode : {GEMM_DOWN_WGRAD, GEMM_UP_WGRAD}) {
    const int Mw = mode_Mw(mode, d, f), N = mode_N(mode, d, f);
    // smallest tile count over the shapes the launcher may pick (128x128 is the fallback)
    const int tiles = G * (Mw / 256 > 0 ? Mw / 256 : 1) * (N / 256 > 0 ? N / 256 : 1);
    const int ks = choose_ksplit(tiles, G, (int)M, Mw, N, (size_t)-1);
    if (ks > 1) best = std::max(best, (size_t)ks * G * Mw * N * sizeof(float));
  }
  return best;
}

namespace {

// Whether the two sets of p go into one launch of the pipelined kernel: it must cover both, and
// each must be a shape the single-set launcher would give it.
bool merge_sets(int mode, const GemmArgs& p) {
  if (!pipe_supports(mode, p)) return false;
  // Weight gradients: set 0 must fill the chip without a split; set 1's row reduction is split so
  // its tiles are about as long as set 0's (see launch_wgrad_sets).
  if (mode == GEMM_DOWN_WGRAD || mode == GEMM_UP_WGRAD)
    return (long long)p.G * (mode_Mw(mode, p.d, p.f) / 256) * (mode_N(mode, p.d, p.f) / 256) >= 2LL * num_cus();
  return true;
}

// Set 1 of p as a single-set problem.
GemmArgs second_set(const GemmArgs& p) {
  GemmArgs q = p;
  q.nseg = 0;
  q.a = p.s1.a;
  q.b0 = p.s1.b0;
  q.b1 = p.s1.b1;
  q.aux0 = p.s1.aux0;
  q.aux1 = p.s1.aux1;
  q.out0 = p.s1.out0;
  q.out1 = p.s1.out1;
  q.out2 = p.s1.out2;
  q.offsets = p.s1.offsets;
  q.G = p.s1.G;
  q.M = p.s1.M;
  q.f = p.s1.f;
  return q;
}

// Weight gradients of two sets in one launch.  A set's tiles reduce over its groups' rows, so the
// shared expert (all T rows in one group) would give tiles many times longer than the routed
// ones and leave most CUs idle behind them: its reduction is split into chunks about as long as a
// routed group (fp32 partials in the workspace, summed in chunk order by splitk_reduce
// afterwards, as for a split single set).
template <int MODE>
hipError_t launch_wgrad_sets(const GemmArgs& p, hipStream_t s) {
  float* partial = p.ws_bytes > gemm_ws_bytes(p.G)
                       ? reinterpret_cast<float*>(reinterpret_cast<char*>(p.tile_prefix) + gemm_ws_bytes(p.G))
                       : nullptr;
  const size_t pb = partial ? p.ws_bytes - gemm_ws_bytes(p.G) : 0;
  const int Mw = mode_Mw(MODE, p.d, p.s1.f), N = mode_N(MODE, p.d, p.s1.f);
  int ks = sets_split(MODE, p.s1.G, p.s1.M, p.d, p.s1.f);
  while (ks > 1 && (size_t)ks * p.s1.G * Mw * N * sizeof(float) > pb) --ks;
  GemmArgs q = p;
  q.s1.ksplit = ks;
  hipError_t e = launch_grouped_gemm_pipe(MODE, q, 1, partial, s, num_cus());
  if (e != hipSuccess || ks <= 1) return e;
  const GemmArgs p1 = second_set(p);
  const size_t n = (size_t)p1.G * Mw * N;
  hipLaunchKernelGGL(splitk_reduce<MODE>, dim3((unsigned)std::min<size_t>((n / 8 + 255) / 256, 4096)), dim3(256), 0, s,
                     p1, partial, ks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(int mode, const GemmArgs& p, bool bf16, hipStream_t s) {
  if (p.nseg == 2) {
    // Two sets (routed experts and the shared expert): one launch when the pipelined kernel can
    // take both, else one launch per set (same results).
    if (bf16 && merge_sets(mode, p)) {
      if (mode == GEMM_DOWN_WGRAD) return launch_wgrad_sets<GEMM_DOWN_WGRAD>(p, s);
      if (mode == GEMM_UP_WGRAD) return launch_wgrad_sets<GEMM_UP_WGRAD>(p, s);
      return launch_grouped_gemm_pipe(mode, p, 1, nullptr, s, num_cus());
    }
    GemmArgs p0 = p;
    p0.nseg = 0;
    const hipError_t e = launch_grouped_gemm(mode, p0, bf16, s);
    if (e != hipSuccess) return e;
    return launch_grouped_gemm(mode, second_set(p), bf16, s);
  }
  // Split-K partials live in the workspace after the tile prefix.
  float* partial = p.ws_bytes > gemm_ws_bytes(p.G)
                       ? reinterpret_cast<float*>(reinterpret_cast<char*>(p.tile_prefix) + gemm_ws_bytes(p.G))
                       : nullptr;
  const size_t pb = partial ? p.ws_bytes - gemm_ws_bytes(p.G) : 0;
  switch (mode) {
    case GEMM_UP_FWD: return launch_mode<GEMM_UP_FWD>(p, bf16, pb, partial, s);
    case GEMM_DOWN_FWD: return launch_mode<GEMM_DOWN_FWD>(p, bf16, pb, partial, s);
    case GEMM_DOWN_BWD: return launch_mode<GEMM_DOWN_BWD>(p, bf16, pb, partial, s);
    case GEMM_UP_DGRAD: return launch_mode<GEMM_UP_DGRAD>(p, bf16, pb, partial, s);
    case GEMM_DOWN_WGRAD: return launch_mode<GEMM_DOWN_WGRAD>(p, bf16, pb, partial, s);
    case GEMM_UP_WGRAD: return launch_mode<GEMM_UP_WGRAD>(p, bf16, pb, partial, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
