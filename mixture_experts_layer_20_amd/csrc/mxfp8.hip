// MXFP8 quantization and grouped GEMMs on gfx950's block-scaled FP8 matrix instruction.
//
// The pages run their largest operating points with an MXFP8 recipe (Olmo-core DDP MoE examples,
// "Production throughput runs", operating-point table, and "Other experiments in the report") but
// do not define the format.  Reading taken: the OCP Microscaling (MX) v1.0 MXFP8 format with E4M3
// elements, one E8M0 scale (a power of two 2^(byte - 127)) per 32 consecutive elements of the
// contraction axis; shared exponent floor(log2(block max)) - 8, clamped to [-127, 127] (-127 for an
// all-zero block); elements rounded to nearest, ties to even, magnitudes past 448 saturated to 448.
//
// The shared exponent comes from the bit pattern of the block maximum; elements are scaled by an exact
// power of two, clamped to +-448 and converted by the hardware's round-to-nearest-even E4M3
// conversion, so every code and every scale byte is exact.  The GEMM uses v_mfma_scale_f32_32x32x64_f8f6f4: lane i + 32h of
// an operand holds row i, bytes 0..15 in the first 32-element block of the 64-wide K step (k =
// 16h..16h+15) and bytes 16..31 in the second (k = 32+16h..); the scale of block b of row i comes
// from lane i + 32b.  Products of E4M3 values and power-of-two scales are exact in fp32, and are
// accumulated in fp32.
//
// Main GEMM (mx_gemm_pipe_kernel): persistent, one workgroup per CU, 256x256 output tiles, 8 waves
// (two per SIMD, 128x64 each), K consumed 64 bytes per step.  Operand codes stream through a ring
// of four 32 KiB LDS stages filled by direct-to-LDS loads; the stream runs across tile boundaries,
// so the next tile's first stages load during an epilogue.  Scale bytes land in their own small
// LDS ring (one dword per row per two K steps, or 16 bytes per eight where sizes allow).  Each XCD
// takes a contiguous run of the real tile count (read from the group tile prefix the workgroup
// computes in LDS), dealt round-robin to its workgroups.  Weight gradients (ragged K) run over each
// group's padded column range and, when there are few output tiles, split K into parts with fp32
// partials summed in part order.  Epilogues exchange accumulator lanes so each lane stores 16
// contiguous bytes: plain store, SwiGLU (also writing the MXFP8 rows of H) and SwiGLU backward
// (also writing the MXFP8 rows of [dA | dB]).
//
// Fallback GEMM (mx_gemm_kernel, shapes the main one does not take): one workgroup = one 128x128
// output tile (4 waves, 2x2, 64x64 each), K consumed 128 bytes (= 128 elements) per step through a
// double-buffered LDS tile (16 KiB per operand and buffer) with 128-byte row segments, 16-byte
// chunks XOR-swizzled by (row >> 1) & 7 so a ds_read_b128 over 16 rows hits 16 distinct bank
// groups.  In both, the B operand is the instruction's first operand, so each lane's accumulators
// hold 4 consecutive output columns of one row.
#include "common.h"
#include "mxfp8.h"

#include <algorithm>

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
// Native vectors: HIP's uint4 is a class, which keeps arrays of it out of registers.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---- E4M3 / E8M0 --------------------------------------------------------------------------

// floor(log2(v)) of a positive finite fp32 magnitude given by its bits.
__device__ __forceinline__ int floor_log2_bits(uint32_t a) {
  const int ex = (int)(a >> 23);
  return ex ? ex - 127 : (31 - __clz(a)) - 149;
}

// Shared exponent of a block from the bits of its largest magnitude.
__device__ __forceinline__ int mx_shared_exp(uint32_t amax) {
  if (amax == 0) return -127;
  const int e = floor_log2_bits(amax) - 8;   // 8: exponent of E4M3's largest binade (448 = 1.75 * 2^8)
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E4M3 codes of v / 2^e: the power-of-two scaling is exact (ldexp), the clamp to +-448 makes the
// saturation explicit, and the hardware conversion rounds to nearest with ties to even (for bf16
// inputs this equals the bit-level definition for every finite value and every shared exponent in
// [-127, 119]; the device tests compare every code with the oracle).  a -> byte 0, b -> byte 1 of
// the half-word selected by HI.
__device__ __forceinline__ float mx_scaled(uint32_t bits, int e) {
  return fminf(fmaxf(ldexpf(__uint_as_float(bits), -e), -448.0f), 448.0f);
}
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(uint32_t old, uint32_t a, uint32_t b, int e) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(a, e), mx_scaled(b, e), (int)old, HI);
}
// Four bf16 values (two dwords of bf16 pairs) -> four codes in one dword, in order.
__device__ __forceinline__ uint32_t e4m3_pack4(uint32_t w0, uint32_t w1, int e) {
  const uint32_t lo = e4m3_pack2<false>(0u, w0 << 16, w0 & 0xffff0000u, e);
  return e4m3_pack2<true>(lo, w1 << 16, w1 & 0xffff0000u, e);
}


// ---- Row quantization: 8 elements per lane, 4 lanes per block ---------------------------------
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(const bf16_t* __restrict__ x, long long R, int K,
                                                            long long ldx, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int nch = K >> 3;
  const long long total = R * nch;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const long long r = i / nch;
    const int c = (int)(i - r * nch);
    const uint4 v = *reinterpret_cast<const uint4*>(x + r * ldx + (long long)c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = max(amax, (w[j] & 0x7fffu) << 16);
      amax = max(amax, (w[j] >> 16 & 0x7fffu) << 16);
    }
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
    const int e = mx_shared_exp(amax);
    *reinterpret_cast<uint2*>(codes + r * K + (long long)c * 8) =
        make_uint2(e4m3_pack4(w[0], w[1], e), e4m3_pack4(w[2], w[3], e));
    if ((c & 3) == 0) scales[r * (K >> 5) + (c >> 2)] = (uint8_t)(e + 127);
  }
}

// ---- Group prefixes -------------------------------------------------------------------------
// out[g] = mult * sum_{j<g} ceil(len_j / unit), len_j the clamped row count of group j (offsets, or
// group_rows each when offsets is null).  One workgroup of 1024 threads, G <= 1024.
__global__ __launch_bounds__(1024) void mx_prefix_kernel(const int32_t* __restrict__ offsets, int G,
                                                         long long group_rows, long long R, int unit, int mult,
                                                         int32_t* __restrict__ out) {
  __shared__ int buf[1024];
  const int t = threadIdx.x;
  int v = 0;
  if (t < G) {
    long long len;
    if (offsets) {
      const long long lo = min(max((long long)offsets[t], 0LL), R);
      const long long hi = min(max((long long)offsets[t + 1], lo), R);
      len = hi - lo;
    } else {
      len = group_rows;
    }
    v = (int)((len + unit - 1) / unit);
  }
  buf[t] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = t >= o ? buf[t - o] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  if (t < G) out[t + 1] = buf[t] * mult;
  if (t == 0) out[0] = 0;
}

// ---- Column quantization: 128 padded rows of one group x 512 columns per workgroup ----------
// Each thread quantizes two columns over four 32-row blocks into LDS ([column][128 codes]) and
// writes their four scale bytes as one dword; after a barrier the workgroup writes the 512 code
// runs of 128 bytes, eight lanes per run, so one store instruction covers eight whole runs.
// Groups are padded to a multiple of 128 rows, so a 128-row chunk never spans two groups.
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(const bf16_t* __restrict__ x, long long R, int N,
                                                            long long ldx, const int32_t* __restrict__ offsets,
                                                            int G, long long group_rows,
                                                            const int32_t* __restrict__ kbase,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, long long ldc) {
  const long long k0 = (long long)blockIdx.x * 128;
  const int n = (blockIdx.y * 256 + threadIdx.x) * 2;
  const long long ktot = kbase[G];
  long long r0 = 0, rhi = 0;  // source rows of this chunk: [r0, min(r0 + 128, rhi))
  if (k0 < ktot) {
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (kbase[mid] <= k0) lo = mid; else hi = mid;
    }
    long long glo, ghi;
    if (offsets) {
      glo = min(max((long long)offsets[lo], 0LL), R);
      ghi = min(max((long long)offsets[lo + 1], glo), R);
    } else {
      glo = (long long)lo * group_rows;
      ghi = glo + group_rows;
    }
    r0 = glo + (k0 - kbase[lo]);
    rhi = ghi;
  }
  // Codes of this thread's two columns, block by block, staged in LDS ([column][128 codes]) so that
  // only one block's loads are live at a time; each column's 128 codes then go out as one run.
  __shared__ __attribute__((aligned(16))) uint8_t stage[512][128];
  const int lc = threadIdx.x * 2;
  const bool active = n < N;
  uint32_t sc[2] = {0u, 0u};
  for (int blk = 0; blk < 4; ++blk) {
    uint32_t v[32];
    const long long rb = r0 + 32 * blk;
#pragma unroll
    for (int j = 0; j < 32; ++j)
      v[j] = active && rb + j < rhi ? *reinterpret_cast<const uint32_t*>(x + (rb + j) * ldx + n) : 0u;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t amax = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = max(amax, ((v[j] >> (16 * c)) & 0x7fffu) << 16);
      const int e = mx_shared_exp(amax);
      sc[c] |= (uint32_t)(e + 127) << (8 * blk);
      u32x4_t w[2];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        // column c of rows 4q .. 4q+3 of the block, as bf16 bit patterns in the upper halves
        const uint32_t x0 = c ? (v[4 * q] & 0xffff0000u) : (v[4 * q] << 16);
        const uint32_t x1 = c ? (v[4 * q + 1] & 0xffff0000u) : (v[4 * q + 1] << 16);
        const uint32_t x2 = c ? (v[4 * q + 2] & 0xffff0000u) : (v[4 * q + 2] << 16);
        const uint32_t x3 = c ? (v[4 * q + 3] & 0xffff0000u) : (v[4 * q + 3] << 16);
        w[q >> 2][q & 3] = e4m3_pack2<true>(e4m3_pack2<false>(0u, x0, x1, e), x2, x3, e);
      }
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(&stage[lc + c][32 * blk]);
      dst[0] = w[0];
      dst[1] = w[1];
    }
  }
  if (active) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      *reinterpret_cast<uint32_t*>(scales + (long long)(n + c) * (ldc >> 5) + (k0 >> 5)) = sc[c];
  }
  __syncthreads();
  const int n0 = blockIdx.y * 512, runs = min(512, N - n0), part = threadIdx.x & 7;
#pragma unroll 4
  for (int run = threadIdx.x >> 3; run < runs; run += 32) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&stage[run][16 * part]);
    *reinterpret_cast<u32x4_t*>(codes + (long long)(n0 + run) * ldc + k0 + 16 * part) = v;
  }
}

// ---- Grouped GEMM ---------------------------------------------------------------------------
constexpr int TB = 128;               // tile rows = tile columns = K step (bytes)
constexpr int OPBYTES = TB * TB;      // one operand tile of one buffer: 16 KiB

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ uint32_t bf16pack(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// Operand fragment of a 32-row block for K step half s: row i = lane & 31, chunks 4s + h and
// 4s + 2 + h (h = lane >> 5) of the 128-byte row.
__device__ __forceinline__ i32x8_t read_frag(const uint8_t* tile, int row, int s, int h) {
  const uint8_t* base = tile + row * TB;
  const int sw = swz(row);
  const u32x4_t p = *reinterpret_cast<const u32x4_t*>(base + 16 * ((4 * s + h) ^ sw));
  const u32x4_t q = *reinterpret_cast<const u32x4_t*>(base + 16 * ((4 * s + 2 + h) ^ sw));
  i32x8_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (int)p[j];
    r[4 + j] = (int)q[j];
  }
  return r;
}

template <int EPI, bool RK>
__global__ __launch_bounds__(256, 2) void mx_gemm_kernel(MxGemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][OPBYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, li = lane & 31, h = lane >> 5;
  // Output columns per tile: the SwiGLU tile multiplies 64 gate and 64 up columns.
  constexpr int OC = EPI == MX_EPI_SWIGLU ? 64 : 128;
  const int NT = p.N / OC;

  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD one contiguous run of tiles.
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int per = nb >> 3;
  int Lt;
  {
    const int xcd = b & 7, idx = b >> 3;
    const int rem = nb & 7;  // the first `rem` XCDs get one more
    const int start = xcd * per + min(xcd, rem);
    Lt = start + idx;
  }
  const int nt = Lt % NT;
  int g, m0, m_end;
  long long kb0, kb1;
  if constexpr (!RK) {
    const int mt = Lt / NT;
    if (mt >= p.tile_prefix[p.G]) return;
    int lo = 0, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_prefix[mid] <= mt) lo = mid; else hi = mid;
    }
    g = lo;
    const int r0 = min(max(p.offsets[g], 0), p.M);
    const int r1 = min(max(p.offsets[g + 1], r0), p.M);
    m0 = r0 + (mt - p.tile_prefix[g]) * TB;
    m_end = r1;
    kb0 = 0;
    kb1 = p.K;
  } else {
    const int MT = p.M / TB;
    const int r = Lt / NT;
    if (r >= p.G * MT) return;
    g = r / MT;
    m0 = (r - g * MT) * TB;
    m_end = p.M;
    kb0 = p.offsets[g];
    kb1 = p.offsets[g + 1];
  }
  const int nk = (int)((kb1 - kb0) / TB);

  // Global load slots: thread loads rows (tid >> 3) + 32j, 16-byte chunk tid & 7, of both operands.
  const int lrow = tid >> 3, lch = tid & 7;
  const uint8_t* ga[4];
  const uint8_t* gb[4];
  const uint8_t* gb2[4];   // K columns >= ksplit (store / SwiGLU backward with a second source)
  const long long gofs = RK ? 0 : (long long)g * p.b_gstride;
  const bool split = EPI != MX_EPI_SWIGLU && p.b2 != nullptr;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = lrow + 32 * j;
    const int ar = RK ? m0 + r : min(m0 + r, m_end - 1);
    ga[j] = p.a + (long long)ar * p.lda + kb0 + 16 * lch;
    if constexpr (EPI == MX_EPI_SWIGLU) {
      // tile row r: wave column r >> 6, block (r >> 5) & 1 (0: gate rows of b, 1: up rows of b2)
      const int br = nt * 64 + (r >> 6) * 32 + (r & 31);
      gb[j] = (((r >> 5) & 1) ? p.b2 : p.b) + gofs + (long long)br * p.ldb + kb0 + 16 * lch;
      gb2[j] = gb[j];
    } else {
      const int br = nt * TB + r;
      gb[j] = p.b + gofs + (long long)br * p.ldb + kb0 + 16 * lch;
      gb2[j] = (split ? p.b2 : p.b) + gofs + (long long)br * p.ldb + 16 * lch - p.ksplit;
    }
  }
  const int lofs = lrow * TB + 16 * (lch ^ swz(lrow));  // + 32 * TB * j

  // Scale words (4 blocks of one K step) of this lane's fragment rows, shifted by 8h so that byte 0
  // (step half 0) and byte 2 (step half 1) are this lane's blocks.
  const uint8_t* sa_p[2];
  const uint8_t* sb_p[2];
  const uint8_t* sb2_p[2];
  const long long lda_s = p.lda >> 5, ldb_s = p.ldb >> 5;
  const long long gofs_s = gofs >> 5;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = wm * 64 + q * 32 + li;
    const int ar = RK ? m0 + r : min(m0 + r, m_end - 1);
    sa_p[q] = p.as + (long long)ar * lda_s + (kb0 >> 5);
    if constexpr (EPI == MX_EPI_SWIGLU) {
      const int br = nt * 64 + wn * 32 + li;
      sb_p[q] = (q ? p.bs2 : p.bs) + gofs_s + (long long)br * ldb_s + (kb0 >> 5);
      sb2_p[q] = sb_p[q];
    } else {
      const int br = nt * TB + wn * 64 + q * 32 + li;
      sb_p[q] = p.bs + gofs_s + (long long)br * ldb_s + (kb0 >> 5);
      sb2_p[q] = (split ? p.bs2 : p.bs) + gofs_s + (long long)br * ldb_s - (p.ksplit >> 5);
    }
  }
  const int ks = split ? p.ksplit : 0x7fffffff;   // K columns from the second source start here

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4_t ra[4], rb[4];
  uint32_t sa_c[2], sb_c[2], sa_n[2] = {0, 0}, sb_n[2] = {0, 0};
  if (nk > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[j] = *reinterpret_cast<const u32x4_t*>(ga[j]);
      rb[j] = *reinterpret_cast<const u32x4_t*>(ks <= 0 ? gb2[j] : gb[j]);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      sa_c[q] = *reinterpret_cast<const uint32_t*>(sa_p[q]) >> (8 * h);
      sb_c[q] = *reinterpret_cast<const uint32_t*>(ks <= 0 ? sb2_p[q] : sb_p[q]) >> (8 * h);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4_t*>(&lds[0][0][lofs + 32 * TB * j]) = ra[j];
      *reinterpret_cast<u32x4_t*>(&lds[0][1][lofs + 32 * TB * j]) = rb[j];
    }
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const long long off = (long long)(kt + 1) * TB;
      const bool second = kb0 + off >= ks;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = *reinterpret_cast<const u32x4_t*>(ga[j] + off);
        rb[j] = *reinterpret_cast<const u32x4_t*>((second ? gb2[j] + kb0 : gb[j]) + off);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        sa_n[q] = *reinterpret_cast<const uint32_t*>(sa_p[q] + 4 * (kt + 1)) >> (8 * h);
        sb_n[q] = *reinterpret_cast<const uint32_t*>((second ? sb2_p[q] + (kb0 >> 5) : sb_p[q]) + 4 * (kt + 1)) >>
                  (8 * h);
      }
    }
    const uint8_t* ta = lds[cur][0];
    const uint8_t* tb = lds[cur][1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x8_t fa[2], fb[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        fa[q] = read_frag(ta, wm * 64 + q * 32 + li, s, h);
        fb[q] = read_frag(tb, wn * 64 + q * 32 + li, s, h);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (s == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0,
                                                                        (int)sb_c[j], 0, (int)sa_c[i]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 2,
                                                                        (int)sb_c[j], 2, (int)sa_c[i]);
        }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<u32x4_t*>(&lds[cur ^ 1][0][lofs + 32 * TB * j]) = ra[j];
        *reinterpret_cast<u32x4_t*>(&lds[cur ^ 1][1][lofs + 32 * TB * j]) = rb[j];
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        sa_c[q] = sa_n[q];
        sb_c[q] = sb_n[q];
      }
    }
    __syncthreads();
  }

  // Epilogue: lane holds row li of each 32-row block, columns 8*(r/4) + 4h + (r%4).
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = m0 + wm * 64 + i * 32 + li;
    if (!RK && row >= m_end) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (EPI == MX_EPI_SWIGLU) {
        const int col = nt * 64 + wn * 32 + 8 * q + 4 * h;
        float hv[4];
        const long long o = (long long)row * p.N + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = acc[i][0][4 * q + r], bb = acc[i][1][4 * q + r];
          hv[r] = a * sigmoid_f32(a) * bb;
        }
        if (p.out0)
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(p.out0) + o) =
              make_uint2(bf16pack(acc[i][0][4 * q], acc[i][0][4 * q + 1]),
                         bf16pack(acc[i][0][4 * q + 2], acc[i][0][4 * q + 3]));
        if (p.out1)
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(p.out1) + o) =
              make_uint2(bf16pack(acc[i][1][4 * q], acc[i][1][4 * q + 1]),
                         bf16pack(acc[i][1][4 * q + 2], acc[i][1][4 * q + 3]));
        *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(p.out2) + o) =
            make_uint2(bf16pack(hv[0], hv[1]), bf16pack(hv[2], hv[3]));
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nt * TB + wn * 64 + j * 32 + 8 * q + 4 * h;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
          if constexpr (EPI == MX_EPI_SWIGLU_BWD) {
            const long long o = (long long)row * p.N + col;
            const uint2 av = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(p.aux0) + o);
            const uint2 bv = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(p.aux1) + o);
            const uint32_t aw[2] = {av.x, av.y}, bw[2] = {bv.x, bv.y};
            float da[4], db[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float a = bf16_to_f32((bf16_t)(aw[r >> 1] >> (16 * (r & 1))));
              const float bb = bf16_to_f32((bf16_t)(bw[r >> 1] >> (16 * (r & 1))));
              const float sg = sigmoid_f32(a);
              da[r] = v[r] * bb * sg * (1.0f + a * (1.0f - sg));
              db[r] = v[r] * a * sg;
            }
            bf16_t* dab = reinterpret_cast<bf16_t*>(p.out0) + (long long)row * (2 * p.N);
            *reinterpret_cast<uint2*>(dab + col) = make_uint2(bf16pack(da[0], da[1]), bf16pack(da[2], da[3]));
            *reinterpret_cast<uint2*>(dab + p.N + col) =
                make_uint2(bf16pack(db[0], db[1]), bf16pack(db[2], db[3]));
          } else {
            bf16_t* dst;
            if constexpr (RK) {
              dst = row < p.split
                        ? reinterpret_cast<bf16_t*>(p.out0) + ((long long)g * p.split + row) * p.N + col
                        : reinterpret_cast<bf16_t*>(p.out1) +
                              ((long long)g * (p.M - p.split) + (row - p.split)) * p.N + col;
            } else {
              dst = reinterpret_cast<bf16_t*>(p.out0) + (long long)row * p.N + col;
            }
            *reinterpret_cast<uint2*>(dst) = make_uint2(bf16pack(v[0], v[1]), bf16pack(v[2], v[3]));
          }
        }
      }
    }
  }
}

// ---- Pipelined grouped GEMM: 256x256 tiles ----------------------------------------------------
// 8 waves (2 per SIMD): wave w covers rows 128*(w & 1) .. +128 and columns 64*(w >> 1) .. +64 of
// the tile (4 x 2 blocks of 32x32).  K step = 64 bytes.  Codes stream through a ring of four
// 32 KiB LDS stages filled by direct loads (global_load_lds_dwordx4: lane l's 16 bytes land at
// M0 + 16 l); the stage three steps ahead is issued right after the barrier that publishes the
// current one, so three stages (96 KiB) are in flight per CU.  Scale bytes: one dword per row
// covers two K steps (4 blocks); the 512 dwords of a tile's two steps land in a three-slot LDS
// ring.  LDS reads are inline assembly that waits for its own results; the ring is governed by
// explicit vmcnt waits (a compiler-generated LDS read would first wait for every direct load in
// flight).  K-contiguous rows of 64 bytes are stored with 16-byte chunk c at c ^ ((row >> 2) & 3).
constexpr int PB = 256;                 // tile rows / columns
constexpr int PK = 64;                  // K step (bytes = elements)
constexpr int PSTAGE = 2 * PB * PK;     // 32 KiB: A then B
constexpr int PNST = 4;
// Scale ring: each row's scale bytes arrive SW at a time (SW = 4: two K steps per dword; SW = 16: eight
// K steps per 16-byte load, four times fewer scattered requests, when K and the group strides allow).
// A slot holds 256 A rows, then 256 B rows, SW bytes each.
template <int SW> struct ScaleRing {
  static constexpr int STEPS = SW / 2;               // K steps per load
  static constexpr int SLOT = 2 * PB * SW;
  static constexpr int SLOTS = SW == 4 ? 3 : 2;      // a slot is reloaded only after its last read
  static constexpr int PREF = PNST * PSTAGE + SLOTS * SLOT;   // group tile prefix (ragged rows): 1025 ints
  static constexpr int LDS = PREF + 4 * 1032;
};

// One LDS dword read with its own wait (a compiler-generated LDS read would first wait for every
// direct load in flight).
__device__ __forceinline__ int lds_i32(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

__device__ __forceinline__ uint32_t lds_off(const void* ptr) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)ptr);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | (0xf << 8));
}
__device__ __forceinline__ void pbarrier() { asm volatile("s_barrier" ::: "memory"); }

// Fragments and scales of one K step, read from LDS with the wait inside the same block.  Outputs
// are early-clobber: a result may land while later reads of the block still need their addresses.
struct PFrag {
  u32x4_t a[4][2];
  u32x4_t b[2][2];
  uint32_t sa[4], sb[2];
};

template <int SW>
__device__ __forceinline__ void read_step(PFrag& f, uint32_t a0, uint32_t a2, uint32_t b0, uint32_t b2, uint32_t sa,
                                          uint32_t sb) {
  asm volatile(
      "ds_read_b128 %0, %18\n\t"
      "ds_read_b128 %1, %19\n\t"
      "ds_read_b128 %2, %18 offset:2048\n\t"
      "ds_read_b128 %3, %19 offset:2048\n\t"
      "ds_read_b128 %4, %18 offset:4096\n\t"
      "ds_read_b128 %5, %19 offset:4096\n\t"
      "ds_read_b128 %6, %18 offset:6144\n\t"
      "ds_read_b128 %7, %19 offset:6144\n\t"
      "ds_read_b128 %8, %20\n\t"
      "ds_read_b128 %9, %21\n\t"
      "ds_read_b128 %10, %20 offset:2048\n\t"
      "ds_read_b128 %11, %21 offset:2048\n\t"
      "ds_read_u8 %12, %22\n\t"
      "ds_read_u8 %13, %22 offset:%24\n\t"
      "ds_read_u8 %14, %22 offset:%25\n\t"
      "ds_read_u8 %15, %22 offset:%26\n\t"
      "ds_read_u8 %16, %23\n\t"
      "ds_read_u8 %17, %23 offset:%24\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.a[0][0]), "=&v"(f.a[0][1]), "=&v"(f.a[1][0]), "=&v"(f.a[1][1]), "=&v"(f.a[2][0]), "=&v"(f.a[2][1]),
        "=&v"(f.a[3][0]), "=&v"(f.a[3][1]), "=&v"(f.b[0][0]), "=&v"(f.b[0][1]), "=&v"(f.b[1][0]), "=&v"(f.b[1][1]),
        "=&v"(f.sa[0]), "=&v"(f.sa[1]), "=&v"(f.sa[2]), "=&v"(f.sa[3]), "=&v"(f.sb[0]), "=&v"(f.sb[1])
      : "v"(a0), "v"(a2), "v"(b0), "v"(b2), "v"(sa), "v"(sb), "i"(32 * SW), "i"(64 * SW), "i"(96 * SW)
      : "memory");
}

__device__ __forceinline__ i32x8_t frag8(const u32x4_t& lo, const u32x4_t& hi) {
  i32x8_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (int)lo[j];
    r[4 + j] = (int)hi[j];
  }
  return r;
}

// One output tile of the pipelined kernel.
struct PTile {
  int g, m0, m_end, nt, nk, part;
  long long kb0;
};

__device__ __forceinline__ int ufirst(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Tile Lt of the launch (tile order: group by group, row tiles, column tiles fastest); false past the
// last tile.
template <bool RK>
__device__ __forceinline__ bool pipe_tile(const MxGemmArgs& p, int Lt, int NT, uint32_t pref, PTile& t) {
  t.nt = Lt % NT;
  if constexpr (!RK) {
    // pref: LDS address of the group tile prefix (pref[g] = row tiles of groups before g)
    const int mt = Lt / NT;
    if (mt >= ufirst(lds_i32(pref + 4 * p.G))) return false;
    int lo = 0, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ufirst(lds_i32(pref + 4 * mid)) <= mt) lo = mid; else hi = mid;
    }
    t.g = lo;
    const int r0 = min(max(ufirst(p.offsets[lo]), 0), p.M);
    const int r1 = min(max(ufirst(p.offsets[lo + 1]), r0), p.M);
    t.m0 = r0 + (mt - ufirst(lds_i32(pref + 4 * lo))) * PB;
    t.m_end = r1;
    t.kb0 = 0;
    t.nk = p.K / PK;
  } else {
    // Tile order: column tiles fastest, then row tiles, then K parts, then groups.  Part q of a
    // group covers [q c, (q + 1) c) of its K range, c = its length / kparts rounded up to 128.
    const int MT = p.M / PB, S = p.kparts;
    int r = Lt / NT;
    if (r >= p.G * S * MT) return false;
    const int mt = r % MT;
    r /= MT;
    t.part = r % S;
    t.g = r / S;
    t.m0 = mt * PB;
    t.m_end = p.M;
    const int k0 = ufirst(p.offsets[t.g]), k1 = ufirst(p.offsets[t.g + 1]);
    const int len = k1 - k0;
    const int chunk = ((len + S - 1) / S + 127) / 128 * 128;
    const int a = min(len, t.part * chunk), e = min(len, (t.part + 1) * chunk);
    t.kb0 = k0 + a;
    t.nk = (e - a) / PK;
  }
  return true;
}

// This lane's load sources for one tile: code loads (instruction j of each operand fills slot
// q = (2 wave + j) 64 + lane = row q >> 2, physical chunk q & 3; gb2: the same rows in the second
// source at K column 0) and the scale dword (wave w < 4: A row 64 w + lane; else B row 64 (w - 4) +
// lane).
struct PLoad {
  const uint8_t* ga[2];
  const uint8_t* gb[2];
  const uint8_t* gb2[2];
  const uint8_t* gs;
  const uint8_t* gs2;
};

template <int EPI, bool RK>
__device__ __forceinline__ void pipe_sources(const MxGemmArgs& p, const PTile& t, bool split, int wave, int lane,
                                             PLoad& L) {
  const long long lda_s = p.lda >> 5, ldb_s = p.ldb >> 5;
  const long long gofs = RK ? 0 : (long long)t.g * p.b_gstride;
  // B tile row r: its source (first or second) and row.  The SwiGLU tile holds gate rows (first
  // source) and up rows (second source) of 128 output columns.
  auto bsrc2 = [&](int r) -> bool { return EPI == MX_EPI_SWIGLU && ((r >> 5) & 1); };
  auto brow = [&](int r) -> int {
    if constexpr (EPI == MX_EPI_SWIGLU) return t.nt * 128 + (r >> 6) * 32 + (r & 31);
    else return t.nt * PB + r;
  };
  auto arow = [&](int r) -> int { return RK ? t.m0 + r : min(t.m0 + r, t.m_end - 1); };
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = (2 * wave + j) * 64 + lane;
    const int row = q >> 2;
    const int c = (q & 3) ^ ((row >> 2) & 3);
    L.ga[j] = p.a + (long long)arow(row) * p.lda + t.kb0 + 16 * c;
    const long long bo = gofs + (long long)brow(row) * p.ldb + 16 * c;
    L.gb[j] = (bsrc2(row) ? p.b2 : p.b) + bo + t.kb0;
    L.gb2[j] = (split ? p.b2 : p.b) + bo;
  }
  const int r = (wave & 3) * 64 + lane;
  const long long bo = (gofs >> 5) + (long long)brow(r) * ldb_s;
  L.gs = wave < 4 ? p.as + (long long)arow(r) * lda_s + (t.kb0 >> 5)
                  : (bsrc2(r) ? p.bs2 : p.bs) + bo + (t.kb0 >> 5);
  L.gs2 = wave < 4 ? L.gs : (split ? p.bs2 : p.bs) + bo;
}

// Stage s of the load stream = step j of tile t: codes into ring slot s & 3, and every STEPS steps the
// scale bytes of the next STEPS steps into scale slot (s / STEPS) % SLOTS (a tile's step count is a
// multiple of STEPS, so s and j agree modulo STEPS).
template <int SW>
__device__ __forceinline__ void pipe_issue(const PLoad& L, long long kb0, int j, int s, int ks, char* ring,
                                           char* sring, int wave) {
  using SR = ScaleRing<SW>;
  char* st = ring + (s & 3) * PSTAGE;
  const long long off = (long long)j * PK;
  const bool second = kb0 + off >= ks;   // B columns of this stage come from the second source
  if (j % SR::STEPS == 0) {
    const uint8_t* src = (second && wave >= 4) ? L.gs2 + ((kb0 + off - ks) >> 5) : L.gs + 2 * j;
    lvoid_t* dst = (lvoid_t*)(sring + ((s / SR::STEPS) % SR::SLOTS) * SR::SLOT + wave * 64 * SW);
    if constexpr (SW == 16) __builtin_amdgcn_global_load_lds((gvoid_t*)src, dst, 16, 0, 0);
    else __builtin_amdgcn_global_load_lds((gvoid_t*)src, dst, 4, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    __builtin_amdgcn_global_load_lds((gvoid_t*)(L.ga[q] + off), (lvoid_t*)(st + (2 * wave + q) * 1024), 16, 0, 0);
    const uint8_t* bs = second ? L.gb2[q] + (kb0 + off - ks) : L.gb[q] + off;
    __builtin_amdgcn_global_load_lds((gvoid_t*)bs, (lvoid_t*)(st + PB * PK + (2 * wave + q) * 1024), 16, 0, 0);
  }
}

// Accumulator block exchange for wide stores.  After the transposed MFMA, lane l holds row l % 32 and,
// for element v, column 8 (v / 4) + 4 (l / 32) + v % 4 of the 32x32 block: a store covers 32 rows
// with 16 bytes each.  v_permlane32_swap of the 4-column pieces of each 16-column half gives lane l
// 8 consecutive columns 16 H + 8 (l / 32) of its row; v_permlane16_swap of the two halves then
// leaves x0 = row l % 16 and x1 = row 16 + l % 16, both at columns 16 ((l / 16) % 2) + 8 (l / 32):
// each 16-byte store covers 16 rows with 64 contiguous bytes.
__device__ __forceinline__ int xcol(int lane) { return 16 * ((lane >> 4) & 1) + 8 * (lane >> 5); }

__device__ __forceinline__ void xchg_block(const f32x16_t& c, float (&x0)[8], float (&x1)[8]) {
  float hv[2][8];
#pragma unroll
  for (int H = 0; H < 2; ++H)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[8 * H + e]), __float_as_uint(c[8 * H + 4 + e]),
                                                      false, false);
      hv[H][e] = __uint_as_float(r[0]);
      hv[H][4 + e] = __uint_as_float(r[1]);
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(hv[0][e]), __float_as_uint(hv[1][e]), false, false);
    x0[e] = __uint_as_float(r[0]);
    x1[e] = __uint_as_float(r[1]);
  }
}

__device__ __forceinline__ u32x4_t pack8(const float (&v)[8]) {
  u32x4_t w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = bf16pack(v[2 * e], v[2 * e + 1]);
  return w;
}
__device__ __forceinline__ void unpack8(const u32x4_t& w, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

// MXFP8 of 8 consecutive bf16 values of a row (packed in w) whose 32-column block is spread over
// lanes l, l ^ 16, l ^ 32, l ^ 48 (the exchanged layout): codes to dst (8 bytes), the scale byte by
// the lane holding the block's first columns.
__device__ __forceinline__ void quant8_xchg(const u32x4_t& w, uint8_t* dst, uint8_t* scale, bool first) {
  uint32_t am = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) am = max(am, max((w[e] & 0x7fffu) << 16, ((w[e] >> 16) & 0x7fffu) << 16));
  am = max(am, (uint32_t)__shfl_xor((int)am, 16));
  am = max(am, (uint32_t)__shfl_xor((int)am, 32));
  const int e = mx_shared_exp(am);
  *reinterpret_cast<uint2*>(dst) = make_uint2(e4m3_pack4(w[0], w[1], e), e4m3_pack4(w[2], w[3], e));
  if (first) *scale = (uint8_t)(e + 127);
}

template <int EPI, bool RK>
__device__ __forceinline__ void pipe_epilogue(const MxGemmArgs& p, const PTile& t, const f32x16_t (&acc)[4][2],
                                              int wm, int wn, int lane) {
  const int cl = xcol(lane), rl = lane & 15;
  if constexpr (EPI == MX_EPI_SWIGLU_BWD) {
    // The A/B stash of a 32-row block is loaded, all of it, before the block's first store: the
    // stores through out0 and qc may alias the stash as far as the compiler knows, so a load
    // written after one would wait for it and then for a whole memory round trip.  (Loading the
    // next block's stash as well, before these stores, needs more registers than are left.)
    // Rows past the group are clamped on load and dropped on store.
    u32x4_t sa[1][2][2], sb[1][2][2];   // [buffer][column block][16-row piece]
    auto load_blk = [&](int i, int buf) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
          const int row = min(t.m0 + wm * 128 + i * 32 + rl + 16 * pc, t.m_end - 1);
          const long long o = (long long)row * p.N + t.nt * PB + wn * 64 + c * 32 + cl;
          sa[buf][c][pc] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const bf16_t*>(p.aux0) + o);
          sb[buf][c][pc] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const bf16_t*>(p.aux1) + o);
        }
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load_blk(i, 0);
      const int rbase = t.m0 + wm * 128 + i * 32 + rl;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float x[2][8];
        xchg_block(acc[i][c], x[0], x[1]);
        const int col = t.nt * PB + wn * 64 + c * 32 + cl;
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
          const int row = rbase + 16 * pc;
          if (row >= t.m_end) continue;
          float a[8], bb[8], da[8], db[8];
          unpack8(sa[0][c][pc], a);
          unpack8(sb[0][c][pc], bb);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sg = sigmoid_f32(a[e]);
            da[e] = x[pc][e] * bb[e] * sg * (1.0f + a[e] * (1.0f - sg));
            db[e] = x[pc][e] * a[e] * sg;
          }
          bf16_t* dab = reinterpret_cast<bf16_t*>(p.out0) + (long long)row * (2 * p.N);
          const u32x4_t aw = pack8(da), bw = pack8(db);
          *reinterpret_cast<u32x4_t*>(dab + col) = aw;
          *reinterpret_cast<u32x4_t*>(dab + p.N + col) = bw;
          if (p.qc) {
            uint8_t* qrow = p.qc + (long long)row * (2 * p.N);
            uint8_t* srow = p.qs + (long long)row * (p.N >> 4);
            quant8_xchg(aw, qrow + col, srow + (col >> 5), cl == 0);
            quant8_xchg(bw, qrow + p.N + col, srow + ((p.N + col) >> 5), cl == 0);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rbase = t.m0 + wm * 128 + i * 32 + rl;   // + 16 for the second piece
    if constexpr (EPI == MX_EPI_SWIGLU) {
      float g[2][8], u[2][8];
      xchg_block(acc[i][0], g[0], g[1]);
      xchg_block(acc[i][1], u[0], u[1]);
      const int col = t.nt * 128 + wn * 32 + cl;
#pragma unroll
      for (int pc = 0; pc < 2; ++pc) {
        const int row = rbase + 16 * pc;
        if (row >= t.m_end) continue;
        float hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = g[pc][e] * sigmoid_f32(g[pc][e]) * u[pc][e];
        const long long o = (long long)row * p.N + col;
        if (p.out0) *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(p.out0) + o) = pack8(g[pc]);
        if (p.out1) *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(p.out1) + o) = pack8(u[pc]);
        const u32x4_t hw = pack8(hv);
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(p.out2) + o) = hw;
        if (p.qc) quant8_xchg(hw, p.qc + o, p.qs + (long long)row * (p.N >> 5) + (col >> 5), cl == 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float x[2][8];
        xchg_block(acc[i][c], x[0], x[1]);
        const int col = t.nt * PB + wn * 64 + c * 32 + cl;
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
          const int row = rbase + 16 * pc;
          if (!RK && row >= t.m_end) continue;
          {
            if constexpr (RK) {
              if (p.kparts > 1) {   // fp32 partial of K part t.part
                float* dst = p.partial + (((long long)t.part * p.G + t.g) * p.M + row) * p.N + col;
                u32x4_t w0, w1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  w0[e] = __float_as_uint(x[pc][e]);
                  w1[e] = __float_as_uint(x[pc][4 + e]);
                }
                reinterpret_cast<u32x4_t*>(dst)[0] = w0;
                reinterpret_cast<u32x4_t*>(dst)[1] = w1;
                continue;
              }
            }
            bf16_t* dst;
            if constexpr (RK) {
              dst = row < p.split
                        ? reinterpret_cast<bf16_t*>(p.out0) + ((long long)t.g * p.split + row) * p.N + col
                        : reinterpret_cast<bf16_t*>(p.out1) +
                              ((long long)t.g * (p.M - p.split) + (row - p.split)) * p.N + col;
            } else {
              dst = reinterpret_cast<bf16_t*>(p.out0) + (long long)row * p.N + col;
            }
            *reinterpret_cast<u32x4_t*>(dst) = pack8(x[pc]);
          }
        }
      }
    }
  }
}

// Persistent: one workgroup per CU walks its list of tiles; the load stream runs across tile
// boundaries, so the next tile's first stages are in flight during a tile's epilogue.  The tile
// list: each XCD (workgroup b runs on XCD b % 8) takes one contiguous eighth of the tiles, dealt
// round-robin to its workgroups.
template <int EPI, bool RK, int SW>
__global__ __launch_bounds__(512, 1) void mx_gemm_pipe_kernel(MxGemmArgs p) {
  using SR = ScaleRing<SW>;
  extern __shared__ __attribute__((aligned(16))) char plds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1, li = lane & 31, h = lane >> 5;
  constexpr int OC = EPI == MX_EPI_SWIGLU ? 128 : PB;   // output columns per tile
  const int NT = p.N / OC;
  // Ragged rows: the group tile prefix, computed by every workgroup into LDS before any direct
  // load is issued (G <= 1024; a Hillis-Steele scan over 1024 entries, two per thread).
  int* pref_lds = reinterpret_cast<int*>(plds + SR::PREF);
  const uint32_t pref = lds_off(pref_lds);
  if constexpr (!RK) {
    int* scan = pref_lds + 1;   // scan[g] = row tiles of groups 0..g
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int g = tid + 512 * q;
      int v = 0;
      if (g < p.G) {
        const int r0 = min(max(p.offsets[g], 0), p.M);
        const int r1 = min(max(p.offsets[g + 1], r0), p.M);
        v = (r1 - r0 + PB - 1) / PB;
      }
      scan[g] = v;
    }
    if (tid == 0) pref_lds[0] = 0;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      int add[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int g = tid + 512 * q;
        add[q] = g >= o ? scan[g - o] : 0;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 2; ++q) scan[tid + 512 * q] += add[q];
      __syncthreads();
    }
  }
  // Tiles to share out: ragged rows count the row tiles the groups really have (the launch size
  // assumes the worst case; an even split of that would leave the XCDs at its end idle).
  const int U = RK ? p.tiles : ufirst(pref_lds[p.G]) * NT;

  const int nb = gridDim.x, b = blockIdx.x;
  int first, stride, last;   // this workgroup's tiles: first, first + stride, ... < last
  if (nb < 8) {
    first = b;
    stride = nb;
    last = U;
  } else {
    const int xcd = b & 7;
    const int nwx = nb / 8 + (xcd < nb % 8 ? 1 : 0);
    const int per = U / 8, rem = U % 8;
    const int c0 = xcd * per + min(xcd, rem);
    first = c0 + (b >> 3);
    stride = nwx;
    last = c0 + per + (xcd < rem ? 1 : 0);
  }

  const bool split = EPI != MX_EPI_SWIGLU && p.b2 != nullptr;
  const int ks = split ? p.ksplit : 0x7fffffff;   // K columns from the second source start here
  char* ring = plds;
  char* sring = plds + PNST * PSTAGE;

  // Producer: the next stage to load (tile position pl, step pj).
  int pl = first, pj = 0;
  bool pvalid = false;
  PTile pt;
  PLoad L;
  auto pseek = [&]() {   // move to the first tile at or after pl with steps to load
    pvalid = false;
    while (pl < last) {
      if (!pipe_tile<RK>(p, pl, NT, pref, pt)) { pl = last; break; }
      if (pt.nk > 0) {
        pipe_sources<EPI, RK>(p, pt, split, wave, lane, L);
        pvalid = true;
        break;
      }
      pl += stride;
    }
  };
  int issued = 0;   // stages issued so far
  auto produce = [&]() {
    if (!pvalid) return;
    pipe_issue<SW>(L, pt.kb0, pj, issued, ks, ring, sring, wave);
    ++issued;
    if (++pj == pt.nk) {
      pj = 0;
      pl += stride;
      pseek();
    }
  };
  pseek();
  for (int q = 0; q < 3; ++q) produce();

  // LDS read offsets of this lane: A rows 128 wm + 32 i + li, B rows 64 wn + 32 j + li; chunks h, 2 + h.
  const int sw = (li >> 2) & 3;
  const uint32_t ring0 = lds_off(ring), sring0 = lds_off(sring);
  const uint32_t oa0 = (uint32_t)((wm * 128 + li) * PK + 16 * (h ^ sw));
  const uint32_t oa2 = (uint32_t)((wm * 128 + li) * PK + 16 * ((2 + h) ^ sw));
  const uint32_t ob0 = (uint32_t)(PB * PK + (wn * 64 + li) * PK + 16 * (h ^ sw));
  const uint32_t ob2 = (uint32_t)(PB * PK + (wn * 64 + li) * PK + 16 * ((2 + h) ^ sw));
  const uint32_t osa = (uint32_t)((wm * 128 + li) * SW + h);
  const uint32_t osb = (uint32_t)(PB * SW + (wn * 64 + li) * SW + h);

  int c = 0;            // consumer: next stage to multiply
  bool after_epi = false;
  for (int Lt = first; Lt < last; Lt += stride) {
    PTile t;
    if (!pipe_tile<RK>(p, Lt, NT, pref, t)) break;
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int j = 0; j < t.nk; ++j, ++c) {
      // Stage c complete for this wave.  After an epilogue its stores follow the later stages'
      // loads in the counter, so wait for everything; otherwise at most the loads of the (up to two)
      // later stages may still be in flight.
      const int later = issued - 1 - c;
      if (after_epi || later <= 0) wait_vm<0>();
      else if (later == 1) wait_vm<4>();
      else wait_vm<8>();
      after_epi = false;
      pbarrier();
      produce();
      PFrag f;
      const uint32_t sb = ring0 + (uint32_t)((c & 3) * PSTAGE);
      const uint32_t ss = sring0 + (uint32_t)(((c / SR::STEPS) % SR::SLOTS) * SR::SLOT + 2 * (c % SR::STEPS));
      read_step<SW>(f, sb + oa0, sb + oa2, sb + ob0, sb + ob2, ss + osa, ss + osb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x8_t fa = frag8(f.a[i][0], f.a[i][1]);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag8(f.b[q][0], f.b[q][1]), fa, acc[i][q], 0,
                                                                      0, 0, (int)f.sb[q], 0, (int)f.sa[i]);
      }
    }
    pipe_epilogue<EPI, RK>(p, t, acc, wm, wn, lane);
    after_epi = true;
  }
}

// Compute units of the current device (one persistent workgroup each).
int device_cus() {
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

template <int EPI, bool RK, int SW>
hipError_t launch_mx_pipe_sw(const MxGemmArgs& a, int tiles, hipStream_t s) {
  // The dynamic LDS limit above 64 KiB is a per-device attribute of the kernel: set it once per
  // device (bit d of the mask; devices past 63 set it on every launch).
  static unsigned long long attr_set = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 64 || !((attr_set >> dev) & 1ull)) {
    hipError_t e = hipFuncSetAttribute((const void*)mx_gemm_pipe_kernel<EPI, RK, SW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, ScaleRing<SW>::LDS);
    if (e != hipSuccess) return e;
    if (dev < 64) attr_set |= 1ull << dev;
  }
  MxGemmArgs q = a;
  q.tiles = tiles;
  const int blocks = std::min(tiles, device_cus());
  hipLaunchKernelGGL((mx_gemm_pipe_kernel<EPI, RK, SW>), dim3(blocks), dim3(512), ScaleRing<SW>::LDS, s, q);
  return hipGetLastError();
}

// 16-byte scale loads need every row's scale run, group offset and K split on 16-byte boundaries of
// the scale arrays (K, row strides, group stride and split multiples of 512 elements), and no K offset.
inline bool wide_scales(const MxGemmArgs& a, bool ragged_k) {
  auto al = [](const void* ptr) { return ptr == nullptr || ((uintptr_t)ptr & 15) == 0; };
  return !ragged_k && a.K % 512 == 0 && a.lda % 512 == 0 && a.ldb % 512 == 0 && a.b_gstride % 512 == 0 &&
         (a.ksplit == 0 || a.ksplit % 512 == 0) && al(a.as) && al(a.bs) && al(a.bs2);
}

template <int EPI, bool RK>
hipError_t launch_mx_pipe(const MxGemmArgs& a, int tiles, hipStream_t s) {
  if (wide_scales(a, RK)) return launch_mx_pipe_sw<EPI, RK, 16>(a, tiles, s);
  return launch_mx_pipe_sw<EPI, RK, 4>(a, tiles, s);
}

// Sum of the K parts of a weight-gradient product, in part order, rounded once to bf16; rows
// [0, split) of each group to out0, the others to out1.  8 consecutive elements per thread.
__global__ __launch_bounds__(256) void mx_k_reduce_kernel(const float* __restrict__ partial, int S, int G, int M,
                                                          int N, int split, bf16_t* __restrict__ out0,
                                                          bf16_t* __restrict__ out1) {
  const long long per = (long long)M * N;
  const long long total = (long long)G * per / 8;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const long long e0 = i * 8;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int q = 0; q < S; ++q) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(partial + (long long)q * G * per + e0);
      const u32x4_t a = src[0], b = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] += __uint_as_float(a[e]);
        v[4 + e] += __uint_as_float(b[e]);
      }
    }
    const long long g = e0 / per, rem = e0 - g * per;
    const int row = (int)(rem / N), col = (int)(rem - (long long)row * N);
    bf16_t* dst = row < split ? out0 + ((long long)g * split + row) * N + col
                              : out1 + ((long long)g * (M - split) + (row - split)) * N + col;
    *reinterpret_cast<u32x4_t*>(dst) = pack8(v);
  }
}

template <int EPI, bool RK>
hipError_t launch_mx(const MxGemmArgs& a, int blocks, hipStream_t s) {
  hipLaunchKernelGGL((mx_gemm_kernel<EPI, RK>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quant_rows(const void* x, long long R, int K, long long ldx, uint8_t* codes,
                                uint8_t* scales, hipStream_t s) {
  const long long total = R * (K / 8);
  if (total == 0) return hipSuccess;
  const int blocks = (int)std::min<long long>((total + 255) / 256, 256LL * 16);
  hipLaunchKernelGGL(mx_quant_rows_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const bf16_t*>(x), R,
                     K, ldx, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quant_cols(const void* x, long long R, int N, long long ldx, const int32_t* offsets,
                                int G, long long group_rows, int kpad, uint8_t* codes, uint8_t* scales,
                                long long ldc, int32_t* kbase, hipStream_t s) {
  hipLaunchKernelGGL(mx_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, G, group_rows, R, kpad, kpad, kbase);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ldc == 0 || N == 0) return e;
  hipLaunchKernelGGL(mx_quant_cols_kernel, dim3((unsigned)(ldc / 128), (unsigned)((N + 511) / 512)), dim3(256), 0,
                     s, reinterpret_cast<const bf16_t*>(x), R, N, ldx, offsets, G, group_rows, kbase, codes,
                     scales, ldc);
  return hipGetLastError();
}

int mx_k_parts(int G, int M, int N) {
  if (M % PB != 0 || N % PB != 0) return 1;   // the 128x128 kernel does not split
  const long long tiles = (long long)G * (M / PB) * (N / PB);
  const int cus = device_cus();
  if (tiles >= cus) return 1;
  return (int)std::min<long long>(16, (cus + tiles - 1) / tiles);
}

size_t mx_k_workspace_bytes(int G, int M, int N) {
  const int S = mx_k_parts(G, M, N);
  return S > 1 ? (size_t)S * G * M * N * sizeof(float) : 0;
}

hipError_t launch_mx_gemm(int epi, bool ragged_k, const MxGemmArgs& a, hipStream_t s) {
  // The pipelined 256x256 kernel covers output widths that are multiples of its tile (128 columns
  // for SwiGLU) and, for weight gradients, output heights that are multiples of 256.
  const bool pipe = (epi == MX_EPI_SWIGLU ? a.N % 128 == 0 : a.N % PB == 0) && (!ragged_k || a.M % PB == 0);
  const int TM = pipe ? PB : TB;
  const int OC = epi == MX_EPI_SWIGLU ? TM / 2 : TM;
  const long long NT = a.N / OC;
  long long tiles;
  if (!ragged_k) {
    if (!pipe) {   // the pipelined kernel computes its tile prefix itself
      hipLaunchKernelGGL(mx_prefix_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.G, 0LL, (long long)a.M, TM, 1,
                         a.tile_prefix);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    tiles = ((long long)(a.M + TM - 1) / TM + a.G) * NT;
  } else {
    tiles = (long long)a.G * (a.M / TM) * NT;
  }
  if (tiles == 0) return hipSuccess;
  const int blocks = (int)tiles;
  if (pipe) {
    if (ragged_k) {
      if (a.kparts <= 1) return launch_mx_pipe<MX_EPI_STORE, true>(a, blocks, s);
      hipError_t e = launch_mx_pipe<MX_EPI_STORE, true>(a, blocks * a.kparts, s);
      if (e != hipSuccess) return e;
      const long long n8 = (long long)a.G * a.M * a.N / 8;
      const int rb = (int)std::min<long long>((n8 + 255) / 256, 4096);
      hipLaunchKernelGGL(mx_k_reduce_kernel, dim3(rb), dim3(256), 0, s, a.partial, a.kparts, a.G, a.M, a.N, a.split,
                         reinterpret_cast<bf16_t*>(a.out0), reinterpret_cast<bf16_t*>(a.out1));
      return hipGetLastError();
    }
    switch (epi) {
      case MX_EPI_SWIGLU: return launch_mx_pipe<MX_EPI_SWIGLU, false>(a, blocks, s);
      case MX_EPI_SWIGLU_BWD: return launch_mx_pipe<MX_EPI_SWIGLU_BWD, false>(a, blocks, s);
      default: return launch_mx_pipe<MX_EPI_STORE, false>(a, blocks, s);
    }
  }
  if (ragged_k) return launch_mx<MX_EPI_STORE, true>(a, blocks, s);
  hipError_t e;
  switch (epi) {
    case MX_EPI_SWIGLU: e = launch_mx<MX_EPI_SWIGLU, false>(a, blocks, s); break;
    case MX_EPI_SWIGLU_BWD: e = launch_mx<MX_EPI_SWIGLU_BWD, false>(a, blocks, s); break;
    default: return launch_mx<MX_EPI_STORE, false>(a, blocks, s);
  }
  if (e != hipSuccess || !a.qc) return e;
  // The 128x128 kernel does not quantize in its epilogue: quantize the stored rows afterwards.
  const int K = epi == MX_EPI_SWIGLU ? a.N : 2 * a.N;
  return launch_mx_quant_rows(epi == MX_EPI_SWIGLU ? a.out2 : a.out0, a.M, K, K, a.qc, a.qs, s);
}

}  // namespace moe
