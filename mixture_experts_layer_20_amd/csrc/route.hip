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

#include <type_traits>

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int RT = 32;   // tokens per block
constexpr int RE = 64;   // experts per block
constexpr int RK = 128;  // features per LDS step (long enough to cover the next step's global loads)
constexpr int RTH = 256; // threads per block: 16 x 16, each 2 tokens x 4 experts (4 waves per CU)

// 8 consecutive elements k0.. of a row as fp32 (0 past n; a 16-byte load when the row is aligned and
// all 8 are in range).
template <bool BF16>
__device__ __forceinline__ void row8(const void* base, size_t row_off, int k0, int n, bool valid, float (&v)[8]) {
  if (BF16) {
    const bf16_t* r = reinterpret_cast<const bf16_t*>(base) + row_off;
    if (valid && k0 + 8 <= n && ((row_off + k0) & 7) == 0) {
      const uint4 u = *reinterpret_cast<const uint4*>(r + k0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (valid && k0 + i < n) ? bf16_to_f32(r[k0 + i]) : 0.0f;
    }
  } else {
    const float* r = reinterpret_cast<const float*>(base) + row_off;
    if (valid && k0 + 8 <= n && ((row_off + k0) & 3) == 0) {
      const float4 a = *reinterpret_cast<const float4*>(r + k0), b = *reinterpret_cast<const float4*>(r + k0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (valid && k0 + i < n) ? r[k0 + i] : 0.0f;
    }
  }
}

// One feature of the 2x4 block: products in the canonical order (see router_logits_kernel).
template <bool BF16>
__device__ __forceinline__ void logits_step(const float* xrow, const float* wrow, int tx, int ty, float (&acc)[2][4]) {
  const float2 av = *reinterpret_cast<const float2*>(xrow + ty * 2);
  const float4 bv = *reinterpret_cast<const float4*>(wrow + tx * 4);
  const float a[2] = {av.x, av.y}, b[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float prod = a[i] * b[j];
      acc[i][j] = acc[i][j] + prod;
    }
}

// Logits on the vector ALU (fp32 inputs, and bf16 rows whose length is not a multiple of 8): one
// thread owns 2 tokens x 4 experts and walks the features in increasing order, each product and
// each sum rounded separately.  The next 128-feature tile is loaded into registers while the
// current one is multiplied.
template <bool BF16>
__global__ __launch_bounds__(RTH) void router_logits_kernel(const void* xv, const void* wv,
                                                            const float* bias, float* logits,
                                                            int T, int d, int E) {
  __shared__ __attribute__((aligned(16))) float xs[RK][RT];
  __shared__ __attribute__((aligned(16))) float ws[RK][RE];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * RT, e0 = blockIdx.y * RE;
  // staging: thread q loads features (q % 8) * 16 .. + 16 of token row q / 8, and features
  // (q % 4) * 32 .. + 32 of expert row q / 4
  const int xr_row = tid >> 3, xk = (tid & 7) * 16;
  const int wr_row = tid >> 2, wk = (tid & 3) * 32;
  const bool xok = t0 + xr_row < T, wok = e0 + wr_row < E;
  const size_t xoff = (size_t)(xok ? t0 + xr_row : 0) * d, woff = (size_t)(wok ? e0 + wr_row : 0) * d;
  float xr[2][8], wr[4][8];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) row8<BF16>(xv, xoff, k0 + xk + 8 * c, d, xok, xr[c]);
#pragma unroll
    for (int c = 0; c < 4; ++c) row8<BF16>(wv, woff, k0 + wk + 8 * c, d, wok, wr[c]);
  };
  fetch(0);
  float acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < d; k0 += RK) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) xs[xk + 8 * c + i][xr_row] = xr[c][i];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) ws[wk + 8 * c + i][wr_row] = wr[c][i];
    __syncthreads();
    if (k0 + RK < d) fetch(k0 + RK);
    const int kn = d - k0 < RK ? d - k0 : RK;
    if (kn == RK) {
#pragma unroll
      for (int kk = 0; kk < RK; ++kk) logits_step<BF16>(xs[kk], ws[kk], tx, ty, acc);
    } else {
      for (int kk = 0; kk < kn; ++kk) logits_step<BF16>(xs[kk], ws[kk], tx, ty, acc);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + ty * 2 + i;
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

// Logits of bf16 inputs on the matrix core.  v_mfma_f32_16x16x1_4b_f32 adds one product per output
// per instruction (K = 1), rounding each step to nearest like an FMA, and a product of two bf16
// values is exact in fp32 (while it is not below the normal range, see below), so a chain of them
// over k = 0, 1, ... is the canonical sequential sum bit for bit at twice the rate of unpacked fp32
// FMAs.  The instruction issues every 32 cycles, dependent or not (measured), so one wave per SIMD
// runs one chain: 16 tokens (operand A, the same in the instruction's four 16x16 blocks) by 64
// experts (operand B, one per lane, block b = experts 16b..16b+15).  Output register r of lane l is
// block r/4, token row 4*(l/16) + r%4, expert column l%16.
//
// A vector-ALU instruction of the wave that runs the chain waits for the matrix core (measured:
// each one adds about 7 cycles to the chain), while one from another wave on the same SIMD runs
// beside it.  So a workgroup is 4 chain waves (64 tokens by 64 experts) and 4 staging waves.  The
// staging waves load 128-k slices of the token and expert rows (whole 256-byte row segments per
// instruction, one slice ahead), widen the bf16 values to fp32 and store them in LDS (rows padded
// by 16 bytes so 16 rows read at one offset hit distinct banks), double buffered, one barrier per
// slice.  A chain wave only reads its fp32 operands from LDS, the next 8 k while the current 8
// products run, and issues matrix-core instructions.  Chunks past d are staged as zeros: a product
// 0 * 0 = +0 leaves every partial sum unchanged (the canonical sum starts at +0 and so is never
// -0).  Rows past T or E are clamped to the last row and their results not stored.
//
// The matrix core rounds a subnormal partial sum differently from IEEE fp32, and a product below
// fp32's normal range is not exact.  Neither can arise when every nonzero input has magnitude
// >= 2^-50: every product (at most 16 significant bits) is then a multiple of 2^-114, and so is
// every partial sum, which is therefore zero or at least 2^-114.  The staging threads keep the
// minimum over the values they stage of 2|v| - 1 (16-bit integers, so zero wraps to the top); a
// workgroup that saw a nonzero |v| below 2^-50 recomputes its outputs on the vector ALU in the
// canonical order.
typedef float f32x16_r __attribute__((ext_vector_type(16)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
constexpr uint16_t RM_TINY = 77 << 7;   // bf16 magnitude bits of 2^-50
constexpr int RM_TOK = 16, RM_EXP = 64, RM_CW = 4;   // tokens per chain, experts, chain waves
constexpr int RM_ROWS = RM_TOK * RM_CW;              // token rows of a workgroup (= staging rows)
constexpr int RM_CH = 16;                            // chunks of 8 k per slice
constexpr int RM_PITCH = RM_CH * 8 + 4;              // floats per staged row (16-byte pad)
constexpr int RM_BUF = RM_ROWS * RM_PITCH;           // floats per staged operand slice
constexpr int RM_LDS = 4 * RM_BUF * 4;               // bytes: 2 buffers x (tokens, experts)
constexpr int RM_NTH = 64 * 2 * RM_CW;
static_assert(RM_ROWS == RM_EXP && RM_ROWS * RM_CH == 4 * 64 * RM_CW, "staging map: 4 rows per thread");
static_assert(RM_LDS > (160 << 10) / 2, "one workgroup per compute unit");

// Packed running minimum of 2|v| - 1 over the 8 bf16 values of a chunk.
__device__ __forceinline__ u16x2_t tiny_scan(u16x2_t mn, const uint4& v) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u16x2_t two = {2, 2}, mone = {0xffff, 0xffff};
    mn = __builtin_elementwise_min(mn, __builtin_bit_cast(u16x2_t, w4[i]) * two + mone);
  }
  return mn;
}
__device__ __forceinline__ bool tiny_seen(u16x2_t mn) {
  return mn.x < 2 * RM_TINY - 1 || mn.y < 2 * RM_TINY - 1;
}
__device__ __forceinline__ void widen_store(float* dst, const uint4& v) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                                                  __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  reinterpret_cast<float4*>(dst)[1] = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xffff0000u),
                                                  __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xffff0000u));
}

__global__ __launch_bounds__(RM_NTH) void router_logits_mfma_kernel(const bf16_t* x, const bf16_t* w,
                                                                   const float* bias, float* logits, int T,
                                                                   int d, int E) {
  extern __shared__ __attribute__((aligned(16))) float rlds[];   // [buffer][tokens | experts][row][RM_PITCH]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * RM_ROWS, e0 = blockIdx.y * RM_EXP;
  const int nch = d >> 3, nkb = (nch + RM_CH - 1) / RM_CH;
  u16x2_t mn = {0xffff, 0xffff};
  f32x16_r acc = {};
  if (wave >= RM_CW) {
    // staging: thread i copies chunk i % 16 of rows i / 16 + 16 q, q = 0..3 (a row is 16 threads)
    const int st = tid - 64 * RM_CW, sr = st >> 4, sc = st & 15;
    const uint4* xsrc[4];
    const uint4* wsrc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xsrc[q] = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + sr + 16 * q, T - 1) * d);
      wsrc[q] = reinterpret_cast<const uint4*>(w + (size_t)min(e0 + sr + 16 * q, E - 1) * d);
    }
    uint4 sx[4], sw[4];
    // Global loads are never under a branch (the chunk index is clamped and the value zeroed when
    // staged): a load under a condition makes the compiler wait for every load in flight.
    auto stage_load = [&](int kb) {
      const int c = min(kb * RM_CH + sc, nch - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sx[q] = xsrc[q][c];
        sw[q] = wsrc[q][c];
      }
    };
    auto stage_store = [&](int buf, int kb) {
      if ((kb + 1) * RM_CH > nch) {   // the last, partial slice: chunks past d become zeros
        const uint32_t keep = kb * RM_CH + sc < nch ? 0xffffffffu : 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sx[q] = make_uint4(sx[q].x & keep, sx[q].y & keep, sx[q].z & keep, sx[q].w & keep);
          sw[q] = make_uint4(sw[q].x & keep, sw[q].y & keep, sw[q].z & keep, sw[q].w & keep);
        }
      }
      float* xd = rlds + (2 * buf) * RM_BUF + sr * RM_PITCH + sc * 8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 vx = sx[q], vw = sw[q];
        mn = tiny_scan(tiny_scan(mn, vx), vw);
        widen_store(xd + 16 * q * RM_PITCH, vx);
        widen_store(xd + RM_BUF + 16 * q * RM_PITCH, vw);
      }
    };
    stage_load(0);
    stage_store(0, 0);
    stage_load(min(1, nkb - 1));
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
      // slice kb+1 into the other buffer (last read in slice kb-1, before the previous barrier)
      if (kb + 1 < nkb) stage_store((kb + 1) & 1, kb + 1);
      stage_load(min(kb + 2, nkb - 1));
      __syncthreads();
    }
  } else {
    // chain wave: token row wave*16 + lane%16 (operand A), expert row lane (operand B)
    const float4* xr = reinterpret_cast<const float4*>(rlds + (wave * RM_TOK + (lane & 15)) * RM_PITCH);
    const float4* wr = reinterpret_cast<const float4*>(rlds + RM_BUF + lane * RM_PITCH);
    constexpr int BUF4 = 2 * RM_BUF / 4;   // float4s from one buffer to the next
    __syncthreads();
    float4 xn0 = xr[0], xn1 = xr[1], wn0 = wr[0], wn1 = wr[1];
    for (int kb = 0; kb < nkb; ++kb) {
      const int o = (kb & 1) * BUF4;
#pragma unroll
      for (int r = 0; r < RM_CH; ++r) {
        const float4 x0 = xn0, x1 = xn1, w0 = wn0, w1 = wn1;
        if (r + 1 < RM_CH) {
          xn0 = xr[o + 2 * r + 2];
          xn1 = xr[o + 2 * r + 3];
          wn0 = wr[o + 2 * r + 2];
          wn1 = wr[o + 2 * r + 3];
        }
        __builtin_amdgcn_sched_barrier(0);   // keeps the reads ahead of this chunk's products
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        const float ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x1f32(xs[i], ws[i], acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      const int on = ((kb + 1) & 1) * BUF4;
      xn0 = xr[on];
      xn1 = xr[on + 1];
      wn0 = wr[on];
      wn1 = wr[on + 1];
    }
  }
  const bool tiny = __syncthreads_or(tiny_seen(mn)) != 0;
  const int tw = t0 + wave * RM_TOK;
  if (wave >= RM_CW || tw >= T) return;
  if (tiny) {
    // canonical order on the vector ALU: each product rounded, then the sum (contraction is off)
#pragma unroll 1
    for (int r = 0; r < 16; ++r) {
      const int tt = min(tw + 4 * (lane >> 4) + (r & 3), T - 1), ee = min(e0 + 16 * (r >> 2) + (lane & 15), E - 1);
      const bf16_t* xt = x + (size_t)tt * d;
      const bf16_t* we = w + (size_t)ee * d;
      float s = 0.0f;
      for (int kk = 0; kk < d; ++kk) {
        const float prod = bf16_to_f32(xt[kk]) * bf16_to_f32(we[kk]);
        s = s + prod;
      }
      acc[r] = s;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tt = tw + 4 * (lane >> 4) + (r & 3), ee = e0 + 16 * (r >> 2) + (lane & 15);
    if (tt < T && ee < E) {
      float v = acc[r];
      if (bias) v = v + bias[ee];
      logits[(size_t)tt * E + ee] = v;
    }
  }
}

// Selection key of a (logit, expert) pair: a larger key is selected first.  The high word orders
// the logits (the sign-magnitude bits mapped to a monotone unsigned code, -0 taken as +0 so equal
// logits tie), a NaN gets code 0, below every number (whose codes are at least 0x007fffff); the
// low word is ~e, so equal codes go to the lower expert index.  Keys of distinct experts differ,
// and every real key exceeds 0, the key of an empty or already taken slot.
__device__ __forceinline__ uint64_t select_key(float v, int e) {
  uint32_t b = __float_as_uint(v);
  b = b == 0x80000000u ? 0u : b;
  const uint32_t flip = (uint32_t)((int32_t)b >> 31) | 0x80000000u;   // ~b below zero, b | sign above
  const uint32_t code = (b & 0x7fffffffu) > 0x7f800000u ? 0u : b ^ flip;
  return ((uint64_t)code << 32) | (uint32_t)~e;
}
// The logit a key was made from (a NaN for code 0; +0 for -0).
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t code = (uint32_t)(key >> 32);
  if (code == 0u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(code & 0x80000000u ? code & 0x7fffffffu : ~code);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }

// The larger of key and the key of the lane that DPP control CTRL names (within a 16-lane row).
template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp(uint64_t key) {
  const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)key, CTRL, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(key >> 32), CTRL, 0xf, 0xf, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > key ? o : key;
}

// Top-k and gates: L lanes per token (16 or 32), S logits per lane (lane j of a token holds experts
// j, j + L, ..., j + (S-1) L), so L * S >= E.  Round r takes the largest key of the token (the
// lane's best slot, then a maximum over the token's lanes: quad swaps and row rotations by DPP,
// and one exchange across rows for L = 32), clears that slot, and lane r keeps it.
template <int L, int S>
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* logits, int T, int E, int k,
                                                        int renormalize, int32_t* topk_idx,
                                                        float* topk_gate) {
  const long long gl = (long long)blockIdx.x * 256 + threadIdx.x;   // T * L may exceed 2^31
  const int t = (int)(gl / L), j = (int)(gl % L);
  if (__builtin_amdgcn_readfirstlane(t) >= T) return;   // the wave's first token is past T
  const int tc = min(t, T - 1);
  float v[S];
  uint64_t key[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {   // unconditional loads (clamped expert), so all are in flight together
    const int e = j + s * L;
    v[s] = logits[(size_t)tc * E + min(e, E - 1)];
    key[s] = e < E ? select_key(v[s], e) : 0ull;
  }
  uint64_t top = 0, mine = 0;
  float denom = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (r >= k) break;
    uint64_t best = key[0];
#pragma unroll
    for (int s = 1; s < S; ++s) best = key[s] > best ? key[s] : best;
    best = max_dpp<0xB1>(best);    // quad_perm 1,0,3,2
    best = max_dpp<0x4E>(best);    // quad_perm 2,3,0,1
    best = max_dpp<0x124>(best);   // row_ror 4
    best = max_dpp<0x128>(best);   // row_ror 8: every lane of the row holds the row's best
    if constexpr (L == 32) {
      const uint32_t lo = __shfl_xor((int)(uint32_t)best, 16, 64);
      const uint32_t hi = __shfl_xor((int)(uint32_t)(best >> 32), 16, 64);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      best = o > best ? o : best;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) key[s] = key[s] == best ? 0ull : key[s];
    if (r == 0) top = best;
    if (j == r) mine = best;
    if (renormalize) denom += expf(key_logit(best) - key_logit(top));
  }
  const float vmax = key_logit(top);   // the token's largest logit
  if (!renormalize) {
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (j + s * L < E) part += expf(v[s] - vmax);
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    denom = part;
  }
  if (t < T && j < k) {
    topk_idx[(size_t)t * k + j] = key_expert(mine);
    topk_gate[(size_t)t * k + j] = expf(key_logit(mine) - vmax) / denom;
  }
}

// ------------------------------------------------------------------------------------------
// Router backward (gates = softmax over the chosen logits).

// The logit gradients of a token's K (>= k) chosen experts: dl_j = g_j (dg_j - sum_i g_i dg_i),
// evaluated as g_j * sum_i g_i (dg_j - dg_i), equal because the gates sum to one; this form has no
// cancellation between large terms when one gate is close to 1 and the others are tiny.  Entries
// j >= k are 0.  Every kernel below takes its dl from here, so all of them see the same values.
template <int K>
__device__ __forceinline__ void token_logit_grads(const float* gate, const float* dgate, size_t t, int k,
                                                  float (&dl)[K]) {
  float g[K], dg[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {   // loads at a clamped index, never under a condition
    const size_t a = t * k + (i < k ? i : k - 1);
    g[i] = i < k ? gate[a] : 0.0f;
    dg[i] = i < k ? dgate[a] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (i < k) s += g[i] * (dg[j] - dg[i]);
    dl[j] = j < k ? g[j] * s : 0.0f;
  }
}
// The logit gradient of assignment a = t*k + j.
__device__ __forceinline__ float assignment_logit_grad(const float* gate, const float* dgate, int a, int k) {
  float dl[8];
  token_logit_grads<8>(gate, dgate, (size_t)(a / k), k, dl);
  const int j = a % k;
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i == j) r = dl[i];
  return r;
}

// dx_router[t] = sum_j dl[t,j] * w_router[idx[t,j]], one block per token (any d).
template <typename T>
__global__ __launch_bounds__(256) void route_dx_kernel(const float* dgate, const float* gate, const int32_t* idx,
                                                       const T* w, int d, int k, T* dx) {
  const int t = blockIdx.x;
  float dl[8];
  token_logit_grads<8>(gate, dgate, (size_t)t, k, dl);
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) acc += dl[j] * to_f32<T>(w[(size_t)idx[(size_t)t * k + j] * d + c]);
    dx[(size_t)t * d + c] = from_f32<T>(acc);
  }
}

constexpr int SEG = 64;        // permuted rows per partial sum of the router weight gradient
constexpr int DWCOLS = 1024;   // columns per block (any d)
constexpr int DWCOLS8 = 2048;  // columns per block, 8 per thread (d a multiple of 8)
constexpr int DXCOLS = 2048;   // dx_router columns per block, 8 per thread (d a multiple of 8)
constexpr int DXL = 16;        // 16-byte expert-row loads in flight per thread in a dx_router block
// Tokens per dx_router block for K expert rows per token (T: element type of the rows).
template <typename T, int K>
constexpr int dx_tokens() { return DXL / (K * (sizeof(T) == 2 ? 1 : 2)) > 0 ? DXL / (K * (sizeof(T) == 2 ? 1 : 2)) : 1; }

// pre[e] = SEG-row segments of the experts before e, pre[E] = all of them, in LDS, computed by the
// block itself (blockDim 256, E <= 256) from the clamped offsets.
__device__ __forceinline__ void seg_prefix_lds(const int32_t* offsets, int E, int Tk, int* pre) {
  const int tid = threadIdx.x;
  int c = 0;
  if (tid < E) {
    int lo = offsets[tid], hi = offsets[tid + 1];
    lo = lo < 0 ? 0 : (lo > Tk ? Tk : lo);
    hi = hi < lo ? lo : (hi > Tk ? Tk : hi);
    c = (hi - lo + SEG - 1) / SEG;
  }
  pre[tid + 1] = c;
  if (tid == 0) pre[0] = 0;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? pre[tid + 1 - off] : 0;
    __syncthreads();
    pre[tid + 1] += v;
    __syncthreads();
  }
}

// The segment of a partial-sum block: its expert e and permuted rows [p0, p1); false past the last.
__device__ __forceinline__ bool find_segment(const int* pre, const int32_t* offsets, int E, int Tk, int seg, int& e,
                                             int& p0, int& p1) {
  if (seg >= pre[E]) return false;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= seg) lo = mid; else hi = mid;
  }
  e = lo;
  int r0 = offsets[e], r1 = offsets[e + 1];
  r0 = r0 < 0 ? 0 : (r0 > Tk ? Tk : r0);
  r1 = r1 < r0 ? r0 : (r1 > Tk ? Tk : r1);
  p0 = r0 + (seg - pre[e]) * SEG;
  p1 = p0 + SEG < r1 ? p0 + SEG : r1;
  return true;
}

// The segment's token rows and logit gradients, staged in LDS in permuted-row order.
__device__ __forceinline__ void stage_segment(const float* dgate, const float* gate, const int32_t* src_row, int k,
                                              int Tk, int p0, int n, int* tok_s, float* w_s) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int a = src_row[p0 + i];
    a = a < 0 ? 0 : (a >= Tk ? Tk - 1 : a);   // a valid row even for a corrupt plan
    tok_s[i] = a / k;
    w_s[i] = assignment_logit_grad(gate, dgate, a, k);
  }
  __syncthreads();
}

// Partial dW_router rows: segment s of expert e sums dl(a) * x[a / k] over its rows in order.
template <typename T>
__global__ __launch_bounds__(256) void route_dw_partial_kernel(const float* dgate, const float* gate,
                                                               const int32_t* src_row, const int32_t* offsets,
                                                               const T* x, int E, int Tk, int d, int k,
                                                               float* partial) {
  __shared__ int pre[257];
  __shared__ int tok_s[SEG];
  __shared__ float w_s[SEG];
  seg_prefix_lds(offsets, E, Tk, pre);
  const int seg = blockIdx.x;
  int e, p0, p1;
  if (!find_segment(pre, offsets, E, Tk, seg, e, p0, p1)) return;
  const int cbase = blockIdx.y * DWCOLS;
  const int n = p1 - p0;
  stage_segment(dgate, gate, src_row, k, Tk, p0, n, tok_s, w_s);
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
        const float wgt = w_s[r0 + u];
#pragma unroll
        for (int i = 0; i < NC; ++i) acc[i] += wgt * xv[u][i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = cbase + threadIdx.x + i * 256;
    if (c < d) partial[(size_t)seg * d + c] = acc[i];
  }
}

// 8 columns of one expert row as floats, from 16-byte loads already issued (RW of them: 1 for bf16,
// 2 for fp32).
template <typename T, int RW>
__device__ __forceinline__ void unpack8(const uint4 (&u)[RW], float (&v)[8]) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const uint32_t wd[4] = {u[0].x, u[0].y, u[0].z, u[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(wd[i] << 16);
      v[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      v[4 * r + 0] = __uint_as_float(u[r].x);
      v[4 * r + 1] = __uint_as_float(u[r].y);
      v[4 * r + 2] = __uint_as_float(u[r].z);
      v[4 * r + 3] = __uint_as_float(u[r].w);
    }
  }
}

// The router backward for d a multiple of 8, in one launch: blocks [0, ndw) form the dW_router
// partial sums (block b: segment b / ncw, 2048 columns b % ncw, 8 per thread), the rest dx_router
// (dx_tokens tokens per block, 2048 columns, 8 per thread).  The two kinds share no data; one launch
// lets the latency-bound dx_router blocks run beside the bandwidth-bound partial sums.  A dx_router
// thread issues all DXL expert-row loads of its tokens before it multiplies (a block per token kept
// too few bytes in flight per CU); rows j >= k of a token (K > k) load a valid row and are skipped.
template <typename T, int K>
__global__ __launch_bounds__(256) void route_bwd8_kernel(const float* dgate, const float* gate, const int32_t* idx,
                                                         const int32_t* src_row, const int32_t* offsets, const T* x,
                                                         const T* w, int Tn, int d, int E, int k, int ndw, int ncw,
                                                         float* partial, T* dx) {
  constexpr int RW = sizeof(T) == 2 ? 1 : 2;   // 16-byte loads per 8 columns
  const int Tk = Tn * k;
  if ((int)blockIdx.x < ndw) {
    __shared__ int pre[257];
    __shared__ int tok_s[SEG];
    __shared__ float w_s[SEG];
    seg_prefix_lds(offsets, E, Tk, pre);
    const int seg = blockIdx.x / ncw;
    int e, p0, p1;
    if (!find_segment(pre, offsets, E, Tk, seg, e, p0, p1)) return;
    const int n = p1 - p0;
    stage_segment(dgate, gate, src_row, k, Tk, p0, n, tok_s, w_s);
    const int c = (blockIdx.x % ncw) * DWCOLS8 + threadIdx.x * 8;
    if (c >= d) return;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    for (int rr = 0; rr < n; rr += 8) {
      uint4 raw[8][RW];
#pragma unroll
      for (int u = 0; u < 8; ++u) {   // rows past the segment load its first row (never used)
        const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)tok_s[rr + u < n ? rr + u : 0] * d + c);
#pragma unroll
        for (int r = 0; r < RW; ++r) raw[u][r] = src[r];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (rr + u < n) {
          float xv[8];
          unpack8<T, RW>(raw[u], xv);
          const float wgt = w_s[rr + u];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += wgt * xv[q];
        }
      }
    }
    float* out = partial + (size_t)seg * d + c;
    reinterpret_cast<float4*>(out)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(out)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    return;
  }
  constexpr int NT = dx_tokens<T, K>();
  const int ncx = (d + DXCOLS - 1) / DXCOLS;
  const int b = blockIdx.x - ndw, tb = b / ncx;
  const int c = (b % ncx) * DXCOLS + threadIdx.x * 8;
  if (c >= d) return;
  float dl[NT][K];
  uint4 raw[NT][K][RW];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int t = min(tb * NT + tt, Tn - 1);
    token_logit_grads<K>(gate, dgate, (size_t)t, k, dl[tt]);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      int e = idx[(size_t)t * k + (j < k ? j : k - 1)];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);   // a valid row even for a corrupt selection
      const uint4* src = reinterpret_cast<const uint4*>(w + (size_t)e * d + c);
#pragma unroll
      for (int r = 0; r < RW; ++r) raw[tt][j][r] = src[r];
    }
  }
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int t = tb * NT + tt;
    if (t >= Tn) break;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (j < k) {
        float wv[8];
        unpack8<T, RW>(raw[tt][j], wv);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += dl[tt][j] * wv[q];
      }
    }
    T* out = dx + (size_t)t * d + c;
    if constexpr (std::is_same<T, bf16_t>::value) {
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u[i] = (uint32_t)from_f32<bf16_t>(acc[2 * i]) | ((uint32_t)from_f32<bf16_t>(acc[2 * i + 1]) << 16);
      *reinterpret_cast<uint4*>(out) = make_uint4(u[0], u[1], u[2], u[3]);
    } else {
      reinterpret_cast<float4*>(out)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      reinterpret_cast<float4*>(out)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// dW_router[e] = sum of the expert's segment partials, in segment order (zeros if none).  Segments
// past nseg (the partial sums that exist) are never read.  The form for d a multiple of 4 takes four
// columns per thread in 16-byte loads, one column quad per thread, so all of a thread's segment
// loads are in flight together; the other form strides over the block's columns.
__global__ __launch_bounds__(256) void route_dw_reduce_kernel(const float* partial, const int32_t* offsets, int E,
                                                              int Tk, int d, int nseg, float* dw) {
  __shared__ int pre[257];
  seg_prefix_lds(offsets, E, Tk, pre);
  const int e = blockIdx.x;
  const int s0 = min(pre[e], nseg), s1 = min(pre[e + 1], nseg);
  for (int c = blockIdx.y * DWCOLS + threadIdx.x; c < d && c < (blockIdx.y + 1) * DWCOLS; c += 256) {
    float acc = 0.0f;
#pragma unroll 16
    for (int s = s0; s < s1; ++s) acc += partial[(size_t)s * d + c];   // in order; loads overlap
    dw[(size_t)e * d + c] = acc;
  }
}

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

hipError_t launch_router_logits(const void* x, const void* w, const float* bias, float* logits,
                                int T, int d, int E, bool bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16 && d % 8 == 0) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(router_logits_mfma_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, RM_LDS);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(router_logits_mfma_kernel, dim3(ceil_div(T, RM_ROWS), ceil_div(E, RM_EXP)), dim3(RM_NTH),
                       RM_LDS, s, reinterpret_cast<const bf16_t*>(x), reinterpret_cast<const bf16_t*>(w), bias,
                       logits, T, d, E);
    return hipGetLastError();
  }
  dim3 grid(ceil_div(T, RT), ceil_div(E, RE));
  if (bf16) hipLaunchKernelGGL(router_logits_kernel<true>, grid, dim3(RTH), 0, s, x, w, bias, logits, T, d, E);
  else hipLaunchKernelGGL(router_logits_kernel<false>, grid, dim3(RTH), 0, s, x, w, bias, logits, T, d, E);
  return hipGetLastError();
}

hipError_t launch_topk_gate(const float* logits, int T, int E, int k, int renormalize,
                            int32_t* topk_idx, float* topk_gate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E <= 64)
    hipLaunchKernelGGL((topk_gate_kernel<16, 4>), dim3(ceil_div(T, 16)), dim3(256), 0, s, logits, T, E, k,
                       renormalize, topk_idx, topk_gate);
  else if (E <= 128)
    hipLaunchKernelGGL((topk_gate_kernel<16, 8>), dim3(ceil_div(T, 16)), dim3(256), 0, s, logits, T, E, k,
                       renormalize, topk_idx, topk_gate);
  else
    hipLaunchKernelGGL((topk_gate_kernel<32, 8>), dim3(ceil_div(T, 8)), dim3(256), 0, s, logits, T, E, k,
                       renormalize, topk_idx, topk_gate);
  return hipGetLastError();
}
__global__ __launch_bounds__(256) void route_dw_reduce4_kernel(const float* partial, const int32_t* offsets, int E,
                                                               int Tk, int d, int nseg, float* dw) {
  __shared__ int pre[257];
  seg_prefix_lds(offsets, E, Tk, pre);
  const int e = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  const int s0 = min(pre[e], nseg), s1 = min(pre[e + 1], nseg);
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 8
  for (int s = s0; s < s1; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(partial + (size_t)s * d + c);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(dw + (size_t)e * d + c) = acc;
}

static inline long long max_segments(long long Tk, int E) { return (Tk + SEG - 1) / SEG + E; }

size_t route_bwd_ws_bytes(long long T, long long d, int E, int k) {
  const long long Tk = T * k;
  return align256((size_t)max_segments(Tk, E) * d * sizeof(float));
}

template <typename T>
static void launch_route_bwd8(const float* dgate, const float* gate, const int32_t* idx, const int32_t* src_row,
                              const int32_t* offsets, const T* x, const T* w, int Tn, int d, int E, int k,
                              float* partial, T* dx, hipStream_t s) {
  const int ncw = ceil_div(d, DWCOLS8), ncx = ceil_div(d, DXCOLS);
  const int ndw = (int)max_segments((long long)Tn * k, E) * ncw;
  auto grid = [&](int nt) { return dim3((unsigned)(ndw + ceil_div(Tn, nt) * ncx)); };
  switch (k) {
    case 1:
      hipLaunchKernelGGL((route_bwd8_kernel<T, 1>), grid(dx_tokens<T, 1>()), dim3(256), 0, s, dgate, gate, idx, src_row, offsets, x,
                         w, Tn, d, E, k, ndw, ncw, partial, dx);
      break;
    case 2:
      hipLaunchKernelGGL((route_bwd8_kernel<T, 2>), grid(dx_tokens<T, 2>()), dim3(256), 0, s, dgate, gate, idx, src_row, offsets, x,
                         w, Tn, d, E, k, ndw, ncw, partial, dx);
      break;
    case 3:
    case 4:
      hipLaunchKernelGGL((route_bwd8_kernel<T, 4>), grid(dx_tokens<T, 4>()), dim3(256), 0, s, dgate, gate, idx, src_row, offsets, x,
                         w, Tn, d, E, k, ndw, ncw, partial, dx);
      break;
    default:
      hipLaunchKernelGGL((route_bwd8_kernel<T, 8>), grid(dx_tokens<T, 8>()), dim3(256), 0, s, dgate, gate, idx, src_row, offsets, x,
                         w, Tn, d, E, k, ndw, ncw, partial, dx);
  }
}

hipError_t launch_route_bwd(const float* dgate, const float* gate, const int32_t* topk_idx,
                            const int32_t* offsets, const int32_t* src_row, const void* x,
                            const void* w, int T, int d, int E, int k, bool bf16, float* dw,
                            void* dx_router, void* ws, hipStream_t s) {
  const int Tk = T * k;
  float* partial = reinterpret_cast<float*>(ws);
  if (T > 0 && d % 8 == 0) {
    if (bf16)
      launch_route_bwd8<bf16_t>(dgate, gate, topk_idx, src_row, offsets, reinterpret_cast<const bf16_t*>(x),
                                reinterpret_cast<const bf16_t*>(w), T, d, E, k, partial,
                                reinterpret_cast<bf16_t*>(dx_router), s);
    else
      launch_route_bwd8<float>(dgate, gate, topk_idx, src_row, offsets, reinterpret_cast<const float*>(x),
                               reinterpret_cast<const float*>(w), T, d, E, k, partial,
                               reinterpret_cast<float*>(dx_router), s);
  } else if (T > 0) {
    const dim3 gdw((unsigned)max_segments(Tk, E), ceil_div(d, DWCOLS));
    if (bf16) {
      hipLaunchKernelGGL(route_dx_kernel<bf16_t>, dim3(T), dim3(256), 0, s, dgate, gate, topk_idx,
                         reinterpret_cast<const bf16_t*>(w), d, k, reinterpret_cast<bf16_t*>(dx_router));
      hipLaunchKernelGGL(route_dw_partial_kernel<bf16_t>, gdw, dim3(256), 0, s, dgate, gate, src_row, offsets,
                         reinterpret_cast<const bf16_t*>(x), E, Tk, d, k, partial);
    } else {
      hipLaunchKernelGGL(route_dx_kernel<float>, dim3(T), dim3(256), 0, s, dgate, gate, topk_idx,
                         reinterpret_cast<const float*>(w), d, k, reinterpret_cast<float*>(dx_router));
      hipLaunchKernelGGL(route_dw_partial_kernel<float>, gdw, dim3(256), 0, s, dgate, gate, src_row, offsets,
                         reinterpret_cast<const float*>(x), E, Tk, d, k, partial);
    }
  }
  if (d % 4 == 0)
    hipLaunchKernelGGL(route_dw_reduce4_kernel, dim3(E, ceil_div(d, 1024)), dim3(256), 0, s, partial, offsets, E, Tk,
                       d, (int)max_segments(Tk, E), dw);
  else
    hipLaunchKernelGGL(route_dw_reduce_kernel, dim3(E, ceil_div(d, DWCOLS)), dim3(256), 0, s, partial, offsets, E, Tk,
                       d, (int)max_segments(Tk, E), dw);
  return hipGetLastError();
}

}  // namespace moe
