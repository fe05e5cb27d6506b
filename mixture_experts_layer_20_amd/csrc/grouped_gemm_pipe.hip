// Pipelined grouped GEMM for gfx950: the six GEMM stages of the SwiGLU expert MLP (forward,
// dgrad, wgrad) over expert-ragged row groups, at the layer's large shapes.
//
// Tokens are moved to experts that stay resident ("Olmo-core 3 Opens Large MoE Training",
// "Technical Deep Dive"); each expert's rows form one ragged group of the grouped GEMM.
//
// Design (one workgroup = 256x256 output tile, 4 waves in a 2x2 grid, 128x128 per wave):
//  * K is consumed 32 at a time through a ring of four 32 KiB LDS stages that global loads fill
//    directly (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16*l).  Three stages are
//    in flight while one is multiplied; no registers are spent on staging.
//  * An operand that is K-contiguous in memory is kept [row][32 k] in LDS (64-byte rows, 16-byte
//    chunks XOR-swizzled) and read with ds_read_b128.  An operand that is K-strided (weights in
//    dgrad, activations in wgrad) is kept [32 k][256 rows] (512-byte rows, 64-byte windows
//    XOR-swizzled by k) and read with ds_read_b64_tr_b16, which hands each lane 4 consecutive k
//    of one column: two such reads form a 32x32x16 MFMA operand.  No transposition pass.
//  * v_mfma_f32_32x32x16_bf16, fp32 accumulators (256 per lane).
//  * LDS reads are inline assembly with explicit lgkmcnt waits; the ring is governed by explicit
//    vmcnt waits and a plain s_barrier.  (The compiler's own waits would drain every load in
//    flight before each LDS read, and a fenced barrier drains them too.)
//  * Epilogue: the accumulators go through LDS in fp32, are read back as rows of 8 consecutive
//    columns, get the mode's elementwise math (SwiGLU, SwiGLU backward) and are written with
//    16-byte stores.
//  * Persistent grid, per-expert tile prefix computed in-kernel, tiles dealt so each XCD walks one
//    contiguous run (workgroup b runs on XCD b % 8).
#include "common.h"
#include "gemm_common.h"

#include <algorithm>

namespace moe {
namespace {

using namespace gemm;

constexpr int BM = 256, BN = 256, BKS = 32, NSTAGE = 4, NTH = 256, WGM = 2, WGN = 2, MI = 4, NI = 4;
constexpr int OPB = 256 * BKS * 2;         // one operand tile of one stage: 16 KiB
constexpr int STAGE = 2 * OPB;             // 32 KiB
constexpr int LDS_BYTES = NSTAGE * STAGE;  // 128 KiB
constexpr int PMAXG = 1024;

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;
// Native vectors (HIP's uint2/uint4 are classes, which inline-assembly operands would force into
// memory).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Zero source for the direct loads of K rows past an expert's end (weight gradients).
__device__ __attribute__((aligned(16))) uint4 g_zero_rows[64];

__device__ __forceinline__ uint32_t lds_addr_of(const void* ptr) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)ptr);
}

// ---- K-contiguous operand: [256 rows][32 k], 64-byte rows; chunk swizzle (row >> 2) & 3 makes
// 16 consecutive rows read at one chunk hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kc_swz(int row) { return (row >> 2) & 3; }

// ---- K-strided operand: [32 k][256 columns], 512-byte rows; 64-byte window w of row k is stored
// at window w ^ (k & 3) (within its 256-byte half), so the 4 k-rows of one transposed read hit
// distinct bank groups.
__device__ __forceinline__ int mc_phys_chunk(int k, int chunk) { return chunk ^ ((k & 3) << 2); }

// Direct loads of one operand tile for the K step starting at k0 (4 instructions per wave).
// KC: slot q = (row q/4, physical chunk q%4).  MC: slot q = (k q/32, physical chunk q%32).
template <int MODE, bool A_OP>
__device__ __forceinline__ void issue_operand(const GemmArgs& p, char* dst, int g, int m0, int m_end, int nt,
                                              int k0, int k_end, int wave, int lane) {
  constexpr bool kc = A_OP ? Traits<MODE>::a_kcontig : Traits<MODE>::b_kcontig;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = (wave * 4 + j) * 64 + lane;
    const bf16_t* src;
    if constexpr (kc) {
      const int row = q >> 2;
      const int kk = k0 + (((q & 3) ^ kc_swz(row)) << 3);
      if constexpr (A_OP) {
        src = a_ptr_kc<MODE, bf16_t>(p, min(m0 + row, m_end - 1), kk);
      } else {
        src = b_ptr_kc<MODE, bf16_t, BN>(p, g, nt, row, kk);
      }
    } else {
      const int kr = q >> 5;
      const int col = ((q & 31) ^ ((kr & 3) << 2)) << 3;   // logical column of this physical chunk
      const int k = k0 + kr;
      if (k < k_end) {
        if constexpr (A_OP) src = a_ptr_mc<MODE, bf16_t>(p, k, m0 + col);
        else src = b_ptr_mc<MODE, bf16_t>(p, g, k, nt * BN + col);
      } else {
        src = reinterpret_cast<const bf16_t*>(g_zero_rows);
      }
    }
    __builtin_amdgcn_global_load_lds((gvoid_t*)src, (lvoid_t*)(dst + (wave * 4 + j) * 1024), 16, 0, 0);
  }
}

template <int MODE>
__device__ __forceinline__ void issue_stage(const GemmArgs& p, char* st, int g, int m0, int m_end, int nt, int k0,
                                            int k_end, int wave, int lane) {
  issue_operand<MODE, true>(p, st, g, m0, m_end, nt, k0, k_end, wave, lane);
  issue_operand<MODE, false>(p, st + OPB, g, m0, m_end, nt, k0, k_end, wave, lane);
}

// Row (A) / column (B) of the wave's MFMA block i inside the 256-wide operand tile.
template <int MODE, bool A_OP>
__device__ __forceinline__ int block_row(int wm, int wn, int i) {
  if constexpr (A_OP) {
    return wm * 128 + 32 * i;
  } else if constexpr (MODE == GEMM_UP_FWD) {
    // gate (W1) columns in blocks 0,1 and the same up (W3) columns in blocks 2,3
    return (i < 2) ? wn * 64 + 32 * i : 128 + wn * 64 + 32 * (i - 2);
  } else {
    return wn * 128 + 32 * i;
  }
}

// Per-lane LDS offset (within a stage, operand base included) of the first fragment read of each
// 16-deep substep; the other blocks follow from it:
//  KC: block i is a constant offset away (its rows are 32*i or, for the gate/up B tile, the listed
//      rows further; the swizzle repeats every 16 rows), applied as the instruction's offset field.
//  MC: block i is 32 columns = 4 chunks further; with the window swizzle that is an XOR of i into
//      address bits 6-7.  The second transposed read of a block is 4 k-rows = 2048 bytes further.
template <int MODE, bool A_OP>
__device__ __forceinline__ uint32_t frag_base(int s, int wm, int wn, int lane) {
  constexpr bool kc = A_OP ? Traits<MODE>::a_kcontig : Traits<MODE>::b_kcontig;
  const uint32_t base = A_OP ? 0 : OPB;
  const int rb = block_row<MODE, A_OP>(wm, wn, 0);
  if constexpr (kc) {
    const int row = rb + (lane & 31);
    const int chunk = s * 2 + (lane >> 5);
    return base + row * 64 + ((chunk ^ kc_swz(row)) << 4);
  } else {
    // 16-lane block b = lane/16 covers columns rb + 16*(b&1) + [0,16) and k-rows
    // s*16 + (b>>1)*8 + [0,8); lane j = 4c + q of the block points at k-row c, columns +4q..+4q+3.
    const int b = lane >> 4, j = lane & 15, c = j >> 2, q = j & 3;
    const int k = s * 16 + (b >> 1) * 8 + c;
    const int col = rb + 16 * (b & 1) + 4 * q;
    return base + k * 512 + (mc_phys_chunk(k, col >> 3) << 4) + (col & 7) * 2;
  }
}

// Offset of block i relative to block 0 (KC operands), in bytes.
template <int MODE, bool A_OP>
constexpr int kc_block_off(int i) {
  return A_OP ? 2048 * i
              : (MODE == GEMM_UP_FWD ? (i < 2 ? 2048 * i : 8192 + 2048 * (i - 2)) : 2048 * i);
}

#define MOE_DS_READ_B128(OUT, ADDR, OFF) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(OUT) : "v"(ADDR), "i"(OFF))
#define MOE_DS_READ_TR(OUT, ADDR, OFF) asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(OUT) : "v"(ADDR), "i"(OFF))

// Fragments of one 16-deep substep.  For MC operands the two 64-bit halves are kept apart until
// the wait, then packed (4 k from the first read, 4 from the second).
template <bool KC>
struct Frag;
template <>
struct Frag<true> {
  bf16x8_t v[4];
  template <int MODE, bool A_OP>
  __device__ __forceinline__ void read(uint32_t addr) {
    MOE_DS_READ_B128(v[0], addr, (kc_block_off<MODE, A_OP>(0)));
    MOE_DS_READ_B128(v[1], addr, (kc_block_off<MODE, A_OP>(1)));
    MOE_DS_READ_B128(v[2], addr, (kc_block_off<MODE, A_OP>(2)));
    MOE_DS_READ_B128(v[3], addr, (kc_block_off<MODE, A_OP>(3)));
  }
  __device__ __forceinline__ bf16x8_t get(int i) const { return v[i]; }
};
template <>
struct Frag<false> {
  u32x2_t h[2][4];
  template <int MODE, bool A_OP>
  __device__ __forceinline__ void read(uint32_t addr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ai = addr ^ (uint32_t)(i << 6);
      MOE_DS_READ_TR(h[0][i], ai, 0);
      MOE_DS_READ_TR(h[1][i], ai, 2048);
    }
  }
  __device__ __forceinline__ bf16x8_t get(int i) const {
    const u32x4_t u = {h[0][i].x, h[0][i].y, h[1][i].x, h[1][i].y};
    return __builtin_bit_cast(bf16x8_t, u);
  }
};
#undef MOE_DS_READ_B128
#undef MOE_DS_READ_TR

// Wait until at most N LDS reads are outstanding (the reads issued after fa/fb); fa and fb are
// in-out operands so no use of them can be scheduled before the wait.  lgkmcnt is 4 bits wide:
// N is clamped to 15, which is conservative (it also waits for the oldest of the newer reads).
#define MOE_LGKM_ASM(NSTR, ...) asm volatile("s_waitcnt lgkmcnt(" NSTR ")" : __VA_ARGS__)
#define MOE_LGKM_SWITCH(N, ...)                       \
  do {                                                 \
    if constexpr ((N) == 0) MOE_LGKM_ASM("0", __VA_ARGS__);   \
    else if constexpr ((N) == 8) MOE_LGKM_ASM("8", __VA_ARGS__); \
    else if constexpr ((N) == 12) MOE_LGKM_ASM("12", __VA_ARGS__); \
    else MOE_LGKM_ASM("15", __VA_ARGS__);              \
  } while (0)

template <int N>
__device__ __forceinline__ void frag_wait(Frag<true>& a, Frag<true>& b) {
  MOE_LGKM_SWITCH(N, "+v"(a.v[0]), "+v"(a.v[1]), "+v"(a.v[2]), "+v"(a.v[3]), "+v"(b.v[0]), "+v"(b.v[1]),
                  "+v"(b.v[2]), "+v"(b.v[3]));
}
template <int N>
__device__ __forceinline__ void frag_wait(Frag<true>& a, Frag<false>& b) {
  MOE_LGKM_SWITCH(N, "+v"(a.v[0]), "+v"(a.v[1]), "+v"(a.v[2]), "+v"(a.v[3]), "+v"(b.h[0][0]), "+v"(b.h[0][1]),
                  "+v"(b.h[0][2]), "+v"(b.h[0][3]), "+v"(b.h[1][0]), "+v"(b.h[1][1]), "+v"(b.h[1][2]),
                  "+v"(b.h[1][3]));
}
template <int N>
__device__ __forceinline__ void frag_wait(Frag<false>& a, Frag<false>& b) {
  MOE_LGKM_SWITCH(N, "+v"(a.h[0][0]), "+v"(a.h[0][1]), "+v"(a.h[0][2]), "+v"(a.h[0][3]), "+v"(a.h[1][0]),
                  "+v"(a.h[1][1]), "+v"(a.h[1][2]), "+v"(a.h[1][3]), "+v"(b.h[0][0]), "+v"(b.h[0][1]),
                  "+v"(b.h[0][2]), "+v"(b.h[0][3]), "+v"(b.h[1][0]), "+v"(b.h[1][1]), "+v"(b.h[1][2]),
                  "+v"(b.h[1][3]));
}
#undef MOE_LGKM_SWITCH
#undef MOE_LGKM_ASM

// Number of LDS read instructions of one substep's fragments, and the wait count that lets one
// substep's worth of newer reads stay in flight.
template <bool KC> constexpr int nreads() { return KC ? 4 : 8; }
template <bool KA, bool KB> constexpr int newer_reads() {
  return nreads<KA>() + nreads<KB>() > 15 ? 15 : nreads<KA>() + nreads<KB>();
}

// s_waitcnt vmcnt(N) lgkmcnt(0), N a multiple of 8 below 64.
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 16) __builtin_amdgcn_s_waitcnt(0x4070);   // vmcnt 16 = low bits 0, high bits 1
  else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0070 | 8);
  else __builtin_amdgcn_s_waitcnt(0x0070);
}

template <int MODE>
__device__ __forceinline__ void mma_substep(const Frag<Traits<MODE>::a_kcontig>& fa,
                                            const Frag<Traits<MODE>::b_kcontig>& fb, f32x16_t (&acc)[MI][NI]) {
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const bf16x8_t a = fa.get(i);
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, fb.get(j), acc[i][j], 0, 0, 0);
  }
}

// ---- Epilogue ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_sigmoid(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// Four fp32 values to packed bf16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ u32x2_t pack4_bf16(const float (&x)[4]) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t lo = {x[0], x[1]}, hi = {x[2], x[3]};
  u32x2_t w;
  w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, b16x2_t));
  w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, b16x2_t));
  return w;
}
__device__ __forceinline__ void st8(void* base, size_t elem, const float (&x)[4]) {
  *reinterpret_cast<u32x2_t*>(reinterpret_cast<bf16_t*>(base) + elem) = pack4_bf16(x);
}

// Store 4 consecutive outputs (row m, columns n..n+3) of the mode; u holds the up-projection values
// of the gate/up GEMM.
template <int MODE>
__device__ __forceinline__ void store4(const GemmArgs& p, int g, int m, int n, const float (&v)[4], const float (&u)[4],
                                       int split, int ksplit, float* partial) {
  if constexpr (MODE == GEMM_UP_FWD) {
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = v[i] * fast_sigmoid(v[i]) * u[i];
    const size_t idx = (size_t)m * p.f + n;
    if (p.out0) st8(p.out0, idx, v);
    if (p.out1) st8(p.out1, idx, u);
    st8(p.out2, idx, h);
  } else if constexpr (MODE == GEMM_DOWN_FWD || MODE == GEMM_UP_DGRAD) {
    st8(p.out0, (size_t)m * p.d + n, v);
  } else if constexpr (MODE == GEMM_DOWN_BWD) {
    const size_t idx = (size_t)m * p.f + n;
    const u32x2_t au = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const bf16_t*>(p.aux0) + idx);
    const u32x2_t bu = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const bf16_t*>(p.aux1) + idx);
    const uint32_t aw[2] = {au.x, au.y}, bw[2] = {bu.x, bu.y};
    float da[4], db[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __uint_as_float(i & 1 ? (aw[i >> 1] & 0xffff0000u) : (aw[i >> 1] << 16));
      const float b = __uint_as_float(i & 1 ? (bw[i >> 1] & 0xffff0000u) : (bw[i >> 1] << 16));
      const float s = fast_sigmoid(a);
      da[i] = v[i] * b * s * (1.0f + a * (1.0f - s));
      db[i] = v[i] * a * s;
    }
    const size_t row = (size_t)m * (2 * p.f);
    st8(p.out0, row + n, da);
    st8(p.out0, row + p.f + n, db);
  } else {  // weight gradients: m is the gradient row, n its column
    const int Mw = mode_Mw(MODE, p.d, p.f), Nw = mode_N(MODE, p.d, p.f);
    if (ksplit > 1) {
      float* dst = partial + (((size_t)split * p.G + g) * Mw + m) * Nw + n;
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (MODE == GEMM_DOWN_WGRAD) {
      st8(p.out0, ((size_t)g * p.d + m) * p.f + n, v);
    } else {
      void* out = m < p.f ? p.out0 : p.out1;
      const int mm = m < p.f ? m : m - p.f;
      st8(out, ((size_t)g * p.f + mm) * p.d + n, v);
    }
  }
}

// 4x4 transpose inside each quad of lanes (DPP quad permutes): on entry lane j of a quad holds
// x[e] = M[j][e]; on exit it holds x[e] = M[e][j].
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ void quad_transpose(float (&x)[4], int lane) {
  const bool hi = lane & 2, odd = lane & 1;
  const float u0 = dpp_xor2(x[0]), u1 = dpp_xor2(x[1]), u2 = dpp_xor2(x[2]), u3 = dpp_xor2(x[3]);
  const float n0 = hi ? u2 : x[0], n1 = hi ? u3 : x[1], n2 = hi ? x[2] : u0, n3 = hi ? x[3] : u1;
  const float w0 = dpp_xor1(n0), w1 = dpp_xor1(n1), w2 = dpp_xor1(n2), w3 = dpp_xor1(n3);
  x[0] = odd ? w1 : n0;
  x[1] = odd ? n1 : w0;
  x[2] = odd ? w3 : n2;
  x[3] = odd ? n3 : w2;
}

// Copies of four accumulator registers to VGPRs.  Written out so that each value leaves its AGPR
// only where it is used: left to itself the compiler moves the whole accumulator set to VGPRs at
// the end of the K loop and spills.  The hazard checker does not look into inline asm, so the
// two wait states a DPP read of a freshly written VGPR needs are added here.
#define MOE_AGPR_READ4(C, E0, X)                                                                  \
  asm volatile(                                                                                   \
      "v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\tv_accvgpr_read_b32 %2, %6\n\t"     \
      "v_accvgpr_read_b32 %3, %7\n\ts_nop 1"                                                       \
      : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3])                                            \
      : "a"(C[(E0)]), "a"(C[(E0) + 1]), "a"(C[(E0) + 2]), "a"(C[(E0) + 3]))

// Epilogue straight from the accumulators.  In the 32x32 accumulator layout lane l holds column
// l % 32 and, for element v, row 8*(v/4) + 4*(l/32) + v%4; after the quad transpose of elements
// 4g..4g+3 lane l holds row 8g + 4*(l/32) + l%4 and columns 4*((l%32)/4) .. +3.
template <int MODE>
__device__ __forceinline__ void epilogue_block(const GemmArgs& p, const f32x16_t& c, const f32x16_t& cu, int g,
                                               int row, int m_end, int n, int lane, int split, int ksplit,
                                               float* partial) {
#pragma unroll
  for (int vg = 0; vg < 4; ++vg) {
    const int m = row + 8 * vg;
    float v[4], u[4];
    MOE_AGPR_READ4(c, 4 * vg, v);
    quad_transpose(v, lane);
    if constexpr (MODE == GEMM_UP_FWD) {
      MOE_AGPR_READ4(cu, 4 * vg, u);
      quad_transpose(u, lane);
    }
    if (m < m_end) store4<MODE>(p, g, m, n, v, u, split, ksplit, partial);
  }
}

// Blocks IDX.. of the wave's accumulators, unrolled at compile time (the loop unroller gives up on
// the larger epilogues, and a run-time block index would put the accumulators in scratch memory).
template <int MODE, int IDX>
__device__ __forceinline__ void epilogue_from(const GemmArgs& p, const f32x16_t (&acc)[MI][NI], int g, int row0,
                                              int m_end, int col0, int lane, int split, int ksplit, float* partial) {
  constexpr int NJ = (MODE == GEMM_UP_FWD) ? NI / 2 : NI;
  if constexpr (IDX < MI * NJ) {
    constexpr int mi = IDX / NJ, ni = IDX % NJ;
    constexpr int nu = (MODE == GEMM_UP_FWD) ? ni + NI / 2 : ni;
    epilogue_block<MODE>(p, acc[mi][ni], acc[mi][nu], g, row0 + mi * 32 + 4 * (lane >> 5) + (lane & 3), m_end,
                         col0 + ni * 32 + 4 * ((lane & 31) >> 2), lane, split, ksplit, partial);
    epilogue_from<MODE, IDX + 1>(p, acc, g, row0, m_end, col0, lane, split, ksplit, partial);
  }
}

template <int MODE>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& p, const f32x16_t (&acc)[MI][NI], int g, int row0,
                                              int m_end, int col0, int lane, int split, int ksplit, float* partial) {
  // The accumulator reads are opaque to the hazard checker: leave the last MFMA's write-back
  // (at most 18 wait states) behind before the first of them.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  epilogue_from<MODE, 0>(p, acc, g, row0, m_end, col0, lane, split, ksplit, partial);
}

// Per-group tile prefix (ragged-M modes): pref[g] = 256-row tiles of the groups before g.
__device__ __forceinline__ void tile_prefix_lds(const GemmArgs& p, int* pref, int* scratch) {
  const int tid = threadIdx.x;
  if (tid == 0) scratch[NTH] = 0;
  __syncthreads();
  for (int base = 0; base < p.G; base += NTH) {
    const int g = base + tid;
    int c = 0;
    if (g < p.G) {
      int lo, hi;
      group_rows(p.offsets, g, p.M, lo, hi);
      c = (hi - lo + BM - 1) / BM;
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

template <int MODE>
__global__ __launch_bounds__(NTH, 1) void grouped_gemm_pipe(GemmArgs p, int NT, int MT, int ksplit, float* partial) {
  typedef Traits<MODE> TR;
  constexpr bool AKC = TR::a_kcontig, BKC = TR::b_kcontig;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  __shared__ int pref[PMAXG + 1];
  __shared__ int scan_scratch[NTH + 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave % WGM, wn = wave / WGM;
  const uint32_t lds0 = lds_addr_of(lds);

  const uint32_t fa0 = lds0 + frag_base<MODE, true>(0, wm, wn, lane), fa1 = lds0 + frag_base<MODE, true>(1, wm, wn, lane);
  const uint32_t fb0 = lds0 + frag_base<MODE, false>(0, wm, wn, lane), fb1 = lds0 + frag_base<MODE, false>(1, wm, wn, lane);

  int total;
  if constexpr (!TR::raggedK) {
    tile_prefix_lds(p, pref, scan_scratch);
    total = pref[p.G] * NT;
  } else {
    total = p.G * ksplit * MT * NT;
  }
  const int per = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int nbx = gridDim.x >> 3;
  const int L_end = min(total, (xcd + 1) * per);

  // Tile decode: group, row range and K range of logical tile L.
  struct Tile {
    int g, m0, m_end, nt, k_begin, k_end, split, nk;
  };
  auto decode = [&](int L) {
    Tile t;
    t.split = 0;
    if constexpr (!TR::raggedK) {
      const int mt = L / NT;
      t.nt = L - mt * NT;
      int lo = 0, hi = p.G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] <= mt) lo = mid; else hi = mid;
      }
      t.g = lo;
      int r0, r1;
      group_rows(p.offsets, t.g, p.M, r0, r1);
      t.m0 = r0 + (mt - pref[t.g]) * BM;
      t.m_end = r1;
      t.k_begin = 0;
      t.k_end = mode_K(MODE, p.d, p.f);
    } else {
      t.nt = L % NT;
      int r = L / NT;
      const int mt = r % MT;
      r /= MT;
      t.split = r % ksplit;
      t.g = r / ksplit;
      t.m0 = mt * BM;
      t.m_end = t.m0 + BM;
      int r0, r1;
      group_rows(p.offsets, t.g, p.M, r0, r1);
      const int chunk = ((r1 - r0 + ksplit - 1) / ksplit + BKS - 1) / BKS * BKS;
      t.k_begin = min(r1, r0 + t.split * chunk);
      t.k_end = min(r1, t.k_begin + chunk);
    }
    t.nk = (t.k_end - t.k_begin + BKS - 1) / BKS;
    return t;
  };
  // First three K stages of a tile into ring slots 0..2.
  auto prefetch = [&](const Tile& t) {
    for (int s = 0; s < 3 && s < t.nk; ++s)
      issue_stage<MODE>(p, lds + s * STAGE, t.g, t.m0, t.m_end, t.nt, t.k_begin + s * BKS, t.k_end, wave, lane);
  };

  int L = xcd * per + (blockIdx.x >> 3);
  Tile cur;
  if (L < L_end) {
    cur = decode(L);
    prefetch(cur);
  }
  for (; L < L_end; L += nbx) {
    const int g = cur.g, m0 = cur.m0, m_end = cur.m_end, nt = cur.nt, k_begin = cur.k_begin, k_end = cur.k_end;
    const int nk = cur.nk, split = cur.split;

    f32x16_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    if (nk > 0) {
      // Everything older than stage 0's loads (the previous tile's stores) is also waited for;
      // stages 1 and 2 stay in flight.
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): stores of the previous tile may be younger
      asm volatile("s_barrier" ::: "memory");
      Frag<AKC> a0, a1;
      Frag<BKC> b0, b1;
      a0.template read<MODE, true>(fa0);
      b0.template read<MODE, false>(fb0);
      for (int kt = 0; kt < nk; ++kt) {
        const uint32_t sb = (kt & 3) * STAGE;
        a1.template read<MODE, true>(fa1 + sb);
        b1.template read<MODE, false>(fb1 + sb);
        frag_wait<newer_reads<AKC, BKC>()>(a0, b0);
        mma_substep<MODE>(a0, b0, acc);
        if (kt + 1 < nk) {
          wait_vm(kt + 2 < nk ? 8 : 0);
          asm volatile("s_barrier" ::: "memory");
          if (kt + 3 < nk)
            issue_stage<MODE>(p, lds + ((kt + 3) & 3) * STAGE, g, m0, m_end, nt, k_begin + (kt + 3) * BKS, k_end,
                              wave, lane);
          const uint32_t sn = ((kt + 1) & 3) * STAGE;
          a0.template read<MODE, true>(fa0 + sn);
          b0.template read<MODE, false>(fb0 + sn);
          frag_wait<newer_reads<AKC, BKC>()>(a1, b1);
        } else {
          frag_wait<0>(a1, b1);
        }
        mma_substep<MODE>(a1, b1, acc);
      }
    }
    // The ring is free once every wave has finished its reads: start the next tile's loads now so
    // they overlap this tile's epilogue.
    asm volatile("s_barrier" ::: "memory");
    if (L + nbx < L_end) {
      cur = decode(L + nbx);
      prefetch(cur);
    }

    const int row0 = m0 + wm * 128;
    const int col0 = (MODE == GEMM_UP_FWD) ? nt * (BN / 2) + wn * 64 : nt * BN + wn * 128;
    epilogue_tile<MODE>(p, acc, g, row0, m_end, col0, lane, split, ksplit, partial);
  }
}

template <int MODE>
hipError_t launch_pipe(const GemmArgs& p, int ksplit, float* partial, hipStream_t s, int num_cus) {
  typedef Traits<MODE> TR;
  const int NT = mode_N(MODE, p.d, p.f) / BN;
  int MT = 0;
  long long tiles;
  if constexpr (!TR::raggedK) {
    if (p.M == 0) return hipSuccess;
    tiles = ((long long)ceil_div(p.M, BM) + p.G) * NT;
  } else {
    MT = mode_Mw(MODE, p.d, p.f) / BM;
    tiles = (long long)p.G * MT * NT * ksplit;
  }
  long long grid = std::min<long long>(tiles, (long long)num_cus);
  grid = (grid + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_pipe<MODE>, dim3((unsigned)grid), dim3(NTH), 0, s, p, NT, MT, ksplit, partial);
  return hipGetLastError();
}

}  // namespace

bool pipe_supports(int mode, const GemmArgs& p) {
  if (p.G > PMAXG) return false;
  const int N = gemm::mode_N(mode, p.d, p.f);
  if (N % BN) return false;
  if (mode == GEMM_DOWN_WGRAD || mode == GEMM_UP_WGRAD) return gemm::mode_Mw(mode, p.d, p.f) % BM == 0;
  return gemm::mode_K(mode, p.d, p.f) % BKS == 0;
}

hipError_t launch_grouped_gemm_pipe(int mode, const GemmArgs& p, int ksplit, float* partial, hipStream_t s,
                                    int num_cus) {
  switch (mode) {
    case GEMM_UP_FWD: return launch_pipe<GEMM_UP_FWD>(p, 1, nullptr, s, num_cus);
    case GEMM_DOWN_FWD: return launch_pipe<GEMM_DOWN_FWD>(p, 1, nullptr, s, num_cus);
    case GEMM_DOWN_BWD: return launch_pipe<GEMM_DOWN_BWD>(p, 1, nullptr, s, num_cus);
    case GEMM_UP_DGRAD: return launch_pipe<GEMM_UP_DGRAD>(p, 1, nullptr, s, num_cus);
    case GEMM_DOWN_WGRAD: return launch_pipe<GEMM_DOWN_WGRAD>(p, ksplit, partial, s, num_cus);
    case GEMM_UP_WGRAD: return launch_pipe<GEMM_UP_WGRAD>(p, ksplit, partial, s, num_cus);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
