// Pipelined grouped GEMM for gfx950: the six GEMM stages of the SwiGLU expert MLP (forward,
// dgrad, wgrad) over expert-ragged row groups, at the layer's large shapes.
//
// Tokens are moved to experts that stay resident ("Olmo-core 3 Opens Large MoE Training",
// "Technical Deep Dive"); each expert's rows form one ragged group of the grouped GEMM.
//
// Design (one workgroup = 256x256 output tile, 8 waves in a 2x4 grid, 128x64 per wave; a group of
// 257..320 rows in the forward and data-gradient products takes one 320x256 tile, 160x64 per wave):
//  * K is consumed 64 at a time ("K step") through two 64 KiB LDS stages that global loads fill
//    directly (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16*l).  The loads form one
//    continuous stream over all tiles of the workgroup: a stage is refilled with the stage two steps
//    ahead as soon as every wave has read it, also across tile boundaries, so the next tile's first
//    stages are in flight during the current tile's epilogue.
//  * The vector memory path of a CU keeps a limited number of cache-line requests in flight, so the
//    operand stream runs at (lines in flight x bytes per request) / latency.  A K-contiguous operand
//    row of a 64-deep stage is 128 bytes, one whole line per request (a 32-deep stage requested half
//    lines and streamed at half the rate).  Such an operand is kept [row][64 k] in LDS (128-byte
//    rows, 16-byte chunks XOR-swizzled) and read with ds_read_b128.  An operand that is K-strided
//    (weights in dgrad, activations in wgrad) is kept [64 k][256 rows] (512-byte rows, 64-byte
//    windows XOR-swizzled by k) and read with ds_read_b64_tr_b16, which hands each lane 4 consecutive
//    k of one column: two such reads form a 32x32x16 MFMA operand.  No transposition pass.
//  * v_mfma_f32_32x32x16_bf16, fp32 accumulators (128 per lane, 160 in a 320-row tile).
//  * Two waves per SIMD (one per row half), so one can feed the matrix core while the other waits
//    on a load issue, a fragment read or the barrier.  A K step is four phases of 8 MFMAs (one per
//    16-deep substep); every LDS fragment read and every global load is placed between two MFMAs
//    (scheduling barriers pin the order).  One s_barrier per K step, before the last phase, which
//    issues the stage loads.  LDS reads are inline assembly with explicit lgkmcnt waits and the ring
//    is governed by explicit vmcnt waits (the compiler's own waits would drain every load in flight
//    before each LDS access).
//  * Epilogue straight from the accumulators: a v_permlane32_swap gives each lane 8 consecutive
//    columns of one row, the mode's elementwise math (SwiGLU, SwiGLU backward, whose A/B stash is
//    loaded in the same layout a block ahead) is applied and 16-byte bf16 stores go out, as whole
//    128-byte rows where the mode has one output.  Weight gradients are stored nontemporally, and
//    three quarters of a weight-gradient tile's stores are issued during the next tile's first K
//    step, between its MFMAs.
//  * Persistent grid, per-expert tile prefix computed in-kernel, tiles dealt so each XCD walks one
//    contiguous run of each expert set (workgroup b runs on XCD b % 8); an XCD's last round of
//    tiles, when it would keep at most half of its workgroups busy, is dealt as 128-row half tiles,
//    whose second row half of waves issues its loads but no MFMAs.
#include "common.h"
#include "gemm_common.h"

#include <algorithm>

namespace moe {
namespace {

using namespace gemm;

constexpr int BM = 256, BN = 256, BKS = 64, NSTAGE = 2;
constexpr int NW = 8, NTH = 64 * NW;  // two waves per SIMD
constexpr int WGN = 4;                // wave w: row half wm = w / WGN, column quarter wn = w % WGN
constexpr int MI = 4, NI = 2;         // 32x32 blocks per wave: 128 rows x 64 columns
constexpr int MIX = 5, BMX = 320;     // a tile of 257..BMX rows (modes with row capacity BMX): 160 x 64
constexpr int LPB = 4;                // direct loads (1 KiB each) per wave per stage of operand B
constexpr int OPB = 256 * BKS * 2;    // operand B tile of one stage: 32 KiB

// Modes whose tiles hold up to BMX rows (operand A K-contiguous): an expert of 257..320 rows is one
// tile rather than a full tile and a remainder tile that streams the same weights again.  The
// weight gradients hold up to BM rows.
template <int MODE>
constexpr bool has_x() { return MODE == GEMM_UP_FWD || MODE == GEMM_DOWN_FWD || MODE == GEMM_UP_DGRAD || MODE == GEMM_DOWN_BWD; }
template <int MODE>
constexpr int rows_a() { return has_x<MODE>() ? BMX : BM; }          // operand A rows per stage
template <int MODE>
constexpr int opa() { return rows_a<MODE>() * BKS * 2; }             // operand A bytes per stage
template <int MODE>
constexpr int lpa() { return opa<MODE>() / 1024 / NW; }              // its direct loads per wave
template <int MODE>
constexpr int lpw() { return lpa<MODE>() + LPB; }                    // direct loads per wave per stage
template <int MODE>
constexpr int stage_bytes() { return opa<MODE>() + OPB; }
template <int MODE>
constexpr int mi_max() { return has_x<MODE>() ? MIX : MI; }
// Operand A loads per wave that a tile of at most BM rows needs; the others (rows BM..BMX-1 of a
// BMX-row stage) are issued only for tiles of more than BM rows.
constexpr int LPA_BM = BM * BKS * 2 / 1024 / NW;
template <int MODE>
constexpr int lpa_skip() { return lpa<MODE>() - LPA_BM; }
// 1 KiB slot of a stage's operand tile that load j of a wave fills.  K-contiguous operand A is
// slot-major over the waves (load j of wave w: slot j * NW + w), so loads j >= LPA_BM are exactly
// the rows past BM; every other operand is wave-major (slot w * lp + j), which keeps the loads of
// one wave LP consecutive slots apart by a fixed step.
template <int MODE, bool A_OP>
__device__ __forceinline__ int load_slot(int wave, int j) {
  if constexpr (A_OP && Traits<MODE>::a_kcontig) return j * NW + wave;
  else return wave * (A_OP ? lpa<MODE>() : LPB) + j;
}
constexpr int PMAXG = 1024;   // groups of the first set
constexpr int PMAXG1 = 64;    // groups of the second set (the shared expert: 1)
constexpr int WG_NB = 4;      // tile columns per block of the weight-gradient tile order

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

// One 32-bit LDS load, waited for.  Written out because a compiler-generated LDS access would be
// preceded by a wait for every direct-to-LDS load in flight.
__device__ __forceinline__ int lds_load_i32(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// ---- K-contiguous operand: [256 rows][64 k], 128-byte rows (each 128-byte row segment is one
// whole cache line of the source, loaded by 8 lanes of one instruction); chunk swizzle
// (row >> 1) & 7 makes 16 consecutive rows read at one chunk hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kc_swz(int row) { return (row >> 1) & 7; }

// ---- K-strided operand: [64 k][256 columns], 512-byte rows; 64-byte window w of row k is stored
// at window w ^ (k & 3) (within its 256-byte half), so the 4 k-rows of one transposed read hit
// distinct bank groups.
__device__ __forceinline__ int mc_phys_chunk(int k, int chunk) { return chunk ^ ((k & 3) << 2); }

// ---- Tiles -------------------------------------------------------------------------------
// Output tile: set seg, group g, rows [m0, m_end), tile column nt, K range [k_begin, k_end) in nk
// steps of 64 (split: K chunk index of a split weight gradient; ks: the split count).  half: at
// most 128 rows (ragged M only), multiplied as a 128x256 tile.  x: more than 256 rows (at most
// BMX), multiplied as a 320x256 tile, 160 rows per wave.
struct Tile {
  int seg, g, m0, m_end, nt, k_begin, k_end, nk, split, ks;
  bool half, x;
};

// The arguments of one set of groups (set 1: the second set of a merged launch), in the layout
// the addressing helpers read.
__device__ __forceinline__ GemmArgs seg_args(const GemmArgs& p, int seg) {
  GemmArgs q = p;
  const bool s1 = seg != 0;
  q.a = s1 ? p.s1.a : p.a;
  q.b0 = s1 ? p.s1.b0 : p.b0;
  q.b1 = s1 ? p.s1.b1 : p.b1;
  q.aux0 = s1 ? p.s1.aux0 : p.aux0;
  q.aux1 = s1 ? p.s1.aux1 : p.aux1;
  q.out0 = s1 ? p.s1.out0 : p.out0;
  q.out1 = s1 ? p.s1.out1 : p.out1;
  q.out2 = s1 ? p.s1.out2 : p.out2;
  q.offsets = s1 ? p.s1.offsets : p.offsets;
  q.G = s1 ? p.s1.G : p.G;
  q.M = s1 ? p.s1.M : p.M;
  q.f = s1 ? p.s1.f : p.f;
  return q;
}

// Division of non-negative 31-bit integers by a divisor fixed for the whole launch, as a multiply
// and a shift (the round-up method of Granlund and Montgomery, "Division by invariant integers
// using multiplication", 1994): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (mulhi(m, n) + n) >> l.  The tile decode runs once or twice per tile in every wave, and a
// weight-gradient tile is only a few K steps long.
struct FastDiv {
  uint32_t m, l;
};
__device__ __forceinline__ FastDiv make_fastdiv(uint32_t d) {   // d >= 1
  const uint32_t l = d > 1 ? 32u - (uint32_t)__clz((int)(d - 1)) : 0u;
  const uint64_t m = ((((uint64_t)1 << l) - d) << 32) / d + 1;
  return FastDiv{(uint32_t)m, l};
}
__device__ __forceinline__ int fdiv(int n, uint32_t m, uint32_t l) {
  return (int)(((uint64_t)__umulhi((uint32_t)n, m) + (uint32_t)n) >> l);
}

// Tile geometry of one set: tile columns, weight-gradient row tiles, split, tiles, the row-tile
// band of the tile order, the LDS tables (clamped group offsets, per-group tile prefix) and, for
// the weight-gradient decode, divisions by MT * NT, MT * WG_NB, NT and the split.
struct SegGeo {
  int NT, MT, ks, total, band;
  bool rows256;   // the set's groups take 256-row tiles (and a remainder) even where 320-row ones fit
  uint32_t offs, pref;
  FastDiv fd_mn, fd_mb, fd_nt, fd_ks;
};

// The tiles of one XCD: n list positions; position i < n1 is tile total0 + lo1 + i (set 1), the
// others are lo0 + (i - n1) (set 0 numbering, which set 1 continues).  Positions from q on are
// half tiles (ragged M only): q + 2h + s is row half s of tile position q + h.  When the XCD's
// last round of tiles would keep at most half of its workgroups busy, those tiles are dealt as
// halves, so every workgroup ends with at most one half tile instead of some running a whole
// extra tile while the others wait.
struct Deal {
  int n, n1, lo0, lo1, total0, q;
};
__device__ __forceinline__ int tile_at(const Deal& dl, int i) {
  return i < dl.n1 ? dl.total0 + dl.lo1 + i : dl.lo0 + (i - dl.n1);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// A pointer that is the same in every lane, kept in scalar registers (the compiler cannot always
// tell, and then addresses it per lane or loops over the lanes for a buffer resource).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (T*)(uintptr_t)((hi << 32) | lo);
}

// Group row range from the clamped offsets kept in LDS (the clamping of group_rows).
__device__ __forceinline__ void group_rows_lds(uint32_t offs, int g, int& lo, int& hi) {
  lo = uniform(lds_load_i32(offs + 4 * g));
  hi = max(lo, uniform(lds_load_i32(offs + 4 * (g + 1))));
}

// Rows per tile of a group of R rows (ragged M) and the group's tiles: ceil(R / BMX) tiles of
// equal height where the mode has row capacity BMX (so no tile is a short remainder that streams
// the weights again), else 256-row tiles and a remainder.  The SwiGLU-backward product (down_bwd)
// takes a BMX-row tile only for a group that it holds whole: its 320-row tile spills registers at
// tile boundaries, which costs more than a remainder tile once a group has two or more tiles.
template <int MODE>
__device__ __forceinline__ int group_tiles(int R, bool rows256 = false) {
  if constexpr (MODE == GEMM_DOWN_BWD) return R <= BMX ? (R > 0) : (R + BM - 1) / BM;
  return has_x<MODE>() && !rows256 ? (R + BMX - 1) / BMX : (R + BM - 1) / BM;
}
template <int MODE>
__device__ __forceinline__ int tile_rows(int R, bool rows256 = false) {
  if constexpr (!has_x<MODE>()) return BM;
  if constexpr (MODE == GEMM_DOWN_BWD) return R <= BMX ? BMX : BM;
  if (rows256) return BM;
  const int n = max(1, group_tiles<MODE>(R));
  return (R + n - 1) / n;
}

template <int MODE>
__device__ __forceinline__ Tile decode_tile(const GemmArgs& p0, const SegGeo (&geo)[2], int L) {
  Tile t;
  t.seg = L >= geo[0].total;
  if (t.seg) L -= geo[0].total;
  const GemmArgs p = seg_args(p0, t.seg);
  const int NT = t.seg ? geo[1].NT : geo[0].NT, MT = t.seg ? geo[1].MT : geo[0].MT;
  const int ksplit = t.seg ? geo[1].ks : geo[0].ks;
  t.ks = ksplit;
  const uint32_t pref = t.seg ? geo[1].pref : geo[0].pref, offs = t.seg ? geo[1].offs : geo[0].offs;
  t.split = 0;
  t.half = false;
  t.x = false;
  if constexpr (!Traits<MODE>::raggedK) {
    // Tile order: group by group; inside a group, bands of `band` (4) row tiles, and inside a band
    // column by column.  An XCD's round of 32 tiles then covers 4 row tiles by 8 column tiles of a
    // large group (the shared expert), which reads the fewest distinct operand panels per round
    // (4 + 8); the row tiles that read one weight tile run together.
    int lo = 0, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (uniform(lds_load_i32(pref + 4 * mid)) * NT <= L) lo = mid; else hi = mid;
    }
    t.g = lo;
    const int p0 = uniform(lds_load_i32(pref + 4 * t.g)), p1 = uniform(lds_load_i32(pref + 4 * (t.g + 1)));
    const int MB = t.seg ? geo[1].band : geo[0].band;
    const int l = L - p0 * NT;
    const int b = l / (MB * NT);
    const int mb = min(MB, p1 - p0 - b * MB);
    const int r = l - b * MB * NT;
    t.nt = r / mb;
    const int mt = b * MB + (r - t.nt * mb);
    int r0, r1;
    group_rows_lds(offs, t.g, r0, r1);
    const int rpt = tile_rows<MODE>(r1 - r0, t.seg ? geo[1].rows256 : geo[0].rows256);
    t.m0 = r0 + mt * rpt;
    t.m_end = min(r1, t.m0 + rpt);
    t.half = t.m_end - t.m0 <= BM / 2;
    t.x = t.m_end - t.m0 > BM;
    t.k_begin = 0;
    t.k_end = mode_K(MODE, p.d, p.f);
  } else {
    const SegGeo& g0 = geo[0];
    const SegGeo& g1 = geo[1];
    const uint32_t mn_m = t.seg ? g1.fd_mn.m : g0.fd_mn.m, mn_l = t.seg ? g1.fd_mn.l : g0.fd_mn.l;
    const uint32_t ks_m = t.seg ? g1.fd_ks.m : g0.fd_ks.m, ks_l = t.seg ? g1.fd_ks.l : g0.fd_ks.l;
    const int r = fdiv(L, mn_m, mn_l);
    const int idx = L - r * (MT * NT);
    // Inside one (group, split): blocks of WG_NB tile columns, walked row tile by row tile, so an
    // XCD's round of workgroups covers a compact block of the expert's gradient and the next round
    // reuses its column operand (wide gradients: 16 tile columns at d = 4096).
    int mt;
    if (NT > WG_NB && NT % WG_NB == 0) {
      const int jb = fdiv(idx, t.seg ? g1.fd_mb.m : g0.fd_mb.m, t.seg ? g1.fd_mb.l : g0.fd_mb.l);
      const int rem = idx - jb * (MT * WG_NB);
      mt = rem / WG_NB;
      t.nt = jb * WG_NB + (rem - mt * WG_NB);
    } else {
      mt = fdiv(idx, t.seg ? g1.fd_nt.m : g0.fd_nt.m, t.seg ? g1.fd_nt.l : g0.fd_nt.l);
      t.nt = idx - mt * NT;
    }
    t.g = fdiv(r, ks_m, ks_l);
    t.split = r - t.g * ksplit;
    t.m0 = mt * BM;
    t.m_end = t.m0 + BM;
    int r0, r1;
    group_rows_lds(offs, t.g, r0, r1);
    const int chunk = (fdiv(r1 - r0 + ksplit - 1, ks_m, ks_l) + BKS - 1) / BKS * BKS;
    t.k_begin = min(r1, r0 + t.split * chunk);
    t.k_end = min(r1, t.k_begin + chunk);
  }
  t.nk = (t.k_end - t.k_begin + BKS - 1) / BKS;
  return t;
}

// The tile at list position i of an XCD's deal.  A half with no rows (the second half of a tile
// of at most 128 rows) has nk = 0 and is skipped.
template <int MODE>
__device__ __forceinline__ Tile deal_tile(const GemmArgs& p, const SegGeo (&geo)[2], const Deal& dl, int i) {
  if (Traits<MODE>::raggedK || i < dl.q) return decode_tile<MODE>(p, geo, tile_at(dl, i));
  const int h = (i - dl.q) >> 1, s = (i - dl.q) & 1;
  Tile t = decode_tile<MODE>(p, geo, tile_at(dl, dl.q + h));
  const int hb = t.x ? BMX / 2 : BM / 2;   // a tile of more than 256 rows: two of at most 160
  t.m0 += s * hb;
  t.m_end = min(t.m_end, t.m0 + hb);
  t.half = t.m_end - t.m0 <= BM / 2;
  t.x = false;
  if (t.m0 >= t.m_end) t.nk = 0;
  return t;
}

// ---- Direct loads ------------------------------------------------------------------------
// Load IDX (below lpa: operand A, else operand B) of the stage starting at k0 of tile t: 16 bytes
// per lane into LDS slot q = (wave * lp + j) * 64 + lane of the operand tile (lp: the operand's
// loads per wave).
// KC: slot q = (row q/8, physical chunk q%8).  MC: slot q = (k q/32, physical chunk q%32).
template <int MODE, int IDX>
__device__ __forceinline__ void issue_load(const GemmArgs& p, char* stage, const Tile& t, int k0, int wave, int lane) {
  constexpr bool A_OP = IDX < lpa<MODE>();
  constexpr int j = A_OP ? IDX : IDX - lpa<MODE>();
  constexpr bool kc = A_OP ? Traits<MODE>::a_kcontig : Traits<MODE>::b_kcontig;
  if constexpr (A_OP && j >= LPA_BM) {
    if (!t.x) return;   // as in issue_fast
  }
  const int q = load_slot<MODE, A_OP>(wave, j) * 64 + lane;
  const bf16_t* src;
  if constexpr (kc) {
    const int row = q >> 3;
    const int kk = k0 + (((q & 7) ^ kc_swz(row)) << 3);
    if constexpr (A_OP) {
      src = a_ptr_kc<MODE, bf16_t>(p, min(t.m0 + row, t.m_end - 1), kk);
    } else {
      src = b_ptr_kc<MODE, bf16_t, BN>(p, t.g, t.nt, row, kk);
    }
  } else {
    const int kr = q >> 5;
    const int col = ((q & 31) ^ ((kr & 3) << 2)) << 3;   // logical column of this physical chunk
    const int k = k0 + kr;
    if (k < t.k_end) {
      if constexpr (A_OP) src = a_ptr_mc<MODE, bf16_t>(p, k, t.m0 + col);
      else src = b_ptr_mc<MODE, bf16_t>(p, t.g, k, t.nt * BN + col);
    } else {
      src = reinterpret_cast<const bf16_t*>(g_zero_rows);
    }
  }
  __builtin_amdgcn_global_load_lds((gvoid_t*)src, (lvoid_t*)(stage + (A_OP ? 0 : opa<MODE>()) + load_slot<MODE, A_OP>(wave, j) * 1024),
                                   16, 0, 0);
}

// Loads inside the K loop: source = wave-uniform stage base + per-lane 32-bit byte offset.  The
// offsets depend on the tile only through the row clamp of the K-contiguous A operand; the bases
// carry k0 and the tile position.
template <int MODE>
__device__ __forceinline__ uint32_t load_offset(const GemmArgs& p, const Tile& t, int idx, int wave, int lane) {
  const bool a_op = idx < lpa<MODE>();
  const int q = (a_op ? load_slot<MODE, true>(wave, idx) : load_slot<MODE, false>(wave, idx - lpa<MODE>())) * 64 + lane;
  const bool kc = a_op ? Traits<MODE>::a_kcontig : Traits<MODE>::b_kcontig;
  if (kc) {
    const int row = q >> 3;
    const uint32_t c16 = (uint32_t)(((q & 7) ^ kc_swz(row)) << 4);
    if (a_op) {
      const int K = mode_K(MODE, p.d, p.f);
      return (uint32_t)(min(t.m0 + row, t.m_end - 1) - t.m0) * (uint32_t)K * 2u + c16;
    }
    if constexpr (MODE == GEMM_UP_FWD) return (uint32_t)(row & (BN / 2 - 1)) * (uint32_t)p.d * 2u + c16;
    return (uint32_t)row * (uint32_t)p.f * 2u + c16;   // GEMM_DOWN_FWD: W2 rows of length f
  }
  const int kr = q >> 5;
  const uint32_t col = (uint32_t)(((q & 31) ^ ((kr & 3) << 2)) << 3);
  uint32_t stride;   // elements per K row of the operand
  if (a_op) stride = MODE == GEMM_DOWN_WGRAD ? p.d : 2 * p.f;
  else if constexpr (MODE == GEMM_DOWN_BWD || MODE == GEMM_DOWN_WGRAD) stride = p.f;
  else stride = p.d;
  return ((uint32_t)kr * stride + col) * 2u;
}

// Per-lane byte offsets of a wave's loads from the stage bases.  Only the K-contiguous A operand
// (rows clamped at the group end) needs one per load; load j of any other operand is its first
// load's offset plus j times a wave-uniform step, with the swizzle change of odd j applied as an
// XOR (issue_fast).
struct LoadOffs {
  uint32_t a[MIX];   // lpa loads (at most 5)
  uint32_t b;
  uint32_t sa, sb;   // steps (bytes) between consecutive loads of A (not K-contiguous) and of B
};

// Step between consecutive loads of a wave (load j covers 8 K-contiguous rows, or 2 K rows of a
// K-strided operand, after load j - 1).
template <int MODE, bool A_OP>
__device__ __forceinline__ uint32_t load_step(const GemmArgs& p) {
  constexpr bool kc = A_OP ? Traits<MODE>::a_kcontig : Traits<MODE>::b_kcontig;
  uint32_t ld;   // elements per row (KC) or per K row (MC) of the operand
  if constexpr (A_OP) {
    if constexpr (kc) ld = mode_K(MODE, p.d, p.f);
    else ld = MODE == GEMM_DOWN_WGRAD ? p.d : 2 * p.f;
  } else if constexpr (kc) {
    ld = MODE == GEMM_UP_FWD ? p.d : p.f;
  } else {
    ld = (MODE == GEMM_DOWN_BWD || MODE == GEMM_DOWN_WGRAD) ? p.f : p.d;
  }
  return kc ? 16u * ld : 4u * ld;
}

// Wave-uniform byte bases of operands A and B for the stage starting at k0.
template <int MODE>
__device__ __forceinline__ void stage_bases(const GemmArgs& p, const Tile& t, int k0, int wave, const char*& sa,
                                            const char*& sb) {
  const char* a = reinterpret_cast<const char*>(p.a);
  const char* b0 = reinterpret_cast<const char*>(p.b0);
  const size_t d = p.d, f = p.f, g = t.g;
  if constexpr (MODE == GEMM_UP_FWD) {
    sa = a + ((size_t)t.m0 * d + k0) * 2;
    // B tile rows 0..127 are W1 (gate) rows, 128..255 the same W3 (up) rows; wave w loads rows
    // 8 * LPB * w .. + 8 * LPB - 1
    sb = reinterpret_cast<const char*>(wave < NW / 2 ? p.b0 : p.b1) + ((g * f + (size_t)t.nt * (BN / 2)) * d + k0) * 2;
  } else if constexpr (MODE == GEMM_DOWN_FWD) {
    sa = a + ((size_t)t.m0 * f + k0) * 2;
    sb = b0 + ((g * d + (size_t)t.nt * BN) * f + k0) * 2;
  } else if constexpr (MODE == GEMM_DOWN_BWD) {
    sa = a + ((size_t)t.m0 * d + k0) * 2;
    sb = b0 + ((g * d + k0) * f + (size_t)t.nt * BN) * 2;
  } else if constexpr (MODE == GEMM_UP_DGRAD) {
    sa = a + ((size_t)t.m0 * 2 * f + k0) * 2;
    const bool up = k0 >= p.f;
    sb = reinterpret_cast<const char*>(up ? p.b1 : p.b0) + ((g * f + (size_t)(up ? k0 - p.f : k0)) * d +
                                                            (size_t)t.nt * BN) * 2;
  } else if constexpr (MODE == GEMM_DOWN_WGRAD) {
    sa = a + ((size_t)k0 * d + t.m0) * 2;
    sb = b0 + ((size_t)k0 * f + (size_t)t.nt * BN) * 2;
  } else {
    sa = a + ((size_t)k0 * 2 * f + t.m0) * 2;
    sb = b0 + ((size_t)k0 * d + (size_t)t.nt * BN) * 2;
  }
}

template <int MODE, int IDX>
__device__ __forceinline__ void issue_fast(char* stage, const char* sa, const char* sb, const LoadOffs& lo,
                                           int k_left, bool x, int wave, int lane) {
  constexpr bool A_OP = IDX < lpa<MODE>();
  constexpr int J = A_OP ? IDX : IDX - lpa<MODE>();
  if constexpr (A_OP && J >= LPA_BM) {
    if (!x) return;   // wave-uniform: rows past BM of a tile that has none
  }
  // Load J is 8 K-contiguous rows (2 K rows) after load 0, which moves the row swizzle by 4
  // chunks (the window swizzle by 8 chunks) for odd J: a 64-byte (128-byte) XOR on top of the step.
  constexpr bool KC = A_OP ? Traits<MODE>::a_kcontig : Traits<MODE>::b_kcontig;
  constexpr uint32_t FLIP = (J & 1) ? (KC ? 64u : 128u) : 0u;
  uint32_t off;
  if constexpr (A_OP && Traits<MODE>::a_kcontig) off = lo.a[J];
  else if constexpr (A_OP) off = (lo.a[0] + (uint32_t)J * lo.sa) ^ FLIP;
  else off = (lo.b + (uint32_t)J * lo.sb) ^ FLIP;
  const char* src = (A_OP ? sa : sb) + off;
  if constexpr (Traits<MODE>::raggedK) {
    // K-strided operands: lane reads K row (load slot) * 2 + lane / 32 of the stage; rows past
    // the group's end read zeros.
    const int kr = load_slot<MODE, A_OP>(wave, J) * 2 + (lane >> 5);
    if (kr >= k_left) src = reinterpret_cast<const char*>(g_zero_rows);
  }
  __builtin_amdgcn_global_load_lds((gvoid_t*)src, (lvoid_t*)(stage + (A_OP ? 0 : opa<MODE>()) + load_slot<MODE, A_OP>(wave, J) * 1024),
                                   16, 0, 0);
}

// The next stage to load: operand bases and the number of its K rows inside the tile's K range.
struct StageSrc {
  const char* sa;
  const char* sb;
  int k_left;
  bool x;   // the stage belongs to a tile of more than BM rows (all lpa operand A loads)
};

// ---- Fragments ---------------------------------------------------------------------------
// Every tile is multiplied as 256x256: eight waves in a 2x4 grid, wave w = 4*wm + wn owning rows
// wm*128.. and 64 columns (4x2 MFMA blocks).  The two waves of a SIMD (w and w + 4, one per row
// half) take turns on its matrix core, so one of them can issue MFMAs while the other waits on a
// load issue, a fragment read or the barrier.  A tile with at most 128 rows (the last rows of a
// group) keeps the same load stream; the waves of the second row half skip its MFMAs.

// Row (A) / column (B) of the wave's MFMA block i inside the operand tile (M blocks per wave row:
// the wave's rows are wm * 32M ..).
template <int MODE, bool A_OP>
__device__ __forceinline__ int block_row(int wm, int wn, int i, int M = MI) {
  if constexpr (A_OP) return wm * 32 * M + 32 * i;
  // gate/up: the wave's 32 gate (W1) columns in block 0, the same up (W3) columns in block 1
  else if constexpr (MODE == GEMM_UP_FWD) return i == 0 ? wn * 32 : 128 + wn * 32;
  else return wn * 64 + 32 * i;
}

// Per-lane LDS offset (within a stage, operand base included) of the first fragment read of each
// 16-deep substep; the other blocks follow from it:
//  KC: block i is a constant offset away (its rows are 32*i or, for the gate/up B tile, 128 rows
//      further; the swizzle repeats every 16 rows), applied as the instruction's offset field.
//  The substep s (0..3) picks the 16-deep quarter of the stage's 64 k.
//  MC: block i is 32 columns = 4 chunks further; with the window swizzle that is an XOR of i into
//      address bits 6-7 (block 0 starts at a multiple of 64 columns).  The second transposed read
//      of a block is 4 k-rows = 2048 bytes further.
template <int MODE, bool A_OP>
__device__ __forceinline__ uint32_t frag_base(int s, int wm, int wn, int lane, int M = MI) {
  constexpr bool kc = A_OP ? Traits<MODE>::a_kcontig : Traits<MODE>::b_kcontig;
  const uint32_t base = A_OP ? 0 : opa<MODE>();
  const int rb = block_row<MODE, A_OP>(wm, wn, 0, M);
  if constexpr (kc) {
    const int row = rb + (lane & 31);
    const int chunk = s * 2 + (lane >> 5);
    return base + row * 128 + ((chunk ^ kc_swz(row)) << 4);
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
  if (!A_OP && MODE == GEMM_UP_FWD) return 16384 * i;
  return 4096 * i;
}

// Fragments of one 16-deep substep for NB blocks, read one instruction at a time (IDX).  KC: one
// read per block.  MC: two reads per block (4 k each), kept apart until packed for the MFMA.
template <bool KC, int NB>
struct Frag;
template <int NB>
struct Frag<true, NB> {
  static constexpr int PER_BLOCK = 1;
  bf16x8_t v[NB];
  template <int MODE, bool A_OP, int IDX>
  __device__ __forceinline__ void read_one(uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2"
                 : "=v"(v[IDX])
                 : "v"(addr), "i"(kc_block_off<MODE, A_OP>(IDX)));
  }
  __device__ __forceinline__ bf16x8_t get(int i) const { return v[i]; }
  // after an lgkmcnt wait: the values are in-out operands here, so no use moves above the wait
  __device__ __forceinline__ void landed() {
#pragma unroll
    for (int i = 0; i < NB; ++i) asm volatile("" : "+v"(v[i]));
  }
};
template <int NB>
struct Frag<false, NB> {
  static constexpr int PER_BLOCK = 2;
  u32x2_t h[2][NB];
  template <int MODE, bool A_OP, int IDX>
  __device__ __forceinline__ void read_one(uint32_t addr) {
    constexpr int i = IDX >> 1, r = IDX & 1;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(h[r][i]) : "v"(addr ^ (uint32_t)(i << 6)), "i"(r * 2048));
  }
  __device__ __forceinline__ bf16x8_t get(int i) const {
    const u32x4_t u = {h[0][i].x, h[0][i].y, h[1][i].x, h[1][i].y};
    return __builtin_bit_cast(bf16x8_t, u);
  }
  __device__ __forceinline__ void landed() {
#pragma unroll
    for (int i = 0; i < NB; ++i) asm volatile("" : "+v"(h[0][i]), "+v"(h[1][i]));
  }
};

template <int MODE>
using FragA = Frag<Traits<MODE>::a_kcontig, mi_max<MODE>()>;
template <int MODE>
using FragB = Frag<Traits<MODE>::b_kcontig, NI>;

// Wait until every LDS read is done; then the fragments count as written (no use of them can be
// scheduled before the wait).
template <int MODE>
__device__ __forceinline__ void frag_wait(FragA<MODE>& a, FragB<MODE>& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  a.landed();
  b.landed();
}

// ---- K step phases -------------------------------------------------------------------------
// Slot Q of a phase: MFMA Q (block row Q/NI, block column Q%NI), then the memory instructions that
// belong to the slot.  The scheduling barriers keep this order: the matrix core always has the
// next MFMA queued while the wave issues a read or a load.  ACT = false: a wave of the idle row
// half of a 128-row tile, which issues only the loads.

// MFMAs per phase and fragment reads per substep of a tile with M blocks per wave row.
template <int M>
constexpr int n_slots() { return M * NI; }
template <int MODE, int M>
constexpr int nreads_a() { return M * FragA<MODE>::PER_BLOCK; }
template <int MODE>
constexpr int nreads_b() { return NI * FragB<MODE>::PER_BLOCK; }

// The B fragment goes in as the MFMA's first operand: the accumulator block is then the
// transpose of the output block, so each lane ends up with consecutive output columns of one row.
template <int MODE, int Q, int M>
__device__ __forceinline__ void mfma_slot(f32x16_t (&acc)[M][NI], const FragA<MODE>& a, const FragB<MODE>& b) {
  constexpr int i = Q / NI, j = Q % NI;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b.get(j), a.get(i), acc[i][j], 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Fragment read R of a substep (A's reads first, then B's).
template <int MODE, int R, int M>
__device__ __forceinline__ void read_slot(FragA<MODE>& a, FragB<MODE>& b, uint32_t ra, uint32_t rb) {
  constexpr int NRA = nreads_a<MODE, M>(), NRB = nreads_b<MODE>();
  if constexpr (R < NRA) a.template read_one<MODE, true, R>(ra);
  else if constexpr (R < NRA + NRB) b.template read_one<MODE, false, R - NRA>(rb);
}

// Reads spread over the slots: ceil(reads / slots) per slot.
template <int MODE, int M>
constexpr int reads_per_slot() { return (nreads_a<MODE, M>() + nreads_b<MODE>() + n_slots<M>() - 1) / n_slots<M>(); }
template <int MODE, int Q, int I, int M>
__device__ __forceinline__ void slot_reads(FragA<MODE>& a, FragB<MODE>& b, uint32_t ra, uint32_t rb) {
  if constexpr (I < reads_per_slot<MODE, M>()) {
    read_slot<MODE, Q + I * n_slots<M>(), M>(a, b, ra, rb);
    slot_reads<MODE, Q, I + 1, M>(a, b, ra, rb);
  }
}

// Direct loads of slot Q: the lpw loads of a stage are spread evenly over the slots of a phase
// (a burst of direct loads stalls the issuing wave).
template <int MODE, int Q, int I, int M>
__device__ __forceinline__ void slot_loads(char* stage, const StageSrc& ss, const LoadOffs& voff, int wave,
                                           int lane) {
  constexpr int NS = n_slots<M>(), LPW = lpw<MODE>();
  constexpr int PER = (LPW + NS - 1) / NS, EVERY = NS > LPW ? NS / LPW : 1;
  if constexpr (I < PER && Q % EVERY == 0 && (Q / EVERY) * PER + I < LPW) {
    issue_fast<MODE, (Q / EVERY) * PER + I>(stage, ss.sa, ss.sb, voff, ss.k_left, ss.x, wave, lane);
    slot_loads<MODE, Q, I + 1, M>(stage, ss, voff, wave, lane);
  }
}

// Deferred epilogue stores of the unsplit weight gradients.  A weight-gradient tile has a short K
// loop (the expert's rows, 4 K steps at 256 rows), and its epilogue writes half as many bytes as
// the loop loads from L2; issued all at once, the stores hold the matrix cores idle.  So the epilogue
// stores block row 0 of the wave and keeps block rows 1..3 (DEFER store instructions) as packed
// bf16 rows, which the first K step of the wave's next tile issues between its MFMAs, four per
// phase in the first three phases.  The K loop's wait arithmetic is unchanged: the step's wait
// comes after them, and an epilogue plus the deferred stores still issue epilogue_stores().
constexpr int DEFER_ROWS = 3;
constexpr int DEFER = 4 * DEFER_ROWS;
struct Pending {
  u32x4_t v[DEFER];
  __amdgpu_buffer_rsrc_t r;
  uint32_t row_bytes;
  int offa, offb;   // per-lane byte offsets of the A and B rows of a pair (row 0 of the window)
};
struct NoPending {};
template <int MODE>
using PendingOf = typename std::conditional<Traits<MODE>::raggedK, Pending, NoPending>::type;
// Deferred store I: block row MI - DEFER_ROWS + I / 4, row half q, the pair's A (rows 0..7) or B
// (rows 8..15) store of st_rows128.
template <int I>
__device__ __forceinline__ void pending_store(const Pending& pd) {
  constexpr int mi = MI - DEFER_ROWS + I / 4, q = (I / 2) % 2;
  constexpr bool isb = I % 2;
  const int off = (isb ? pd.offb : pd.offa) + (int)((mi * 32 + 16 * q + (isb ? 8 : 0)) * pd.row_bytes);
  __builtin_amdgcn_raw_buffer_store_b128(pd.v[I], pd.r, off, 0, 2);
}

template <int I>
__device__ __forceinline__ void flush_pending(const Pending& pd) {
  if constexpr (I < DEFER) {
    pending_store<I>(pd);
    flush_pending<I + 1>(pd);
  }
}

// One phase of a K step: the MFMAs of the current substep (fragments ac, bc); the reads of the
// next substep into an, bn at ra/rb; with LOADS, the loads of the stage two steps ahead into this
// step's slot; with PS >= 0, the deferred stores of phase PS of a tile's first K step.
template <int MODE, bool ACT, bool LOADS, int Q, int M, int PS = -1>
__device__ __forceinline__ void phase(f32x16_t (&acc)[M][NI], const FragA<MODE>& ac, const FragB<MODE>& bc,
                                      FragA<MODE>& an, FragB<MODE>& bn, uint32_t ra, uint32_t rb, char* stage,
                                      const StageSrc& ss, const LoadOffs& voff, int wave, int lane,
                                      const PendingOf<MODE>* pd = nullptr) {
  if constexpr (Q < n_slots<M>()) {
    if constexpr (ACT) {
      mfma_slot<MODE, Q, M>(acc, ac, bc);
      slot_reads<MODE, Q, 0, M>(an, bn, ra, rb);
    }
    if constexpr (LOADS) slot_loads<MODE, Q, 0, M>(stage, ss, voff, wave, lane);
    constexpr int SPP = (DEFER + 2) / 3, EVERY = n_slots<M>() / SPP;   // deferred stores per phase
    if constexpr (PS >= 0 && Q % EVERY == EVERY - 1 && PS * SPP + Q / EVERY < DEFER)
      pending_store<PS * SPP + Q / EVERY>(*pd);
    __builtin_amdgcn_sched_barrier(0);
    phase<MODE, ACT, LOADS, Q + 1, M, PS>(acc, ac, bc, an, bn, ra, rb, stage, ss, voff, wave, lane, pd);
  }
}

// All reads of one substep's fragments (prologue, start of a tile).
template <int MODE, int R, int M>
__device__ __forceinline__ void read_all(FragA<MODE>& a, FragB<MODE>& b, uint32_t ra, uint32_t rb) {
  if constexpr (R < nreads_a<MODE, M>() + nreads_b<MODE>()) {
    read_slot<MODE, R, M>(a, b, ra, rb);
    read_all<MODE, R + 1, M>(a, b, ra, rb);
  }
}

template <int MODE, int IDX>
__device__ __forceinline__ void issue_all(const GemmArgs& p, char* stage, const Tile& t, int k0, int wave, int lane) {
  if constexpr (IDX < lpw<MODE>()) {
    issue_load<MODE, IDX>(p, stage, t, k0, wave, lane);
    issue_all<MODE, IDX + 1>(p, stage, t, k0, wave, lane);
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
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Output window of one wave: the tensor region that starts at the wave's first output row and
// column, as a buffer resource whose size ends with the last row inside the group.  Stores to
// rows past it are dropped by the hardware, so no store is branched around and every epilogue
// issues a fixed number of memory instructions (the K loop's vmcnt arithmetic relies on it).
struct OutWin {
  __amdgpu_buffer_rsrc_t r;
  uint32_t row_bytes;
};
__device__ __forceinline__ OutWin out_win(const void* base, size_t elem_off, int rows, int row_elems, int esize) {
  OutWin w;
  w.row_bytes = (uint32_t)uniform(row_elems * esize);
  char* b = uniform_ptr(const_cast<char*>(reinterpret_cast<const char*>(base)) + elem_off * esize);
  w.r = __builtin_amdgcn_make_buffer_rsrc(b, 0, uniform(max(rows, 0) * (int)w.row_bytes), 0x00020000);
  return w;
}
// 8 fp32 values to packed bf16 (16 bytes).
__device__ __forceinline__ u32x4_t pack8_bf16(const float (&x)[8]) {
  const float lo[4] = {x[0], x[1], x[2], x[3]}, hi[4] = {x[4], x[5], x[6], x[7]};
  const u32x2_t a = pack4_bf16(lo), b = pack4_bf16(hi);
  const u32x4_t w = {a.x, a.y, b.x, b.y};
  return w;
}
// The output windows of one wave's block of a tile (wrows rows).
struct OutWins {
  OutWin w[3];
};

template <int MODE>
__device__ __forceinline__ OutWins out_wins(const GemmArgs& p, const Tile& t, int row0, int col0, float* partial,
                                            int wrows = 128) {
  OutWins o;
  const int rows = min(wrows, t.m_end - row0);
  const size_t d = p.d, f = p.f;
  if constexpr (MODE == GEMM_UP_FWD) {
    const size_t e = (size_t)row0 * f + col0;
    o.w[0] = out_win(p.out0, e, rows, p.f, 2);
    o.w[1] = out_win(p.out1, e, rows, p.f, 2);
    o.w[2] = out_win(p.out2, e, rows, p.f, 2);
  } else if constexpr (MODE == GEMM_DOWN_FWD || MODE == GEMM_UP_DGRAD) {
    o.w[0] = out_win(p.out0, (size_t)row0 * d + col0, rows, p.d, 2);
  } else if constexpr (MODE == GEMM_DOWN_BWD) {
    o.w[0] = out_win(p.out0, (size_t)row0 * 2 * f + col0, rows, 2 * p.f, 2);
  } else {
    const int Mw = mode_Mw(MODE, p.d, p.f), Nw = mode_N(MODE, p.d, p.f);
    if (t.ks > 1) {
      o.w[0] = out_win(partial, (((size_t)t.split * p.G + t.g) * Mw + row0) * Nw + col0, 128, Nw, 4);
    } else if constexpr (MODE == GEMM_DOWN_WGRAD) {
      o.w[0] = out_win(p.out0, ((size_t)t.g * d + row0) * f + col0, 128, p.f, 2);
    } else {  // rows [0, f) of the gradient go to dW1, [f, 2f) to dW3; a wave's 128 rows lie in one
      const bool up = row0 >= p.f;
      o.w[0] = out_win(up ? p.out1 : p.out0, ((size_t)t.g * f + (up ? row0 - p.f : row0)) * d + col0, 128, p.d, 2);
    }
  }
  return o;
}

// Output layout of a 32x32 accumulator block after block_half: lane l holds row l % 32, and for
// half H the 8 columns 16H + 8*(l/32) + 0..7, so a store of 16 bytes per lane covers 32 rows with
// 32 contiguous bytes each, which the CU's store path takes at a quarter of its rate for rows of
// 64 bytes or more.  Exchanging lane groups (v_permlane16_swap, one per dword) between the two
// 16-byte pieces a, b of each lane turns them into r0, covering rows 0..15, and r1, rows 16..31,
// four lanes and 64 contiguous bytes per row: lane l then holds row l % 16 (+16 in r1), piece
// (l/16) % 2 of lane (l % 16) + 32*(l/32).  The exchange is its own inverse.
__device__ __forceinline__ void swap16(const u32x4_t& a, const u32x4_t& b, u32x4_t& r0, u32x4_t& r1) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const auto r = __builtin_amdgcn_permlane16_swap(a[e], b[e], false, false);
    r0[e] = r[0];
    r1[e] = r[1];
  }
}
// Column offset (elements) of lane's 16 bytes in the exchanged layout: bf16 pieces are the two
// halves of the block (8 columns each), fp32 pieces the two quarters of one half (4 columns).
__device__ __forceinline__ int xcol_bf16(int lane) { return 16 * ((lane >> 4) & 1) + 8 * (lane >> 5); }
__device__ __forceinline__ int xcol_f32(int lane) { return 4 * ((lane >> 4) & 1) + 8 * (lane >> 5); }

// Store two packed pieces (the lane's halves H = 0, 1 of a block) as rows rl and rl + 16 at
// column cl of the exchanged layout.
__device__ __forceinline__ void st_pair(const OutWin& w, int rl, int cl, int esize, const u32x4_t& a,
                                        const u32x4_t& b) {
  u32x4_t r0, r1;
  swap16(a, b, r0, r1);
  const int off = (int)(rl * w.row_bytes) + cl * esize;
  __builtin_amdgcn_raw_buffer_store_b128(r0, w.r, off, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(r1, w.r, off + 16 * (int)w.row_bytes, 0, 0);
}
__device__ __forceinline__ void st_pair_bf16(const OutWin& w, int rl, int cl, const float (&x)[2][8]) {
  st_pair(w, rl, cl, 2, pack8_bf16(x[0]), pack8_bf16(x[1]));
}
__device__ __forceinline__ u32x4_t bits4(float a, float b, float c, float d) {
  const u32x4_t r = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
  return r;
}

// Stashed pre-activations (a, b) of the down-projection dgrad for one block, as loaded: rows 0..15
// (a0, b0) and 16..31 (a1, b1) of the exchanged layout.
struct AuxBlock {
  u32x4_t a0, a1, b0, b1;
};

// Store one 32x32 output block (rows br.., columns bc.. of the wave's window) of the mode: v holds
// the lane's two halves of the accumulator block, u the up-projection halves of the gate/up GEMM,
// x the stashed pre-activations of the down-projection dgrad.
template <int MODE>
__device__ __forceinline__ void store_block(const GemmArgs& p, const OutWins& o, int br, int bc, const float (&v)[2][8],
                                            const float (&u)[2][8], const AuxBlock& x, int ksplit, int lane) {
  const int rl = br + (lane & 15);
  const int cl = bc + xcol_bf16(lane);
  if constexpr (MODE == GEMM_UP_FWD) {
    float h[2][8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 8; ++i) h[hh][i] = v[hh][i] * fast_sigmoid(v[hh][i]) * u[hh][i];
    if (p.out0) st_pair_bf16(o.w[0], rl, cl, v);
    if (p.out1) st_pair_bf16(o.w[1], rl, cl, u);
    st_pair_bf16(o.w[2], rl, cl, h);
  } else if constexpr (MODE == GEMM_DOWN_FWD || MODE == GEMM_UP_DGRAD) {
    st_pair_bf16(o.w[0], rl, cl, v);
  } else if constexpr (MODE == GEMM_DOWN_BWD) {
    // back to the accumulator layout: halves 0 and 1 of a and b
    u32x4_t ah[2], bh[2];
    swap16(x.a0, x.a1, ah[0], ah[1]);
    swap16(x.b0, x.b1, bh[0], bh[1]);
    u32x4_t pa[2], pb[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float da[8], db[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = (i & 1) ? bf16_hi(ah[hh][i >> 1]) : bf16_lo(ah[hh][i >> 1]);
        const float b = (i & 1) ? bf16_hi(bh[hh][i >> 1]) : bf16_lo(bh[hh][i >> 1]);
        const float s = fast_sigmoid(a);
        da[i] = v[hh][i] * b * s * (1.0f + a * (1.0f - s));
        db[i] = v[hh][i] * a * s;
      }
      pa[hh] = pack8_bf16(da);
      pb[hh] = pack8_bf16(db);
    }
    st_pair(o.w[0], rl, cl, 2, pa[0], pa[1]);
    st_pair(o.w[0], rl, p.f + cl, 2, pb[0], pb[1]);
  } else {  // weight gradients
    if (ksplit > 1) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        st_pair(o.w[0], rl, bc + 16 * hh + xcol_f32(lane), 4, bits4(v[hh][0], v[hh][1], v[hh][2], v[hh][3]),
                bits4(v[hh][4], v[hh][5], v[hh][6], v[hh][7]));
    } else {
      st_pair_bf16(o.w[0], rl, cl, v);
    }
  }
}

// Store instructions every epilogue issues at least (per wave; the optional pre-activation stashes
// of the gate/up GEMM not counted; an unsplit weight-gradient epilogue with the deferred stores the
// next tile's first K step issues before its wait).
template <int MODE>
constexpr int epilogue_stores() {
  return MODE == GEMM_UP_FWD ? 8 : (MODE == GEMM_DOWN_BWD ? 32 : 16);
}

// Copies of four accumulator registers to VGPRs.  Written out so that each value leaves its AGPR
// only where it is used: left to itself the compiler moves the whole accumulator set to VGPRs at
// the end of the K loop and spills.  The hazard checker does not look into inline asm, so two
// wait states for a cross-lane read of a freshly written VGPR are added here.
#define MOE_AGPR_READ4(C, E0, X)                                                                  \
  asm volatile(                                                                                   \
      "v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\tv_accvgpr_read_b32 %2, %6\n\t"     \
      "v_accvgpr_read_b32 %3, %7\n\ts_nop 1"                                                       \
      : "=v"(X[0]), "=v"(X[1]), "=v"(X[2]), "=v"(X[3])                                            \
      : "a"(C[(E0)]), "a"(C[(E0) + 1]), "a"(C[(E0) + 2]), "a"(C[(E0) + 3]))

// Half H of an accumulator block as 8 consecutive output columns.  With the transposed MFMA, lane
// l holds output row l % 32 and, for element v, column 8*(v/4) + 4*(l/32) + v%4 of the block.
// Swapping the upper lanes of group 2H with the lower lanes of group 2H+1 (v_permlane32_swap)
// leaves lane l with columns 16H + 8*(l/32) + 0..7.
__device__ __forceinline__ void block_half(const f32x16_t& c, int h, float (&x)[8]) {
  float lo[4], hi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = c[8 * h + e];
    hi[e] = c[8 * h + 4 + e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo[e]), __float_as_uint(hi[e]), false, false);
    x[e] = __uint_as_float(r[0]);
    x[4 + e] = __uint_as_float(r[1]);
  }
}

// Pre-activations of one block for the down-projection dgrad, loaded in the exchanged layout
// (64 contiguous bytes per row) with inline assembly and waited for explicitly: a compiler-tracked
// load would be preceded and followed by waits that drain the load stream of the next tile.  Rows
// clamped into the group.
__device__ __forceinline__ void load_aux(const GemmArgs& p, int row, int m_end, int col, AuxBlock& x, int lane) {
  const int rl = row + (lane & 15), cl = col + xcol_bf16(lane);
  const size_t e0 = (size_t)min(rl, m_end - 1) * p.f + cl, e1 = (size_t)min(rl + 16, m_end - 1) * p.f + cl;
  const bf16_t* a = reinterpret_cast<const bf16_t*>(p.aux0);
  const bf16_t* b = reinterpret_cast<const bf16_t*>(p.aux1);
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x.a0) : "v"(a + e0) : "memory");
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x.a1) : "v"(a + e1) : "memory");
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x.b0) : "v"(b + e0) : "memory");
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x.b1) : "v"(b + e1) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_aux(AuxBlock& x) {
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(x.a0), "+v"(x.a1), "+v"(x.b0), "+v"(x.b1) : "n"(N) : "memory");
}

// Output blocks per wave row (the gate/up GEMM pairs a gate block with an up block).
template <int MODE>
constexpr int out_nj() { return MODE == GEMM_UP_FWD ? NI / 2 : NI; }

// Window row and column of accumulator block IDX.
template <int MODE, int IDX>
constexpr int block_r() { return (IDX / out_nj<MODE>()) * 32; }
template <int MODE, int IDX>
constexpr int block_c() { return (IDX % out_nj<MODE>()) * 32; }

template <int MODE>
__device__ __forceinline__ void epilogue_block(const GemmArgs& p, const OutWins& o, const f32x16_t& c,
                                               const f32x16_t& cu, int br, int bc, const AuxBlock& x, int ksplit,
                                               int lane) {
  float v[2][8], u[2][8];
  block_half(c, 0, v[0]);
  block_half(c, 1, v[1]);
  if constexpr (MODE == GEMM_UP_FWD) {
    block_half(cu, 0, u[0]);
    block_half(cu, 1, u[1]);
  }
  store_block<MODE>(p, o, br, bc, v, u, x, ksplit, lane);
}

// Blocks whose pre-activations are in flight ahead of the block being stored.
constexpr int AUX_AHEAD = 1;

// Memory instructions issued after the pre-activation loads of block IDX and before the wait for
// them: the stores of the AUX_AHEAD blocks before it and the loads of the AUX_AHEAD blocks after
// it (4 each; block j's loads are issued before the wait of block j - AUX_AHEAD).
template <int IDX, int NB>
constexpr int aux_younger() {
  return 4 * (IDX < AUX_AHEAD ? IDX : AUX_AHEAD) + 4 * (NB - 1 - IDX < AUX_AHEAD ? NB - 1 - IDX : AUX_AHEAD);
}

// Blocks IDX.. of the wave's accumulators, unrolled at compile time (the loop unroller gives up on
// the larger epilogues, and a run-time block index would put the accumulators in scratch memory).
// The down-projection dgrad keeps the pre-activation loads AUX_AHEAD blocks ahead of their use.
template <int MODE, int IDX, int M>
__device__ __forceinline__ void epilogue_from(const GemmArgs& p, const OutWins& o, const f32x16_t (&acc)[M][NI],
                                              int row0, int col0, int m_end, int lane,
                                              AuxBlock (&aux)[AUX_AHEAD + 1], int ksplit) {
  constexpr int NJ = out_nj<MODE>();
  constexpr int NB = M * NJ;
  constexpr int NA = AUX_AHEAD + 1;
  if constexpr (IDX < NB) {
    if constexpr (MODE == GEMM_DOWN_BWD) {
      if constexpr (IDX + AUX_AHEAD < NB)
        load_aux(p, row0 + block_r<MODE, IDX + AUX_AHEAD>(), m_end, col0 + block_c<MODE, IDX + AUX_AHEAD>(),
                 aux[(IDX + AUX_AHEAD) % NA], lane);
      wait_aux<aux_younger<IDX, NB>()>(aux[IDX % NA]);
    }
    constexpr int mi = IDX / NJ, ni = IDX % NJ;
    constexpr int nu = (MODE == GEMM_UP_FWD) ? ni + NJ : ni;
    epilogue_block<MODE>(p, o, acc[mi][ni], acc[mi][nu], block_r<MODE, IDX>(), block_c<MODE, IDX>(), aux[IDX % NA],
                         ksplit, lane);
    epilogue_from<MODE, IDX + 1, M>(p, o, acc, row0, col0, m_end, lane, aux, ksplit);
  }
}

// Rows of 128 bytes: blocks (mi, 0) and (mi, 1) stored together.  After swap16 each block has r0
// (rows 0..15) and r1 (rows 16..31), lane l holding row l % 16 and 16 bytes at xcol_bf16(l).  A
// rotation by 8 lanes inside each 16-lane row (DPP row_ror:8) of block 1's pieces and a select on
// lane bit 3 give A (rows 0..7: block 0 where bit 3 is clear, block 1 where it is set) and B (rows
// 8..15): 8 lanes and 128 contiguous bytes (a whole cache line) per row, in as many store
// instructions as two blocks stored apart.  NT: a nontemporal store (weight gradients, which nothing
// in the layer pass reads again: with normal stores the 4 MB of gradient lines an XCD writes per
// round of tiles evicted the operand panels from L2, and the panels were fetched again).
__device__ __forceinline__ void rows128_data(const float (&x0)[2][8], const float (&x1)[2][8], int lane,
                                             u32x4_t (&A)[2], u32x4_t (&B)[2]) {
  u32x4_t a[2], c[2];
  swap16(pack8_bf16(x0[0]), pack8_bf16(x0[1]), a[0], a[1]);
  swap16(pack8_bf16(x1[0]), pack8_bf16(x1[1]), c[0], c[1]);
  const bool hi8 = (lane & 8) != 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)c[q][e], 0x128, 0xf, 0xf, false);
      A[q][e] = hi8 ? t : a[q][e];
      B[q][e] = hi8 ? a[q][e] : t;
    }
  }
}
template <bool NT>
__device__ __forceinline__ void st_rows128(const OutWin& w, int br, const float (&x0)[2][8], const float (&x1)[2][8],
                                           int lane) {
  constexpr int AUX = NT ? 2 : 0;   // cache policy bits of the buffer store: nt
  u32x4_t A[2], B[2];
  rows128_data(x0, x1, lane, A, B);
  const bool hi8 = (lane & 8) != 0;
  const int rl = br + (lane & 7);
  const int cx = xcol_bf16(lane);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = rl + 16 * q;
    __builtin_amdgcn_raw_buffer_store_b128(A[q], w.r, (int)(r * w.row_bytes) + (cx + (hi8 ? 32 : 0)) * 2, 0, AUX);
    __builtin_amdgcn_raw_buffer_store_b128(B[q], w.r, (int)((r + 8) * w.row_bytes) + (cx + (hi8 ? 0 : 32)) * 2, 0, AUX);
  }
}
// The epilogue of the modes with one bf16 output and no elementwise math (down projection, gate/up
// data gradient, unsplit weight gradients), block row MIDX.. of the wave.
template <int MIDX, int M, bool NT, int END = M>
__device__ __forceinline__ void epilogue_rows128(const OutWins& o, const f32x16_t (&acc)[M][NI], int lane) {
  if constexpr (MIDX < END) {
    float v0[2][8], v1[2][8];
    block_half(acc[MIDX][0], 0, v0[0]);
    block_half(acc[MIDX][0], 1, v0[1]);
    block_half(acc[MIDX][1], 0, v1[0]);
    block_half(acc[MIDX][1], 1, v1[1]);
    st_rows128<NT>(o.w[0], MIDX * 32, v0, v1, lane);
    epilogue_rows128<MIDX + 1, M, NT, END>(o, acc, lane);
  }
}
// The last DEFER_ROWS block rows of a wave's unsplit weight gradient, packed for pending_store.
template <int M>
__device__ __forceinline__ void defer_rows(const OutWin& w, const f32x16_t (&acc)[M][NI], int lane, Pending& pd) {
#pragma unroll
  for (int mi = M - DEFER_ROWS; mi < M; ++mi) {
    float v0[2][8], v1[2][8];
    block_half(acc[mi][0], 0, v0[0]);
    block_half(acc[mi][0], 1, v0[1]);
    block_half(acc[mi][1], 0, v1[0]);
    block_half(acc[mi][1], 1, v1[1]);
    u32x4_t A[2], B[2];
    rows128_data(v0, v1, lane, A, B);
    const int i = 4 * (mi - (M - DEFER_ROWS));
    pd.v[i + 0] = A[0];
    pd.v[i + 1] = B[0];
    pd.v[i + 2] = A[1];
    pd.v[i + 3] = B[1];
  }
  const bool hi8 = (lane & 8) != 0;
  const int cx = xcol_bf16(lane);
  pd.r = w.r;
  pd.row_bytes = w.row_bytes;
  pd.offa = (int)((lane & 7) * w.row_bytes) + (cx + (hi8 ? 32 : 0)) * 2;
  pd.offb = (int)((lane & 7) * w.row_bytes) + (cx + (hi8 ? 0 : 32)) * 2;
}

// Pre-activation loads of blocks IDX..AUX_AHEAD-1, issued in block order before the first store.
template <int MODE, int IDX>
__device__ __forceinline__ void aux_prologue(const GemmArgs& p, int row0, int col0, int m_end,
                                             AuxBlock (&aux)[AUX_AHEAD + 1], int lane) {
  if constexpr (IDX < AUX_AHEAD && IDX < MI * out_nj<MODE>()) {
    load_aux(p, row0 + block_r<MODE, IDX>(), m_end, col0 + block_c<MODE, IDX>(), aux[IDX], lane);
    aux_prologue<MODE, IDX + 1>(p, row0, col0, m_end, aux, lane);
  }
}

// The wave's output block of a tile: rows wm*32M.. and its 64 columns (32 H columns for the gate/up
// GEMM).  The idle row half of a 128-row tile runs it too: its window holds no rows, so every store
// is dropped, and it issues the same number of memory instructions as the others.
template <int MODE, int M>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& p, const f32x16_t (&acc)[M][NI], const Tile& t,
                                              int wm, int wn, int lane, float* partial, PendingOf<MODE>& pd, bool& pd_on) {
  // The accumulator reads are opaque to the hazard checker: leave the last MFMA's write-back
  // (at most 18 wait states) behind before the first of them.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  // The lane index through a volatile move: the per-lane addressing below is then computed here,
  // not hoisted out of the tile loop into registers the K loop would have to keep (or spill).
  asm volatile("v_mov_b32 %0, %0" : "+v"(lane));
  const int row0 = t.m0 + wm * 32 * M;
  const int col0 = (MODE == GEMM_UP_FWD) ? t.nt * (BN / 2) + wn * 32 : t.nt * BN + wn * 64;
  const OutWins o = out_wins<MODE>(p, t, row0, col0, partial, 32 * M);
  const int ksplit = t.ks;
  AuxBlock aux[AUX_AHEAD + 1];
  if constexpr (MODE == GEMM_DOWN_BWD) aux_prologue<MODE, 0>(p, row0, col0, t.m_end, aux, lane);
  if constexpr (Traits<MODE>::raggedK && M == MI) {
    if (ksplit == 1) {   // block rows past MI - DEFER_ROWS go out in the next tile's first K step
      epilogue_rows128<0, M, true, M - DEFER_ROWS>(o, acc, lane);
      defer_rows<M>(o.w[0], acc, lane, pd);
      pd_on = true;
      return;
    }
  }
  if constexpr (MODE != GEMM_UP_FWD && MODE != GEMM_DOWN_BWD) {
    if (ksplit == 1) {   // same store count as the per-block path (two per block)
      epilogue_rows128<0, M, Traits<MODE>::raggedK>(o, acc, lane);
      return;
    }
  }
  epilogue_from<MODE, 0, M>(p, o, acc, row0, col0, t.m_end, lane, aux, ksplit);
}

// Output of a tile with an empty K range (a weight gradient of an expert without tokens): zeros.
template <int MODE>
__device__ __forceinline__ void zero_tile(const GemmArgs& p, const Tile& t, int wm, int wn, int lane,
                                          float* partial) {
  const float z[2][8] = {};
  const AuxBlock zx = {};
  const int row0 = t.m0 + wm * 128, col0 = t.nt * BN + wn * 64;
  const OutWins o = out_wins<MODE>(p, t, row0, col0, partial);
  const int ksplit = t.ks;
#pragma unroll 1
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll 1
    for (int ni = 0; ni < NI; ++ni) store_block<MODE>(p, o, mi * 32, ni * 32, z, z, zx, ksplit, lane);
}

// Per-group tile prefix (ragged-M modes): pref[g] = tiles (group_tiles) of the groups before g,
// from the clamped offsets in offs.
template <int MODE>
__device__ __forceinline__ void tile_prefix_lds(int G, const int* offs, int* pref, int* scratch, bool rows256) {
  const int tid = threadIdx.x;
  if (tid == 0) scratch[NTH] = 0;
  __syncthreads();
  for (int base = 0; base < G; base += NTH) {
    const int g = base + tid;
    int c = 0;
    if (g < G) {
      const int lo = offs[g], hi = max(lo, offs[g + 1]);
      c = group_tiles<MODE>(hi - lo, rows256);
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
    if (g < G) pref[g] = carry + scratch[tid] - c;
    __syncthreads();
    if (tid == NTH - 1) scratch[NTH] = carry + scratch[NTH - 1];
    __syncthreads();
  }
  if (tid == 0) pref[G] = scratch[NTH];
  __syncthreads();
}

// Weight gradients: a tile's cost in K steps, plus WG_TILE_COST for its epilogue and the
// pipeline's turn at a tile boundary (a tile of chunk rows of one split of a group of R rows).
constexpr int WG_TILE_COST = 5;
__device__ __forceinline__ int wg_tile_cost(int R, int ks) {
  const int chunk = (R + ks - 1) / ks;
  return (chunk + BKS - 1) / BKS + WG_TILE_COST;
}

// cpref[g] = summed cost of the tiles of the groups before g, cpref[G] the total (every group has
// tpg tiles, all of one cost), from the clamped offsets in offs.  A group's share is capped so the
// total stays below 2^30 (only groups far beyond any memory size reach the cap).
__device__ __forceinline__ void cost_prefix_lds(int G, int ks, int tpg, const int* offs, int* cpref,
                                                int* scratch) {
  const int tid = threadIdx.x;
  const long long cap = (1LL << 30) / (G + 1);
  if (tid == 0) scratch[NTH] = 0;
  __syncthreads();
  for (int base = 0; base < G; base += NTH) {
    const int g = base + tid;
    int c = 0;
    if (g < G) {
      const int lo = offs[g], hi = max(lo, offs[g + 1]);
      c = (int)min(cap, (long long)tpg * wg_tile_cost(hi - lo, ks));
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
    if (g < G) cpref[g] = carry + scratch[tid] - c;
    __syncthreads();
    if (tid == NTH - 1) scratch[NTH] = carry + scratch[NTH - 1];
    __syncthreads();
  }
  if (tid == 0) cpref[G] = scratch[NTH];
  __syncthreads();
}

// Summed cost of the tiles before tile i (i <= G * tpg).
__device__ __forceinline__ int cost_before(const int* cpref, const int* offs, int tpg, int ks, int i) {
  const int g = i / tpg, r = i - g * tpg;
  if (r == 0) return cpref[g];
  const int lo = offs[g], hi = max(lo, offs[g + 1]);
  return cpref[g] + r * wg_tile_cost(hi - lo, ks);
}

// First tile of XCD x under a cost-balanced cut: the first tile whose preceding cost reaches x/8
// of the total.
__device__ __forceinline__ int cost_cut(const int* cpref, const int* offs, int G, int tpg, int ks, int x) {
  if (x >= 8) return G * tpg;
  const int target = (int)((long long)x * cpref[G] / 8);
  int lo = 0, hi = G;   // largest g with cpref[g] <= target
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cpref[mid] <= target) lo = mid; else hi = mid;
  }
  const int glo = offs[lo], ghi = max(glo, offs[lo + 1]);
  const int tc = wg_tile_cost(ghi - glo, ks);
  const int j = (target - cpref[lo] + tc - 1) / tc;
  return lo * tpg + min(j, tpg);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): everything but the N newest loads or stores is done.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Producer of the load stream: the tile and K step of the next stage to load.  Once the stream
// runs out it keeps reloading the last stage (valid memory, into slots nobody reads again).  The
// K loop's waits (everything, or everything but the last epilogue's stores) do not depend on how
// many loads a stage has, so a stage of a tile of at most BM rows skips the A loads past row BM.
struct Producer {
  Tile t;
  int i, k;        // this XCD's tile list position, K step
  LoadOffs lo;     // per-lane load offsets
  StageSrc ss;     // sources of stage k
  long long da, db;  // byte step of the sources from one K step to the next
};

template <int MODE>
__device__ __forceinline__ StageSrc stage_src(const Producer& pr, const GemmArgs& p, int wave) {
  StageSrc ss;
  const int k0 = pr.t.k_begin + pr.k * BKS;
  ss.k_left = pr.t.k_end - k0;
  ss.x = pr.t.x;
  stage_bases<MODE>(seg_args(p, pr.t.seg), pr.t, k0, wave, ss.sa, ss.sb);
  ss.sa = uniform_ptr(ss.sa);
  ss.sb = uniform_ptr(ss.sb);
  return ss;
}

// A new tile for the producer: per-lane load offsets, the sources of its first stage and the
// per-step source strides (K-contiguous operands move 32 elements, K-strided ones 32 rows).
template <int MODE>
__device__ __forceinline__ void set_offsets(Producer& pr, const GemmArgs& p, int wave, int lane) {
  const GemmArgs q = seg_args(p, pr.t.seg);
  constexpr bool kca = Traits<MODE>::a_kcontig;
#pragma unroll
  for (int i = 0; i < (kca ? lpa<MODE>() : 1); ++i) pr.lo.a[i] = load_offset<MODE>(q, pr.t, i, wave, lane);
  pr.lo.b = load_offset<MODE>(q, pr.t, lpa<MODE>(), wave, lane);
  pr.lo.sa = (uint32_t)uniform((int)load_step<MODE, true>(q));
  pr.lo.sb = (uint32_t)uniform((int)load_step<MODE, false>(q));
  pr.ss = stage_src<MODE>(pr, p, wave);
  const long long d = q.d, f = q.f, kc = 2 * BKS;
  if constexpr (MODE == GEMM_UP_FWD || MODE == GEMM_DOWN_FWD) { pr.da = kc; pr.db = kc; }
  else if constexpr (MODE == GEMM_DOWN_BWD) { pr.da = kc; pr.db = kc * f; }
  else if constexpr (MODE == GEMM_UP_DGRAD) { pr.da = kc; pr.db = kc * d; }
  else if constexpr (MODE == GEMM_DOWN_WGRAD) { pr.da = kc * d; pr.db = kc * f; }
  else { pr.da = kc * 2 * f; pr.db = kc * d; }
}

template <int MODE>
__device__ __forceinline__ void advance(Producer& pr, const GemmArgs& p, const SegGeo (&geo)[2], const Deal& dl,
                                        int nbx, int wave, int lane) {
  if (pr.k + 1 < pr.t.nk) {
    ++pr.k;
    if (MODE == GEMM_UP_DGRAD && pr.t.k_begin + pr.k * BKS == (pr.t.seg ? p.s1.f : p.f)) {
      pr.ss = stage_src<MODE>(pr, p, wave);   // K moves from the gate half (W1) to the up half (W3)
    } else {
      pr.ss.sa += pr.da;
      pr.ss.sb += pr.db;
      pr.ss.k_left -= BKS;
    }
    return;
  }
  for (int i = pr.i + nbx; i < dl.n; i += nbx) {
    const Tile t = deal_tile<MODE>(p, geo, dl, i);
    if (t.nk > 0) {
      pr.t = t;
      pr.i = i;
      pr.k = 0;
      set_offsets<MODE>(pr, p, wave, lane);
      return;
    }
  }
  pr.i = dl.n;
}

// Per-lane fragment read bases of substep 0, both operands.  Substep s of a slot at sb:
//  KC: the logical chunk is 2s + lane/32 and the swizzle XORs bits 4-6 of the address only, so the
//      address is (base + sb) XOR 32s (sb and base's row part leave bits 5-6 clear);
//  MC: the window swizzle depends on k mod 4, the same in every substep, so it is base + sb + 8192s.
struct FragBases {
  uint32_t a, ax, b;   // ax: operand A of a tile of more than 256 rows (160 rows per wave)
};
template <int MODE>
__device__ __forceinline__ FragBases frag_bases(uint32_t lds0, int wm, int wn, int lane) {
  FragBases f;
  f.a = lds0 + frag_base<MODE, true>(0, wm, wn, lane);
  f.ax = lds0 + frag_base<MODE, true>(0, wm, wn, lane, MIX);
  f.b = lds0 + frag_base<MODE, false>(0, wm, wn, lane);
  return f;
}
template <int MODE, bool A_OP, int S>
__device__ __forceinline__ uint32_t sub_addr(uint32_t base, uint32_t sb) {
  constexpr bool kc = A_OP ? Traits<MODE>::a_kcontig : Traits<MODE>::b_kcontig;
  if constexpr (kc) return (base + sb) ^ (uint32_t)(32 * S);
  else return base + sb + (uint32_t)(8192 * S);
}

// One K step (stage j, slot j & 1): four phases of 16-deep substeps whose fragments alternate
// between the register sets 0 and 1; the fourth phase reads substep 0 of stage j + 1 from the other
// slot and loads stage j + 2 into this one, which every wave has finished reading by then.  PD: the
// first three phases also issue the previous tile's deferred stores.
template <int MODE, bool ACT, int M, bool PD>
__device__ __forceinline__ void kstep(const GemmArgs& p, f32x16_t (&acc)[M][NI], uint32_t fa, const FragBases& fb,
                                      FragA<MODE>& a0, FragB<MODE>& b0, FragA<MODE>& a1, FragB<MODE>& b1, int j,
                                      int since_epi, Producer& pr, const SegGeo (&geo)[2], const Deal& dl, int nbx,
                                      int wave, int lane, char* lds, const PendingOf<MODE>& pd) {
  constexpr uint32_t STAGE = stage_bytes<MODE>();
  const uint32_t sb = (j & 1) * STAGE;
  phase<MODE, ACT, false, 0, M, PD ? 0 : -1>(acc, a0, b0, a1, b1, sub_addr<MODE, true, 1>(fa, sb), sub_addr<MODE, false, 1>(fb.b, sb), nullptr, pr.ss, pr.lo, wave, lane, &pd);
  if constexpr (ACT) frag_wait<MODE>(a1, b1);
  phase<MODE, ACT, false, 0, M, PD ? 1 : -1>(acc, a1, b1, a0, b0, sub_addr<MODE, true, 2>(fa, sb), sub_addr<MODE, false, 2>(fb.b, sb), nullptr, pr.ss, pr.lo, wave, lane, &pd);
  if constexpr (ACT) frag_wait<MODE>(a0, b0);
  phase<MODE, ACT, false, 0, M, PD ? 2 : -1>(acc, a0, b0, a1, b1, sub_addr<MODE, true, 3>(fa, sb), sub_addr<MODE, false, 3>(fb.b, sb), nullptr, pr.ss, pr.lo, wave, lane, &pd);
  if constexpr (ACT) frag_wait<MODE>(a1, b1);
  // Stage j+1 has landed once nothing issued before the last epilogue's stores is outstanding
  // (the first step after an epilogue; at least epilogue_stores() of them follow the stage's
  // loads), or nothing at all; the barrier makes every wave's part visible and frees slot j & 1.
  if (since_epi == 0) wait_vm<epilogue_stores<MODE>()>();
  else wait_vm<0>();
  barrier();
  const uint32_t sn = ((j + 1) & 1) * STAGE;
  phase<MODE, ACT, true, 0, M>(acc, a1, b1, a0, b0, sub_addr<MODE, true, 0>(fa, sn), sub_addr<MODE, false, 0>(fb.b, sn), lds + sb, pr.ss, pr.lo, wave, lane);
  advance<MODE>(pr, p, geo, dl, nbx, wave, lane);
  if constexpr (ACT) frag_wait<MODE>(a0, b0);
}

// One output tile: its K steps j, j+1, ... and its epilogue.  M blocks per wave row (MI, or MIX
// for a tile of more than 256 rows).  ACT: on entry a0/b0 hold substep 0 of stage j.  !ACT (the
// idle row half of a 128-row tile): the wave issues its share of the load stream and the
// epilogue's memory instructions only, and reads no fragments.  pd_on: pd holds the previous
// tile's deferred stores.
template <int MODE, bool ACT, int M>
__device__ __forceinline__ void run_tile(const GemmArgs& p, const Tile& ct, const FragBases& fb, FragA<MODE>& a0,
                                         FragB<MODE>& b0, FragA<MODE>& a1, FragB<MODE>& b1, int& j,
                                         int& since_epi, Producer& pr, const SegGeo (&geo)[2], const Deal& dl,
                                         int nbx, int wm, int wn, int wave, int lane, char* lds, float* partial,
                                         PendingOf<MODE>& pd, bool& pd_on) {
  const uint32_t fa = M == MIX ? fb.ax : fb.a;
  f32x16_t acc[M][NI];
#pragma unroll
  for (int i = 0; i < M; ++i)
#pragma unroll
    for (int jj = 0; jj < NI; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.0f;
  int kc = 0;
  if constexpr (Traits<MODE>::raggedK && M == MI && ACT) {
    if (pd_on) {
      kstep<MODE, ACT, M, true>(p, acc, fa, fb, a0, b0, a1, b1, j, since_epi, pr, geo, dl, nbx, wave, lane, lds, pd);
      pd_on = false;
      ++kc, ++j, ++since_epi;
    }
  }
  for (; kc < ct.nk; ++kc, ++j) {
    kstep<MODE, ACT, M, false>(p, acc, fa, fb, a0, b0, a1, b1, j, since_epi, pr, geo, dl, nbx, wave, lane, lds, pd);
    ++since_epi;
  }
  epilogue_tile<MODE, M>(seg_args(p, ct.seg), acc, ct, wm, wn, lane, partial, pd, pd_on);
  since_epi = 0;
}

template <int MODE>
__global__ __launch_bounds__(NTH, 1) void grouped_gemm_pipe(GemmArgs p, int ksplit, float* partial) {
  typedef Traits<MODE> TR;
  constexpr int STAGE = stage_bytes<MODE>();
  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE];
  __shared__ int pref_s[PMAXG + 1];
  __shared__ int offs_s[PMAXG + 1];
  __shared__ int pref1_s[PMAXG1 + 1];
  __shared__ int offs1_s[PMAXG1 + 1];
  __shared__ int scan_scratch[NTH + 1];

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6), lane = tid & 63;
  // the two waves of a SIMD (w, w + 4) take the two row halves
  const int wm = wave / WGN, wn = wave % WGN;
  const uint32_t lds0 = lds_addr_of(lds);

  const FragBases fb = frag_bases<MODE>(lds0, wm, wn, lane);

  // Per set: clamped group offsets (the clamping of group_rows), tile geometry and, for ragged M,
  // the per-group tile prefix.  Set 1 (if any) follows set 0 in the tile order.
  const bool two = p.nseg == 2;
  for (int g = tid; g <= p.G; g += NTH) offs_s[g] = clampi(p.offsets[g], 0, p.M);
  if (two)
    for (int g = tid; g <= p.s1.G; g += NTH) offs1_s[g] = clampi(p.s1.offsets[g], 0, p.s1.M);
  __syncthreads();
  SegGeo geo[2];
  geo[0].offs = lds_addr_of(offs_s);
  geo[0].pref = lds_addr_of(pref_s);
  geo[1].offs = lds_addr_of(offs1_s);
  geo[1].pref = lds_addr_of(pref1_s);
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const int f = sg ? p.s1.f : p.f, G = sg ? p.s1.G : p.G;
    geo[sg].NT = mode_N(MODE, p.d, f) / BN;
    geo[sg].MT = TR::raggedK ? mode_Mw(MODE, p.d, f) / BM : 0;
    geo[sg].ks = sg ? max(1, p.s1.ksplit) : ksplit;
    geo[sg].band = 4;
    // The second set's groups (the shared expert: T rows in one group) take 256-row tiles where
    // its tiles are the longer ones (its K is its own d_ff, larger than the routed experts') and
    // 256-row tiles deal them to each XCD's workgroups in whole rounds while 320-row ones do not:
    // it is dealt first, and a partial round of its long tiles leaves some workgroups carrying one
    // more than the others for the whole stage.
    geo[sg].rows256 = false;
    if constexpr (has_x<MODE>() && MODE != GEMM_DOWN_BWD) {
      if (sg == 1 && two && mode_K(MODE, p.d, p.s1.f) > mode_K(MODE, p.d, p.f)) {
        int n256 = 0, nx = 0;
        for (int g = 0; g < G; ++g) {
          const int lo = offs1_s[g], R = max(lo, offs1_s[g + 1]) - lo;
          n256 += group_tiles<MODE>(R, true);
          nx += group_tiles<MODE>(R, false);
        }
        const int round = 8 * (int)(gridDim.x >> 3);
        geo[sg].rows256 = (n256 * geo[sg].NT) % round == 0 && (nx * geo[sg].NT) % round != 0;
      }
    }
    geo[sg].fd_mn = make_fastdiv((uint32_t)max(1, geo[sg].MT * geo[sg].NT));
    geo[sg].fd_mb = make_fastdiv((uint32_t)max(1, geo[sg].MT * WG_NB));
    geo[sg].fd_nt = make_fastdiv((uint32_t)max(1, geo[sg].NT));
    geo[sg].fd_ks = make_fastdiv((uint32_t)max(1, geo[sg].ks));
    if (sg == 1 && !two) {
      geo[sg].total = 0;
    } else if constexpr (!TR::raggedK) {
      int* offs_tab = sg ? offs1_s : offs_s;
      int* pref_tab = sg ? pref1_s : pref_s;
      tile_prefix_lds<MODE>(G, offs_tab, pref_tab, scan_scratch, geo[sg].rows256);
      geo[sg].total = pref_tab[G] * geo[sg].NT;
    } else {
      geo[sg].total = G * geo[sg].ks * geo[sg].MT * geo[sg].NT;
    }
  }
  // Tiles are dealt so each XCD (workgroup b runs on XCD b % 8) walks one contiguous run of the
  // tile order.  Two sets: each XCD gets a run of each set, set 1 first.  The sets' tiles differ in
  // length (the shared expert's K is its own d_ff in the down and gate/up data-gradient products,
  // and its weight-gradient reduction is split into chunks), so one run over both sets would leave
  // the XCDs that draw set 1 with more work; set 1's tiles are the longer ones where they differ.
  //
  // Weight gradients of skewed routing: set 0's tiles differ in cost with their group's rows, and
  // equal tile counts per XCD can leave one XCD with far more K steps than another.  When the
  // costliest XCD of the equal-count cut would carry more than 1.15x the mean, set 0 is cut by
  // cost instead (a cut may then fall inside a group, whose operand panels two XCDs then read;
  // with balanced routing the equal-count cut is kept for that reason).
  const int xcd = blockIdx.x & 7;
  const int nbx = gridDim.x >> 3;
  const int total0 = geo[0].total, per0 = (total0 + 7) >> 3;
  bool by_cost = false;
  if constexpr (TR::raggedK) {
    const int tpg = geo[0].ks * geo[0].MT * geo[0].NT;
    if (total0 > 0) {
      cost_prefix_lds(p.G, geo[0].ks, tpg, offs_s, pref_s, scan_scratch);
      int worst = 0;
      for (int x = 0; x < 8; ++x)
        worst = max(worst, cost_before(pref_s, offs_s, tpg, geo[0].ks, min(total0, (x + 1) * per0)) -
                               cost_before(pref_s, offs_s, tpg, geo[0].ks, min(total0, x * per0)));
      by_cost = (long long)worst * 800 > (long long)pref_s[p.G] * 115;
    }
  }
  auto cut0 = [&](int x) {
    if constexpr (TR::raggedK) {
      if (by_cost) return cost_cut(pref_s, offs_s, p.G, geo[0].ks * geo[0].MT * geo[0].NT, geo[0].ks, x);
    }
    return min(total0, x * per0);
  };
  Deal dl;
  dl.total0 = total0;
  dl.lo0 = cut0(xcd);
  if (two) {
    const int per1 = (geo[1].total + 7) >> 3;
    dl.lo1 = min(geo[1].total, xcd * per1);
    dl.n1 = min(geo[1].total, (xcd + 1) * per1) - dl.lo1;
  } else {
    dl.lo1 = 0;
    dl.n1 = 0;
  }
  dl.n = dl.n1 + cut0(xcd + 1) - dl.lo0;
  dl.q = dl.n;
  if constexpr (!TR::raggedK) {
    const int rem = dl.n % nbx;
    if (rem > 0 && 2 * rem <= nbx) {
      dl.q = dl.n - rem;
      dl.n += rem;
    }
  }

  // Consumer: the tile being multiplied (the first one with work; empty ones get zeros).
  int ic = blockIdx.x >> 3;
  Tile ct;
  for (;; ic += nbx) {
    if (ic >= dl.n) return;
    ct = deal_tile<MODE>(p, geo, dl, ic);
    if (ct.nk > 0) break;
    if constexpr (TR::raggedK) zero_tile<MODE>(seg_args(p, ct.seg), ct, wm, wn, lane, partial);
  }

  // Prologue: stages 0 and 1 into slots 0 and 1, wait for stage 0.
  Producer pr;
  pr.t = ct;
  pr.i = ic;
  pr.k = 0;
  set_offsets<MODE>(pr, p, wave, lane);
#pragma unroll 1
  for (int s = 0; s < NSTAGE; ++s) {
    issue_all<MODE, 0>(seg_args(p, pr.t.seg), lds + s * STAGE, pr.t, pr.t.k_begin + pr.k * BKS, wave, lane);
    advance<MODE>(pr, p, geo, dl, nbx, wave, lane);
  }
  // stage 0 landed: at most stage 1's loads outstanding (one fewer per skipped A load)
  wait_vm<(NSTAGE - 1) * (lpw<MODE>() - lpa_skip<MODE>())>();
  barrier();
  FragA<MODE> a0, a1;
  FragB<MODE> b0, b1;
  int j = 0, since_epi = 3;
  PendingOf<MODE> pd;
  bool pd_on = false;
  for (;;) {
    // Substep 0 of the tile's first stage is read here rather than kept in registers through the
    // previous epilogue (its slot is refilled only after this wave's next barrier, and the previous
    // tile may have had the other row layout).
    const uint32_t sb = (j & 1) * STAGE;
    if (!TR::raggedK && ct.half && wm == 1) {
      run_tile<MODE, false, MI>(p, ct, fb, a0, b0, a1, b1, j, since_epi, pr, geo, dl, nbx, wm, wn, wave, lane, lds,
                                partial, pd, pd_on);
    } else if (has_x<MODE>() && ct.x) {
      read_all<MODE, 0, mi_max<MODE>()>(a0, b0, sub_addr<MODE, true, 0>(fb.ax, sb), sub_addr<MODE, false, 0>(fb.b, sb));
      frag_wait<MODE>(a0, b0);
      run_tile<MODE, true, mi_max<MODE>()>(p, ct, fb, a0, b0, a1, b1, j, since_epi, pr, geo, dl, nbx, wm, wn, wave,
                                           lane, lds, partial, pd, pd_on);
    } else {
      read_all<MODE, 0, MI>(a0, b0, sub_addr<MODE, true, 0>(fb.a, sb), sub_addr<MODE, false, 0>(fb.b, sb));
      frag_wait<MODE>(a0, b0);
      run_tile<MODE, true, MI>(p, ct, fb, a0, b0, a1, b1, j, since_epi, pr, geo, dl, nbx, wm, wn, wave, lane, lds,
                               partial, pd, pd_on);
    }
    bool more = false;
    for (ic += nbx; ic < dl.n; ic += nbx) {
      ct = deal_tile<MODE>(p, geo, dl, ic);
      if (ct.nk > 0) {
        more = true;
        break;
      }
      if constexpr (TR::raggedK) zero_tile<MODE>(seg_args(p, ct.seg), ct, wm, wn, lane, partial);
    }
    if (!more) break;
  }
  if constexpr (Traits<MODE>::raggedK) {
    if (pd_on) flush_pending<0>(pd);   // the last tile's deferred stores
  }
  // No direct-to-LDS load may still be writing when the workgroup's LDS is released.
  wait_vm<0>();
}

// Upper bound of the tiles of one set (ragged M: every group may add a partial tile).
template <int MODE>
long long set_tiles(int G, int M, int d, int f, int ksplit) {
  const long long NT = mode_N(MODE, d, f) / BN;
  if constexpr (!Traits<MODE>::raggedK) return M > 0 ? ((long long)ceil_div(M, BM) + G) * NT : 0;
  else return (long long)G * (mode_Mw(MODE, d, f) / BM) * NT * ksplit;
}

template <int MODE>
hipError_t launch_pipe(const GemmArgs& p, int ksplit, float* partial, hipStream_t s, int num_cus) {
  long long tiles = set_tiles<MODE>(p.G, p.M, p.d, p.f, ksplit);
  if (p.nseg == 2) tiles += set_tiles<MODE>(p.s1.G, p.s1.M, p.d, p.s1.f, std::max(1, p.s1.ksplit));
  long long grid = std::min<long long>(tiles, (long long)num_cus);
  grid = (grid + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_pipe<MODE>, dim3((unsigned)grid), dim3(NTH), 0, s, p, ksplit, partial);
  return hipGetLastError();
}

}  // namespace

static bool pipe_supports_set(int mode, int G, int d, int f, int gmax) {
  if (G > gmax) return false;
  if (gemm::mode_N(mode, d, f) % BN) return false;
  if (mode == GEMM_DOWN_WGRAD || mode == GEMM_UP_WGRAD) return gemm::mode_Mw(mode, d, f) % BM == 0;
  return gemm::mode_K(mode, d, f) % BKS == 0;
}

bool pipe_supports(int mode, const GemmArgs& p) {
  if (!pipe_supports_set(mode, p.G, p.d, p.f, PMAXG)) return false;
  return p.nseg != 2 || pipe_supports_set(mode, p.s1.G, p.d, p.s1.f, PMAXG1);
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
