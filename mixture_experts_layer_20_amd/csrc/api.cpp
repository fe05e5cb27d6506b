// libmoe C-ABI: argument validation, workspace carving and kernel launches.
// Every entry point checks its arguments on the host before enqueuing anything, never
// synchronises, never allocates, and reports errors through status codes.
#include "libmoe.h"

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "common.h"
#include "mxfp8.h"

namespace {

thread_local std::string g_err;

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status_t hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxInt = 0x7fffffff;

#define CHECK(cond, st, ...)                 \
  do {                                       \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

// Device tensors, index arrays and workspaces are accessed with vector loads and stores of up to
// 16 bytes (the GEMMs also with 16-byte direct-to-LDS loads) at offsets from each base pointer
// that are multiples of the access size, so every device pointer must be 16-byte aligned (hipMalloc
// and PyTorch allocations are 256-byte aligned).  NULL passes.
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  return true;
}

#define CHECK_ALIGN16(...)                                                   \
  CHECK(aligned16({__VA_ARGS__}), MOE_ERR_INVALID_VALUE,                    \
        "device pointers must be 16-byte aligned (" #__VA_ARGS__ ")")

moe_status_t check_dtype(moe_dtype_t dt) {
  CHECK(dt == MOE_F32 || dt == MOE_BF16, MOE_ERR_INVALID_VALUE, "dt must be MOE_F32 or MOE_BF16");
  return MOE_OK;
}

moe_status_t check_tokens(int64_t T, int64_t d, int32_t E, int32_t k) {
  CHECK(T >= 0, MOE_ERR_INVALID_VALUE, "T must be >= 0 (got %lld)", (long long)T);
  CHECK(d > 0, MOE_ERR_INVALID_VALUE, "d must be > 0 (got %lld)", (long long)d);
  CHECK(E > 0, MOE_ERR_INVALID_VALUE, "E must be > 0 (got %d)", E);
  CHECK(k > 0 && k <= E, MOE_ERR_INVALID_VALUE, "k must be in [1, E] (got k=%d, E=%d)", k, E);
  CHECK(E <= 256, MOE_ERR_UNSUPPORTED, "E > 256 is not supported (got %d)", E);
  CHECK(k <= 8, MOE_ERR_UNSUPPORTED, "k > 8 is not supported (got %d)", k);
  CHECK(d <= kMaxInt && T <= kMaxInt, MOE_ERR_UNSUPPORTED, "T and d must fit in int32");
  CHECK(T * k <= kMaxInt - 8, MOE_ERR_UNSUPPORTED, "T*k must be < 2^31");
  CHECK(T * (int64_t)E <= kMaxInt, MOE_ERR_UNSUPPORTED, "T*E must be < 2^31");
  return MOE_OK;
}

moe_status_t check_mlp(int32_t G, int64_t M, int64_t d, int64_t f, moe_dtype_t dt) {
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  CHECK(G > 0, MOE_ERR_INVALID_VALUE, "G must be > 0 (got %d)", G);
  CHECK(M >= 0, MOE_ERR_INVALID_VALUE, "M must be >= 0 (got %lld)", (long long)M);
  CHECK(d > 0 && f > 0, MOE_ERR_INVALID_VALUE, "d and f must be > 0");
  CHECK(d % 128 == 0 && f % 128 == 0, MOE_ERR_UNSUPPORTED,
        "d and f must be multiples of 128 (got d=%lld, f=%lld)", (long long)d, (long long)f);
  CHECK(M <= kMaxInt / 2 && d <= 65536 && f <= 65536 && G <= 1024, MOE_ERR_UNSUPPORTED,
        "sizes out of the supported range");
  CHECK(((M + 127) / 128 + G) * (2 * f / 64 + d / 64) < kMaxInt, MOE_ERR_UNSUPPORTED, "grid too large");
  return MOE_OK;
}

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }
inline size_t esize(moe_dtype_t dt) { return dt == MOE_BF16 ? 2 : 4; }
inline hipStream_t S(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

moe_status_t run_gemm(int mode, const moe::GemmArgs& a, moe_dtype_t dt, moe_stream_t s,
                      const char* what) {
  CHECK_ALIGN16(a.a, a.b0, a.b1, a.aux0, a.aux1, a.out0, a.out1, a.out2, a.offsets, a.tile_prefix);
  if (a.nseg == 2) CHECK_ALIGN16(a.s1.a, a.s1.b0, a.s1.b1, a.s1.aux0, a.s1.aux1, a.s1.out0, a.s1.out1, a.s1.out2,
                                 a.s1.offsets);
  return hip_check(moe::launch_grouped_gemm(mode, a, dt == MOE_BF16, S(s)), what);
}

moe::GemmArgs base_args(const int32_t* offsets, int32_t G, int64_t M, int64_t d, int64_t f, void* ws,
                        size_t ws_bytes) {
  moe::GemmArgs a{};
  a.offsets = offsets;
  a.tile_prefix = reinterpret_cast<int32_t*>(ws);
  a.ws_bytes = ws_bytes;
  a.G = G;
  a.M = (int)M;
  a.d = (int)d;
  a.f = (int)f;
  return a;
}

// ---------------------------------------------------------------------------------------------
// Scratch for the entry point that allocates nothing (moe_permute_noalloc): a file-scope device
// array that each GPU holds from the library's load until the process ends.  In host code the
// array's name only stands in for the symbol; its device address, different on every GPU, comes
// from hipGetSymbolAddress, taken once per device with that device current, and only that address
// is ever handed to a kernel.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that device).
moe_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  CHECK(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "device %d is beyond the %d devices supported", dev,
        kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_VALUE: return "MOE_ERR_INVALID_VALUE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "libmoe 0.1 gfx950"; }

// ---------------------------------------------------------------------------------------------

moe_status_t moe_route(const void* x, const void* w_router, const float* bias, float* logits,
                       int64_t T, int64_t d, int32_t E, int32_t k, int32_t renormalize,
                       moe_dtype_t dt, int32_t* topk_idx, float* topk_gate, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, d, E, k)) != MOE_OK) return st;
  CHECK(renormalize == 0 || renormalize == 1, MOE_ERR_INVALID_VALUE, "renormalize must be 0 or 1");
  CHECK(!w_router || x, MOE_ERR_INVALID_VALUE, "x is NULL with a learned router");
  CHECK(w_router || !bias, MOE_ERR_INVALID_VALUE, "bias given without a learned router");
  if (T == 0) return MOE_OK;
  CHECK(logits && topk_idx && topk_gate, MOE_ERR_INVALID_VALUE, "logits/topk_idx/topk_gate is NULL");
  CHECK_ALIGN16(x, w_router, bias, logits, topk_idx, topk_gate);
  if (w_router) {
    st = hip_check(moe::launch_router_logits(x, w_router, bias, logits, (int)T, (int)d, E,
                                             dt == MOE_BF16, S(stream)),
                   "router logits");
    if (st != MOE_OK) return st;
  }
  return hip_check(moe::launch_topk_gate(logits, (int)T, E, k, renormalize, topk_idx, topk_gate, S(stream)),
                   "top-k");
}

size_t moe_permute_workspace_size(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E <= 0 || k <= 0) return 0;
  return moe::permute_ws_bytes(T, E, k);
}

moe_status_t moe_permute(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E,
                         int32_t k, moe_dtype_t dt, int32_t* counts, int32_t* offsets,
                         int32_t* dest_pos, int32_t* src_row, void* x_perm, void* ws,
                         size_t ws_bytes, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, d, E, k)) != MOE_OK) return st;
  CHECK(counts && offsets, MOE_ERR_INVALID_VALUE, "counts/offsets is NULL");
  CHECK(T == 0 || (topk_idx && dest_pos && src_row), MOE_ERR_INVALID_VALUE,
        "topk_idx/dest_pos/src_row is NULL");
  CHECK(!x_perm || x || T == 0, MOE_ERR_INVALID_VALUE, "x is NULL while x_perm is requested");
  CHECK(!x_perm || d % 8 == 0, MOE_ERR_UNSUPPORTED, "the row gather needs d %% 8 == 0 (got %lld)",
        (long long)d);
  const size_t need = moe::permute_ws_bytes(T, E, k);
  CHECK(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
        ws ? ws_bytes : (size_t)0);
  CHECK_ALIGN16(x, topk_idx, counts, offsets, dest_pos, src_row, x_perm, ws);
  return hip_check(moe::launch_permute(x, topk_idx, (int)T, (int)d, E, k, dt == MOE_BF16, counts,
                                       offsets, dest_pos, src_row, x_perm, ws, S(stream)),
                   "permute");
}

size_t moe_permute_noalloc_max_scratch(void) { return kScratchBytes; }

moe_status_t moe_permute_noalloc(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E, int32_t k,
                                 moe_dtype_t dt, int32_t* counts, int32_t* offsets, int32_t* dest_pos,
                                 int32_t* src_row, void* x_perm, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, d, E, k)) != MOE_OK) return st;
  CHECK(counts && offsets, MOE_ERR_INVALID_VALUE, "counts/offsets is NULL");
  CHECK(T == 0 || (topk_idx && dest_pos && src_row), MOE_ERR_INVALID_VALUE,
        "topk_idx/dest_pos/src_row is NULL");
  CHECK(!x_perm || x || T == 0, MOE_ERR_INVALID_VALUE, "x is NULL while x_perm is requested");
  CHECK(!x_perm || d % 8 == 0, MOE_ERR_UNSUPPORTED, "the row gather needs d %% 8 == 0 (got %lld)",
        (long long)d);
  const size_t need = moe::permute_ws_bytes(T, E, k);
  CHECK(need <= kScratchBytes, MOE_ERR_UNSUPPORTED,
        "T*k = %lld with E = %d needs %zu bytes of scratch; moe_permute_noalloc holds %zu (use moe_permute)",
        (long long)(T * k), E, need, kScratchBytes);
  CHECK_ALIGN16(x, topk_idx, counts, offsets, dest_pos, src_row, x_perm);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MOE_OK) return st;
  // Every scratch element the kernels read they first write in the same call (chunk counts,
  // chunk bases, local ranks), so nothing needs clearing.
  return hip_check(moe::launch_permute(x, topk_idx, (int)T, (int)d, E, k, dt == MOE_BF16, counts,
                                       offsets, dest_pos, src_row, x_perm, ws, S(stream)),
                   "permute (no allocation)");
}

// ---------------------------------------------------------------------------------------------

size_t moe_grouped_mlp_fwd_workspace_size(int64_t M, int32_t G, int64_t d, int64_t f) {
  (void)M; (void)d; (void)f;
  if (G <= 0) return 0;
  return moe::gemm_ws_bytes(G);
}

size_t moe_grouped_mlp_bwd_workspace_size(int64_t M, int32_t G, int64_t d, int64_t f) {
  if (G <= 0 || M < 0 || f <= 0 || d <= 0) return 0;
  // Tile prefix and split-K partials first, dAB (sized for fp32 so one workspace serves both
  // element types) at the end.
  return moe::gemm_ws_bytes(G) + align256(moe::gemm_partial_bytes(G, M, (int)d, (int)f)) +
         align256((size_t)M * 2 * f * 4);
}

#define MLP_COMMON_CHECKS(need)                                                              \
  g_err.clear();                                                                             \
  moe_status_t st = check_mlp(G, M, d, f, dt);                                               \
  if (st != MOE_OK) return st;                                                               \
  CHECK(offsets, MOE_ERR_INVALID_VALUE, "offsets is NULL");                                  \
  CHECK(ws && ws_bytes >= (need), MOE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", \
        (size_t)(need), ws ? ws_bytes : (size_t)0);

moe_status_t moe_expert_gate_up_fwd(const void* x_in, const int32_t* offsets, int32_t G,
                                    int64_t M, int64_t d, int64_t f, const void* w1,
                                    const void* w3, moe_dtype_t dt, void* a_stash, void* b_stash,
                                    void* h, void* ws, size_t ws_bytes, moe_stream_t stream) {
  MLP_COMMON_CHECKS(moe::gemm_ws_bytes(G));
  CHECK(w1 && w3 && (M == 0 || (x_in && h)), MOE_ERR_INVALID_VALUE, "x_in/w1/w3/h is NULL");
  CHECK((a_stash == nullptr) == (b_stash == nullptr), MOE_ERR_INVALID_VALUE,
        "a_stash and b_stash must both be given or both be NULL");
  moe::GemmArgs a = base_args(offsets, G, M, d, f, ws, ws_bytes);
  a.a = x_in; a.b0 = w1; a.b1 = w3; a.out0 = a_stash; a.out1 = b_stash; a.out2 = h;
  return run_gemm(moe::GEMM_UP_FWD, a, dt, stream, "gate/up GEMM");
}

moe_status_t moe_expert_down_fwd(const void* h, const int32_t* offsets, int32_t G, int64_t M,
                                 int64_t d, int64_t f, const void* w2, moe_dtype_t dt, void* y,
                                 void* ws, size_t ws_bytes, moe_stream_t stream) {
  MLP_COMMON_CHECKS(moe::gemm_ws_bytes(G));
  CHECK(w2 && (M == 0 || (h && y)), MOE_ERR_INVALID_VALUE, "h/w2/y is NULL");
  moe::GemmArgs a = base_args(offsets, G, M, d, f, ws, ws_bytes);
  a.a = h; a.b0 = w2; a.out0 = y;
  return run_gemm(moe::GEMM_DOWN_FWD, a, dt, stream, "down GEMM");
}

moe_status_t moe_expert_down_bwd(const void* dy, const void* a_stash, const void* b_stash,
                                 const int32_t* offsets, int32_t G, int64_t M, int64_t d,
                                 int64_t f, const void* w2, moe_dtype_t dt, void* dab, void* ws,
                                 size_t ws_bytes, moe_stream_t stream) {
  MLP_COMMON_CHECKS(moe::gemm_ws_bytes(G));
  CHECK(w2 && (M == 0 || (dy && a_stash && b_stash && dab)), MOE_ERR_INVALID_VALUE,
        "dy/a/b/w2/dab is NULL");
  moe::GemmArgs a = base_args(offsets, G, M, d, f, ws, ws_bytes);
  a.a = dy; a.b0 = w2; a.aux0 = a_stash; a.aux1 = b_stash; a.out0 = dab;
  return run_gemm(moe::GEMM_DOWN_BWD, a, dt, stream, "down dgrad GEMM");
}

moe_status_t moe_expert_down_wgrad(const void* dy, const void* h, const int32_t* offsets,
                                   int32_t G, int64_t M, int64_t d, int64_t f, moe_dtype_t dt,
                                   void* dw2, void* ws, size_t ws_bytes, moe_stream_t stream) {
  MLP_COMMON_CHECKS(moe::gemm_ws_bytes(G));
  CHECK(dw2 && (M == 0 || (dy && h)), MOE_ERR_INVALID_VALUE, "dy/h/dw2 is NULL");
  moe::GemmArgs a = base_args(offsets, G, M, d, f, ws, ws_bytes);
  a.a = dy; a.b0 = h; a.out0 = dw2;
  return run_gemm(moe::GEMM_DOWN_WGRAD, a, dt, stream, "down wgrad GEMM");
}

moe_status_t moe_expert_gate_up_dgrad(const void* dab, const int32_t* offsets, int32_t G,
                                      int64_t M, int64_t d, int64_t f, const void* w1,
                                      const void* w3, moe_dtype_t dt, void* dx_in, void* ws,
                                      size_t ws_bytes, moe_stream_t stream) {
  MLP_COMMON_CHECKS(moe::gemm_ws_bytes(G));
  CHECK(w1 && w3 && (M == 0 || (dab && dx_in)), MOE_ERR_INVALID_VALUE, "dab/w1/w3/dx_in is NULL");
  moe::GemmArgs a = base_args(offsets, G, M, d, f, ws, ws_bytes);
  a.a = dab; a.b0 = w1; a.b1 = w3; a.out0 = dx_in;
  return run_gemm(moe::GEMM_UP_DGRAD, a, dt, stream, "gate/up dgrad GEMM");
}

moe_status_t moe_expert_gate_up_wgrad(const void* dab, const void* x_in, const int32_t* offsets,
                                      int32_t G, int64_t M, int64_t d, int64_t f, moe_dtype_t dt,
                                      void* dw1, void* dw3, void* ws, size_t ws_bytes,
                                      moe_stream_t stream) {
  MLP_COMMON_CHECKS(moe::gemm_ws_bytes(G));
  CHECK(dw1 && dw3 && (M == 0 || (dab && x_in)), MOE_ERR_INVALID_VALUE, "dab/x_in/dw1/dw3 is NULL");
  moe::GemmArgs a = base_args(offsets, G, M, d, f, ws, ws_bytes);
  a.a = dab; a.b0 = x_in; a.out0 = dw1; a.out1 = dw3;
  return run_gemm(moe::GEMM_UP_WGRAD, a, dt, stream, "gate/up wgrad GEMM");
}

size_t moe_expert_stage_workspace_size(const moe_expert_set_t* sets, int32_t nsets, int64_t d) {
  if (!sets || nsets < 1 || nsets > 2 || d <= 0) return 0;
  size_t need = 0;
  for (int i = 0; i < nsets; ++i) {
    const moe_expert_set_t& e = sets[i];
    if (e.G <= 0 || e.M < 0 || e.f <= 0) return 0;
    need = std::max(need, moe::gemm_ws_bytes(e.G) + align256(moe::gemm_partial_bytes(e.G, e.M, (int)d, (int)e.f)));
  }
  if (nsets == 2)
    need = std::max(need, moe::gemm_ws_bytes(sets[0].G) +
                              align256(moe::gemm_sets_partial_bytes(sets[0].G, sets[0].M, sets[1].G, sets[1].M,
                                                                    (int)d, (int)sets[1].f)));
  return need;
}

namespace {

// The GEMM operands of one expert set for a stage, or an error when a member the stage needs is
// missing.
moe_status_t stage_operands(moe_stage_t stage, const moe_expert_set_t& e, moe::GemmArgs& a) {
  const bool rows = e.M > 0;
  switch (stage) {
    case MOE_STAGE_GATE_UP_FWD:
      CHECK(e.w1 && e.w3 && (!rows || (e.x && e.h)), MOE_ERR_INVALID_VALUE, "x/w1/w3/h is NULL");
      CHECK((e.a == nullptr) == (e.b == nullptr), MOE_ERR_INVALID_VALUE,
            "a and b must both be given or both be NULL");
      a.a = e.x; a.b0 = e.w1; a.b1 = e.w3; a.out0 = e.a; a.out1 = e.b; a.out2 = e.h;
      return MOE_OK;
    case MOE_STAGE_DOWN_FWD:
      CHECK(e.w2 && (!rows || (e.h && e.y)), MOE_ERR_INVALID_VALUE, "h/w2/y is NULL");
      a.a = e.h; a.b0 = e.w2; a.out0 = e.y;
      return MOE_OK;
    case MOE_STAGE_DOWN_BWD:
      CHECK(e.w2 && (!rows || (e.dy && e.a && e.b && e.dab)), MOE_ERR_INVALID_VALUE, "dy/a/b/w2/dab is NULL");
      a.a = e.dy; a.b0 = e.w2; a.aux0 = e.a; a.aux1 = e.b; a.out0 = e.dab;
      return MOE_OK;
    case MOE_STAGE_GATE_UP_DGRAD:
      CHECK(e.w1 && e.w3 && (!rows || (e.dab && e.dx)), MOE_ERR_INVALID_VALUE, "dab/w1/w3/dx is NULL");
      a.a = e.dab; a.b0 = e.w1; a.b1 = e.w3; a.out0 = e.dx;
      return MOE_OK;
    case MOE_STAGE_DOWN_WGRAD:
      CHECK(e.dw2 && (!rows || (e.dy && e.h)), MOE_ERR_INVALID_VALUE, "dy/h/dw2 is NULL");
      a.a = e.dy; a.b0 = e.h; a.out0 = e.dw2;
      return MOE_OK;
    case MOE_STAGE_GATE_UP_WGRAD:
      CHECK(e.dw1 && e.dw3 && (!rows || (e.dab && e.x)), MOE_ERR_INVALID_VALUE, "dab/x/dw1/dw3 is NULL");
      a.a = e.dab; a.b0 = e.x; a.out0 = e.dw1; a.out1 = e.dw3;
      return MOE_OK;
  }
  return fail(MOE_ERR_INVALID_VALUE, "unknown stage %d", (int)stage);
}

}  // namespace

moe_status_t moe_expert_stage(moe_stage_t stage, const moe_expert_set_t* sets, int32_t nsets, int64_t d,
                              moe_dtype_t dt, void* ws, size_t ws_bytes, moe_stream_t stream) {
  g_err.clear();
  CHECK(sets && (nsets == 1 || nsets == 2), MOE_ERR_INVALID_VALUE, "nsets must be 1 or 2 (got %d)", (int)nsets);
  CHECK((int)stage >= 0 && (int)stage <= 5, MOE_ERR_INVALID_VALUE, "unknown stage %d", (int)stage);
  size_t need = 0;
  moe::GemmArgs a{};
  for (int i = 0; i < nsets; ++i) {
    const moe_expert_set_t& e = sets[i];
    moe_status_t st = check_mlp(e.G, e.M, d, e.f, dt);
    if (st != MOE_OK) return st;
    CHECK(e.offsets, MOE_ERR_INVALID_VALUE, "offsets of set %d is NULL", i);
    need = std::max(need, moe::gemm_ws_bytes(e.G));
    moe::GemmArgs s = base_args(e.offsets, e.G, e.M, d, e.f, ws, ws_bytes);
    if ((st = stage_operands(stage, e, s)) != MOE_OK) return st;
    if (i == 0) {
      a = s;
    } else {
      a.nseg = 2;
      a.s1 = moe::GemmSeg{s.a, s.b0, s.b1, s.aux0, s.aux1, s.out0, s.out1, s.out2, s.offsets, s.G, s.M, s.f};
    }
  }
  CHECK(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
        ws ? ws_bytes : (size_t)0);
  static const char* names[6] = {"gate/up GEMM", "down GEMM", "down dgrad GEMM", "gate/up dgrad GEMM",
                                 "down wgrad GEMM", "gate/up wgrad GEMM"};
  return run_gemm((int)stage, a, dt, stream, names[(int)stage]);
}

moe_status_t moe_grouped_mlp_fwd(const void* x_in, const int32_t* offsets, int32_t G, int64_t M,
                                 int64_t d, int64_t f, const void* w1, const void* w3,
                                 const void* w2, moe_dtype_t dt, void* a_stash, void* b_stash,
                                 void* h, void* y, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = moe_expert_gate_up_fwd(x_in, offsets, G, M, d, f, w1, w3, dt, a_stash, b_stash,
                                           h, ws, ws_bytes, stream);
  if (st != MOE_OK) return st;
  return moe_expert_down_fwd(h, offsets, G, M, d, f, w2, dt, y, ws, ws_bytes, stream);
}

moe_status_t moe_grouped_mlp_bwd(const void* dy, const void* x_in, const void* a, const void* b,
                                 const void* h, const int32_t* offsets, int32_t G, int64_t M,
                                 int64_t d, int64_t f, const void* w1, const void* w3,
                                 const void* w2, moe_dtype_t dt, void* dx_in, void* dw1, void* dw3,
                                 void* dw2, void* ws, size_t ws_bytes, moe_stream_t stream) {
  MLP_COMMON_CHECKS(moe_grouped_mlp_bwd_workspace_size(M, G, d, f));
  CHECK(w1 && w3 && w2 && dw1 && dw3 && dw2, MOE_ERR_INVALID_VALUE, "weight or gradient pointer is NULL");
  CHECK(M == 0 || (dy && x_in && a && b && h && dx_in), MOE_ERR_INVALID_VALUE,
        "activation pointer is NULL");
  const size_t dab_bytes = align256((size_t)M * 2 * f * 4);
  const size_t gws = moe_grouped_mlp_bwd_workspace_size(M, G, d, f) - dab_bytes;
  void* dab = reinterpret_cast<char*>(ws) + gws;
  if ((st = moe_expert_down_bwd(dy, a, b, offsets, G, M, d, f, w2, dt, dab, ws, gws, stream)) != MOE_OK)
    return st;
  if ((st = moe_expert_down_wgrad(dy, h, offsets, G, M, d, f, dt, dw2, ws, gws, stream)) != MOE_OK)
    return st;
  if ((st = moe_expert_gate_up_dgrad(dab, offsets, G, M, d, f, w1, w3, dt, dx_in, ws, gws, stream)) != MOE_OK)
    return st;
  return moe_expert_gate_up_wgrad(dab, x_in, offsets, G, M, d, f, dt, dw1, dw3, ws, gws, stream);
}

// ---------------------------------------------------------------------------------------------

moe_status_t moe_combine(const void* y_perm, const float* topk_gate, const int32_t* dest_pos,
                         const void* shared_out, int64_t T, int64_t d, int32_t k, moe_dtype_t dt,
                         void* out, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, d, k, k)) != MOE_OK) return st;
  CHECK(d % 8 == 0, MOE_ERR_UNSUPPORTED, "d must be a multiple of 8 (got %lld)", (long long)d);
  if (T == 0) return MOE_OK;
  CHECK(y_perm && topk_gate && dest_pos && out, MOE_ERR_INVALID_VALUE, "y_perm/topk_gate/dest_pos/out is NULL");
  CHECK_ALIGN16(y_perm, topk_gate, dest_pos, shared_out, out);
  return hip_check(moe::launch_combine(y_perm, topk_gate, dest_pos, shared_out, (int)T, (int)d, k,
                                       dt == MOE_BF16, out, S(stream)),
                   "combine");
}

moe_status_t moe_combine_bwd(const void* dout, const void* y_perm, const float* topk_gate,
                             const int32_t* dest_pos, int64_t T, int64_t d, int32_t k,
                             moe_dtype_t dt, void* dy_perm, float* dgate, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, d, k, k)) != MOE_OK) return st;
  CHECK(d % 8 == 0, MOE_ERR_UNSUPPORTED, "d must be a multiple of 8 (got %lld)", (long long)d);
  if (T == 0) return MOE_OK;
  CHECK(dout && topk_gate && dest_pos && dy_perm, MOE_ERR_INVALID_VALUE, "dout/topk_gate/dest_pos/dy_perm is NULL");
  CHECK(!dgate || y_perm, MOE_ERR_INVALID_VALUE, "y_perm is NULL while dgate is requested");
  CHECK_ALIGN16(dout, y_perm, topk_gate, dest_pos, dy_perm, dgate);
  return hip_check(moe::launch_combine_bwd(dout, y_perm, topk_gate, dest_pos, (int)T, (int)d, k,
                                           dt == MOE_BF16, dy_perm, dgate, S(stream)),
                   "combine backward");
}

moe_status_t moe_permute_bwd(const void* dx_perm, const int32_t* dest_pos, const void* dx_add0,
                             const void* dx_add1, int64_t T, int64_t d, int32_t k,
                             moe_dtype_t dt, void* dx, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, d, k, k)) != MOE_OK) return st;
  CHECK(d % 8 == 0, MOE_ERR_UNSUPPORTED, "d must be a multiple of 8 (got %lld)", (long long)d);
  if (T == 0) return MOE_OK;
  CHECK(dx_perm && dest_pos && dx, MOE_ERR_INVALID_VALUE, "dx_perm/dest_pos/dx is NULL");
  CHECK_ALIGN16(dx_perm, dest_pos, dx_add0, dx_add1, dx);
  return hip_check(moe::launch_permute_bwd(dx_perm, dest_pos, dx_add0, dx_add1, (int)T, (int)d, k,
                                           dt == MOE_BF16, dx, S(stream)),
                   "permute backward");
}

size_t moe_route_bwd_workspace_size(int64_t T, int64_t d, int32_t E, int32_t k) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0) return 0;
  return moe::route_bwd_ws_bytes(T, d, E, k);
}

moe_status_t moe_route_bwd(const float* dgate, const float* topk_gate, const int32_t* topk_idx,
                           const int32_t* offsets, const int32_t* src_row, const void* x,
                           const void* w_router, int64_t T, int64_t d, int32_t E, int32_t k,
                           int32_t renormalize, moe_dtype_t dt, float* dw_router, void* dx_router,
                           void* ws, size_t ws_bytes, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, d, E, k)) != MOE_OK) return st;
  CHECK(renormalize == 0 || renormalize == 1, MOE_ERR_INVALID_VALUE, "renormalize must be 0 or 1");
  CHECK(renormalize == 1, MOE_ERR_UNSUPPORTED, "router backward supports renormalized gates only");
  CHECK(offsets && w_router && dw_router, MOE_ERR_INVALID_VALUE, "offsets/w_router/dw_router is NULL");
  CHECK(T == 0 || (dgate && topk_gate && topk_idx && src_row && x && dx_router), MOE_ERR_INVALID_VALUE,
        "a per-token pointer is NULL");
  const size_t need = moe::route_bwd_ws_bytes(T, d, E, k);
  CHECK(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
        ws ? ws_bytes : (size_t)0);
  CHECK_ALIGN16(dgate, topk_gate, topk_idx, offsets, src_row, x, w_router, dw_router, dx_router, ws);
  return hip_check(moe::launch_route_bwd(dgate, topk_gate, topk_idx, offsets, src_row, x, w_router,
                                         (int)T, (int)d, E, k, dt == MOE_BF16, dw_router, dx_router,
                                         ws, S(stream)),
                   "router backward");
}

size_t moe_router_aux_workspace_size(int64_t T, int32_t E) {
  if (T < 0 || E <= 0) return 0;
  return moe::router_aux_ws_bytes(T, E);
}

moe_status_t moe_router_aux(const float* logits, const int32_t* counts, int64_t T, int32_t E, int32_t k,
                            float weight, float* loss, float* prob_mean, float* load_frac, void* ws,
                            size_t ws_bytes, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_tokens(T, 1, E, k);
  if (st != MOE_OK) return st;
  CHECK(counts && loss && prob_mean && load_frac, MOE_ERR_INVALID_VALUE, "counts/loss/prob_mean/load_frac is NULL");
  CHECK(T == 0 || logits, MOE_ERR_INVALID_VALUE, "logits is NULL");
  const size_t need = moe::router_aux_ws_bytes(T, E);
  CHECK(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
        ws ? ws_bytes : (size_t)0);
  CHECK_ALIGN16(logits, counts, loss, prob_mean, load_frac, ws);
  return hip_check(moe::launch_router_aux(logits, counts, (int)T, E, k, weight, loss, prob_mean, load_frac, ws,
                                          S(stream)),
                   "router statistics");
}

size_t moe_router_aux_bwd_workspace_size(int64_t T, int64_t d, int32_t E) {
  if (T < 0 || d <= 0 || E <= 0) return 0;
  return moe::router_aux_bwd_ws_bytes(T, d, E);
}

moe_status_t moe_router_aux_bwd(const float* logits, const float* load_frac, const void* x, const void* w_router,
                                int64_t T, int64_t d, int32_t E, float weight, moe_dtype_t dt, float* dw_router,
                                void* dx_router, void* ws, size_t ws_bytes, moe_stream_t stream) {
  g_err.clear();
  moe_status_t st = check_dtype(dt);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, d, E, 1)) != MOE_OK) return st;
  CHECK(d % 8 == 0, MOE_ERR_UNSUPPORTED, "d must be a multiple of 8 (got %lld)", (long long)d);
  CHECK(load_frac && w_router && dw_router, MOE_ERR_INVALID_VALUE, "load_frac/w_router/dw_router is NULL");
  CHECK(T == 0 || (logits && x && dx_router), MOE_ERR_INVALID_VALUE, "logits/x/dx_router is NULL");
  const size_t need = moe::router_aux_bwd_ws_bytes(T, d, E);
  CHECK(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
        ws ? ws_bytes : (size_t)0);
  CHECK_ALIGN16(logits, load_frac, x, w_router, dw_router, dx_router, ws);
  return hip_check(moe::launch_router_aux_bwd(logits, load_frac, x, w_router, (int)T, (int)d, E, weight,
                                              dt == MOE_BF16, dw_router, dx_router, ws, S(stream)),
                   "router load-balancing backward");
}

// ---------------------------------------------------------------------------------------------
// MXFP8

moe_status_t moe_mx_quantize_rows(const void* x, int64_t R, int64_t K, int64_t ldx, uint8_t* codes,
                                  uint8_t* scales, moe_stream_t stream) {
  g_err.clear();
  CHECK(R >= 0 && K > 0, MOE_ERR_INVALID_VALUE, "R must be >= 0 and K > 0 (got R=%lld, K=%lld)", (long long)R,
        (long long)K);
  CHECK(K % 32 == 0, MOE_ERR_UNSUPPORTED, "K must be a multiple of 32 (got %lld)", (long long)K);
  CHECK(ldx >= K && ldx % 8 == 0, MOE_ERR_INVALID_VALUE, "ldx must be >= K and a multiple of 8 (got %lld)",
        (long long)ldx);
  CHECK(K <= kMaxInt && R <= kMaxInt, MOE_ERR_UNSUPPORTED, "R and K must fit in int32");
  if (R == 0) return MOE_OK;
  CHECK(x && codes && scales, MOE_ERR_INVALID_VALUE, "x/codes/scales is NULL");
  CHECK_ALIGN16(x, codes, scales);
  return hip_check(moe::launch_mx_quant_rows(x, R, (int)K, ldx, codes, scales, S(stream)), "MXFP8 row quantization");
}

int64_t moe_mx_quantize_cols_ld(int64_t R, int32_t G, int32_t kpad) {
  if (R < 0 || G <= 0 || kpad <= 0) return 0;
  // Only a non-empty group adds padding, at most kpad - 1 rows.
  return (R + std::min<int64_t>(G, R) * (kpad - 1)) / kpad * kpad;
}

moe_status_t moe_mx_quantize_cols(const void* x, int64_t R, int64_t N, int64_t ldx, const int32_t* offsets,
                                  int32_t G, int64_t group_rows, int32_t kpad, uint8_t* codes, uint8_t* scales,
                                  int64_t ldc, int32_t* kbase, moe_stream_t stream) {
  g_err.clear();
  CHECK(R >= 0 && N > 0, MOE_ERR_INVALID_VALUE, "R must be >= 0 and N > 0");
  CHECK(N % 2 == 0 && ldx >= N && ldx % 2 == 0, MOE_ERR_UNSUPPORTED, "N and ldx must be even, ldx >= N");
  CHECK(G > 0 && G <= 1024, MOE_ERR_INVALID_VALUE, "G must be in [1, 1024] (got %d)", G);
  CHECK(kpad > 0 && kpad % 128 == 0, MOE_ERR_UNSUPPORTED, "kpad must be a positive multiple of 128 (got %d)",
        kpad);
  CHECK(ldc % 128 == 0 && ldc >= 0, MOE_ERR_INVALID_VALUE, "ldc must be a multiple of 128 (got %lld)",
        (long long)ldc);
  CHECK(R <= kMaxInt && N <= kMaxInt && ldc <= kMaxInt, MOE_ERR_UNSUPPORTED, "sizes must fit in int32");
  int64_t need;
  if (offsets) {
    need = moe_mx_quantize_cols_ld(R, G, kpad);
  } else {
    CHECK(group_rows >= 0 && R == (int64_t)G * group_rows, MOE_ERR_INVALID_VALUE,
          "without offsets R must equal G * group_rows (got R=%lld, G=%d, group_rows=%lld)", (long long)R, G,
          (long long)group_rows);
    need = (int64_t)G * ((group_rows + kpad - 1) / kpad * kpad);
  }
  CHECK(ldc >= need, MOE_ERR_INVALID_VALUE, "ldc must be >= %lld (got %lld)", (long long)need, (long long)ldc);
  CHECK(kbase && (ldc == 0 || (codes && scales)), MOE_ERR_INVALID_VALUE, "kbase/codes/scales is NULL");
  CHECK(R == 0 || x, MOE_ERR_INVALID_VALUE, "x is NULL");
  CHECK_ALIGN16(x, offsets, codes, scales, kbase);
  return hip_check(moe::launch_mx_quant_cols(x, R, (int)N, ldx, offsets, G, group_rows, kpad, codes, scales, ldc,
                                             kbase, S(stream)),
                   "MXFP8 column quantization");
}

size_t moe_mx_gemm_workspace_size(int32_t G) {
  if (G <= 0) return 0;
  return align256((size_t)(G + 1) * sizeof(int32_t));
}

moe_status_t moe_mx_gemm_rows(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                              const uint8_t* b_scales, int64_t b_row_stride, int64_t b_group_stride,
                              const uint8_t* b2_codes, const uint8_t* b2_scales, int64_t b2_k, const int32_t* offsets,
                              int32_t G, int64_t M, int64_t N, int64_t K, int32_t epilogue, void* out0, void* out1,
                              void* out2, const void* aux0, const void* aux1, uint8_t* q_codes, uint8_t* q_scales,
                              void* ws, size_t ws_bytes, moe_stream_t stream) {
  g_err.clear();
  CHECK(epilogue >= MOE_MX_EPI_STORE && epilogue <= MOE_MX_EPI_SWIGLU_BWD, MOE_ERR_INVALID_VALUE,
        "unknown epilogue %d", epilogue);
  CHECK(G > 0 && G <= 1024, MOE_ERR_INVALID_VALUE, "G must be in [1, 1024] (got %d)", G);
  CHECK(M >= 0 && N > 0 && K > 0, MOE_ERR_INVALID_VALUE, "M must be >= 0, N and K > 0");
  const int oc = epilogue == MOE_MX_EPI_SWIGLU ? 64 : 128;
  CHECK(K % 128 == 0 && N % oc == 0, MOE_ERR_UNSUPPORTED, "K must be a multiple of 128 and N of %d", oc);
  // Columns one source holds: all K, or the two parts of a K split.
  const int64_t span = (b2_codes && epilogue != MOE_MX_EPI_SWIGLU) ? std::max<int64_t>(b2_k, K - b2_k) : K;
  CHECK(b_row_stride >= span && b_row_stride % 128 == 0 && b_group_stride >= 0 && b_group_stride % 128 == 0,
        MOE_ERR_INVALID_VALUE, "B strides must be multiples of 128, the row stride >= the columns of a source");
  CHECK(M <= kMaxInt && N <= kMaxInt / 2 && K <= kMaxInt, MOE_ERR_UNSUPPORTED, "sizes must fit in int32");
  CHECK(((M + 127) / 128 + G) * (N / oc) < kMaxInt, MOE_ERR_UNSUPPORTED, "grid too large");
  CHECK(a_codes && a_scales && b_codes && b_scales && offsets, MOE_ERR_INVALID_VALUE, "an operand pointer is NULL");
  CHECK((b2_codes == nullptr) == (b2_scales == nullptr), MOE_ERR_INVALID_VALUE,
        "b2_codes and b2_scales must both be given or both be NULL");
  if (epilogue == MOE_MX_EPI_SWIGLU) {
    CHECK(b2_codes, MOE_ERR_INVALID_VALUE, "the SwiGLU epilogue needs the up-projection rows in b2");
  } else if (b2_codes) {
    CHECK(b2_k > 0 && b2_k < K && b2_k % 128 == 0, MOE_ERR_INVALID_VALUE,
          "b2_k must be a multiple of 128 in (0, K) (got %lld)", (long long)b2_k);
  }
  if (epilogue == MOE_MX_EPI_STORE) CHECK(out0, MOE_ERR_INVALID_VALUE, "out0 is NULL");
  if (epilogue == MOE_MX_EPI_SWIGLU) CHECK(out2, MOE_ERR_INVALID_VALUE, "out2 is NULL");
  if (epilogue == MOE_MX_EPI_SWIGLU_BWD) CHECK(out0 && aux0 && aux1, MOE_ERR_INVALID_VALUE, "out0/aux0/aux1 is NULL");
  CHECK((q_codes == nullptr) == (q_scales == nullptr), MOE_ERR_INVALID_VALUE,
        "q_codes and q_scales must both be given or both be NULL");
  CHECK(!q_codes || epilogue != MOE_MX_EPI_STORE, MOE_ERR_INVALID_VALUE,
        "quantized outputs are produced by the SwiGLU epilogues only");
  const size_t need = moe_mx_gemm_workspace_size(G);
  CHECK(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
        ws ? ws_bytes : (size_t)0);
  if (M == 0) return MOE_OK;
  CHECK_ALIGN16(a_codes, a_scales, b_codes, b_scales, b2_codes, b2_scales, offsets, out0, out1, out2, aux0, aux1, q_codes, q_scales, ws);
  moe::MxGemmArgs a{};
  a.a = a_codes;
  a.as = a_scales;
  a.lda = K;
  a.b = b_codes;
  a.bs = b_scales;
  a.ldb = b_row_stride;
  a.b_gstride = b_group_stride;
  a.b2 = b2_codes;
  a.bs2 = b2_scales;
  a.ksplit = (epilogue != MOE_MX_EPI_SWIGLU && b2_codes) ? (int)b2_k : 0;
  a.kparts = 1;
  a.offsets = offsets;
  a.tile_prefix = reinterpret_cast<int32_t*>(ws);
  a.G = G;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.out0 = out0;
  a.out1 = out1;
  a.out2 = out2;
  a.aux0 = aux0;
  a.aux1 = aux1;
  a.qc = q_codes;
  a.qs = q_scales;
  return hip_check(moe::launch_mx_gemm(epilogue, false, a, S(stream)), "MXFP8 grouped GEMM (rows)");
}

size_t moe_mx_gemm_k_workspace_size(int32_t G, int64_t M, int64_t N) {
  if (G <= 0 || M <= 0 || N <= 0 || M > kMaxInt || N > kMaxInt || G > 1024) return 0;
  return moe::mx_k_workspace_bytes(G, (int)M, (int)N);
}

moe_status_t moe_mx_gemm_k(const uint8_t* a_codes, const uint8_t* a_scales, int64_t lda, const uint8_t* b_codes,
                           const uint8_t* b_scales, int64_t ldb, const int32_t* kbase, int32_t G, int64_t M,
                           int64_t N, int64_t split, void* out0, void* out1, void* ws, size_t ws_bytes,
                           moe_stream_t stream) {
  g_err.clear();
  CHECK(G > 0 && G <= 1024, MOE_ERR_INVALID_VALUE, "G must be in [1, 1024] (got %d)", G);
  CHECK(M > 0 && N > 0 && split >= 0 && split <= M, MOE_ERR_INVALID_VALUE, "M, N must be > 0, split in [0, M]");
  CHECK(M % 128 == 0 && N % 128 == 0, MOE_ERR_UNSUPPORTED, "M and N must be multiples of 128");
  CHECK(lda > 0 && ldb > 0 && lda % 128 == 0 && ldb % 128 == 0, MOE_ERR_INVALID_VALUE,
        "lda and ldb must be positive multiples of 128");
  CHECK(M <= kMaxInt && N <= kMaxInt && lda <= kMaxInt && ldb <= kMaxInt, MOE_ERR_UNSUPPORTED,
        "sizes must fit in int32");
  CHECK((int64_t)G * (M / 128) * (N / 128) < kMaxInt, MOE_ERR_UNSUPPORTED, "grid too large");
  CHECK(a_codes && a_scales && b_codes && b_scales && kbase, MOE_ERR_INVALID_VALUE, "an operand pointer is NULL");
  CHECK((split == 0 || out0) && (split == M || out1), MOE_ERR_INVALID_VALUE, "out0/out1 is NULL");
  const size_t need = moe::mx_k_workspace_bytes(G, (int)M, (int)N);
  CHECK(need == 0 || (ws && ws_bytes >= need), MOE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
        ws ? ws_bytes : (size_t)0);
  CHECK_ALIGN16(a_codes, a_scales, b_codes, b_scales, kbase, out0, out1, ws);
  moe::MxGemmArgs a{};
  a.a = a_codes;
  a.as = a_scales;
  a.lda = lda;
  a.b = b_codes;
  a.bs = b_scales;
  a.ldb = ldb;
  a.offsets = kbase;
  a.G = G;
  a.M = (int)M;
  a.N = (int)N;
  a.out0 = out0;
  a.out1 = out1;
  a.split = (int)split;
  a.kparts = moe::mx_k_parts(G, (int)M, (int)N);
  a.partial = reinterpret_cast<float*>(ws);
  return hip_check(moe::launch_mx_gemm(MOE_MX_EPI_STORE, true, a, S(stream)), "MXFP8 grouped GEMM (K)");
}

// ---------------------------------------------------------------------------------------------

size_t moe_workspace_bytes(int32_t op, int64_t T, int64_t d, int32_t E, int32_t k, int64_t f, int64_t fs) {
  g_err.clear();
  if (check_tokens(T, d, E, k) != MOE_OK) return 0;
  if (f <= 0 || fs < 0) {
    fail(MOE_ERR_INVALID_VALUE, "f must be > 0 and fs >= 0 (got f=%lld, fs=%lld)", (long long)f, (long long)fs);
    return 0;
  }
  const int64_t Tk = T * k;
  // The routed experts and (fs > 0) the shared expert as expert sets, sizes only.
  moe_expert_set_t sets[2] = {};
  sets[0].G = E;
  sets[0].M = Tk;
  sets[0].f = f;
  sets[1].G = 1;
  sets[1].M = T;
  sets[1].f = fs;
  const int nsets = fs > 0 ? 2 : 1;
  switch (op) {
    case MOE_OP_ROUTE:
    case MOE_OP_COMBINE:
    case MOE_OP_COMBINE_BWD:
    case MOE_OP_PERMUTE_BWD: return 0;
    case MOE_OP_PERMUTE: return moe_permute_workspace_size(T, E, k);
    case MOE_OP_GROUPED_MLP_FWD: return moe_grouped_mlp_fwd_workspace_size(Tk, E, d, f);
    case MOE_OP_GROUPED_MLP_BWD: return moe_grouped_mlp_bwd_workspace_size(Tk, E, d, f);
    case MOE_OP_ROUTE_BWD: return moe_route_bwd_workspace_size(T, d, E, k);
    case MOE_OP_EXPERT_STAGE: return moe_expert_stage_workspace_size(sets, nsets, d);
    case MOE_OP_ROUTER_AUX: return moe_router_aux_workspace_size(T, E);
    case MOE_OP_ROUTER_AUX_BWD: return moe_router_aux_bwd_workspace_size(T, d, E);
    case MOE_OP_MX_GEMM_ROWS: return moe_mx_gemm_workspace_size(E);
    case MOE_OP_MX_GEMM_K: {
      size_t need = std::max(moe_mx_gemm_k_workspace_size(E, d, f), moe_mx_gemm_k_workspace_size(E, 2 * f, d));
      if (fs > 0)
        need = std::max(need, std::max(moe_mx_gemm_k_workspace_size(1, d, fs),
                                       moe_mx_gemm_k_workspace_size(1, 2 * fs, d)));
      return need;
    }
    default:
      fail(MOE_ERR_INVALID_VALUE, "unknown op %d", op);
      return 0;
  }
}

}  // extern "C"
