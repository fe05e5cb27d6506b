/*
 * libmoe — one GPU's share of the Olmo-core 3 mixture-of-experts block, for AMD MI355X (gfx950).
 *
 * The layer: every token picks its top-k routed experts (learned router or random routing) and
 * also goes through one shared expert; the routed experts are SwiGLU MLPs that stay resident on
 * the GPU while tokens are moved to them; the output is the gate-weighted sum of the k expert
 * outputs plus the shared expert's output.  Sources: "Olmo-core DDP MoE examples" README,
 * section "Production throughput runs" (top-4 routing, one shared expert, learned vs random
 * routing); "Olmo-core 3 Opens Large MoE Training", "Technical Deep Dive" (experts stay pinned in
 * local memory, tokens are routed to them); "Scaling Trillion-Parameter Models: The Architecture
 * of Olmo-core 3", "Code Snippet" (a per-token expert selection step).
 *
 * Conventions shared by every call
 *   Memory      All tensor pointers are DEVICE pointers owned by the caller.  The library keeps
 *               no pointer after a call returns and allocates no device memory: scratch space is
 *               the caller's workspace, sized by the matching *_workspace_size function (or, for
 *               moe_permute_noalloc, a fixed device array the library holds per GPU).
 *               Every device pointer (tensors, index arrays, workspaces) must be 16-byte
 *               aligned: the kernels use 16-byte vector and direct-to-LDS accesses from each base
 *               (hipMalloc and PyTorch allocations are 256-byte aligned); a misaligned pointer
 *               returns MOE_ERR_INVALID_VALUE.
 *   Layout      Row-major, contiguous.  Weights are [out_features, in_features]:
 *                 w_router [E, d]; w1, w3 [G, f, d]; w2 [G, d, f].
 *   Types       dt = MOE_F32: every activation and weight is float.  dt = MOE_BF16: activations,
 *               weights and their gradients are bfloat16 (uint16 bit patterns); router logits,
 *               gates, gate gradients and the router weight gradient are always float32;
 *               accumulation is always float32.
 *   Streams     Every call only enqueues work on `stream` (a hipStream_t; NULL = null stream)
 *               and returns.  No call synchronises with the host or copies to the host.
 *   Errors      Arguments are checked on the host before anything is enqueued.  Invalid values
 *               return MOE_ERR_INVALID_VALUE, valid but unsupported sizes MOE_ERR_UNSUPPORTED,
 *               a too small workspace MOE_ERR_WORKSPACE, a failed launch MOE_ERR_HIP.  Detail is
 *               in moe_last_error() (per thread).  Nothing aborts and nothing throws.
 *   Results     Every output is bitwise deterministic from run to run (no floating-point
 *               atomics).  Gradients are written, never accumulated into.
 *   Sizes       1 <= k <= min(E, 8), E <= 256, T*k < 2^31; for the expert MLP calls d and f must
 *               be multiples of 128.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_VALUE = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef void* moe_stream_t; /* hipStream_t */

/* ------------------------------------------------------------------------------------------ */
/* Routing                                                                                     */

/* Router: logits, top-k selection and gate weights.
 * Source: "Scaling Trillion-Parameter Models ...", "Code Snippet" (one expert choice per token);
 * "Olmo-core DDP MoE examples", "Production throughput runs" (top-4; learned or random routing).
 *   x          [T, d]  (dt)            tokens; read only when w_router != NULL
 *   w_router   [E, d]  (dt) or NULL    learned router.  NULL selects random routing: `logits`
 *                                       is then an INPUT (caller-drawn scores)
 *   bias       [E] float or NULL       constant per-expert logit bias (learned routing only)
 *   logits     [T, E] float            learned: OUTPUT, L[t,e] = x[t,:].w_router[e,:] summed in
 *                                       index order with one fp32 rounding per product and per
 *                                       addition, then + bias[e]; random: INPUT
 *   topk_idx   [T, k] int32  OUTPUT    the k largest logits of each token, largest first; equal
 *                                       logits ordered by lower expert index (-0 equals +0)
 *   topk_gate  [T, k] float  OUTPUT    renormalize=1: softmax over the k chosen logits;
 *                                       renormalize=0: full softmax probability over all E
 * A NaN logit ranks after every number (-inf included) and NaNs among themselves by lower index,
 * so every topk_idx value is in [0, E) whatever the logits hold; the gates of a token with a NaN
 * or infinite logit are unspecified. */
moe_status_t moe_route(const void* x, const void* w_router, const float* bias, float* logits,
                       int64_t T, int64_t d, int32_t E, int32_t k, int32_t renormalize,
                       moe_dtype_t dt, int32_t* topk_idx, float* topk_gate, moe_stream_t stream);

/* Token dispatch: per-expert histogram, exclusive prefix sum, stable permutation and row gather.
 * Source: "Olmo-core 3 Opens Large MoE Training", "Enhanced Key Takeaways" and "Technical Deep
 * Dive" (tokens are routed to experts that stay in place).
 * Assignment a = t*k + j (token t, slot j) belongs to expert topk_idx[a].  Rows are expert-major;
 * inside an expert they keep ascending a (a stable counting sort).
 *   topk_idx  [T, k] int32  INPUT, each value in [0, E) (out-of-range values are not checked)
 *   counts    [E] int32     OUTPUT  rows per expert
 *   offsets   [E+1] int32   OUTPUT  exclusive prefix sum of counts; offsets[E] = T*k
 *   dest_pos  [T*k] int32   OUTPUT  row of assignment a
 *   src_row   [T*k] int32   OUTPUT  assignment held by row p (inverse of dest_pos)
 *   x_perm    [T*k, d] (dt) OUTPUT or NULL: x_perm[p] = x[src_row[p] / k] (exact copy)
 *   ws        device workspace of moe_permute_workspace_size(T, E, k) bytes */
size_t moe_permute_workspace_size(int64_t T, int32_t E, int32_t k);
moe_status_t moe_permute(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E,
                         int32_t k, moe_dtype_t dt, int32_t* counts, int32_t* offsets,
                         int32_t* dest_pos, int32_t* src_row, void* x_perm, void* ws,
                         size_t ws_bytes, moe_stream_t stream);

/* moe_permute for callers that cannot allocate device memory or pass a workspace: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and checks as moe_permute without ws/ws_bytes; no call allocates or frees anything.  Its scratch
 * is a fixed array in device memory that the library holds on every GPU it runs on until the
 * process ends: moe_permute_noalloc_max_scratch() bytes (4 MiB).  Sizes whose moe_permute
 * workspace (moe_permute_workspace_size(T, E, k)) exceeds that return MOE_ERR_UNSUPPORTED; with
 * E = 256 this allows T*k up to about 690,000.  All calls on one GPU share that GPU's array, which
 * keeps the last call's contents: calls that may overlap on one GPU (different streams, no ordering
 * between them) race on it and give undefined results; calls ordered on one stream are safe. */
size_t moe_permute_noalloc_max_scratch(void);
moe_status_t moe_permute_noalloc(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E,
                                 int32_t k, moe_dtype_t dt, int32_t* counts, int32_t* offsets,
                                 int32_t* dest_pos, int32_t* src_row, void* x_perm, moe_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Grouped SwiGLU expert MLP.  G groups (experts) over M rows; group g owns rows                */
/* [offsets[g], offsets[g+1]) of x_in (offsets is a DEVICE array, non-decreasing, offsets[0]=0,  */
/* offsets[G]=M).  Group g computes A = X W1[g]^T, B = X W3[g]^T, H = silu(A)*B, Y = H W2[g]^T.  */
/* The shared expert is the same computation with G = 1 and offsets = {0, T}.                   */
/* Source: "Olmo-core DDP MoE examples", "Interpreting the eight-layer DDP vs FSDP comparison"   */
/* (sparse expert kernels; shared-branch mixing) and "Production throughput runs" (one shared    */
/* expert).  The SwiGLU form is the reading taken where the pages are silent.                    */

/* Workspace for the forward calls (tile schedule only). */
size_t moe_grouped_mlp_fwd_workspace_size(int64_t M, int32_t G, int64_t d, int64_t f);
/* Workspace for moe_grouped_mlp_bwd: the tile schedule plus dAB [M, 2f] (dt). */
size_t moe_grouped_mlp_bwd_workspace_size(int64_t M, int32_t G, int64_t d, int64_t f);

/* Forward: gate/up GEMM with fused SwiGLU, then the down GEMM.
 *   x_in [M, d]; w1, w3 [G, f, d]; w2 [G, d, f]           INPUT  (dt)
 *   a_stash, b_stash [M, f]                               OUTPUT (dt) or both NULL (no backward)
 *   h [M, f]                                              OUTPUT (dt) (also the down GEMM input)
 *   y [M, d]                                              OUTPUT (dt) */
moe_status_t moe_grouped_mlp_fwd(const void* x_in, const int32_t* offsets, int32_t G, int64_t M,
                                 int64_t d, int64_t f, const void* w1, const void* w3,
                                 const void* w2, moe_dtype_t dt, void* a_stash, void* b_stash,
                                 void* h, void* y, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Backward of moe_grouped_mlp_fwd (all four steps below, dAB kept in the workspace).
 * Source: the same expert kernels trained end to end ("Olmo-core DDP MoE examples", "Production
 * throughput runs": every operating point is a training run, so each expert product has its data
 * and weight gradient; "Interpreting the eight-layer DDP vs FSDP comparison": sparse expert kernels).
 *   dy [M, d], x_in [M, d], a, b, h [M, f]                INPUT  (dt)
 *   dx_in [M, d]                                          OUTPUT (dt)
 *   dw1, dw3 [G, f, d]; dw2 [G, d, f]                     OUTPUT (dt); a group with no rows
 *                                                         gets exact zeros */
moe_status_t moe_grouped_mlp_bwd(const void* dy, const void* x_in, const void* a, const void* b,
                                 const void* h, const int32_t* offsets, int32_t G, int64_t M,
                                 int64_t d, int64_t f, const void* w1, const void* w3,
                                 const void* w2, moe_dtype_t dt, void* dx_in, void* dw1, void* dw3,
                                 void* dw2, void* ws, size_t ws_bytes, moe_stream_t stream);

/* The individual GEMM stages of the two calls above, each a single kernel launch, for callers
 * that schedule or time the stages themselves.  Same argument meanings; ws needs
 * moe_grouped_mlp_fwd_workspace_size bytes.  dab [M, 2f] (dt) holds dA in columns [0, f) and
 * dB in columns [f, 2f):
 *   gate_up_fwd:   A = X W1^T, B = X W3^T; h = silu(A) * B (a_stash/b_stash may be NULL)
 *   down_fwd:      y = h W2^T
 *   down_bwd:      dH = dy W2; dA = dH * B * s * (1 + A (1 - s)), s = sigmoid(A); dB = dH*silu(A)
 *   down_wgrad:    dw2[g] = dy_g^T h_g
 *   gate_up_dgrad: dx_in = dA W1 + dB W3
 *   gate_up_wgrad: dw1[g] = dA_g^T x_g, dw3[g] = dB_g^T x_g */
moe_status_t moe_expert_gate_up_fwd(const void* x_in, const int32_t* offsets, int32_t G,
                                    int64_t M, int64_t d, int64_t f, const void* w1,
                                    const void* w3, moe_dtype_t dt, void* a_stash, void* b_stash,
                                    void* h, void* ws, size_t ws_bytes, moe_stream_t stream);
moe_status_t moe_expert_down_fwd(const void* h, const int32_t* offsets, int32_t G, int64_t M,
                                 int64_t d, int64_t f, const void* w2, moe_dtype_t dt, void* y,
                                 void* ws, size_t ws_bytes, moe_stream_t stream);
moe_status_t moe_expert_down_bwd(const void* dy, const void* a, const void* b,
                                 const int32_t* offsets, int32_t G, int64_t M, int64_t d,
                                 int64_t f, const void* w2, moe_dtype_t dt, void* dab, void* ws,
                                 size_t ws_bytes, moe_stream_t stream);
moe_status_t moe_expert_down_wgrad(const void* dy, const void* h, const int32_t* offsets,
                                   int32_t G, int64_t M, int64_t d, int64_t f, moe_dtype_t dt,
                                   void* dw2, void* ws, size_t ws_bytes, moe_stream_t stream);
moe_status_t moe_expert_gate_up_dgrad(const void* dab, const int32_t* offsets, int32_t G,
                                      int64_t M, int64_t d, int64_t f, const void* w1,
                                      const void* w3, moe_dtype_t dt, void* dx_in, void* ws,
                                      size_t ws_bytes, moe_stream_t stream);
moe_status_t moe_expert_gate_up_wgrad(const void* dab, const void* x_in, const int32_t* offsets,
                                      int32_t G, int64_t M, int64_t d, int64_t f, moe_dtype_t dt,
                                      void* dw1, void* dw3, void* ws, size_t ws_bytes,
                                      moe_stream_t stream);

/* The same GEMM stages over two sets of experts in one call: the routed experts and the shared
 * expert (the pages' block has top-k routed experts plus one shared expert on every token:
 * "Olmo-core DDP MoE examples", "Production throughput runs").  The shared expert is a set with
 * G = 1, offsets = {0, T} and x = the layer input.  Where the pipelined kernel takes both sets
 * the stage is one launch, whose tiles fill the CUs that a lone one-group GEMM would leave idle;
 * otherwise the sets run one after the other.  Results are identical either way.
 * Each stage reads the members listed above for its single-set call:
 *   GATE_UP_FWD:   x, w1, w3 -> a, b (both NULL or both given), h
 *   DOWN_FWD:      h, w2 -> y
 *   DOWN_BWD:      dy, w2, a, b -> dab
 *   GATE_UP_DGRAD: dab, w1, w3 -> dx
 *   DOWN_WGRAD:    dy, h -> dw2
 *   GATE_UP_WGRAD: dab, x -> dw1, dw3
 * Unused members may be NULL.  Every set needs d common; f may differ between sets. */
typedef struct {
  const int32_t* offsets; /* [G+1] device, as for the single-set calls */
  int32_t G;
  int64_t M;              /* rows of this set */
  int64_t f;              /* hidden width of this set's experts */
  const void* x;          /* [M, d] */
  const void* w1;         /* [G, f, d] */
  const void* w3;         /* [G, f, d] */
  const void* w2;         /* [G, d, f] */
  void* a;                /* [M, f] */
  void* b;                /* [M, f] */
  void* h;                /* [M, f] */
  void* y;                /* [M, d] */
  const void* dy;         /* [M, d] */
  void* dab;              /* [M, 2f] */
  void* dx;               /* [M, d] */
  void* dw1;              /* [G, f, d] */
  void* dw3;              /* [G, f, d] */
  void* dw2;              /* [G, d, f] */
} moe_expert_set_t;

typedef enum {
  MOE_STAGE_GATE_UP_FWD = 0,
  MOE_STAGE_DOWN_FWD = 1,
  MOE_STAGE_DOWN_BWD = 2,
  MOE_STAGE_GATE_UP_DGRAD = 3,
  MOE_STAGE_DOWN_WGRAD = 4,
  MOE_STAGE_GATE_UP_WGRAD = 5
} moe_stage_t;

/* Workspace bytes for moe_expert_stage over these sets (nsets = 1 or 2). */
size_t moe_expert_stage_workspace_size(const moe_expert_set_t* sets, int32_t nsets, int64_t d);
/* One GEMM stage over nsets (1 or 2) expert sets; sets is a HOST array, the tensors it points to
 * are device memory.  Errors as for the single-set calls; MOE_ERR_INVALID_VALUE for a bad stage or
 * nsets. */
moe_status_t moe_expert_stage(moe_stage_t stage, const moe_expert_set_t* sets, int32_t nsets, int64_t d,
                              moe_dtype_t dt, void* ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Combine                                                                                     */

/* Weighted combine / unpermute: out[t] = shared_out[t] + sum_j topk_gate[t,j] * y_perm[dest_pos[t*k+j]],
 * summed in fp32.  Source: "Olmo-core DDP MoE examples", "Production throughput runs" (top-k
 * experts plus one shared expert); the shared branch is added with weight 1.
 *   y_perm [T*k, d] (dt), topk_gate [T, k] float, dest_pos [T*k] int32   INPUT
 *   shared_out [T, d] (dt) INPUT or NULL;  out [T, d] (dt) OUTPUT */
moe_status_t moe_combine(const void* y_perm, const float* topk_gate, const int32_t* dest_pos,
                         const void* shared_out, int64_t T, int64_t d, int32_t k, moe_dtype_t dt,
                         void* out, moe_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Backward                                                                                    */

/* Backward of moe_combine: the gradient of its gate-weighted sum of the k routed outputs plus the
 * shared output.  Source: "Olmo-core DDP MoE examples", "Production throughput runs" (top-k routed
 * experts plus one shared expert, trained; learned routing, whose gates receive this gradient).
 *   dy_perm[dest_pos[t*k+j]] = topk_gate[t,j] * dout[t]                 OUTPUT [T*k, d] (dt)
 *   dgate[t,j] = <dout[t], y_perm[dest_pos[t*k+j]]> (fp32)              OUTPUT [T, k] or NULL
 * (the shared expert's output gradient is dout itself). */
moe_status_t moe_combine_bwd(const void* dout, const void* y_perm, const float* topk_gate,
                             const int32_t* dest_pos, int64_t T, int64_t d, int32_t k,
                             moe_dtype_t dt, void* dy_perm, float* dgate, moe_stream_t stream);

/* Backward of the row gather plus the other contributions to dx.  Source: "Olmo-core 3 Opens Large
 * MoE Training", "Technical Deep Dive" (tokens travel to resident experts, so their gradients
 * travel back to the tokens); the shared expert and the learned router also read x ("Olmo-core DDP
 * MoE examples", "Production throughput runs"), whence the two addends.
 *   dx[t] = sum_j dx_perm[dest_pos[t*k+j]] + dx_add0[t] + dx_add1[t]   (fp32 sum)
 *   dx_perm [T*k, d] (dt) INPUT; dx_add0, dx_add1 [T, d] (dt) INPUT or NULL; dx [T, d] OUTPUT */
moe_status_t moe_permute_bwd(const void* dx_perm, const int32_t* dest_pos, const void* dx_add0,
                             const void* dx_add1, int64_t T, int64_t d, int32_t k,
                             moe_dtype_t dt, void* dx, moe_stream_t stream);

/* Router backward (learned routing, renormalize = 1).  With g the gates and dg their gradient,
 * the logit gradient is dL[t, S_j] = g_j (dg_j - sum_i g_i dg_i) on the chosen experts and 0
 * elsewhere (the bias, a constant, gets none).  Then
 *   dw_router = dL^T x   [E, d] float OUTPUT (an expert no token chose gets exact zeros)
 *   dx_router = dL w_router  [T, d] (dt) OUTPUT
 * Inputs: dgate, topk_gate [T, k] float; topk_idx [T, k]; offsets [E+1] and src_row [T*k] from
 * moe_permute; x [T, d]; w_router [E, d].  ws: moe_route_bwd_workspace_size(T, d, E, k) bytes.
 * Source: "Olmo-core DDP MoE examples", "Production throughput runs" (learned routing is
 * trained).  renormalize = 0 returns MOE_ERR_UNSUPPORTED. */
size_t moe_route_bwd_workspace_size(int64_t T, int64_t d, int32_t E, int32_t k);
moe_status_t moe_route_bwd(const float* dgate, const float* topk_gate, const int32_t* topk_idx,
                           const int32_t* offsets, const int32_t* src_row, const void* x,
                           const void* w_router, int64_t T, int64_t d, int32_t E, int32_t k,
                           int32_t renormalize, moe_dtype_t dt, float* dw_router, void* dx_router,
                           void* ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Router statistics and the auxiliary load-balancing loss (learned routing)                   */
/* The pages run load-balancing experiments at loss weights 0.02 to 0.50 ("Olmo-core DDP MoE
 * examples", "Other experiments in the report") without stating the loss.  Implemented reading:
 *   loss = weight * E * sum_e f_e P_e,  f_e = counts[e] / (T k),  P_e = mean_t softmax(logits[t])_e
 * (softmax over all E logits).  f comes from the selection and carries no gradient.            */

/* Forward: prob_mean [E] float OUTPUT (P), load_frac [E] float OUTPUT (f), loss [1] float OUTPUT.
 *   logits [T, E] float INPUT (the router logits; NULL allowed when T = 0); counts [E] int32 INPUT
 *   (from moe_permute).  All device pointers.  ws: moe_router_aux_workspace_size(T, E) bytes.
 *   Sums in fixed orders (bitwise reproducible).  Errors: NULL output, bad sizes, small workspace. */
size_t moe_router_aux_workspace_size(int64_t T, int32_t E);
moe_status_t moe_router_aux(const float* logits, const int32_t* counts, int64_t T, int32_t E, int32_t k,
                            float weight, float* loss, float* prob_mean, float* load_frac, void* ws,
                            size_t ws_bytes, moe_stream_t stream);

/* Backward: with G[t, j] = (weight E / T) p[t, j] (f_j - sum_e f_e p[t, e]) the gradient of the
 * loss with respect to the logits, ADDS
 *   G^T x        to dw_router [E, d] float (IN/OUT),
 *   G w_router   to dx_router [T, d] (dt) (IN/OUT; the sum is rounded once to dt),
 * so it runs after moe_route_bwd on the same buffers.  Inputs: logits [T, E] float, load_frac [E]
 * float (from moe_router_aux), x [T, d] (dt), w_router [E, d] (dt).  d must be a multiple of 8.
 * ws: moe_router_aux_bwd_workspace_size(T, d, E) bytes.  Fixed summation orders. */
size_t moe_router_aux_bwd_workspace_size(int64_t T, int64_t d, int32_t E);
moe_status_t moe_router_aux_bwd(const float* logits, const float* load_frac, const void* x, const void* w_router,
                                int64_t T, int64_t d, int32_t E, float weight, moe_dtype_t dt, float* dw_router,
                                void* dx_router, void* ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* MXFP8 grouped GEMMs                                                                          */
/* The pages train their largest operating points with an MXFP8 recipe ("Olmo-core DDP MoE
 * examples", "Production throughput runs", operating-point table; "Other experiments in the
 * report", MXFP8 ablation of the MLP) without defining the format.  Reading implemented: OCP
 * Microscaling (MX) v1.0 MXFP8 -- E4M3 elements (bias 7, largest magnitude 448, no infinities)
 * and one E8M0 scale byte s (value 2^(s - 127)) per 32 consecutive elements of the CONTRACTION
 * axis.  Quantizing a block: shared exponent = floor(log2(max |v|)) - 8 clamped to [-127, 127]
 * (-127 for an all-zero block); each element becomes E4M3(v / 2^shared), rounded to nearest with
 * ties to even, magnitudes above 448 saturated to 448.  Codes and scales are exact (bitwise equal
 * to that definition).  A product of MX operands is the product of the dequantized matrices; it is
 * accumulated in fp32 and stored as bf16.  Inputs of the quantizers are bf16; NaN/Inf unsupported. */

/* Quantize x [R, K] (bf16, row stride ldx elements) along its rows:
 *   codes  [R, K] uint8 OUTPUT (E4M3), scales [R, K/32] uint8 OUTPUT (E8M0).
 * K must be a multiple of 32, ldx a multiple of 8 and >= K.  R = 0 is a no-op. */
moe_status_t moe_mx_quantize_rows(const void* x, int64_t R, int64_t K, int64_t ldx, uint8_t* codes,
                                  uint8_t* scales, moe_stream_t stream);

/* Minimum row stride (bytes) of moe_mx_quantize_cols' output for R rows in G groups padded to kpad. */
int64_t moe_mx_quantize_cols_ld(int64_t R, int32_t G, int32_t kpad);

/* Quantize x [R, N] (bf16, row stride ldx elements) along its COLUMNS, one row range per group,
 * and store it transposed (contraction axis last), for the weight gradients whose contraction
 * runs over the rows an expert received:
 *   group g = rows offsets[g]..offsets[g+1]-1 (offsets [G+1] int32 device, clamped to [0, R]) or,
 *   when offsets is NULL, rows g*group_rows..(g+1)*group_rows-1 (then R must equal G*group_rows);
 *   each group is padded with zero rows to a multiple of kpad (a multiple of 128);
 *   kbase  [G+1] int32 OUTPUT: first column of each group (kbase[G] = total padded length);
 *   codes  [N, ldc] uint8 OUTPUT, group g at columns kbase[g]..kbase[g+1]-1, columns past
 *          kbase[G] hold zero codes; scales [N, ldc/32] uint8 OUTPUT alike.
 * ldc must be a multiple of 128 and >= moe_mx_quantize_cols_ld(R, G, kpad) (offsets given) or
 * G * round_up(group_rows, kpad) (offsets NULL).  N and ldx must be even; G <= 1024. */
moe_status_t moe_mx_quantize_cols(const void* x, int64_t R, int64_t N, int64_t ldx, const int32_t* offsets,
                                  int32_t G, int64_t group_rows, int32_t kpad, uint8_t* codes, uint8_t* scales,
                                  int64_t ldc, int32_t* kbase, moe_stream_t stream);

typedef enum {
  MOE_MX_EPI_STORE = 0,      /* out0 [M, N] bf16 = C */
  MOE_MX_EPI_SWIGLU = 1,     /* B = gate rows (W1), B2 = up rows (W3), N rows each per group;
                                G1 = A B^T, G3 = A B2^T; out2 [M, N] = silu(G1) * G3,
                                out0 / out1 [M, N] = G1 / G3 (each may be NULL) */
  MOE_MX_EPI_SWIGLU_BWD = 2  /* C = dH; aux0, aux1 [M, N] bf16 = the stashed G1, G3;
                                out0 [M, 2N] = [dH * G3 * s (1 + G1 (1 - s)) | dH * G1 * s],
                                s = sigmoid(G1) */
} moe_mx_epilogue_t;

/* Grouped product over ragged ROW ranges (forward and data-gradient GEMMs):
 *   C[m, n] = sum_k A[m, k] B_g[n, k] for rows m of group g = offsets[g]..offsets[g+1]-1
 *   a_codes [M, K], a_scales [M, K/32] (from moe_mx_quantize_rows);
 *   B_g row n at b_codes + g*b_group_stride + n*b_row_stride, its scales at
 *   b_scales + (g*b_group_stride + n*b_row_stride)/32 (N rows per group);
 *   b2_codes / b2_scales: a second B source with the same strides, NULL or given together.  With
 *   MOE_MX_EPI_SWIGLU it holds the up-projection rows (required).  Otherwise, if given, columns
 *   k >= b2_k of B come from it, at column k - b2_k (b2_k a multiple of 128 in (0, K)): the gate/up
 *   data gradient contracts [dA | dB] with W1 and W3 stacked along K;
 *   offsets [G+1] int32 device (clamped to [0, M]; rows outside every group are not written).
 *   q_codes / q_scales (NULL or given together; SwiGLU epilogues only): also write the MXFP8 of the
 *   bf16 rows just stored, along the rows (as moe_mx_quantize_rows would): H [M, N] for
 *   MOE_MX_EPI_SWIGLU, [dA | dB] [M, 2N] for MOE_MX_EPI_SWIGLU_BWD; codes [M, N or 2N], scales /32.
 * K must be a multiple of 128, N of 128 (64 for MOE_MX_EPI_SWIGLU), both strides multiples of 128.
 * ws: moe_mx_gemm_workspace_size(G) bytes. */
size_t moe_mx_gemm_workspace_size(int32_t G);
moe_status_t moe_mx_gemm_rows(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                              const uint8_t* b_scales, int64_t b_row_stride, int64_t b_group_stride,
                              const uint8_t* b2_codes, const uint8_t* b2_scales, int64_t b2_k, const int32_t* offsets,
                              int32_t G, int64_t M, int64_t N, int64_t K, int32_t epilogue, void* out0, void* out1,
                              void* out2, const void* aux0, const void* aux1, uint8_t* q_codes, uint8_t* q_scales,
                              void* ws, size_t ws_bytes, moe_stream_t stream);

/* Grouped product over ragged CONTRACTION ranges (weight gradients):
 *   C_g[m, n] = sum_{k in [kbase[g], kbase[g+1])} A[m, k] B[n, k]
 *   a_codes [M, lda], b_codes [N, ldb] (from moe_mx_quantize_cols, same kbase), scales alike /32;
 *   rows m < split go to out0 [G, split, N], rows m >= split to out1 [G, M - split, N] (bf16);
 *   a group with no rows gets exact zeros.  kbase is device data the call cannot check: it must be
 *   non-decreasing with kbase[G] <= min(lda, ldb) (moe_mx_quantize_cols writes such a kbase).
 * M and N must be multiples of 128, lda and ldb multiples of 128, kbase multiples of 128.
 * ws: moe_mx_gemm_k_workspace_size(G, M, N) bytes (NULL allowed when that is 0; the size depends
 * on the compute units of the current device, so query it with the same device current).  When the product
 * has fewer 256x256 output tiles than the GPU has compute units, each group's K range is split and
 * the fp32 partial sums are added in split order before the single rounding to bf16 (deterministic). */
size_t moe_mx_gemm_k_workspace_size(int32_t G, int64_t M, int64_t N);
moe_status_t moe_mx_gemm_k(const uint8_t* a_codes, const uint8_t* a_scales, int64_t lda, const uint8_t* b_codes,
                           const uint8_t* b_scales, int64_t ldb, const int32_t* kbase, int32_t G, int64_t M,
                           int64_t N, int64_t split, void* out0, void* out1, void* ws, size_t ws_bytes,
                           moe_stream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* Utilities                                                                                   */

/* The calls that take a workspace, for moe_workspace_bytes. */
typedef enum {
  MOE_OP_ROUTE = 0,           /* none */
  MOE_OP_PERMUTE = 1,         /* moe_permute */
  MOE_OP_GROUPED_MLP_FWD = 2, /* moe_grouped_mlp_fwd and the single-set forward stages, routed experts */
  MOE_OP_GROUPED_MLP_BWD = 3, /* moe_grouped_mlp_bwd (routed experts) */
  MOE_OP_COMBINE = 4,         /* none */
  MOE_OP_COMBINE_BWD = 5,     /* none */
  MOE_OP_PERMUTE_BWD = 6,     /* none */
  MOE_OP_ROUTE_BWD = 7,       /* moe_route_bwd */
  MOE_OP_EXPERT_STAGE = 8,    /* moe_expert_stage, any stage, over the routed set and (fs > 0) the
                                 shared expert as a second set */
  MOE_OP_ROUTER_AUX = 9,      /* moe_router_aux */
  MOE_OP_ROUTER_AUX_BWD = 10, /* moe_router_aux_bwd */
  MOE_OP_MX_GEMM_ROWS = 11,   /* moe_mx_gemm_rows over the routed experts (and the shared expert) */
  MOE_OP_MX_GEMM_K = 12       /* moe_mx_gemm_k, both weight-gradient products of each set */
} moe_op_t;

/* Device workspace bytes that call `op` needs in a layer of T tokens of width d, each routed to
 * k of E experts of hidden width f, plus a shared expert of hidden width fs (0: none) that sees
 * every token: the routed experts are G = E groups over M = T*k rows, the shared expert one group
 * over T rows.  Equal to the matching *_workspace_size query (the largest one where the call runs
 * on both sets); a workspace of this size serves every call of that kind in such a layer.  Returns
 * 0 for a call that needs none, and 0 with the reason in moe_last_error() for an unknown op or
 * sizes outside the ranges the calls accept.  Some sizes depend on the compute units of the current
 * device: query with the device current that will run the call. */
size_t moe_workspace_bytes(int32_t op, int64_t T, int64_t d, int32_t E, int32_t k, int64_t f, int64_t fs);

const char* moe_status_string(moe_status_t status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);
/* Library version, e.g. "libmoe 0.1 gfx950". */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
