"""CPU oracle of one GPU's share of the Olmo-core 3 mixture-of-experts block.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module. The product path (the HIP library and its Python binding) never does.

What the layer computes, and where the pages state it:
  * a router picks experts for every token separately (Scaling Trillion-Parameter Models: The
    Architecture of Olmo-core 3, "Code Snippet": route_input calls select_expert per token);
  * each token goes to its top-4 experts and to one shared expert; routing is either learned or
    random (Olmo-core DDP MoE examples, "Production throughput runs" and its operating-point table);
  * tokens move to experts that stay resident; the experts do not move (Olmo-core 3 Opens Large
    MoE Training, "Enhanced Key Takeaways" and "Technical Deep Dive").
The pages give no formulas. Readings taken where they are silent:
  router logits are fp32, summed in index order one rounding per step, then + bias; selection is
  the k largest logits, ties to the lowest expert index, -0 equal to +0; gates are a softmax over
  the k chosen logits; the expert MLP is SwiGLU, silu(x W1^T) * (x W3^T) then W2^T, no biases; the
  shared expert is added with weight 1; no capacity limit (dropless); within one expert, rows keep
  ascending token order.

Precision: the router logits decide integers (the selection), so they are computed in fp32 in
the fixed order above, exactly as the GPU must. Everything after the selection is computed in
``dt`` (float64 unless a caller asks otherwise). No blocking, fusion or reordering: each function
is the plain definition, with numpy matmul, sort and exp as the only library steps.

Pins (tests/test_oracle_*.py): brute-force top-k with forced ties and signed zeros; a scalar
fp32 loop for the logits; bijection/stability/count invariants of the permutation; E=1,k=1 equal
to torch's dense SwiGLU; identical experts; k=E equal to a dense soft mixture; central finite
differences; torch fp64 autograd on a dense masked formulation; for the load-balancing loss, the
balanced-routing and single-expert closed forms, zero row sums of its gradient, finite differences
and autograd.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------------------------
# Router


def canonical_router_logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None = None
                            ) -> np.ndarray:
    """fp32 router logits L[t, e] = fl(...fl(fl(x[t,0] w[e,0]) + fl(x[t,1] w[e,1]))... + b[e]).

    One fp32 rounding after every product and every addition, index order 0..d-1, no fused
    multiply-add; the bias (if any) is added last.  Routing decisions are taken on these bits.
    """
    x = np.asarray(x, np.float32)
    w = np.asarray(w_router, np.float32)
    T, d = x.shape
    E = w.shape[0]
    assert w.shape == (E, d)
    acc = np.zeros((T, E), np.float32)
    for i in range(d):
        prod = x[:, i:i + 1] * w[None, :, i]          # fp32 product, rounded
        acc = acc + prod                              # fp32 sum, rounded
    if bias is not None:
        acc = acc + np.asarray(bias, np.float32)[None, :]
    return acc


def dense_router_logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None = None,
                        dt=np.float64) -> np.ndarray:
    """Router logits in ``dt`` by matmul (used only where the logits must be differentiable in
    high precision, e.g. finite-difference checks; routing on the GPU uses the fp32 bits)."""
    L = np.asarray(x, dt) @ np.asarray(w_router, dt).T
    if bias is not None:
        L = L + np.asarray(bias, dt)[None, :]
    return L


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, largest first, equal values by lower index.

    A stable sort of the negated logits is exactly that order (IEEE comparison, so -0 == +0).
    numpy's sort places NaN after every number, so a NaN logit ranks below -inf and NaNs rank among
    themselves by index: every selected index is a real expert whatever the logits hold.
    """
    order = np.argsort(-np.asarray(logits), axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def gate_weights(logits: np.ndarray, topk_idx: np.ndarray, renormalize: bool = True, dt=np.float64
                 ) -> np.ndarray:
    """Gate weight of each chosen expert.

    renormalize=True: softmax over the k chosen logits (equal, up to rounding, to a softmax over
    all E followed by renormalisation over the chosen k).  renormalize=False: the full softmax
    probability of each chosen expert.
    """
    L = np.asarray(logits, dt)
    if renormalize:
        sel = np.take_along_axis(L, topk_idx.astype(np.int64), axis=1)
        z = np.exp(sel - sel[:, :1])                 # sel[:, 0] is the row maximum
        return z / z.sum(axis=1, keepdims=True)
    m = L.max(axis=1, keepdims=True)
    p = np.exp(L - m)
    p = p / p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, topk_idx.astype(np.int64), axis=1)


# ---------------------------------------------------------------------------------------------
# Dispatch: histogram, prefix sum, permutation


def dispatch_plan(topk_idx: np.ndarray, E: int):
    """Expert-major layout of the T*k (token, slot) assignments.

    Assignment a = t*k + j goes to expert topk_idx[t, j].  Rows are ordered by expert, and within
    an expert by a (a stable sort of the assignments by expert id).  Returns
      counts[E]      rows per expert
      offsets[E+1]   exclusive prefix sum of counts (offsets[E] = T*k)
      dest_pos[T*k]  row of assignment a in the expert-major layout
      src_row[T*k]   assignment held by row p (inverse of dest_pos)
    """
    flat = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    src_row = np.argsort(flat, kind="stable")
    dest_pos = np.empty_like(src_row)
    dest_pos[src_row] = np.arange(flat.size)
    return (counts.astype(np.int32), offsets.astype(np.int32), dest_pos.astype(np.int32),
            src_row.astype(np.int32))


def permute_rows(x: np.ndarray, src_row: np.ndarray, k: int) -> np.ndarray:
    """Row p of the permuted activations is token src_row[p] // k (a pure copy)."""
    return np.asarray(x)[np.asarray(src_row, np.int64) // k]


# ---------------------------------------------------------------------------------------------
# Expert MLP (SwiGLU)


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def swiglu_forward(X, w1, w3, w2, dt=np.float64):
    """A = X W1^T, B = X W3^T, H = silu(A) * B, Y = H W2^T (w1, w3: [f, d]; w2: [d, f])."""
    X = np.asarray(X, dt)
    A = X @ np.asarray(w1, dt).T
    B = X @ np.asarray(w3, dt).T
    H = A * sigmoid(A) * B
    Y = H @ np.asarray(w2, dt).T
    return A, B, H, Y


def swiglu_backward(dY, X, A, B, H, w1, w3, w2, dt=np.float64):
    """Gradients of swiglu_forward given dL/dY.

    dH = dY W2; dA = dH * B * s * (1 + A (1 - s)) with s = sigmoid(A); dB = dH * silu(A);
    dW2 = dY^T H; dW1 = dA^T X; dW3 = dB^T X; dX = dA W1 + dB W3.
    """
    dY = np.asarray(dY, dt)
    X = np.asarray(X, dt)
    w1 = np.asarray(w1, dt)
    w3 = np.asarray(w3, dt)
    w2 = np.asarray(w2, dt)
    dH = dY @ w2
    s = sigmoid(A)
    dA = dH * B * s * (1.0 + A * (1.0 - s))
    dB = dH * A * s
    dW2 = dY.T @ H
    dW1 = dA.T @ X
    dW3 = dB.T @ X
    dX = dA @ w1 + dB @ w3
    return dX, dW1, dW3, dW2, dA, dB


def grouped_swiglu_forward(X_perm, offsets, W1, W3, W2, dt=np.float64):
    """Expert e applies its own SwiGLU to rows offsets[e]:offsets[e+1] of the permuted activations."""
    M = X_perm.shape[0]
    E, f, d = np.asarray(W1).shape
    A = np.zeros((M, f), dt)
    B = np.zeros((M, f), dt)
    H = np.zeros((M, f), dt)
    Y = np.zeros((M, d), dt)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            A[r0:r1], B[r0:r1], H[r0:r1], Y[r0:r1] = swiglu_forward(X_perm[r0:r1], W1[e], W3[e], W2[e], dt)
    return A, B, H, Y


def grouped_swiglu_backward(dY, X_perm, A, B, H, offsets, W1, W3, W2, dt=np.float64):
    """Per-expert swiglu_backward; an expert with no rows gets exactly zero weight gradients."""
    M = X_perm.shape[0]
    E, f, d = np.asarray(W1).shape
    dX = np.zeros((M, d), dt)
    dW1 = np.zeros((E, f, d), dt)
    dW3 = np.zeros((E, f, d), dt)
    dW2 = np.zeros((E, d, f), dt)
    dA = np.zeros((M, f), dt)
    dB = np.zeros((M, f), dt)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            sl = slice(r0, r1)
            dX[sl], dW1[e], dW3[e], dW2[e], dA[sl], dB[sl] = swiglu_backward(
                dY[sl], X_perm[sl], A[sl], B[sl], H[sl], W1[e], W3[e], W2[e], dt)
    return dX, dW1, dW3, dW2, dA, dB


class PlainExperts:
    """The expert MLP arithmetic of the layer: exact SwiGLU in the oracle's precision."""
    grouped_forward = staticmethod(grouped_swiglu_forward)
    forward = staticmethod(swiglu_forward)
    grouped_backward = staticmethod(grouped_swiglu_backward)
    backward = staticmethod(swiglu_backward)


# ---------------------------------------------------------------------------------------------
# Combine and its backward


def combine(Y_perm, gates, dest_pos, shared_out=None, dt=np.float64):
    """out[t] = shared_out[t] + sum_j gates[t, j] * Y_perm[dest_pos[t*k + j]]."""
    T, k = gates.shape
    rows = np.asarray(dest_pos, np.int64).reshape(T, k)
    Yg = np.asarray(Y_perm, dt)[rows]                 # [T, k, d]
    out = (np.asarray(gates, dt)[:, :, None] * Yg).sum(axis=1)
    if shared_out is not None:
        out = out + np.asarray(shared_out, dt)
    return out


def combine_backward(dout, Y_perm, gates, dest_pos, dt=np.float64):
    """dY_perm[dest_pos[t*k+j]] = gates[t,j] dout[t];  dgates[t,j] = <dout[t], Y_perm[dest_pos[t*k+j]]>."""
    T, k = gates.shape
    dout = np.asarray(dout, dt)
    rows = np.asarray(dest_pos, np.int64).reshape(T, k)
    dY = np.zeros((T * k, dout.shape[1]), dt)
    dY[rows] = np.asarray(gates, dt)[:, :, None] * dout[:, None, :]
    dgates = np.einsum("td,tkd->tk", dout, np.asarray(Y_perm, dt)[rows])
    return dY, dgates


def permute_backward(dX_perm, dest_pos, k, addends=(), dt=np.float64):
    """dx[t] = sum_j dX_perm[dest_pos[t*k+j]] + sum of the addends' row t."""
    Tk, d = dX_perm.shape
    T = Tk // k
    rows = np.asarray(dest_pos, np.int64).reshape(T, k)
    dx = np.asarray(dX_perm, dt)[rows].sum(axis=1)
    for a in addends:
        if a is not None:
            dx = dx + np.asarray(a, dt)
    return dx


# ---------------------------------------------------------------------------------------------
# Router backward


def router_logit_grad(dgates, gates, topk_idx, E, renormalize=True, logits=None, dt=np.float64):
    """dL/dlogits [T, E] of the gate weights.

    renormalize=True: softmax over the chosen k, so dL[t, S_j] = g_j (dg_j - sum_i g_i dg_i) and 0
    for experts not chosen (the selection itself is piecewise constant).
    renormalize=False: full softmax p over E, chosen probabilities returned, so
    dL[t, e] = p_e (dp_e - sum_i p_i dp_i) with dp the dgates scattered onto the chosen experts.
    """
    T, k = gates.shape
    idx = np.asarray(topk_idx, np.int64)
    g = np.asarray(gates, dt)
    dg = np.asarray(dgates, dt)
    dL = np.zeros((T, E), dt)
    if renormalize:
        s = (g * dg).sum(axis=1, keepdims=True)
        np.put_along_axis(dL, idx, g * (dg - s), axis=1)
        return dL
    L = np.asarray(logits, dt)
    m = L.max(axis=1, keepdims=True)
    p = np.exp(L - m)
    p = p / p.sum(axis=1, keepdims=True)
    dp = np.zeros((T, E), dt)
    np.put_along_axis(dp, idx, dg, axis=1)
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def load_balancing_loss(logits, counts, k, weight, dt=np.float64):
    """Auxiliary load-balancing loss of the router and the router statistics it is built from.

    The pages name only the loss weights of their runs, 0.02 to 0.50 (Olmo-core DDP MoE examples,
    "Other experiments in the report"), not the formula.  Reading taken: the loss is
        weight * E * sum_e f_e P_e,
    f_e = count_e / (T k), the fraction of the T k assignments routed to expert e, and P_e the mean
    over the tokens of the softmax over all E logits.  f comes from the selection, which is
    piecewise constant, so only P carries a gradient.  Returns (loss, P, f).
    """
    L = np.asarray(logits, dt)
    T, E = L.shape
    m = L.max(axis=1, keepdims=True)
    p = np.exp(L - m)
    p = p / p.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)
    f = np.asarray(counts, dt) / (T * k)
    return weight * E * (f * P).sum(), P, f


def load_balancing_loss_grad(logits, f, weight, dt=np.float64):
    """dloss/dlogits [T, E] of load_balancing_loss at fixed f: the softmax Jacobian applied to
    c f with c = weight E / T, G[t, j] = c p[t, j] (f_j - sum_e f_e p[t, e])."""
    L = np.asarray(logits, dt)
    T, E = L.shape
    m = L.max(axis=1, keepdims=True)
    p = np.exp(L - m)
    p = p / p.sum(axis=1, keepdims=True)
    f = np.asarray(f, dt)
    c = weight * E / T
    return c * p * (f[None, :] - (p * f[None, :]).sum(axis=1, keepdims=True))


def router_backward(dL, x, w_router, dt=np.float64):
    """dW_router = dL^T x  ([E, d]);  dx_router = dL W_router  ([T, d])."""
    x = np.asarray(x, dt)
    w = np.asarray(w_router, dt)
    return dL.T @ x, dL @ w


# ---------------------------------------------------------------------------------------------
# The whole layer


def layer_forward(x, w1, w3, w2, k, *, logits=None, w_router=None, bias=None, ws1=None, ws3=None,
                  ws2=None, renormalize=True, dt=np.float64, logits_mode="canonical_fp32", lbl_weight=0.0,
                  experts=None):
    """Forward pass of the MoE layer. Returns a dict of every intermediate.

    Routing: random routing passes ``logits``; learned routing passes ``w_router`` (and optional
    ``bias``) and the logits are computed here: in the canonical fp32 order by default, or by a
    ``dt`` matmul when ``logits_mode="dense"`` (finite-difference checks only).  With learned
    routing and lbl_weight > 0 the load-balancing loss and its statistics are added (lbl, P, f).
    ``experts``: an object with the expert MLP's arithmetic (grouped_forward, forward,
    grouped_backward, backward, e.g. the MXFP8 variant); default: the plain SwiGLU above.
    """
    x = np.asarray(x)
    T, d = x.shape
    E = np.asarray(w1).shape[0]
    if logits is None:
        if logits_mode == "canonical_fp32":
            logits = canonical_router_logits(x, w_router, bias)
        elif logits_mode == "dense":
            logits = dense_router_logits(x, w_router, bias, dt)
        else:
            raise ValueError(logits_mode)
    topk_idx = select_topk(logits, k)
    gates = gate_weights(logits, topk_idx, renormalize, dt)
    counts, offsets, dest_pos, src_row = dispatch_plan(topk_idx, E)
    X_perm = permute_rows(x, src_row, k).astype(dt)
    ex = experts or PlainExperts
    A, B, H, Y = ex.grouped_forward(X_perm, offsets, w1, w3, w2, dt)
    if ws1 is not None:
        As, Bs, Hs, S = ex.forward(x, ws1, ws3, ws2, dt)
    else:
        As = Bs = Hs = S = None
    out = combine(Y, gates, dest_pos, S, dt)
    res = dict(logits=logits, topk_idx=topk_idx, gates=gates, counts=counts, offsets=offsets,
               dest_pos=dest_pos, src_row=src_row, X_perm=X_perm, A=A, B=B, H=H, Y=Y,
               As=As, Bs=Bs, Hs=Hs, S=S, out=out, lbl_weight=lbl_weight)
    if w_router is not None and lbl_weight > 0:
        res["lbl"], res["P"], res["f"] = load_balancing_loss(logits, counts, k, lbl_weight, dt)
    return res


def layer_backward(fwd, dout, x, w1, w3, w2, k, *, w_router=None, ws1=None, ws3=None, ws2=None,
                   renormalize=True, dt=np.float64, experts=None):
    """Backward pass given the forward dict and dL/dout.

    Random routing (w_router is None): the logits are data, so no router gradient and no
    router contribution to dx.  The bias, when present, is a constant and gets no gradient.
    """
    T, d = np.asarray(x).shape
    E = np.asarray(w1).shape[0]
    dY, dgates = combine_backward(dout, fwd["Y"], fwd["gates"], fwd["dest_pos"], dt)
    ex = experts or PlainExperts
    dX_perm, dW1, dW3, dW2, dA, dB = ex.grouped_backward(
        dY, fwd["X_perm"], fwd["A"], fwd["B"], fwd["H"], fwd["offsets"], w1, w3, w2, dt)
    res = dict(dY=dY, dgates=dgates, dX_perm=dX_perm, dW1=dW1, dW3=dW3, dW2=dW2, dA=dA, dB=dB)
    addends = []
    if ws1 is not None:
        dxs, dWs1, dWs3, dWs2, dAs, dBs = ex.backward(
            dout, x, fwd["As"], fwd["Bs"], fwd["Hs"], ws1, ws3, ws2, dt)
        res.update(dx_shared=dxs, dWs1=dWs1, dWs3=dWs3, dWs2=dWs2)
        addends.append(dxs)
    if w_router is not None:
        dL = router_logit_grad(dgates, fwd["gates"], fwd["topk_idx"], E, renormalize,
                               fwd["logits"], dt)
        if fwd.get("lbl_weight", 0.0) > 0:
            dL = dL + load_balancing_loss_grad(fwd["logits"], fwd["f"], fwd["lbl_weight"], dt)
        dWr, dx_router = router_backward(dL, x, w_router, dt)
        res.update(dlogits=dL, dWr=dWr, dx_router=dx_router)
        addends.append(dx_router)
    res["dx"] = permute_backward(dX_perm, fwd["dest_pos"], k, addends, dt)
    return res


def run_layer(cfg, vals: dict, dt=np.float64, renormalize=True, lbl_weight=0.0, experts=None):
    """Forward (and backward, when the workload has one) on the value dict of the inputs module."""
    fwd = layer_forward(vals["x"], vals["w1"], vals["w3"], vals["w2"], cfg.k, logits=vals["logits"],
                        w_router=vals["w_router"], bias=vals["bias"], ws1=vals["ws1"],
                        ws3=vals["ws3"], ws2=vals["ws2"], renormalize=renormalize, dt=dt,
                        lbl_weight=lbl_weight, experts=experts)
    bwd = None
    if cfg.backward:
        bwd = layer_backward(fwd, vals["dout"], vals["x"], vals["w1"], vals["w3"], vals["w2"], cfg.k,
                             w_router=vals["w_router"], ws1=vals["ws1"], ws3=vals["ws3"],
                             ws2=vals["ws2"], renormalize=renormalize, dt=dt, experts=experts)
    return fwd, bwd


def max_abs_rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor (0 when both are all zero)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
