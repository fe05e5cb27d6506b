"""Pins of the oracle's backward pass: central finite differences in fp64, and torch fp64 autograd
on a dense masked formulation of the same layer (every expert on every token, times a mask).
A planted-mistake test checks that these pins catch plausible errors in the oracle.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

PARAMS = ("x", "w1", "w3", "w2", "ws1", "ws3", "ws2", "wr")


def make_problem(T, d, E, k, f, fs, seed, with_bias=True, min_gap=1e-3):
    # Draw until the k-th and (k+1)-th logits of every token are at least min_gap apart, so that
    # a finite-difference step cannot change the selection.
    rng = np.random.default_rng(seed)
    while True:
        p = dict(x=rng.standard_normal((T, d)),
                 w1=0.4 * rng.standard_normal((E, f, d)), w3=0.4 * rng.standard_normal((E, f, d)),
                 w2=0.4 * rng.standard_normal((E, d, f)),
                 ws1=0.4 * rng.standard_normal((fs, d)) if fs else None,
                 ws3=0.4 * rng.standard_normal((fs, d)) if fs else None,
                 ws2=0.4 * rng.standard_normal((d, fs)) if fs else None,
                 wr=0.5 * rng.standard_normal((E, d)),
                 b=rng.standard_normal(E) if with_bias else None,
                 dout=rng.standard_normal((T, d)))
        L = p["x"] @ p["wr"].T + (p["b"] if with_bias else 0)
        s = np.sort(L, axis=1)[:, ::-1]
        if k == E or np.min(s[:, k - 1] - s[:, k]) > min_gap:
            return p


def oracle_loss_and_grads(p, k, renormalize):
    fwd = O.layer_forward(p["x"], p["w1"], p["w3"], p["w2"], k, w_router=p["wr"], bias=p["b"],
                          ws1=p["ws1"], ws3=p["ws3"], ws2=p["ws2"], renormalize=renormalize,
                          logits_mode="dense")
    bwd = O.layer_backward(fwd, p["dout"], p["x"], p["w1"], p["w3"], p["w2"], k, w_router=p["wr"],
                           ws1=p["ws1"], ws3=p["ws3"], ws2=p["ws2"], renormalize=renormalize)
    loss = float((fwd["out"] * p["dout"]).sum())
    grads = dict(x=bwd["dx"], w1=bwd["dW1"], w3=bwd["dW3"], w2=bwd["dW2"], wr=bwd["dWr"])
    if p["ws1"] is not None:
        grads.update(ws1=bwd["dWs1"], ws3=bwd["dWs3"], ws2=bwd["dWs2"])
    return loss, grads, fwd


@pytest.mark.parametrize("renormalize", [True, False])
def test_backward_matches_central_differences(renormalize):
    T, d, E, k, f, fs = 6, 8, 4, 2, 6, 5
    p = make_problem(T, d, E, k, f, fs, seed=11)
    _, grads, _ = oracle_loss_and_grads(p, k, renormalize)
    h = 1e-6
    for name in PARAMS:
        arr = p[name]
        fd = np.zeros_like(arr)
        for ix in np.ndindex(arr.shape):
            old = arr[ix]
            arr[ix] = old + h
            lp, _, _ = oracle_loss_and_grads(p, k, renormalize)
            arr[ix] = old - h
            lm, _, _ = oracle_loss_and_grads(p, k, renormalize)
            arr[ix] = old
            fd[ix] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - grads[name])) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-6, (name, err)


def torch_dense_layer(p, mask, renormalize):
    """Every expert on every token; the gate of an unchosen expert is zero."""
    t = {n: (None if p[n] is None else torch.tensor(p[n], dtype=torch.float64, requires_grad=True))
         for n in PARAMS}
    x = t["x"]
    L = x @ t["wr"].T + torch.tensor(p["b"], dtype=torch.float64)
    m = torch.from_numpy(mask)
    if renormalize:
        g = torch.softmax(L.masked_fill(~m, float("-inf")), dim=1)
    else:
        g = torch.softmax(L, dim=1) * m
    out = torch.zeros_like(x)
    E = p["w1"].shape[0]
    for e in range(E):
        h = torch.nn.functional.silu(x @ t["w1"][e].T) * (x @ t["w3"][e].T)
        out = out + g[:, e:e + 1] * (h @ t["w2"][e].T)
    if p["ws1"] is not None:
        out = out + (torch.nn.functional.silu(x @ t["ws1"].T) * (x @ t["ws3"].T)) @ t["ws2"].T
    (out * torch.from_numpy(p["dout"])).sum().backward()
    return out.detach().numpy(), {n: t[n].grad.numpy() for n in PARAMS if t[n] is not None}


@pytest.mark.parametrize("renormalize", [True, False])
@pytest.mark.parametrize("shape", [(40, 16, 8, 3, 12, 10), (25, 8, 6, 6, 5, 0), (31, 12, 5, 1, 7, 9)])
def test_backward_matches_torch_autograd_dense_masked(renormalize, shape):
    T, d, E, k, f, fs = shape
    p = make_problem(T, d, E, k, f, fs, seed=sum(shape), min_gap=0.0)
    _, grads, fwd = oracle_loss_and_grads(p, k, renormalize)
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, fwd["topk_idx"].astype(np.int64), True, axis=1)
    out, tgrads = torch_dense_layer(p, mask, renormalize)
    np.testing.assert_allclose(fwd["out"], out, rtol=1e-11, atol=1e-11)
    for n, g in tgrads.items():
        np.testing.assert_allclose(grads[n], g, rtol=1e-10, atol=1e-10, err_msg=n)


def test_empty_expert_gets_zero_weight_gradient():
    T, d, E, k, f = 10, 6, 5, 1, 4
    p = make_problem(T, d, E, k, f, 0, seed=3, min_gap=0.0)
    p["b"] = np.array([0.0, 0.0, -1e3, 0.0, 0.0])      # expert 2 is never chosen
    _, grads, fwd = oracle_loss_and_grads(p, k, True)
    assert fwd["counts"][2] == 0
    assert np.all(grads["w1"][2] == 0) and np.all(grads["w3"][2] == 0) and np.all(grads["w2"][2] == 0)


# ----------------------------------------------------------------------- planted mistakes

def _bad_swiglu_backward(dY, X, A, B, H, w1, w3, w2, dt=np.float64):
    dX, dW1, dW3, dW2, dA, dB = O.__dict__["_orig_swiglu_backward"](dY, X, A, B, H, w1, w3, w2, dt)
    s = O.sigmoid(A)
    dH = np.asarray(dY, dt) @ np.asarray(w2, dt)
    dA_bad = dH * B * s                                  # dropped the A (1 - s) term
    return dA_bad @ np.asarray(w1, dt) + dB @ np.asarray(w3, dt), dA_bad.T @ X, dW3, dW2, dA_bad, dB


def _bad_router_grad(dgates, gates, topk_idx, E, renormalize=True, logits=None, dt=np.float64):
    return -O.__dict__["_orig_router_logit_grad"](dgates, gates, topk_idx, E, renormalize, logits, dt)


def _bad_combine_backward(dout, Y_perm, gates, dest_pos, dt=np.float64):
    dY, dg = O.__dict__["_orig_combine_backward"](dout, Y_perm, gates, dest_pos, dt)
    return dY, dg[:, ::-1].copy()                        # slots swapped


@pytest.mark.parametrize("name,bad", [("swiglu_backward", _bad_swiglu_backward),
                                      ("router_logit_grad", _bad_router_grad),
                                      ("combine_backward", _bad_combine_backward)])
def test_planted_backward_mistakes_are_caught(monkeypatch, name, bad):
    monkeypatch.setitem(O.__dict__, "_orig_" + name, getattr(O, name))
    monkeypatch.setattr(O, name, bad)
    with pytest.raises(AssertionError):
        test_backward_matches_torch_autograd_dense_masked(True, (40, 16, 8, 3, 12, 10))


def test_planted_tie_break_mistake_is_caught(monkeypatch):
    def bad_select(logits, k):      # ties to the highest index
        L = np.asarray(logits)[:, ::-1]
        order = np.argsort(-L, axis=1, kind="stable")
        return (L.shape[1] - 1 - order[:, :k]).astype(np.int32)
    from tests import test_oracle_pins as P
    monkeypatch.setattr(O, "select_topk", bad_select)
    with pytest.raises(AssertionError):
        P.test_topk_matches_brute_force(2, "integer_ties")


def test_planted_unstable_dispatch_is_caught(monkeypatch):
    orig = O.dispatch_plan

    def bad_dispatch(topk_idx, E):   # rows of each expert in descending token order
        counts, offsets, dest_pos, src_row = orig(topk_idx, E)
        src = src_row.copy()
        for e in range(E):
            src[offsets[e]:offsets[e + 1]] = src[offsets[e]:offsets[e + 1]][::-1]
        dp = np.empty_like(src)
        dp[src] = np.arange(src.size)
        return counts, offsets, dp, src
    from tests import test_oracle_pins as P
    monkeypatch.setattr(O, "dispatch_plan", bad_dispatch)
    with pytest.raises(AssertionError):
        P.test_dispatch_invariants(100, 8, 2, 0.0)
