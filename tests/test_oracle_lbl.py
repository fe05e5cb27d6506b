"""Pins of the oracle's load-balancing loss (the reading documented with the oracle: weight * E *
sum_e f_e P_e) and of its gradient: closed forms at balanced routing and with a single expert, the
zero row sums a softmax Jacobian must give, central finite differences, torch fp64 autograd of the
whole layer with the loss added, and a planted mistake.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.test_oracle_grad import make_problem


def _counts(topk_idx, E):
    return np.bincount(np.asarray(topk_idx).reshape(-1), minlength=E)


def test_balanced_routing_gives_the_weight_itself():
    # f_e = 1/E for every expert: the loss is weight * sum_e P_e = weight, whatever the logits.
    rng = np.random.default_rng(0)
    T, E, k = 48, 6, 2
    logits = 3.0 * rng.standard_normal((T, E))
    counts = np.full(E, T * k // E)
    loss, P, f = O.load_balancing_loss(logits, counts, k, 0.2)
    assert abs(loss - 0.2) < 1e-15
    assert abs(P.sum() - 1.0) < 1e-15 and np.all(f == 1.0 / E)


def test_everything_on_one_confident_expert_gives_weight_times_E():
    # All assignments (k = 1) on expert 0 and its probability ~1: loss -> weight * E.
    T, E = 10, 8
    logits = np.zeros((T, E))
    logits[:, 0] = 60.0
    counts = np.zeros(E, np.int64)
    counts[0] = T
    loss, P, f = O.load_balancing_loss(logits, counts, 1, 0.05)
    assert abs(loss - 0.05 * E) < 1e-12
    assert f[0] == 1.0 and np.all(f[1:] == 0)


def test_single_expert_loss_and_zero_gradient():
    T = 7
    logits = np.random.default_rng(1).standard_normal((T, 1))
    loss, P, f = O.load_balancing_loss(logits, np.array([T]), 1, 0.5)
    assert loss == 0.5 and P[0] == 1.0
    assert np.all(O.load_balancing_loss_grad(logits, f, 0.5) == 0)


def test_gradient_rows_sum_to_zero():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((20, 9))
    f = rng.random(9)
    G = O.load_balancing_loss_grad(logits, f, 0.3)
    assert np.max(np.abs(G.sum(axis=1))) < 1e-15
    assert np.max(np.abs(G)) > 1e-4


def test_gradient_matches_central_differences():
    rng = np.random.default_rng(3)
    T, E, k, w = 5, 6, 2, 0.37
    logits = rng.standard_normal((T, E))
    counts = rng.integers(0, 4, E)
    _, _, f = O.load_balancing_loss(logits, counts, k, w)
    G = O.load_balancing_loss_grad(logits, f, w)
    h = 1e-6
    num = np.zeros_like(logits)
    for t in range(T):
        for e in range(E):
            lp, lm = logits.copy(), logits.copy()
            lp[t, e] += h
            lm[t, e] -= h
            num[t, e] = (O.load_balancing_loss(lp, counts, k, w)[0] - O.load_balancing_loss(lm, counts, k, w)[0]) / (2 * h)
    assert np.max(np.abs(num - G)) < 1e-9


@pytest.mark.parametrize("renormalize", [True])
def test_layer_router_gradients_with_the_loss_match_autograd(renormalize):
    # Router weight gradient of (out . dout + loss): torch autograd through a dense formulation
    # (logits by matmul, softmax over the chosen k times the expert outputs, plus the loss with the
    # counts of the actual selection held constant) against the oracle's backward.
    T, d, E, k, f = 6, 5, 4, 2, 3
    p = make_problem(T, d, E, k, f, 0, seed=4, with_bias=False)
    w = 0.25
    fwd = O.layer_forward(p["x"], p["w1"], p["w3"], p["w2"], k, w_router=p["wr"], renormalize=renormalize,
                          logits_mode="dense", lbl_weight=w)
    bwd = O.layer_backward(fwd, p["dout"], p["x"], p["w1"], p["w3"], p["w2"], k, w_router=p["wr"],
                           renormalize=renormalize)
    tt = lambda a: torch.tensor(a, dtype=torch.float64)
    x, wr = tt(p["x"]), tt(p["wr"]).requires_grad_(True)
    w1, w3, w2 = tt(p["w1"]), tt(p["w3"]), tt(p["w2"])
    L = x @ wr.T
    idx = torch.tensor(fwd["topk_idx"])
    mask = torch.zeros(T, E, dtype=torch.float64).scatter_(1, idx, 1.0)
    g = torch.softmax(L.masked_fill(mask == 0, float("-inf")), dim=1)
    outs = []
    for e in range(E):
        a, b = x @ w1[e].T, x @ w3[e].T
        outs.append((torch.nn.functional.silu(a) * b) @ w2[e].T)
    out = sum(g[:, e:e + 1] * outs[e] for e in range(E))
    counts = tt(_counts(fwd["topk_idx"], E).astype(np.float64))
    P = torch.softmax(L, dim=1).mean(dim=0)
    lbl = w * E * ((counts / (T * k)) * P).sum()
    assert abs(lbl.item() - fwd["lbl"]) < 1e-13
    ((out * tt(p["dout"])).sum() + lbl).backward()
    assert np.max(np.abs(wr.grad.numpy() - bwd["dWr"])) < 1e-10


def test_planted_sign_mistake_is_caught(monkeypatch):
    real = O.load_balancing_loss_grad
    monkeypatch.setattr(O, "load_balancing_loss_grad", lambda L, f, w, dt=np.float64: -real(L, f, w, dt))
    with pytest.raises(AssertionError):
        test_gradient_matches_central_differences()
