"""Pins of the contraction axis of each of the six MXFP8 products in the layer oracle (CPU).

Each product of one expert is rebuilt here from the oracle's primitives -- the quantizers
mx_quantize_rows / mx_quantize_grouped_cols and the grouped products mx_grouped_gemm_rows /
mx_grouped_gemm_k -- with the axis every operand is quantized along written out, and must equal what
MXExperts computes (float64, to 1e-12).  The MX recipe (Olmo-core DDP MoE examples, "Other
experiments in the report", MXFP8 ablation of the MLP) is read as: every product quantizes both
operands along the axis that product sums over.

  gate/up forward      A = X W1^T, B = X W3^T      X rows along d, W1/W3 rows along d
  down forward         Y = H W2^T                  H rows along f, W2 rows along f
  down dgrad           dH = dY W2                  dY rows along d, W2 columns along d
  gate/up dgrad        dX = [dA|dB] [W1; W3]       [dA|dB] rows along 2f, [W1; W3] columns along 2f
  down wgrad           dW2 = dY^T H                dY and H columns along the expert's rows
  gate/up wgrad        dW1 = dA^T X, dW3 = dB^T X  [dA|dB] and X columns along the expert's rows

Planted mistakes -- W2 quantized along d in the down forward, dY quantized along its rows in the
down dgrad -- move Y and dX by 3e-2 and 6e-2 of their largest magnitude: far above 1e-12, so the
rebuild catches them, where a whole-layer comparison at 5e-2 could not."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import mxfp8 as MX

TOL = 1e-12


def _one_expert(seed=0, M=70, d=128, f=96):
    """Bf16 data of one expert's products (M rows, not a multiple of 32: a ragged last block)."""
    rng = np.random.default_rng(seed)
    b = lambda *s, std=1.0: MX.bf16_round(std * rng.standard_normal(s))
    return dict(X=b(M, d), W1=b(f, d, std=0.02), W3=b(f, d, std=0.02), W2=b(d, f, std=0.02), dY=b(M, d))


def _rows(m):
    """(codes, scales) of m quantized along its last axis."""
    return MX.mx_quantize_rows(m)


def _prod_rows(a, b):
    """sum_k a[m, k] b[n, k], both quantized along k (one group of all rows)."""
    ac, as_ = _rows(a)
    bc, bs = _rows(b)
    return MX.mx_grouped_gemm_rows(ac, as_, bc[None], bs[None], np.array([0, a.shape[0]]))


def _prod_over_rows(a, b, kpad=128):
    """sum_r a[r, m] b[r, n], both quantized along the rows r (blocks from the first row)."""
    off = np.array([0, a.shape[0]])
    ac, as_, kb = MX.mx_quantize_grouped_cols(a, off, kpad)
    bc, bs, kb2 = MX.mx_quantize_grouped_cols(b, off, kpad)
    assert np.array_equal(kb, kb2)
    return MX.mx_grouped_gemm_k(ac, as_, bc, bs, kb)[0]


def _rebuild(t):
    """The six products of one expert, each operand quantized along the written-out axis."""
    X, W1, W3, W2, dY = t["X"], t["W1"], t["W3"], t["W2"], t["dY"]
    f = W1.shape[0]
    st = MX.bf16_round
    A = _prod_rows(X, W1)                                  # over d: X rows, W1 rows (W1 is [f, d])
    B = _prod_rows(X, W3)
    H = A / (1.0 + np.exp(-A)) * B
    Y = _prod_rows(st(H), W2)                              # over f: H rows, W2 rows (W2 is [d, f])
    dH = _prod_rows(dY, W2.T.copy())                       # over d: dY rows, W2 columns
    a, b = st(A), st(B)
    s = 1.0 / (1.0 + np.exp(-a))
    dAB = st(np.concatenate([dH * b * s * (1.0 + a * (1.0 - s)), dH * a * s], axis=1))
    dX = _prod_rows(dAB, np.concatenate([W1.T, W3.T], axis=1))   # over 2f: [W1; W3] columns
    dW2 = _prod_over_rows(dY, st(H))                       # [d, f] over the rows
    dWab = _prod_over_rows(dAB, X)                         # [2f, d] over the rows
    return dict(A=A, B=B, H=H, Y=Y, dX=dX, dW1=dWab[:f], dW3=dWab[f:], dW2=dW2)


def _mxexperts(t, experts=None):
    ex = experts or MX.MXExperts()
    A, B, H, Y = ex.forward(t["X"], t["W1"], t["W3"], t["W2"])
    dX, dW1, dW3, dW2, _, _ = ex.backward(t["dY"], t["X"], A, B, H, t["W1"], t["W3"], t["W2"])
    return dict(A=A, B=B, H=H, Y=Y, dX=dX, dW1=dW1, dW3=dW3, dW2=dW2)


def _worst(got, ref):
    return {k: O.max_abs_rel_err(got[k], ref[k]) for k in ref}


@pytest.mark.parametrize("seed,M", [(0, 70), (1, 32), (2, 129), (3, 1)])
def test_every_product_is_quantized_along_its_contraction_axis(seed, M):
    t = _one_expert(seed, M=M)
    errs = _worst(_mxexperts(t), _rebuild(t))
    assert all(e <= TOL for e in errs.values()), errs


class _W2AlongD(MX.MXExperts):
    """Planted mistake: the down forward quantizes W2 [d, f] along d instead of f."""

    def forward(self, X, w1, w3, w2, dt=np.float64):
        Xq = self.mx(X)
        A = Xq @ self.mx(w1).T
        B = Xq @ self.mx(w3).T
        H = A / (1.0 + np.exp(-A)) * B
        Y = self.mx(self.st(H)) @ self.mx(np.asarray(w2, np.float64).T)   # W2 blocks of 32 along d
        return A, B, H, Y


class _DYAlongRowsInDgrad(MX.MXExperts):
    """Planted mistake: the down dgrad quantizes dY along its rows (the wgrad's axis) instead of d."""

    def backward(self, dY, X, A, B, H, w1, w3, w2, dt=np.float64):
        out = list(super().backward(dY, X, A, B, H, w1, w3, w2, dt))
        w2 = np.asarray(w2, np.float64)
        dH = self.mx(self.st(dY).T).T @ self.mx(w2.T).T
        a, b = self.st(A), self.st(B)
        s = 1.0 / (1.0 + np.exp(-a))
        dAB = self.st(np.concatenate([dH * b * s * (1.0 + a * (1.0 - s)), dH * a * s], axis=1))
        out[0] = self.mx(dAB) @ self.mx(np.concatenate([w1.T, w3.T], axis=1)).T
        return tuple(out)


@pytest.mark.parametrize("planted,key", [(_W2AlongD, "Y"), (_DYAlongRowsInDgrad, "dX")])
def test_planted_wrong_axis_fails_the_rebuild(planted, key):
    t = _one_expert(5, M=96)
    errs = _worst(_mxexperts(t, planted()), _rebuild(t))
    assert errs[key] > 1e-4, errs          # the plant is caught by a wide margin
    assert errs[key] > 1e6 * TOL


def test_max_abs_rel_err_by_hand():
    # max |got - ref| = |2.5 - 2| = 0.5 and max |ref| = |-4| = 4: 0.125
    assert O.max_abs_rel_err([1.0, 2.5, -4.0], [1.0, 2.0, -4.0]) == 0.125
    # the denominator is the largest reference magnitude, not the entry's own
    assert O.max_abs_rel_err([0.0, 10.0], [1e-9, 10.0]) == pytest.approx(1e-10)
    assert O.max_abs_rel_err([3.0], [-3.0]) == 2.0
    assert O.max_abs_rel_err(np.zeros(4), np.zeros(4)) == 0.0
    assert O.max_abs_rel_err([1e-30], [0.0]) == float("inf")
    assert O.max_abs_rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
