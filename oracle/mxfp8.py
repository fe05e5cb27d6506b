"""CPU oracle of the MXFP8 grouped GEMM: microscaled FP8 quantization and the scaled products.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module. The product path (the HIP library and its Python binding) never does.

The pages name MXFP8 as the precision of the two Ultra operating points (Olmo-core DDP MoE
examples, "Production throughput runs", operating-point table, column "Precision, recompute") and
list an MXFP8 recipe ablation for the MLP (same page, "Other experiments in the report"). They do
not define the format. The reading taken here is the OCP Microscaling Formats (MX) v1.0
specification's MXFP8 with E4M3 elements:
  * elements are OFP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals, no
    infinities, largest finite magnitude 448 (code 0x7E), 0x7F / 0xFF are NaN;
  * one E8M0 scale (a power of two 2**(s - 127), s a byte) per block of 32 consecutive elements
    along the contraction axis;
  * quantizing a block: shared exponent = floor(log2(max |v|)) - 8 (8 = the largest normal
    exponent of E4M3), clamped to the E8M0 range [-127, 127]; an all-zero block takes -127; every
    element v becomes E4M3(v / 2**shared) rounded to nearest, ties to even, magnitudes above 448
    saturated to 448 (the specification leaves overflow handling to the implementation);
  * a product of two MX blocks is the product of their scales times the dot product of their
    elements, so a GEMM over MX operands equals the product of the dequantized matrices.
Contraction lengths that are not a multiple of 32 are padded with zeros to the next multiple
(zeros do not change any block's maximum or any dot product).

Precision: quantization decides integer codes, so it runs on exact values (float64 holds every
fp32 input and every E4M3 value exactly; a division by a power of two is exact). The products are
float64 matmuls of the dequantized operands.

Pins (tests/test_oracle_mxfp8.py): the E4M3 value table from its bit fields against a brute-force
nearest-value search; the format's fixed points (448, 2**-6, 2**-9, tie cases); the scale's
tightness (each non-zero block's largest code is at least 256); the per-element error bound of the
rounding; lossless round trips of blocks already on the grid; exact integer products; a planted
off-by-one in the shared exponent that the pins catch.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32              # elements per shared scale (OCP MX v1.0)
E4M3_MAX = 448.0        # largest finite E4M3 magnitude
E4M3_EMAX = 8           # exponent of the largest normal E4M3 binade (448 = 1.75 * 2**8)
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_QUANTUM = 2.0 ** -9
SCALE_BIAS = 127        # E8M0: value 2**(byte - 127)


def e4m3_round(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value to each y (exact float64 inputs), ties to even, saturated to +-448.

    In the binade [2**E, 2**(E+1)) with E >= -6 the spacing is 2**(E-3) (3 mantissa bits); below
    2**-6 the spacing is the subnormal quantum 2**-9.  numpy's round is half-to-even, and y divided
    by a power of two is exact, so rint(y / q) * q is the correctly rounded value.
    """
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 of a float64 can land one ulp off near a power of two: fix the binade exactly.
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    q = np.where(a >= E4M3_MIN_NORMAL, np.exp2(e - 3), E4M3_SUBNORMAL_QUANTUM)
    r = np.rint(a / q) * q
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, y)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Byte code of E4M3 values (each v must already be an E4M3 value): sign | exponent | mantissa.
    Zero encodes as 0x00 (a negative zero as 0x80)."""
    v = np.asarray(v, np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    code = np.zeros(a.shape, np.uint8)
    sub = (a > 0) & (a < E4M3_MIN_NORMAL)
    code[sub] = np.rint(a[sub] / E4M3_SUBNORMAL_QUANTUM).astype(np.uint8)
    nrm = a >= E4M3_MIN_NORMAL
    if np.any(nrm):
        e = np.floor(np.log2(a[nrm]))
        e = np.where(np.exp2(e) > a[nrm], e - 1, e)
        m = a[nrm] / np.exp2(e) - 1.0                          # in [0, 1), a multiple of 1/8
        mant = np.rint(m * 8).astype(np.int64)
        assert np.all(mant * 0.125 == m), "not an E4M3 value"
        code[nrm] = ((e.astype(np.int64) + 7) << 3 | mant).astype(np.uint8)
    return code | sign


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Value of E4M3 byte codes (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    mt = c & 0x7
    v = np.where(ex == 0, mt * E4M3_SUBNORMAL_QUANTUM, (1.0 + mt / 8.0) * np.exp2(ex - 7.0))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def shared_exponent(block_amax: np.ndarray) -> np.ndarray:
    """floor(log2(amax)) - 8, clamped to [-127, 127]; -127 for an all-zero block (OCP MX v1.0)."""
    a = np.asarray(block_amax, np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = e - E4M3_EMAX
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 of a matrix along its last axis (the contraction axis).

    x: [R, K] float values (any float dtype; taken exactly).  K is padded with zeros to a multiple
    of 32.  Returns (codes [R, Kp] uint8 E4M3, scales [R, Kp/32] uint8 E8M0 bytes)."""
    x = np.asarray(x, np.float64)
    R, K = x.shape
    Kp = -(-K // BLOCK) * BLOCK
    xp = np.zeros((R, Kp))
    xp[:, :K] = x
    blocks = xp.reshape(R, Kp // BLOCK, BLOCK)
    e = shared_exponent(np.abs(blocks).max(axis=2)) if Kp else np.zeros((R, 0), np.int64)
    y = blocks / np.exp2(e)[:, :, None]
    q = e4m3_round(y)
    return e4m3_encode(q).reshape(R, Kp), (e + SCALE_BIAS).astype(np.uint8)


def mx_dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values of MXFP8 rows: element * 2**(scale byte - 127)."""
    R, Kp = codes.shape
    v = e4m3_decode(codes).reshape(R, Kp // BLOCK, BLOCK)
    return (v * np.exp2(scales.astype(np.float64) - SCALE_BIAS)[:, :, None]).reshape(R, Kp)


def mx_quantize_grouped_cols(x: np.ndarray, offsets: np.ndarray, kpad: int
                             ) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """MXFP8 of a [R, N] matrix along its rows, one row range per group (the contraction axis of a
    weight gradient runs over the rows an expert received).

    Group g covers rows offsets[g]..offsets[g+1]-1.  Its rows are padded with zeros to a multiple of
    `kpad` (itself a multiple of 32) and the result is stored transposed, contraction axis last:
    codes [N, Ktot] with group g at columns kbase[g]..kbase[g+1]-1, scales [N, Ktot/32].
    Returns (codes, scales, kbase)."""
    x = np.asarray(x, np.float64)
    R, N = x.shape
    assert kpad % BLOCK == 0
    G = len(offsets) - 1
    lens = np.diff(offsets)
    kp = -(-lens // kpad) * kpad
    kbase = np.concatenate([[0], np.cumsum(kp)]).astype(np.int64)
    Ktot = int(kbase[-1])
    codes = np.zeros((N, Ktot), np.uint8)
    scales = np.full((N, Ktot // BLOCK), SCALE_BIAS - 127, np.uint8)
    for g in range(G):
        seg = x[offsets[g]:offsets[g + 1]].T                  # [N, len_g], contraction axis last
        segp = np.zeros((N, int(kp[g])))
        segp[:, :seg.shape[1]] = seg
        c, s = mx_quantize_rows(segp)
        codes[:, kbase[g]:kbase[g + 1]] = c
        scales[:, kbase[g] // BLOCK:kbase[g + 1] // BLOCK] = s
    return codes, scales, kbase


def mx_grouped_gemm_rows(a_codes, a_scales, b_codes, b_scales, offsets) -> np.ndarray:
    """Grouped product over ragged row ranges: for group g, rows offsets[g]..offsets[g+1]-1 of A
    times group g's B transposed.  A: [M, Kp] MX rows; B: [G, N, Kp] MX rows (one matrix per group).
    Returns C [M, N] float64 = dequant(A_g) @ dequant(B_g)^T."""
    A = mx_dequantize_rows(a_codes, a_scales)
    G, N, Kp = b_codes.shape
    C = np.zeros((A.shape[0], N))
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            Bg = mx_dequantize_rows(b_codes[g], b_scales[g])
            C[lo:hi] = A[lo:hi] @ Bg.T
    return C


def mx_grouped_gemm_k(a_codes, a_scales, b_codes, b_scales, kbase) -> np.ndarray:
    """Grouped product over ragged contraction ranges: for group g, columns kbase[g]..kbase[g+1]-1
    of A [M, Ktot] and B [N, Ktot].  Returns C [G, M, N] float64."""
    A = mx_dequantize_rows(a_codes, a_scales)
    B = mx_dequantize_rows(b_codes, b_scales)
    G = len(kbase) - 1
    C = np.zeros((G, A.shape[0], B.shape[0]))
    for g in range(G):
        lo, hi = int(kbase[g]), int(kbase[g + 1])
        C[g] = A[:, lo:hi] @ B[:, lo:hi].T
    return C


# ---------------------------------------------------------------------------------------------
# The expert MLP with MXFP8 products (forward and backward)
#
# Every product of the SwiGLU expert is taken on MX operands quantized along its own contraction
# axis (the recipe's reading: activations and weights are quantized afresh for each product, along
# the axis it sums over).  Inputs of a quantization are the values the layer stores: x, weights and
# the upstream gradient are bf16 data; H, dY and [dA | dB] are stored as bf16 before they are
# quantized; the SwiGLU backward reads the bf16 stash of A and B.  Quantization decides codes, so it
# runs on those bf16 values; the products are float64.  A weight gradient's contraction runs over
# the rows one expert received, whose 32-row blocks start at the expert's first row.


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each element (via float32; ties to even at both steps)."""
    f = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


class MXExperts:
    """Expert arithmetic for moe_oracle.layer_forward / layer_backward (argument ``experts``).

    quantize=False and store_bf16=False turn every quantization and every bf16 storage rounding into
    the identity: the result is then the plain SwiGLU expert (the structural pin of this class)."""

    def __init__(self, quantize: bool = True, store_bf16: bool = True):
        self.quantize = quantize
        self.store_bf16 = store_bf16

    def mx(self, m: np.ndarray) -> np.ndarray:
        """Values of m after MXFP8 quantization along its last axis."""
        m = np.asarray(m, np.float64)
        if not self.quantize or m.size == 0:
            return m
        c, s = mx_quantize_rows(m.reshape(-1, m.shape[-1]))
        return mx_dequantize_rows(c, s)[:, :m.shape[-1]].reshape(m.shape)

    def st(self, m: np.ndarray) -> np.ndarray:
        """Values of m as the layer stores them (bf16)."""
        return bf16_round(m) if self.store_bf16 else np.asarray(m, np.float64)

    def forward(self, X, w1, w3, w2, dt=np.float64):
        """A = X W1^T, B = X W3^T (contraction over d), H = silu(A) B, Y = H W2^T (over f)."""
        Xq = self.mx(X)
        A = Xq @ self.mx(w1).T
        B = Xq @ self.mx(w3).T
        H = A / (1.0 + np.exp(-A)) * B
        Y = self.mx(self.st(H)) @ self.mx(w2).T
        return A, B, H, Y

    def backward(self, dY, X, A, B, H, w1, w3, w2, dt=np.float64):
        """dH = dY W2 (over d); SwiGLU backward on the stored A, B; dX = [dA | dB] [W1; W3] (over 2f);
        dW2 = dY^T H, dW1 = dA^T X, dW3 = dB^T X (over the rows)."""
        w1, w3, w2 = (np.asarray(w, np.float64) for w in (w1, w3, w2))
        dYs = self.st(dY)
        dH = self.mx(dYs) @ self.mx(w2.T).T
        a, b = self.st(A), self.st(B)
        s = 1.0 / (1.0 + np.exp(-a))
        dA = dH * b * s * (1.0 + a * (1.0 - s))
        dB = dH * a * s
        dAB = self.st(np.concatenate([dA, dB], axis=1))
        dX = self.mx(dAB) @ self.mx(np.concatenate([w1.T, w3.T], axis=1)).T
        Hs, Xs = self.st(H), np.asarray(X, np.float64)
        dYq, Hq, ABq, Xq = (self.mx(m.T) for m in (dYs, Hs, dAB, Xs))
        dW2 = dYq @ Hq.T
        f = w1.shape[0]
        dW1 = ABq[:f] @ Xq.T
        dW3 = ABq[f:] @ Xq.T
        return dX, dW1, dW3, dW2, dA, dB

    def grouped_forward(self, X_perm, offsets, W1, W3, W2, dt=np.float64):
        M = X_perm.shape[0]
        E, f, d = np.asarray(W1).shape
        A, B, H, Y = np.zeros((M, f)), np.zeros((M, f)), np.zeros((M, f)), np.zeros((M, d))
        for e in range(E):
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 > r0:
                A[r0:r1], B[r0:r1], H[r0:r1], Y[r0:r1] = self.forward(X_perm[r0:r1], W1[e], W3[e], W2[e])
        return A, B, H, Y

    def grouped_backward(self, dY, X_perm, A, B, H, offsets, W1, W3, W2, dt=np.float64):
        M = X_perm.shape[0]
        E, f, d = np.asarray(W1).shape
        dX, dA, dB = np.zeros((M, d)), np.zeros((M, f)), np.zeros((M, f))
        dW1, dW3, dW2 = np.zeros((E, f, d)), np.zeros((E, f, d)), np.zeros((E, d, f))
        for e in range(E):
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 > r0:
                sl = slice(r0, r1)
                dX[sl], dW1[e], dW3[e], dW2[e], dA[sl], dB[sl] = self.backward(
                    dY[sl], X_perm[sl], A[sl], B[sl], H[sl], W1[e], W3[e], W2[e])
        return dX, dW1, dW3, dW2, dA, dB
