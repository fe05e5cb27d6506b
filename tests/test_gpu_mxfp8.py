"""MXFP8 quantization and grouped GEMMs of libmoe against the CPU oracle (GPU).

Codes, scale bytes and group column offsets must match the oracle bit for bit.  Products: the
oracle multiplies the dequantized operands in float64; the device accumulates exact products in
fp32 and rounds the result to bf16 once, so the max-abs-relative error is bounded by bf16's half
ulp (2^-9) plus the fp32 accumulation error; the tests allow 4e-3."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_20_amd import libmoe as L
from oracle import mxfp8 as MX
from tests.gpu_helpers import DEV, as_dtype_values, assert_close, dev_tensor, log, tnp

pytestmark = pytest.mark.gpu

TOL = 4e-3


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def u8(t):
    return t.cpu().numpy().astype(np.uint8)


def awkward_blocks(rng, R, K):
    """bf16 values with per-block magnitudes spread over 2^-30..2^30, all-zero blocks, saturating
    blocks (a block maximum just under a power of two) and exact rounding ties."""
    x = rng.standard_normal((R, K))
    nb = K // 32
    scale = np.exp2(rng.integers(-30, 31, size=(R, nb)))
    x = (x.reshape(R, nb, 32) * scale[:, :, None]).reshape(R, K)
    z = rng.random((R, nb)) < 0.05
    x.reshape(R, nb, 32)[z] = 0.0
    sat = rng.random((R, nb)) < 0.05
    blk = x.reshape(R, nb, 32)
    blk[sat, 0] = 500.0 * np.sign(blk[sat, 0] + 0.5)       # rounds past 448: saturates
    tie = rng.random((R, nb)) < 0.05
    blk[tie, 1] = 2.0 ** 8 * 1.0625                        # halfway between two E4M3 values at scale 1
    blk[tie, 2] = 2.0 ** 8 * (1.0 + 3 / 16)                # the other parity
    return as_dtype_values(x, "bf16")


@pytest.mark.parametrize("R,K,pad", [(333, 2048, 0), (1, 32, 0), (1000, 96, 64), (64, 1024, 8)])
def test_quantize_rows_bit_exact(R, K, pad):
    log(f"mx quantize rows R={R} K={K} pad={pad}")
    rng = np.random.default_rng(R + K)
    x = awkward_blocks(rng, R, K)
    ldx = K + pad
    xs = np.zeros((R, ldx), np.float32)
    xs[:, :K] = x
    codes = torch.empty((R, K), dtype=torch.uint8, device=DEV)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=DEV)
    L.moe_mx_quantize_rows(dev_tensor(xs, "bf16"), R, K, ldx, codes, scales)
    torch.cuda.synchronize()
    rc, rs = MX.mx_quantize_rows(x)
    assert np.array_equal(u8(scales), rs), "scale bytes differ"
    assert np.array_equal(u8(codes), rc), "E4M3 codes differ"


def every_finite_bf16_blocks():
    """Every finite bf16 value, twice: once in blocks of 32 values of similar magnitude (sorted, so a
    block's maximum sits just above its elements) and once in blocks led by a power of two far larger
    than the rest (so small elements land in E4M3's subnormal range or round to signed zero)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]                         # drop Inf / NaN
    vals = (bits << 16).view(np.float32).astype(np.float64)
    srt = vals[np.argsort(np.abs(vals), kind="stable")]
    n = len(srt) // 31 * 31
    lead = np.exp2(np.floor(np.log2(np.maximum(np.abs(srt[:n:31]), 2.0 ** -126))) + 12)
    lead = np.minimum(lead, 2.0 ** 127)
    blocks = np.concatenate([lead[:, None], srt[:n].reshape(-1, 31)], axis=1)
    both = np.concatenate([np.resize(srt, (len(srt) + 31) // 32 * 32), blocks.ravel()])
    both = np.resize(both, (len(both) + 1023) // 1024 * 1024)
    return both.reshape(-1, 1024)


def test_quantize_rows_every_bf16_value():
    x = every_finite_bf16_blocks()
    R, K = x.shape
    log(f"mx quantize rows, every finite bf16 value: R={R} K={K}")
    codes = torch.empty((R, K), dtype=torch.uint8, device=DEV)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=DEV)
    L.moe_mx_quantize_rows(dev_tensor(x, "bf16"), R, K, K, codes, scales)
    torch.cuda.synchronize()
    rc, rs = MX.mx_quantize_rows(x)
    assert np.array_equal(u8(scales), rs), "scale bytes differ"
    assert np.array_equal(u8(codes), rc), "E4M3 codes differ"


@pytest.mark.parametrize("R,N,G,kpad,uniform", [(1000, 256, 8, 128, False), (2048, 128, 4, 128, True),
                                                (77, 64, 5, 256, False)])
def test_quantize_cols_bit_exact(R, N, G, kpad, uniform):
    log(f"mx quantize cols R={R} N={N} G={G} kpad={kpad} uniform={uniform}")
    rng = np.random.default_rng(R + N + G)
    x = awkward_blocks(rng, N, -(-R // 32) * 32)[:, :R].T.copy()     # blocks run along the rows
    if uniform:
        offsets = np.arange(G + 1) * (R // G)
        ldc = G * (-(-(R // G) // kpad) * kpad)
    else:
        cuts = np.sort(rng.integers(0, R + 1, size=G - 1))
        cuts[1] = cuts[0]                      # an empty group
        offsets = np.concatenate([[0], cuts, [R]])
        ldc = L.moe_mx_quantize_cols_ld(R, G, kpad)
    codes = torch.full((N, ldc), 0x55, dtype=torch.uint8, device=DEV)
    scales = torch.full((N, ldc // 32), 0x55, dtype=torch.uint8, device=DEV)
    kbase = torch.empty(G + 1, dtype=torch.int32, device=DEV)
    L.moe_mx_quantize_cols(dev_tensor(x, "bf16"), R, N, N, None if uniform else i32(offsets), G, R // G, kpad,
                           codes, scales, ldc, kbase)
    torch.cuda.synchronize()
    rc, rs, rk = MX.mx_quantize_grouped_cols(x, offsets, kpad)
    kt = int(rk[-1])
    assert np.array_equal(tnp(kbase), rk), "group column offsets differ"
    assert np.array_equal(u8(codes)[:, :kt], rc), "E4M3 codes differ"
    assert np.array_equal(u8(scales)[:, :kt // 32], rs), "scale bytes differ"
    assert not u8(codes)[:, kt:].any() and not u8(scales)[:, kt // 32:].any(), "tail not cleared"


def ragged_offsets(rng, M, G):
    cuts = np.sort(rng.integers(0, M + 1, size=G - 1))
    if G > 3:
        cuts[2] = cuts[1]                      # an empty group
    return np.concatenate([[0], cuts, [M]]).astype(np.int64)


def quantize_rows_gpu_t(t):
    """Stand-alone row quantization of a bf16 device tensor (codes, scales)."""
    R, K = t.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device=DEV)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=DEV)
    L.moe_mx_quantize_rows(t, R, K, K, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def quantize_rows_gpu(x):
    R, K = x.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device=DEV)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=DEV)
    L.moe_mx_quantize_rows(dev_tensor(x, "bf16"), R, K, K, codes, scales)
    return codes, scales


# Shapes with N a multiple of 256 run the pipelined 256x256 kernel (K = 128: a two-step ring),
# the others the 128x128 kernel.
@pytest.mark.parametrize("M,N,K,G", [(700, 256, 384, 6), (129, 128, 128, 1), (2000, 384, 1024, 9),
                                     (3000, 512, 1024, 7), (300, 256, 128, 2), (1, 256, 256, 1)])
def test_gemm_rows_store(M, N, K, G):
    log(f"mx gemm rows store M={M} N={N} K={K} G={G}")
    rng = np.random.default_rng(M + N + K)
    a = as_dtype_values(rng.standard_normal((M, K)), "bf16")
    b = as_dtype_values(0.02 * rng.standard_normal((G, N, K)), "bf16")
    offs = ragged_offsets(rng, M, G)
    ac, as_ = quantize_rows_gpu(a)
    bc, bs = quantize_rows_gpu(b.reshape(G * N, K))
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(L.moe_mx_gemm_workspace_size(G), dtype=torch.uint8, device=DEV)
    L.moe_mx_gemm_rows(ac, as_, bc, bs, K, N * K, None, None, 0, i32(offs), G, M, N, K, L.MOE_MX_EPI_STORE, out,
                       None, None, None, None, None, None, ws, ws.numel())
    torch.cuda.synchronize()
    qa = MX.mx_quantize_rows(a)
    qb = [MX.mx_quantize_rows(b[g]) for g in range(G)]
    ref = MX.mx_grouped_gemm_rows(qa[0], qa[1], np.stack([q[0] for q in qb]), np.stack([q[1] for q in qb]), offs)
    assert_close("C", tnp(out), ref, TOL)


def test_gemm_rows_swiglu_and_backward():
    M, f, d, G = 900, 256, 256, 5
    log(f"mx gemm rows swiglu fwd/bwd M={M} f={f} d={d} G={G}")
    rng = np.random.default_rng(7)
    x = as_dtype_values(rng.standard_normal((M, d)), "bf16")
    w1 = as_dtype_values(0.02 * rng.standard_normal((G, f, d)), "bf16")
    w3 = as_dtype_values(0.02 * rng.standard_normal((G, f, d)), "bf16")
    offs = ragged_offsets(rng, M, G)
    w13 = np.concatenate([w1, w3], axis=1)                       # [G, 2f, d]: gate rows, then up rows
    xc, xs = quantize_rows_gpu(x)
    wc, wsc = quantize_rows_gpu(w13.reshape(G * 2 * f, d))
    A = torch.empty((M, f), dtype=torch.bfloat16, device=DEV)
    B = torch.empty_like(A)
    H = torch.empty_like(A)
    ws = torch.empty(L.moe_mx_gemm_workspace_size(G), dtype=torch.uint8, device=DEV)
    # gate rows at the start of each group's [2f, d] block, up rows f rows further (second source)
    hq = torch.empty((M, f), dtype=torch.uint8, device=DEV)
    hs = torch.empty((M, f // 32), dtype=torch.uint8, device=DEV)
    L.moe_mx_gemm_rows(xc, xs, wc, wsc, d, 2 * f * d, wc[f:], wsc[f:], 0, i32(offs), G, M, f, d,
                       L.MOE_MX_EPI_SWIGLU, A, B, H, None, None, hq, hs, ws, ws.numel())
    torch.cuda.synchronize()
    qx = MX.mx_quantize_rows(x)
    q1 = [MX.mx_quantize_rows(w1[g]) for g in range(G)]
    q3 = [MX.mx_quantize_rows(w3[g]) for g in range(G)]
    G1 = MX.mx_grouped_gemm_rows(*qx, np.stack([q[0] for q in q1]), np.stack([q[1] for q in q1]), offs)
    G3 = MX.mx_grouped_gemm_rows(*qx, np.stack([q[0] for q in q3]), np.stack([q[1] for q in q3]), offs)
    Href = G1 / (1.0 + np.exp(-G1)) * G3
    assert_close("A", tnp(A), G1, TOL)
    assert_close("B", tnp(B), G3, TOL)
    assert_close("H", tnp(H), Href, TOL)
    # The fused quantization of H equals the stand-alone quantizer on the stored H (rows in groups).
    rq, rs = quantize_rows_gpu_t(H)
    rows = np.arange(M)[(np.arange(M) >= offs[0]) & (np.arange(M) < offs[-1])]
    assert np.array_equal(u8(hq)[rows], u8(rq)[rows]) and np.array_equal(u8(hs)[rows], u8(rs)[rows]), "fused H codes"

    # Backward through the down projection: dH = dY W2 (contraction over d), SwiGLU backward
    # against the stashed A and B.
    dy = as_dtype_values(rng.standard_normal((M, d)), "bf16")
    w2t = as_dtype_values(0.02 * rng.standard_normal((G, f, d)), "bf16")   # W2^T per group: [f, d]
    dyc, dys = quantize_rows_gpu(dy)
    w2c, w2s = quantize_rows_gpu(w2t.reshape(G * f, d))
    a_in = as_dtype_values(2.0 * rng.standard_normal((M, f)), "bf16")     # stashed gate/up values
    b_in = as_dtype_values(rng.standard_normal((M, f)), "bf16")
    dab = torch.empty((M, 2 * f), dtype=torch.bfloat16, device=DEV)
    dq = torch.empty((M, 2 * f), dtype=torch.uint8, device=DEV)
    dsq = torch.empty((M, 2 * f // 32), dtype=torch.uint8, device=DEV)
    L.moe_mx_gemm_rows(dyc, dys, w2c, w2s, d, f * d, None, None, 0, i32(offs), G, M, f, d, L.MOE_MX_EPI_SWIGLU_BWD,
                       dab, None, None, dev_tensor(a_in, "bf16"), dev_tensor(b_in, "bf16"), dq, dsq, ws, ws.numel())
    torch.cuda.synchronize()
    qdy = MX.mx_quantize_rows(dy)
    q2 = [MX.mx_quantize_rows(w2t[g]) for g in range(G)]
    dH = MX.mx_grouped_gemm_rows(*qdy, np.stack([q[0] for q in q2]), np.stack([q[1] for q in q2]), offs)
    a, b = a_in.astype(np.float64), b_in.astype(np.float64)
    s = 1.0 / (1.0 + np.exp(-a))
    dA = dH * b * s * (1.0 + a * (1.0 - s))
    dB = dH * a * s
    got = tnp(dab)
    assert_close("dA", got[:, :f], dA, TOL)
    assert_close("dB", got[:, f:], dB, TOL)
    rq, rs = quantize_rows_gpu_t(dab)
    assert np.array_equal(u8(dq), u8(rq)) and np.array_equal(u8(dsq), u8(rs)), "fused [dA|dB] codes"



@pytest.mark.parametrize("R,Mw,N,G,split", [(1000, 256, 128, 7, 128), (300, 128, 256, 3, 128),
                                            (4096, 384, 128, 2, 384), (2000, 512, 256, 9, 256),
                                            (700, 256, 512, 4, 0), (8192, 256, 256, 1, 256)])
def test_gemm_k(R, Mw, N, G, split):
    """Weight-gradient form.  With few 256x256 output tiles the K ranges are split (fp32 partials
    summed in split order): the last three cases, including parts with no rows."""
    log(f"mx gemm k R={R} Mw={Mw} N={N} G={G} split={split} parts={L.moe_mx_gemm_k_workspace_size(G, Mw, N) > 0}")
    rng = np.random.default_rng(R + Mw + N)
    a = as_dtype_values(rng.standard_normal((R, Mw)), "bf16")     # e.g. dY rows of the experts' tokens
    b = as_dtype_values(rng.standard_normal((R, N)), "bf16")      # e.g. H rows
    offs = ragged_offsets(rng, R, G)
    kpad = 128
    ld = L.moe_mx_quantize_cols_ld(R, G, kpad)
    ac = torch.empty((Mw, ld), dtype=torch.uint8, device=DEV)
    as_ = torch.empty((Mw, ld // 32), dtype=torch.uint8, device=DEV)
    bc = torch.empty((N, ld), dtype=torch.uint8, device=DEV)
    bs = torch.empty((N, ld // 32), dtype=torch.uint8, device=DEV)
    kb = torch.empty(G + 1, dtype=torch.int32, device=DEV)
    kb2 = torch.empty(G + 1, dtype=torch.int32, device=DEV)
    L.moe_mx_quantize_cols(dev_tensor(a, "bf16"), R, Mw, Mw, i32(offs), G, 0, kpad, ac, as_, ld, kb)
    L.moe_mx_quantize_cols(dev_tensor(b, "bf16"), R, N, N, i32(offs), G, 0, kpad, bc, bs, ld, kb2)
    out0 = torch.full((G, split, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    out1 = torch.full((G, Mw - split, N), float("nan"), dtype=torch.bfloat16, device=DEV) if split < Mw else None
    nws = L.moe_mx_gemm_k_workspace_size(G, Mw, N)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    L.moe_mx_gemm_k(ac, as_, ld, bc, bs, ld, kb, G, Mw, N, split, out0, out1, ws, nws)
    torch.cuda.synchronize()
    qa = MX.mx_quantize_grouped_cols(a, offs, kpad)
    qb = MX.mx_quantize_grouped_cols(b, offs, kpad)
    ref = MX.mx_grouped_gemm_k(qa[0], qa[1], qb[0], qb[1], qa[2])
    got = tnp(out0)
    if out1 is not None:
        got = np.concatenate([got, tnp(out1)], axis=1)
    for g in range(G):
        if offs[g + 1] == offs[g]:
            assert np.all(got[g] == 0), f"empty group {g} not exact zeros"
        else:
            assert_close(f"C[{g}]", got[g], ref[g], TOL)


def test_gemm_rows_k_split():
    """The gate/up data gradient's form: columns [0, K1) of B from one source, [K1, K) from another."""
    M, N, K1, K2, G = 800, 256, 256, 256, 3
    log(f"mx gemm rows K split M={M} N={N} K={K1}+{K2} G={G}")
    rng = np.random.default_rng(11)
    a = as_dtype_values(rng.standard_normal((M, K1 + K2)), "bf16")
    b1 = as_dtype_values(0.02 * rng.standard_normal((G, N, K1)), "bf16")
    b2 = as_dtype_values(0.02 * rng.standard_normal((G, N, K2)), "bf16")
    offs = ragged_offsets(rng, M, G)
    ac, as_ = quantize_rows_gpu(a)
    c1, s1 = quantize_rows_gpu(b1.reshape(G * N, K1))
    c2, s2 = quantize_rows_gpu(b2.reshape(G * N, K2))
    ws = torch.empty(L.moe_mx_gemm_workspace_size(G), dtype=torch.uint8, device=DEV)
    for n_out in (N, N // 2):      # N = 256: pipelined kernel; the 128-column half view: 128x128 kernel
        out = torch.empty((M, n_out), dtype=torch.bfloat16, device=DEV)
        L.moe_mx_gemm_rows(ac, as_, c1, s1, K1, N * K1, c2, s2, K1, i32(offs), G, M, n_out, K1 + K2,
                           L.MOE_MX_EPI_STORE, out, None, None, None, None, None, None, ws, ws.numel())
        torch.cuda.synchronize()
        bb = np.concatenate([b1, b2], axis=2)[:, :n_out]
        qa = MX.mx_quantize_rows(a)
        qb = [MX.mx_quantize_rows(bb[g]) for g in range(G)]
        ref = MX.mx_grouped_gemm_rows(*qa, np.stack([q[0] for q in qb]), np.stack([q[1] for q in qb]), offs)
        assert_close(f"C (N={n_out})", tnp(out), ref, TOL)


# ------------------------------------------------------------------------------------------ layer

LAYER_CASES = {
    # name: (routing, T, d, E, k, f, fs)
    "learned_f256": ("learned", 256, 256, 8, 2, 256, 256),
    "random_f128": ("random", 300, 256, 5, 3, 128, 128),
    # few tokens over many experts: most experts get no rows, one gets most of them
    "learned_sparse_k1": ("learned", 48, 256, 32, 1, 128, 128),
    "learned_sparse_k2": ("learned", 40, 256, 16, 2, 128, 128),
    "learned_single_token": ("learned", 1, 128, 4, 1, 128, 128),
    "random_top8_e256": ("random", 200, 128, 256, 8, 128, 128),
}


@pytest.mark.parametrize("case", sorted(LAYER_CASES))
def test_mx_layer_matches_oracle(case):
    from mixture_experts_layer_20_amd import inputs as I
    from mixture_experts_layer_20_amd import layer as LY
    from oracle import moe_oracle as O
    routing, T, d, E, k, f, fs = LAYER_CASES[case]
    log(f"mx layer {case}")
    base = I.CONFIGS["tiny64e_learned_skew" if routing == "learned" else "tiny64e_random"]
    cfg = base.with_(name="mx_" + case, T=T, d=d, E=E, k=k, f=f, fs=fs, bias_std=1.0)
    inp = I.make_inputs(cfg)
    lay = LY.MoELayer(cfg, LY.upload_inputs(inp, DEV), precision="mxfp8")
    lay.step()
    torch.cuda.synchronize()
    fwd, bwd = O.run_layer(cfg, I.values(inp), experts=MX.MXExperts())
    b = lay.bufs
    assert np.array_equal(tnp(b["topk_idx"]), fwd["topk_idx"])
    assert np.array_equal(tnp(b["dest_pos"]), fwd["dest_pos"])
    checks = {"out": (b["out"], fwd["out"]), "dx": (b["dx"], bwd["dx"]), "dW1": (b["dw1"], bwd["dW1"]),
              "dW3": (b["dw3"], bwd["dW3"]), "dW2": (b["dw2"], bwd["dW2"]), "dWs1": (b["dws1"], bwd["dWs1"]),
              "dWs3": (b["dws3"], bwd["dWs3"]), "dWs2": (b["dws2"], bwd["dWs2"])}
    if routing == "learned":
        checks["dWr"] = (b["dwr"], bwd["dWr"])
    # Layer-level bar: 5e-2.  The MXFP8 layer moves by ~1e-2 (up to 2e-2) under sub-ulp perturbations
    # of its stored intermediates (tests/test_oracle_mx_layer.py), which is the size of the
    # device's fp32-versus-float64 difference; single products are held to 4e-3 above.
    for name, (got, ref) in checks.items():
        assert_close(name, tnp(got), ref, 5e-2)
    counts = np.bincount(np.asarray(fwd["topk_idx"]).reshape(-1), minlength=E)
    for e in np.nonzero(counts == 0)[0]:
        for key in ("dw1", "dw3", "dw2"):
            assert bool((b[key][int(e)] == 0).all()), f"empty expert {e}: {key} is not zero"


@pytest.mark.parametrize("name", ["tiny64e_random", "tiny64e_learned_skew", "e128_2seq", "large_e128"])
def test_mx_layer_full_size_sampled_experts(name):
    """The MXFP8 layer at the full Tiny-64E shape (the bench's launch configuration).  Routing and
    dispatch are bit-exact over the whole batch; an expert's products depend only on its own rows,
    so the oracle runs the MXFP8 expert on the busiest and the least busy non-empty expert and the
    device's Y rows, dX_perm rows and weight gradients of those experts are compared."""
    from mixture_experts_layer_20_amd import inputs as I
    from mixture_experts_layer_20_amd import layer as LY
    from tests.gpu_helpers import full_routing
    cfg = I.CONFIGS[name]
    log(f"mx full-size layer {name}")
    inp = I.make_inputs(cfg)
    vals = I.values(inp)
    lay = LY.MoELayer(cfg, LY.upload_inputs(inp, DEV), precision="mxfp8")
    lay.step()
    torch.cuda.synchronize()
    b = lay.bufs
    R = full_routing(cfg, vals)
    for key in ("topk_idx", "offsets", "dest_pos", "src_row"):
        assert np.array_equal(tnp(b[key]).reshape(-1), np.asarray(R[key]).reshape(-1)), key
    counts, offs, src = R["counts"], R["offsets"], np.asarray(R["src_row"], np.int64)
    nz = np.nonzero(counts)[0]
    ex = MX.MXExperts()
    for e in sorted({int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])}):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        tok, slot = src[r0:r1] // cfg.k, src[r0:r1] % cfg.k
        X = vals["x"][tok].astype(np.float64)
        dY = R["gates"][tok, slot][:, None] * vals["dout"][tok].astype(np.float64)
        A, B, H, Y = ex.forward(X, vals["w1"][e], vals["w3"][e], vals["w2"][e])
        dX, dW1, dW3, dW2, _, _ = ex.backward(dY, X, A, B, H, vals["w1"][e], vals["w3"][e], vals["w2"][e])
        log(f"  expert {e}: {r1 - r0} rows")
        assert_close(f"y[{e}]", tnp(b["y"][r0:r1]), Y, 5e-2)
        assert_close(f"dx_perm[{e}]", tnp(b["dx_perm"][r0:r1]), dX, 5e-2)
        assert_close(f"dw1[{e}]", tnp(b["dw1"][e]), dW1, 5e-2)
        assert_close(f"dw3[{e}]", tnp(b["dw3"][e]), dW3, 5e-2)
        assert_close(f"dw2[{e}]", tnp(b["dw2"][e]), dW2, 5e-2)
    for e in np.nonzero(counts == 0)[0]:
        assert bool((b["dw2"][int(e)] == 0).all()), f"empty expert {e} has a nonzero gradient"


def test_mx_cached_weights_match_per_pass_quantization():
    """Cached MXFP8 weights give bitwise the results of quantizing them in every pass, until the
    weights change; refresh_mx_weights() makes the next pass see the new weights."""
    from mixture_experts_layer_20_amd import inputs as I
    from mixture_experts_layer_20_amd import layer as LY
    cfg = I.CONFIGS["tiny64e_random"].with_(name="mx_cache", T=256, d=256, E=8, k=2, f=256, fs=256)
    log("mx cached weights")
    inp = I.make_inputs(cfg)
    pa, pb = LY.upload_inputs(inp, DEV), LY.upload_inputs(inp, DEV)
    every = LY.MoELayer(cfg, pa, precision="mxfp8")
    cached = LY.MoELayer(cfg, pb, precision="mxfp8", mx_cached_weights=True)
    keys = ("out", "dx", "dw1", "dw3", "dw2", "dws1")
    same = lambda: all(torch.equal(every.bufs[k], cached.bufs[k]) for k in keys)
    for _ in range(2):
        every.step()
        cached.step()
    torch.cuda.synchronize()
    assert same(), "cached weights differ from per-pass quantization"
    for p in (pa, pb):
        p["w1"].mul_(2.0)                       # a weight update (exact in bf16)
    every.step()
    cached.step()
    torch.cuda.synchronize()
    assert not torch.equal(every.bufs["out"], cached.bufs["out"]), "a stale cache should not see the update"
    cached.refresh_mx_weights()
    every.step()
    cached.step()
    torch.cuda.synchronize()
    assert same(), "after refresh_mx_weights() the results differ"
