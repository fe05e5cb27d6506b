"""ctypes binding of libmoe (include/libmoe.h).

Argument marshalling only: every function has the C entry point's name and argument order, takes
torch tensors (or None) where the C call takes device pointers, and raises MoEError on a non-OK
status.  All computation happens in the HIP library; if it is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

MOE_OK = 0
MOE_ERR_INVALID_VALUE = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_F32 = 0
MOE_BF16 = 1

MOE_STAGE_GATE_UP_FWD = 0
MOE_STAGE_DOWN_FWD = 1
MOE_STAGE_DOWN_BWD = 2
MOE_STAGE_GATE_UP_DGRAD = 3
MOE_STAGE_DOWN_WGRAD = 4
MOE_STAGE_GATE_UP_WGRAD = 5

MOE_OP_ROUTE = 0
MOE_OP_PERMUTE = 1
MOE_OP_GROUPED_MLP_FWD = 2
MOE_OP_GROUPED_MLP_BWD = 3
MOE_OP_COMBINE = 4
MOE_OP_COMBINE_BWD = 5
MOE_OP_PERMUTE_BWD = 6
MOE_OP_ROUTE_BWD = 7
MOE_OP_EXPERT_STAGE = 8
MOE_OP_ROUTER_AUX = 9
MOE_OP_ROUTER_AUX_BWD = 10
MOE_OP_MX_GEMM_ROWS = 11
MOE_OP_MX_GEMM_K = 12

MOE_MX_EPI_STORE = 0
MOE_MX_EPI_SWIGLU = 1
MOE_MX_EPI_SWIGLU_BWD = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libmoe.so")

_c = ctypes
_P = _c.c_void_p
_I64 = _c.c_int64
_I32 = _c.c_int32
_SZ = _c.c_size_t



class ExpertSet(ctypes.Structure):
    """moe_expert_set_t: one set of experts of a multi-set GEMM stage."""
    _fields_ = [("offsets", ctypes.c_void_p), ("G", ctypes.c_int32), ("M", ctypes.c_int64),
                ("f", ctypes.c_int64)] + [(n, ctypes.c_void_p) for n in
                                          ("x", "w1", "w3", "w2", "a", "b", "h", "y", "dy", "dab", "dx", "dw1",
                                           "dw3", "dw2")]


# name -> (restype, argtypes); mirrors include/libmoe.h
_SIGS = {
    "moe_route": (_I32, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_permute_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "moe_permute": (_I32, [_P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_noalloc_max_scratch": (_SZ, []),
    "moe_permute_noalloc": (_I32, [_P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_mlp_fwd_workspace_size": (_SZ, [_I64, _I32, _I64, _I64]),
    "moe_grouped_mlp_bwd_workspace_size": (_SZ, [_I64, _I32, _I64, _I64]),
    "moe_grouped_mlp_fwd": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _I32, _P, _P, _P, _P,
                                   _P, _SZ, _P]),
    "moe_grouped_mlp_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _I32,
                                   _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_gate_up_fwd": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _I32, _P, _P, _P, _P,
                                      _SZ, _P]),
    "moe_expert_down_fwd": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _I32, _P, _P, _SZ, _P]),
    "moe_expert_down_bwd": (_I32, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _I32, _P, _P, _SZ, _P]),
    "moe_expert_down_wgrad": (_I32, [_P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P, _SZ, _P]),
    "moe_expert_gate_up_dgrad": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _I32, _P, _P, _SZ, _P]),
    "moe_expert_gate_up_wgrad": (_I32, [_P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _SZ, _P]),
    "moe_expert_stage_workspace_size": (_SZ, [_P, _I32, _I64]),
    "moe_expert_stage": (_I32, [_I32, _P, _I32, _I64, _I32, _P, _SZ, _P]),
    "moe_combine": (_I32, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P]),
    "moe_combine_bwd": (_I32, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P, _P]),
    "moe_permute_bwd": (_I32, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P]),
    "moe_route_bwd_workspace_size": (_SZ, [_I64, _I64, _I32, _I32]),
    "moe_router_aux_workspace_size": (_SZ, [_I64, _I32]),
    "moe_router_aux": (_I32, [_P, _P, _I64, _I32, _I32, _c.c_float, _P, _P, _P, _P, _SZ, _P]),
    "moe_router_aux_bwd_workspace_size": (_SZ, [_I64, _I64, _I32]),
    "moe_router_aux_bwd": (_I32, [_P, _P, _P, _P, _I64, _I64, _I32, _c.c_float, _I32, _P, _P, _P, _SZ, _P]),
    "moe_route_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P,
                             _P, _SZ, _P]),
    "moe_mx_quantize_rows": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "moe_mx_quantize_cols_ld": (_I64, [_I64, _I32, _I32]),
    "moe_mx_quantize_cols": (_I32, [_P, _I64, _I64, _I64, _P, _I32, _I64, _I32, _P, _P, _I64, _P, _P]),
    "moe_mx_gemm_workspace_size": (_SZ, [_I32]),
    "moe_mx_gemm_rows": (_I32, [_P, _P, _P, _P, _I64, _I64, _P, _P, _I64, _P, _I32, _I64, _I64, _I64, _I32, _P, _P,
                                _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mx_gemm_k_workspace_size": (_SZ, [_I32, _I64, _I64]),
    "moe_mx_gemm_k": (_I32, [_P, _P, _I64, _P, _P, _I64, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "moe_workspace_bytes": (_SZ, [_I32, _I64, _I64, _I32, _I32, _I64, _I64]),
    "moe_status_string": (_c.c_char_p, [_I32]),
    "moe_last_error": (_c.c_char_p, []),
    "moe_version": (_c.c_char_p, []),
}

_LIB = None


class MoEError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        self.status = status
        super().__init__(f"{name} failed: {status_string(status)}: {detail}")


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree); raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoe is not built ({LIB_PATH} missing): run "
                               "`python -m mixture_experts_layer_20_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_string(st: int) -> str:
    return lib().moe_status_string(st).decode()


def last_error() -> str:
    return lib().moe_last_error().decode()


def version() -> str:
    return lib().moe_version().decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream if isinstance(stream, int) else stream.cuda_stream


def _call(name: str, *args):
    st = getattr(lib(), name)(*args)
    if st != MOE_OK:
        raise MoEError(st, name, last_error())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------------------ entry points

def moe_route(x, w_router, bias, logits, T, d, E, k, renormalize, dt, topk_idx, topk_gate, stream=None):
    _call("moe_route", _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits), T, d, E, k, renormalize, dt,
          _ptr(topk_idx), _ptr(topk_gate), _stream(stream))


def moe_workspace_bytes(op, T, d, E, k, f, fs=0) -> int:
    return lib().moe_workspace_bytes(op, T, d, E, k, f, fs)


def moe_permute_workspace_size(T, E, k) -> int:
    return lib().moe_permute_workspace_size(T, E, k)


def moe_permute(x, topk_idx, T, d, E, k, dt, counts, offsets, dest_pos, src_row, x_perm, ws, ws_bytes,
                stream=None):
    _call("moe_permute", _ptr(x), _ptr(topk_idx), T, d, E, k, dt, _ptr(counts), _ptr(offsets),
          _ptr(dest_pos), _ptr(src_row), _ptr(x_perm), _ptr(ws), ws_bytes, _stream(stream))


def moe_permute_noalloc_max_scratch() -> int:
    return lib().moe_permute_noalloc_max_scratch()


def moe_permute_noalloc(x, topk_idx, T, d, E, k, dt, counts, offsets, dest_pos, src_row, x_perm, stream=None):
    _call("moe_permute_noalloc", _ptr(x), _ptr(topk_idx), T, d, E, k, dt, _ptr(counts), _ptr(offsets),
          _ptr(dest_pos), _ptr(src_row), _ptr(x_perm), _stream(stream))


def moe_grouped_mlp_fwd_workspace_size(M, G, d, f) -> int:
    return lib().moe_grouped_mlp_fwd_workspace_size(M, G, d, f)


def moe_grouped_mlp_bwd_workspace_size(M, G, d, f) -> int:
    return lib().moe_grouped_mlp_bwd_workspace_size(M, G, d, f)


def moe_grouped_mlp_fwd(x_in, offsets, G, M, d, f, w1, w3, w2, dt, a_stash, b_stash, h, y, ws, ws_bytes,
                        stream=None):
    _call("moe_grouped_mlp_fwd", _ptr(x_in), _ptr(offsets), G, M, d, f, _ptr(w1), _ptr(w3), _ptr(w2), dt,
          _ptr(a_stash), _ptr(b_stash), _ptr(h), _ptr(y), _ptr(ws), ws_bytes, _stream(stream))


def moe_grouped_mlp_bwd(dy, x_in, a, b, h, offsets, G, M, d, f, w1, w3, w2, dt, dx_in, dw1, dw3, dw2, ws,
                        ws_bytes, stream=None):
    _call("moe_grouped_mlp_bwd", _ptr(dy), _ptr(x_in), _ptr(a), _ptr(b), _ptr(h), _ptr(offsets), G, M, d,
          f, _ptr(w1), _ptr(w3), _ptr(w2), dt, _ptr(dx_in), _ptr(dw1), _ptr(dw3), _ptr(dw2), _ptr(ws),
          ws_bytes, _stream(stream))


def moe_expert_gate_up_fwd(x_in, offsets, G, M, d, f, w1, w3, dt, a_stash, b_stash, h, ws, ws_bytes,
                           stream=None):
    _call("moe_expert_gate_up_fwd", _ptr(x_in), _ptr(offsets), G, M, d, f, _ptr(w1), _ptr(w3), dt,
          _ptr(a_stash), _ptr(b_stash), _ptr(h), _ptr(ws), ws_bytes, _stream(stream))


def moe_expert_down_fwd(h, offsets, G, M, d, f, w2, dt, y, ws, ws_bytes, stream=None):
    _call("moe_expert_down_fwd", _ptr(h), _ptr(offsets), G, M, d, f, _ptr(w2), dt, _ptr(y), _ptr(ws),
          ws_bytes, _stream(stream))


def moe_expert_down_bwd(dy, a, b, offsets, G, M, d, f, w2, dt, dab, ws, ws_bytes, stream=None):
    _call("moe_expert_down_bwd", _ptr(dy), _ptr(a), _ptr(b), _ptr(offsets), G, M, d, f, _ptr(w2), dt,
          _ptr(dab), _ptr(ws), ws_bytes, _stream(stream))


def moe_expert_down_wgrad(dy, h, offsets, G, M, d, f, dt, dw2, ws, ws_bytes, stream=None):
    _call("moe_expert_down_wgrad", _ptr(dy), _ptr(h), _ptr(offsets), G, M, d, f, dt, _ptr(dw2), _ptr(ws),
          ws_bytes, _stream(stream))


def moe_expert_gate_up_dgrad(dab, offsets, G, M, d, f, w1, w3, dt, dx_in, ws, ws_bytes, stream=None):
    _call("moe_expert_gate_up_dgrad", _ptr(dab), _ptr(offsets), G, M, d, f, _ptr(w1), _ptr(w3), dt,
          _ptr(dx_in), _ptr(ws), ws_bytes, _stream(stream))


def moe_expert_gate_up_wgrad(dab, x_in, offsets, G, M, d, f, dt, dw1, dw3, ws, ws_bytes, stream=None):
    _call("moe_expert_gate_up_wgrad", _ptr(dab), _ptr(x_in), _ptr(offsets), G, M, d, f, dt, _ptr(dw1),
          _ptr(dw3), _ptr(ws), ws_bytes, _stream(stream))


def expert_set(offsets, G, M, f, **tensors) -> ExpertSet:
    """An ExpertSet from tensors (members not given are NULL)."""
    e = ExpertSet()
    e.offsets = _ptr(offsets)
    e.G, e.M, e.f = G, M, f
    for name, t in tensors.items():
        setattr(e, name, _ptr(t))
    return e


def _set_array(sets):
    arr = (ExpertSet * len(sets))(*sets)
    return arr, len(sets)


def moe_expert_stage_workspace_size(sets, d) -> int:
    arr, n = _set_array(sets)
    return lib().moe_expert_stage_workspace_size(ctypes.cast(arr, _P), n, d)


def moe_expert_stage(stage, sets, d, dt, ws, ws_bytes, stream=None):
    arr, n = _set_array(sets)
    _call("moe_expert_stage", stage, ctypes.cast(arr, _P), n, d, dt, _ptr(ws), ws_bytes, _stream(stream))


def moe_combine(y_perm, topk_gate, dest_pos, shared_out, T, d, k, dt, out, stream=None):
    _call("moe_combine", _ptr(y_perm), _ptr(topk_gate), _ptr(dest_pos), _ptr(shared_out), T, d, k, dt,
          _ptr(out), _stream(stream))


def moe_combine_bwd(dout, y_perm, topk_gate, dest_pos, T, d, k, dt, dy_perm, dgate, stream=None):
    _call("moe_combine_bwd", _ptr(dout), _ptr(y_perm), _ptr(topk_gate), _ptr(dest_pos), T, d, k, dt,
          _ptr(dy_perm), _ptr(dgate), _stream(stream))


def moe_permute_bwd(dx_perm, dest_pos, dx_add0, dx_add1, T, d, k, dt, dx, stream=None):
    _call("moe_permute_bwd", _ptr(dx_perm), _ptr(dest_pos), _ptr(dx_add0), _ptr(dx_add1), T, d, k, dt,
          _ptr(dx), _stream(stream))


def moe_route_bwd_workspace_size(T, d, E, k) -> int:
    return lib().moe_route_bwd_workspace_size(T, d, E, k)


def moe_route_bwd(dgate, topk_gate, topk_idx, offsets, src_row, x, w_router, T, d, E, k, renormalize, dt,
                  dw_router, dx_router, ws, ws_bytes, stream=None):
    _call("moe_route_bwd", _ptr(dgate), _ptr(topk_gate), _ptr(topk_idx), _ptr(offsets), _ptr(src_row),
          _ptr(x), _ptr(w_router), T, d, E, k, renormalize, dt, _ptr(dw_router), _ptr(dx_router), _ptr(ws),
          ws_bytes, _stream(stream))


def moe_router_aux_workspace_size(T, E) -> int:
    return lib().moe_router_aux_workspace_size(T, E)


def moe_router_aux(logits, counts, T, E, k, weight, loss, prob_mean, load_frac, ws, ws_bytes, stream=None):
    _call("moe_router_aux", _ptr(logits), _ptr(counts), T, E, k, weight, _ptr(loss), _ptr(prob_mean),
          _ptr(load_frac), _ptr(ws), ws_bytes, _stream(stream))


def moe_router_aux_bwd_workspace_size(T, d, E) -> int:
    return lib().moe_router_aux_bwd_workspace_size(T, d, E)


def moe_router_aux_bwd(logits, load_frac, x, w_router, T, d, E, weight, dt, dw_router, dx_router, ws, ws_bytes,
                       stream=None):
    _call("moe_router_aux_bwd", _ptr(logits), _ptr(load_frac), _ptr(x), _ptr(w_router), T, d, E, weight, dt,
          _ptr(dw_router), _ptr(dx_router), _ptr(ws), ws_bytes, _stream(stream))


def moe_mx_quantize_rows(x, R, K, ldx, codes, scales, stream=None):
    _call("moe_mx_quantize_rows", _ptr(x), R, K, ldx, _ptr(codes), _ptr(scales), _stream(stream))


def moe_mx_quantize_cols_ld(R, G, kpad) -> int:
    return lib().moe_mx_quantize_cols_ld(R, G, kpad)


def moe_mx_quantize_cols(x, R, N, ldx, offsets, G, group_rows, kpad, codes, scales, ldc, kbase, stream=None):
    _call("moe_mx_quantize_cols", _ptr(x), R, N, ldx, _ptr(offsets), G, group_rows, kpad, _ptr(codes),
          _ptr(scales), ldc, _ptr(kbase), _stream(stream))


def moe_mx_gemm_workspace_size(G) -> int:
    return lib().moe_mx_gemm_workspace_size(G)


def moe_mx_gemm_rows(a_codes, a_scales, b_codes, b_scales, b_row_stride, b_group_stride, b2_codes, b2_scales, b2_k,
                     offsets, G, M, N, K, epilogue, out0, out1, out2, aux0, aux1, q_codes, q_scales, ws, ws_bytes,
                     stream=None):
    _call("moe_mx_gemm_rows", _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), b_row_stride,
          b_group_stride, _ptr(b2_codes), _ptr(b2_scales), b2_k, _ptr(offsets), G, M, N, K, epilogue, _ptr(out0),
          _ptr(out1), _ptr(out2), _ptr(aux0), _ptr(aux1), _ptr(q_codes), _ptr(q_scales), _ptr(ws), ws_bytes,
          _stream(stream))


def moe_mx_gemm_k_workspace_size(G, M, N) -> int:
    return lib().moe_mx_gemm_k_workspace_size(G, M, N)


def moe_mx_gemm_k(a_codes, a_scales, lda, b_codes, b_scales, ldb, kbase, G, M, N, split, out0, out1, ws, ws_bytes,
                  stream=None):
    _call("moe_mx_gemm_k", _ptr(a_codes), _ptr(a_scales), lda, _ptr(b_codes), _ptr(b_scales), ldb, _ptr(kbase),
          G, M, N, split, _ptr(out0), _ptr(out1), _ptr(ws), ws_bytes, _stream(stream))
