"""ctypes binding of libdsmoe.so: one Python function per C entry point, with
the same name. Argument marshalling only (torch tensors supply device memory
and the current stream); every step of the layer runs in the HIP kernels.

The library must have been built (``__graft_entry__.build()`` or
``python sparse_mixture_experts_gate_amd/build.py``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # loaded first so the library binds to torch's HIP runtime

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdsmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dsmoe.h")

MOE_DT_F32, MOE_DT_BF16, MOE_DT_FP8_E4M3 = 0, 1, 2
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_MISALIGNED", 4: "MOE_ERR_WORKSPACE_TOO_SMALL", 5: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


class MoeLayerDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("group_topn", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("near_tie_eps", ctypes.c_float), ("out_dtype", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w13", "w2", "ws13", "ws2", "w13_scale", "w2_scale", "ws13_scale", "ws2_scale")]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logits", "topk_idx", "topk_gate", "counts", "offsets", "perm", "inv", "h", "gu",
                 "y_perm")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dw13", "dw2", "dws13", "dws2", "dw_router")]


def header_symbols() -> list[str]:
    """Names of the functions that include/dsmoe.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*|int)\s+(\w+)\s*\(", txt, re.M)))


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        D = ctypes.POINTER(MoeLayerDesc)
        W = ctypes.POINTER(MoeWeights)
        sig = {
            "moe_workspace_size": [D, ctypes.POINTER(ctypes.c_size_t)],
            "moe_gate": [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P],
            "moe_route_from_logits": [D, P, P, P, P, P, P, P],
            "moe_permute": [D, P, P, P, P, P, P, P, P, P],
            "moe_expert_ffn": [D, W, P, P, P, P, P, P, P, P, ctypes.c_size_t, P],
            "moe_combine": [D, P, P, P, P, P, P],
            "moe_bias_update": [D, P, F, P, P],
            "deepseek_moe_forward": [D, P, P, P, W, P, P, P, P, P, P, P, ctypes.c_size_t, P],
            "deepseek_moe_forward_noalloc": [D, P, P, P, W, P, P, P, P, P, P, P],
            "moe_quantize_fp8_blocks": [P, I32, I64, I32, I32, P, P, P],
            "moe_quantize_fp8_rows": [P, I32, I64, I32, P, P, P],
            "moe_profile_events": [ctypes.POINTER(ctypes.c_void_p), I32],
            "moe_forward_train": [D, P, P, P, W, P, ctypes.POINTER(MoeSaved), P, P,
                                  ctypes.c_size_t, P],
            "moe_backward_workspace_size": [D, ctypes.POINTER(ctypes.c_size_t)],
            "moe_backward": [D, P, P, W, ctypes.POINTER(MoeSaved), P, P, ctypes.POINTER(MoeGrads),
                             P, ctypes.c_size_t, P],
            "moe_transpose_fp8_blocks": [P, P, I64, I32, I32, P, P, P],
            "moe_backward_fp8": [D, P, P, W, W, ctypes.POINTER(MoeSaved), P, P,
                                 ctypes.POINTER(MoeGrads), P, ctypes.c_size_t, P],
            "moe_seq_balance_workspace_size": [D, I32, ctypes.POINTER(ctypes.c_size_t)],
            "moe_seq_balance_loss": [D, I32, F, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, fn: str) -> None:
    if status != 0:
        raise MoeError(status, fn, lib().moe_last_error().decode())


def _p(t) -> ctypes.c_void_p | None:
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_workspace_size(desc: MoeLayerDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def moe_gate(desc, x, w_router, bias, logits, topk_idx, topk_gate, counts, near_tie, ws,
             stream=None):
    _check(lib().moe_gate(ctypes.byref(desc), _p(x), _p(w_router), _p(bias), _p(logits),
                          _p(topk_idx), _p(topk_gate), _p(counts), _p(near_tie), _p(ws),
                          ws.numel() * ws.element_size(), _stream(stream)), "moe_gate")


def moe_route_from_logits(desc, logits, bias, topk_idx, topk_gate, counts, near_tie, stream=None):
    _check(lib().moe_route_from_logits(ctypes.byref(desc), _p(logits), _p(bias), _p(topk_idx),
                                       _p(topk_gate), _p(counts), _p(near_tie), _stream(stream)),
           "moe_route_from_logits")


def moe_permute(desc, topk_idx, counts, x, offsets, perm, inv, x_perm=None, x_perm_scale=None,
                stream=None):
    _check(lib().moe_permute(ctypes.byref(desc), _p(topk_idx), _p(counts), _p(x), _p(offsets),
                             _p(perm), _p(inv), _p(x_perm), _p(x_perm_scale), _stream(stream)),
           "moe_permute")


def make_weights(w13, w2, ws13=None, ws2=None, w13_scale=None, w2_scale=None, ws13_scale=None,
                 ws2_scale=None) -> MoeWeights:
    return MoeWeights(*(None if t is None else _p(t).value for t in
                        (w13, w2, ws13, ws2, w13_scale, w2_scale, ws13_scale, ws2_scale)))


def moe_expert_ffn(desc, weights: MoeWeights, x, perm, x_perm, x_perm_scale, offsets, y_perm,
                   y_shared, ws, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(desc), ctypes.byref(weights), _p(x), _p(perm),
                                _p(x_perm), _p(x_perm_scale), _p(offsets), _p(y_perm),
                                _p(y_shared), _p(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "moe_expert_ffn")


def moe_combine(desc, y_perm, inv, topk_gate, y_shared, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(desc), _p(y_perm), _p(inv), _p(topk_gate),
                             _p(y_shared), _p(y), _stream(stream)), "moe_combine")


def moe_bias_update(desc, counts, gamma: float, bias, stream=None):
    _check(lib().moe_bias_update(ctypes.byref(desc), _p(counts), ctypes.c_float(gamma), _p(bias),
                                 _stream(stream)), "moe_bias_update")


def deepseek_moe_forward(desc, x, w_router, bias, weights: MoeWeights, y, topk_idx, topk_gate,
                         counts, near_tie, logits, ws, stream=None):
    _check(lib().deepseek_moe_forward(ctypes.byref(desc), _p(x), _p(w_router), _p(bias),
                                      ctypes.byref(weights), _p(y), _p(topk_idx), _p(topk_gate),
                                      _p(counts), _p(near_tie), _p(logits), _p(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "deepseek_moe_forward")


def deepseek_moe_forward_noalloc(desc, x, w_router, bias, weights: MoeWeights, y, topk_idx,
                                 topk_gate, counts, near_tie, logits, stream=None):
    _check(lib().deepseek_moe_forward_noalloc(ctypes.byref(desc), _p(x), _p(w_router), _p(bias),
                                              ctypes.byref(weights), _p(y), _p(topk_idx),
                                              _p(topk_gate), _p(counts), _p(near_tie), _p(logits),
                                              _stream(stream)),
           "deepseek_moe_forward_noalloc")


def _dt(t) -> int:
    return {torch.float32: MOE_DT_F32, torch.bfloat16: MOE_DT_BF16}[t.dtype]


def moe_quantize_fp8_blocks(src, q, scale, stream=None):
    """src [n_mats, rows, cols] (or [rows, cols]) fp32/bf16 -> q uint8 same shape,
    scale fp32 [n_mats, rows/128, cols/128]."""
    shp = src.shape if src.dim() == 3 else (1, *src.shape)
    _check(lib().moe_quantize_fp8_blocks(_p(src), _dt(src), shp[0], shp[1], shp[2], _p(q),
                                         _p(scale), _stream(stream)), "moe_quantize_fp8_blocks")


def moe_profile_events(events) -> None:
    """events: six torch.cuda.Event(enable_timing=True) already recorded once
    (so that they exist), or None to switch the hook off."""
    if events is None:
        _check(lib().moe_profile_events(None, 0), "moe_profile_events")
        return
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check(lib().moe_profile_events(arr, len(events)), "moe_profile_events")


def moe_quantize_fp8_rows(src, q, scale, stream=None):
    _check(lib().moe_quantize_fp8_rows(_p(src), _dt(src), src.shape[0], src.shape[1], _p(q),
                                       _p(scale), _stream(stream)), "moe_quantize_fp8_rows")


def _struct(cls, **tensors):
    return cls(**{k: (None if v is None else _p(v).value) for k, v in tensors.items()})


def make_saved(**tensors) -> MoeSaved:
    """MoeSaved from tensors named like its fields."""
    return _struct(MoeSaved, **tensors)


def make_grads(dw13, dw2, dws13, dws2, dw_router) -> MoeGrads:
    return _struct(MoeGrads, dw13=dw13, dw2=dw2, dws13=dws13, dws2=dws2, dw_router=dw_router)


def moe_forward_train(desc, x, w_router, bias, weights: MoeWeights, y, saved: MoeSaved, near_tie,
                      ws, stream=None):
    _check(lib().moe_forward_train(ctypes.byref(desc), _p(x), _p(w_router), _p(bias),
                                   ctypes.byref(weights), _p(y), ctypes.byref(saved), _p(near_tie),
                                   _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_forward_train")


def moe_backward_workspace_size(desc: MoeLayerDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "moe_backward_workspace_size")
    return n.value


def moe_backward(desc, x, w_router, weights: MoeWeights, saved: MoeSaved, dy, dx, grads: MoeGrads,
                 ws, stream=None):
    _check(lib().moe_backward(ctypes.byref(desc), _p(x), _p(w_router), ctypes.byref(weights),
                              ctypes.byref(saved), _p(dy), _p(dx), ctypes.byref(grads), _p(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "moe_backward")


def moe_seq_balance_workspace_size(desc: MoeLayerDesc, seq_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_seq_balance_workspace_size(ctypes.byref(desc), seq_len, ctypes.byref(n)),
           "moe_seq_balance_workspace_size")
    return n.value


def moe_seq_balance_loss(desc, seq_len: int, alpha: float, x, w_router, logits, topk_idx, loss,
                         dlogits, dx, dw_router, ws, stream=None):
    _check(lib().moe_seq_balance_loss(ctypes.byref(desc), seq_len, alpha, _p(x), _p(w_router),
                                      _p(logits), _p(topk_idx), _p(loss), _p(dlogits), _p(dx),
                                      _p(dw_router), _p(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)), "moe_seq_balance_loss")


def moe_transpose_fp8_blocks(q, scale, qt, scale_t, stream=None):
    """q [n_mats, rows, cols] uint8 (or [rows, cols]), scale fp32
    [n_mats, rows/128, cols/128] -> qt [.., cols, rows], scale_t
    [.., cols/128, rows/128]."""
    shp = q.shape if q.dim() == 3 else (1, *q.shape)
    _check(lib().moe_transpose_fp8_blocks(_p(q), _p(scale), shp[0], shp[1], shp[2], _p(qt),
                                          _p(scale_t), _stream(stream)),
           "moe_transpose_fp8_blocks")


def moe_backward_fp8(desc, x, w_router, weights: MoeWeights, weights_t: MoeWeights,
                     saved: MoeSaved, dy, dx, grads: MoeGrads, ws, stream=None):
    _check(lib().moe_backward_fp8(ctypes.byref(desc), _p(x), _p(w_router), ctypes.byref(weights),
                                  ctypes.byref(weights_t), ctypes.byref(saved), _p(dy), _p(dx),
                                  ctypes.byref(grads), _p(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "moe_backward_fp8")
