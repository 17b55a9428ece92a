"""ctypes binding of libmoe.so: the C ABI of include/moe.h under the same names.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  Tensors are passed by ``data_ptr()``; device-pointer arguments must be
contiguous tensors on a GPU (a host pointer handed to a kernel would fault), and
raw integers are passed through as addresses.  A non-zero status raises MoeError.
There is no fallback: if libmoe.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_E4M3, MOE_E4M3_POW2 = 0, 1, 2, 3
DTYPE_CODES = {"f32": MOE_F32, "bf16": MOE_BF16, "e4m3": MOE_E4M3, "e4m3_pow2": MOE_E4M3_POW2}


class MoeConfig(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_shared", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("top_groups", ctypes.c_int32),
                ("group_topn", ctypes.c_int32), ("act_dtype", ctypes.c_int),
                ("w_dtype", ctypes.c_int)]


class MoeExpertWeights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {code})")
        self.code = code


_lib = None
_P = ctypes.c_void_p
_CFG = ctypes.POINTER(MoeConfig)
_SIGS = {
    "moe_workspace_bytes": (ctypes.c_size_t, [_CFG]),
    "moe_route": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_permute": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_act_quant_e4m3": (ctypes.c_int, [_CFG, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "moe_grouped_ffn": (ctypes.c_int, [_CFG, _P, _P, _P, ctypes.POINTER(MoeExpertWeights), _P,
                                       _P, ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P]),
    "moe_bias_update": (ctypes.c_int, [_CFG, _P, ctypes.c_float, _P, _P]),
    "moe_layer_forward": (ctypes.c_int, [_CFG, _P, _P, _P, ctypes.POINTER(MoeExpertWeights), _P,
                                         _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [_CFG, _P, _P, _P, ctypes.POINTER(MoeExpertWeights),
                                                 _P, _P, _P, _P, _P, _P]),
    "moe_router_scores": (ctypes.c_int, [_CFG, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_balance_loss": (ctypes.c_int, [_CFG, _P, _P, ctypes.c_int32, ctypes.c_float, _P, _P, _P,
                                        _P, _P, ctypes.c_size_t, _P]),
    "moe_combine_backward": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P]),
    "moe_gate_backward": (ctypes.c_int, [_CFG, _P, _P, _P, _P, ctypes.c_int32, _P]),
    "moe_swiglu_backward": (ctypes.c_int, [_CFG, _P, _P, _P, ctypes.c_int32, _P, _P, _P]),
    "moe_backward_workspace_bytes": (ctypes.c_size_t, [_CFG]),
    "moe_router_backward": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_router_backward_workspace_bytes": (ctypes.c_size_t, [_CFG]),
    "moe_expert_backward": (ctypes.c_int, [_CFG, _P, _P, _P, _P, ctypes.POINTER(MoeExpertWeights),
                                           _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_backward_input": (ctypes.c_int, [_CFG, _P, _P, _P, _P,
                                                 ctypes.POINTER(MoeExpertWeights), _P, _P, _P,
                                                 ctypes.c_size_t, _P]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


def lib() -> ctypes.CDLL:
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m "
                               "sparse_moe_layer_affinity_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_symbols() -> list:
    """Function names declared in include/moe.h."""
    hdr = os.path.join(os.path.dirname(_HERE), "include", "moe.h")
    text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def make_config(T, hidden, inter, E, K, G, M, topn, Ns=1, act="bf16", w="bf16") -> MoeConfig:
    return MoeConfig(int(T), int(hidden), int(inter), int(E), int(Ns), int(K), int(G), int(M),
                     int(topn), DTYPE_CODES[act], DTYPE_CODES[w])


def _dev(t, name, nullable=False):
    """Device address of a tensor (or a raw int address)."""
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} must not be None")
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (a host pointer would fault the kernel)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, code: int):
    if code != MOE_OK:
        raise MoeError(fn, code, lib().moe_status_string(code).decode())


def _weights(w: dict) -> MoeExpertWeights:
    return MoeExpertWeights(_dev(w["w_gate"], "w_gate"), _dev(w["w_up"], "w_up"),
                            _dev(w["w_down"], "w_down"), _dev(w.get("s_gate"), "s_gate", True),
                            _dev(w.get("s_up"), "s_up", True), _dev(w.get("s_down"), "s_down", True))


def moe_workspace_bytes(cfg: MoeConfig) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg)))


def moe_route(cfg, x, w_router, bias, topk_idx, topk_gate, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_route", lib().moe_route(
        ctypes.byref(cfg), _dev(x, "x"), _dev(w_router, "w_router"), _dev(bias, "bias"),
        _dev(topk_idx, "topk_idx"), _dev(topk_gate, "topk_gate"), _dev(ws, "ws"), ws_bytes,
        _stream(stream)))


def moe_permute(cfg, topk_idx, expert_load, expert_offsets, row_token, pair_row, ws,
                ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_permute", lib().moe_permute(
        ctypes.byref(cfg), _dev(topk_idx, "topk_idx"), _dev(expert_load, "expert_load"),
        _dev(expert_offsets, "expert_offsets"), _dev(row_token, "row_token"),
        _dev(pair_row, "pair_row"), _dev(ws, "ws"), ws_bytes, _stream(stream)))


def moe_act_quant_e4m3(cfg, x, rows, cols, q, scales, stream=None):
    _check("moe_act_quant_e4m3", lib().moe_act_quant_e4m3(
        ctypes.byref(cfg), _dev(x, "x"), int(rows), int(cols), _dev(q, "q"),
        _dev(scales, "scales"), _stream(stream)))


def moe_grouped_ffn(cfg, x, expert_offsets, row_token, weights: dict, y_rows, ws,
                    ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    w = _weights(weights)
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        ctypes.byref(cfg), _dev(x, "x"), _dev(expert_offsets, "expert_offsets"),
        _dev(row_token, "row_token"), ctypes.byref(w), _dev(y_rows, "y_rows"), _dev(ws, "ws"),
        ws_bytes, _stream(stream)))


def moe_combine(cfg, y_rows, pair_row, topk_gate, residual, y, stream=None):
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(cfg), _dev(y_rows, "y_rows"), _dev(pair_row, "pair_row"),
        _dev(topk_gate, "topk_gate"), _dev(residual, "residual", True), _dev(y, "y"),
        _stream(stream)))


def moe_bias_update(cfg, expert_load, gamma, bias, stream=None):
    _check("moe_bias_update", lib().moe_bias_update(
        ctypes.byref(cfg), _dev(expert_load, "expert_load"), float(gamma), _dev(bias, "bias"),
        _stream(stream)))


def moe_layer_forward(cfg, x, w_router, bias, weights: dict, residual, y, topk_idx, topk_gate,
                      expert_load, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    w = _weights(weights)
    _check("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(cfg), _dev(x, "x"), _dev(w_router, "w_router"), _dev(bias, "bias"),
        ctypes.byref(w), _dev(residual, "residual", True), _dev(y, "y"),
        _dev(topk_idx, "topk_idx"), _dev(topk_gate, "topk_gate"),
        _dev(expert_load, "expert_load"), _dev(ws, "ws"), ws_bytes, _stream(stream)))


def moe_layer_forward_noalloc(cfg, x, w_router, bias, weights: dict, residual, y, topk_idx,
                              topk_gate, expert_load, stream=None):
    w = _weights(weights)
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        ctypes.byref(cfg), _dev(x, "x"), _dev(w_router, "w_router"), _dev(bias, "bias"),
        ctypes.byref(w), _dev(residual, "residual", True), _dev(y, "y"),
        _dev(topk_idx, "topk_idx"), _dev(topk_gate, "topk_gate"),
        _dev(expert_load, "expert_load"), _stream(stream)))


def moe_router_scores(cfg, x, w_router, scores, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_router_scores", lib().moe_router_scores(
        ctypes.byref(cfg), _dev(x, "x"), _dev(w_router, "w_router"), _dev(scores, "scores"),
        _dev(ws, "ws"), ws_bytes, _stream(stream)))


def moe_balance_loss(cfg, scores, topk_idx, seq_len, alpha, seq_loss, expert_frac, expert_prob,
                     grad_logits, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_balance_loss", lib().moe_balance_loss(
        ctypes.byref(cfg), _dev(scores, "scores"), _dev(topk_idx, "topk_idx"), int(seq_len),
        float(alpha), _dev(seq_loss, "seq_loss"), _dev(expert_frac, "expert_frac", True),
        _dev(expert_prob, "expert_prob", True), _dev(grad_logits, "grad_logits", True),
        _dev(ws, "ws"), ws_bytes, _stream(stream)))


def moe_combine_backward(cfg, dy, y_rows, pair_row, topk_gate, dgate, dy_rows, stream=None):
    _check("moe_combine_backward", lib().moe_combine_backward(
        ctypes.byref(cfg), _dev(dy, "dy"), _dev(y_rows, "y_rows"), _dev(pair_row, "pair_row"),
        _dev(topk_gate, "topk_gate"), _dev(dgate, "dgate"), _dev(dy_rows, "dy_rows"),
        _stream(stream)))


def moe_gate_backward(cfg, scores, topk_idx, dgate, grad_logits, accumulate=False, stream=None):
    _check("moe_gate_backward", lib().moe_gate_backward(
        ctypes.byref(cfg), _dev(scores, "scores"), _dev(topk_idx, "topk_idx"),
        _dev(dgate, "dgate"), _dev(grad_logits, "grad_logits"), int(bool(accumulate)),
        _stream(stream)))


def moe_swiglu_backward(cfg, a, b, dh, rows, da, db, stream=None):
    _check("moe_swiglu_backward", lib().moe_swiglu_backward(
        ctypes.byref(cfg), _dev(a, "a"), _dev(b, "b"), _dev(dh, "dh"), int(rows), _dev(da, "da"),
        _dev(db, "db"), _stream(stream)))


def moe_backward_workspace_bytes(cfg: MoeConfig) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(cfg)))


def moe_expert_backward_input(cfg, x, expert_offsets, row_token, pair_row, weights: dict, dy_rows,
                              dx, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    w = _weights(weights)
    _check("moe_expert_backward_input", lib().moe_expert_backward_input(
        ctypes.byref(cfg), _dev(x, "x"), _dev(expert_offsets, "expert_offsets"),
        _dev(row_token, "row_token"), _dev(pair_row, "pair_row"), ctypes.byref(w),
        _dev(dy_rows, "dy_rows"), _dev(dx, "dx"), _dev(ws, "ws"), ws_bytes, _stream(stream)))


def moe_expert_backward(cfg, x, expert_offsets, row_token, pair_row, weights: dict, dy_rows, dx,
                        dw_gate, dw_up, dw_down, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    w = _weights(weights)
    _check("moe_expert_backward", lib().moe_expert_backward(
        ctypes.byref(cfg), _dev(x, "x"), _dev(expert_offsets, "expert_offsets"),
        _dev(row_token, "row_token"), _dev(pair_row, "pair_row"), ctypes.byref(w),
        _dev(dy_rows, "dy_rows"), _dev(dx, "dx", True), _dev(dw_gate, "dw_gate", True),
        _dev(dw_up, "dw_up", True), _dev(dw_down, "dw_down", True), _dev(ws, "ws"), ws_bytes,
        _stream(stream)))


def moe_router_backward_workspace_bytes(cfg: MoeConfig) -> int:
    return int(lib().moe_router_backward_workspace_bytes(ctypes.byref(cfg)))


def moe_router_backward(cfg, x, w_router, grad_logits, dx, dw_router, ws, ws_bytes=None,
                        stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_router_backward", lib().moe_router_backward(
        ctypes.byref(cfg), _dev(x, "x"), _dev(w_router, "w_router"),
        _dev(grad_logits, "grad_logits"), _dev(dx, "dx", True), _dev(dw_router, "dw_router", True),
        _dev(ws, "ws"), ws_bytes, _stream(stream)))


def moe_status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()
