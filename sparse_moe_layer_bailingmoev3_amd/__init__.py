"""Python binding of libmoe, the HIP (gfx950) forward pass of one BailingMoeV3 sparse MoE
layer (Ling-3.0-flash / Ling-3.0-flash-VL).

Argument marshalling only: every step of the layer runs in the library's kernels.  The
functions carry the C-ABI names of include/moe.h and take torch tensors that already live on
the GPU (torch provides device memory and streams).  The library must be built first:

    python -m sparse_moe_layer_bailingmoev3_amd.build

There is no fallback: if libmoe.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = ["MoEConfig", "MoEExpertWeights", "MoEError", "lib_path", "load_library", "moe_workspace_size",
           "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_forward_traced",
           "moe_forward_timed", "moe_update_expert_bias", "moe_dense_ffn_workspace_size", "moe_dense_ffn",
           "moe_forward_noalloc", "moe_quantise_mxfp8", "moe_pack_mxfp4", "moe_pack_mxfp8", "moe_status_string",
           "MOE_WEIGHTS_BF16", "MOE_WEIGHTS_MXFP4", "MOE_WEIGHTS_MXFP8", "MOE_WEIGHTS_MXFP4_TILED",
           "MOE_WEIGHTS_MXFP8_TILED",
           "MOE_ACT_BF16", "MOE_ACT_MXFP8",
           "EXPORTED_SYMBOLS"]

MOE_WEIGHTS_BF16 = 0
MOE_WEIGHTS_MXFP4 = 1
MOE_WEIGHTS_MXFP8 = 2
MOE_WEIGHTS_MXFP4_TILED = 3
MOE_WEIGHTS_MXFP8_TILED = 4
MOE_ACT_BF16 = 0
MOE_ACT_MXFP8 = 1

EXPORTED_SYMBOLS = ("moe_workspace_size", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                    "moe_forward", "moe_forward_traced", "moe_forward_timed", "moe_update_expert_bias",
                    "moe_dense_ffn_workspace_size", "moe_dense_ffn", "moe_forward_noalloc", "moe_quantise_mxfp8",
                    "moe_pack_mxfp4", "moe_pack_mxfp8", "moe_status_string", "moe_last_error")

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libmoe.so")


class MoEConfig(ctypes.Structure):
    """moe_config_t; field names follow the model's text_config."""
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_experts_per_tok", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("moe_intermediate_size", ctypes.c_int32),
                ("num_shared_experts", ctypes.c_int32), ("shared_intermediate_size", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("swiglu_limit", ctypes.c_float), ("shared_swiglu_limit", ctypes.c_float),
                ("expert_weight_format", ctypes.c_int32), ("expert_act_format", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale",
                                                "shared_gate", "shared_up", "shared_down")]


class MoEExpertWeights:
    """moe_expert_weights_t built from device tensors (references are kept alive here)."""

    def __init__(self, gate, up, down, gate_scale=None, up_scale=None, down_scale=None,
                 shared_gate=None, shared_up=None, shared_down=None):
        self._keep = (gate, up, down, gate_scale, up_scale, down_scale, shared_gate, shared_up, shared_down)
        self.struct = _Weights(*[_ptr(t) for t in self._keep])


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{moe_status_string(status)}: {message}")
        self.status = status


_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run: python -m sparse_moe_layer_bailingmoev3_amd.build")
    lib = ctypes.CDLL(path)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    C = ctypes.POINTER(MoEConfig)
    W = ctypes.POINTER(_Weights)
    sigs = {
        "moe_workspace_size": [C, I64, ctypes.POINTER(SZ)],
        "moe_route": [C, I64, P, P, P, P, P, P, SZ, P],
        "moe_dispatch": [C, I64, P, P, P, P, P, P, SZ, P],
        "moe_expert_ffn": [C, I64, P, P, P, W, P, P, SZ, P],
        "moe_combine": [C, I64, P, P, P, P, P],
        "moe_forward": [C, I64, P, P, P, W, P, P, P, P, P, SZ, P],
        "moe_forward_traced": [C, I64, P, P, P, W, P, P, SZ, P, ctypes.POINTER(P), ctypes.c_int32,
                               ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int32)],
        "moe_forward_timed": [C, I64, P, P, P, W, P, P, SZ, P, ctypes.c_int32, P, P],
        "moe_update_expert_bias": [C, P, P, ctypes.c_float, P],
        "moe_dense_ffn_workspace_size": [ctypes.c_int32, ctypes.c_int32, I64, ctypes.POINTER(SZ)],
        "moe_dense_ffn": [ctypes.c_int32, ctypes.c_int32, ctypes.c_float, I64, P, P, P, P, P, P, SZ, P],
        "moe_forward_noalloc": [C, I64, P, P, P, W, P, P, P, P, P],
        "moe_quantise_mxfp8": [P, I64, ctypes.c_int32, P, P, P],
        "moe_pack_mxfp4": [P, P, I64, ctypes.c_int32, ctypes.c_int32, P, P, P],
        "moe_pack_mxfp8": [P, P, I64, ctypes.c_int32, ctypes.c_int32, P, P, P],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != 0:
        raise MoEError(status, load_library().moe_last_error().decode())


def _ws(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def moe_workspace_size(cfg: MoEConfig, T: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().moe_workspace_size(ctypes.byref(cfg), T, ctypes.byref(n)))
    return n.value


def moe_route(cfg, T, x, router_w, expert_bias, topk_idx, topk_w, ws, stream=None):
    p, n = _ws(ws)
    _check(load_library().moe_route(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w), _ptr(expert_bias),
                                    _ptr(topk_idx), _ptr(topk_w), p, n, _stream(stream)))


def moe_dispatch(cfg, T, topk_idx, expert_counts, expert_offsets, sorted_token, inv_perm, ws, stream=None):
    p, n = _ws(ws)
    _check(load_library().moe_dispatch(ctypes.byref(cfg), T, _ptr(topk_idx), _ptr(expert_counts),
                                       _ptr(expert_offsets), _ptr(sorted_token), _ptr(inv_perm), p, n,
                                       _stream(stream)))


def moe_expert_ffn(cfg, T, x, expert_offsets, sorted_token, weights: MoEExpertWeights, y_sorted, ws, stream=None):
    p, n = _ws(ws)
    _check(load_library().moe_expert_ffn(ctypes.byref(cfg), T, _ptr(x), _ptr(expert_offsets), _ptr(sorted_token),
                                         ctypes.byref(weights.struct), _ptr(y_sorted), p, n, _stream(stream)))


def moe_combine(cfg, T, y_sorted, inv_perm, topk_w, out, stream=None):
    _check(load_library().moe_combine(ctypes.byref(cfg), T, _ptr(y_sorted), _ptr(inv_perm), _ptr(topk_w),
                                      _ptr(out), _stream(stream)))


def moe_forward(cfg, T, x, router_w, expert_bias, weights: MoEExpertWeights, out, topk_idx_out=None,
                topk_w_out=None, expert_counts_out=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(load_library().moe_forward(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w), _ptr(expert_bias),
                                      ctypes.byref(weights.struct), _ptr(out), _ptr(topk_idx_out),
                                      _ptr(topk_w_out), _ptr(expert_counts_out), p, n, _stream(stream)))


def moe_forward_traced(cfg, T, x, router_w, expert_bias, weights: MoEExpertWeights, out, ws, events, stream=None):
    """moe_forward recording events[0] before and events[i+1] after the i-th kernel.  `events`
    are raw hipEvent_t handles (ints).  Returns the list of kernel names in launch order."""
    p, n = _ws(ws)
    ev = (ctypes.c_void_p * len(events))(*events)
    names = (ctypes.c_char_p * max(1, len(events) - 1))()
    nk = ctypes.c_int32()
    _check(load_library().moe_forward_traced(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w), _ptr(expert_bias),
                                             ctypes.byref(weights.struct), _ptr(out), p, n, _stream(stream), ev,
                                             len(events), names, ctypes.byref(nk)))
    return [names[i].decode() for i in range(nk.value)]


def moe_forward_timed(cfg, T, x, router_w, expert_bias, weights: MoEExpertWeights, out, ws, kernel_index,
                      start_event, stop_event, stream=None):
    """moe_forward with kernel `kernel_index` (its position in moe_forward_traced's list) timed
    by two raw hipEvent_t handles bound to its dispatch; adds nothing else to the queue."""
    p, n = _ws(ws)
    _check(load_library().moe_forward_timed(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w), _ptr(expert_bias),
                                            ctypes.byref(weights.struct), _ptr(out), p, n, _stream(stream),
                                            kernel_index, start_event, stop_event))


def moe_update_expert_bias(cfg, expert_counts, expert_bias, gamma, stream=None):
    """In-place sign-rule update of the routed experts' selection bias from a step's counts."""
    _check(load_library().moe_update_expert_bias(ctypes.byref(cfg), _ptr(expert_counts), _ptr(expert_bias),
                                                 float(gamma), _stream(stream)))


def moe_dense_ffn_workspace_size(hidden_size, intermediate_size, T) -> int:
    n = ctypes.c_size_t()
    _check(load_library().moe_dense_ffn_workspace_size(hidden_size, intermediate_size, T, ctypes.byref(n)))
    return n.value


def moe_dense_ffn(hidden_size, intermediate_size, swiglu_limit, T, x, gate, up, down, out, ws, stream=None):
    """Dense SwiGLU FFN out = (silu(x gate^T) * (x up^T)) down^T (bf16 in and out)."""
    p, n = _ws(ws)
    _check(load_library().moe_dense_ffn(hidden_size, intermediate_size, float(swiglu_limit), T, _ptr(x), _ptr(gate),
                                        _ptr(up), _ptr(down), _ptr(out), p, n, _stream(stream)))


def moe_forward_noalloc(cfg, T, x, router_w, expert_bias, weights: MoEExpertWeights, out, topk_idx_out=None,
                        topk_w_out=None, expert_counts_out=None, stream=None):
    """moe_forward on the library's static 64 MiB device scratch instead of a caller workspace
    (for callers that cannot allocate); rejects T whose workspace does not fit."""
    _check(load_library().moe_forward_noalloc(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w), _ptr(expert_bias),
                                              ctypes.byref(weights.struct), _ptr(out), _ptr(topk_idx_out),
                                              _ptr(topk_w_out), _ptr(expert_counts_out), _stream(stream)))


def moe_pack_mxfp4(codes, scales, mats, N, Kd, codes_out, scales_out, stream=None):
    """Row-major MXFP4 codes [mats, N, Kd/2] and scales [mats, N, Kd/32] -> the tiled order of
    MOE_WEIGHTS_MXFP4_TILED (same sizes)."""
    _check(load_library().moe_pack_mxfp4(_ptr(codes), _ptr(scales), mats, N, Kd, _ptr(codes_out), _ptr(scales_out),
                                         _stream(stream)))


def moe_pack_mxfp8(codes, scales, mats, N, Kd, codes_out, scales_out, stream=None):
    """Row-major MXFP8 codes [mats, N, Kd] and scales [mats, N, Kd/32] -> the tiled order of
    MOE_WEIGHTS_MXFP8_TILED (same sizes)."""
    _check(load_library().moe_pack_mxfp8(_ptr(codes), _ptr(scales), mats, N, Kd, _ptr(codes_out), _ptr(scales_out),
                                         _stream(stream)))


def moe_quantise_mxfp8(x, rows, cols, codes, scales, stream=None):
    """bf16 [rows, cols] -> MXFP8 E4M3 codes [rows, cols] and e8m0 scales [rows, cols/32] (the
    rounding the MXFP8-activation path applies to x)."""
    _check(load_library().moe_quantise_mxfp8(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))
