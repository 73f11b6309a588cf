"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Tensors are torch tensors already resident on the GPU; their data pointers,
the current HIP stream and the sizes are passed through unchanged.  The
library must be built (python -m top_routing_grouped_amd.build); there is no
fallback when it is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

F32, BF16, U4 = 0, 1, 2
SOFTMAX_TOPK, SIGMOID_GROUP_TOPK = 0, 1
_DT = {"f32": F32, "bf16": BF16, "u4": U4}
_FAM = {"softmax": SOFTMAX_TOPK, "sigmoid_group": SIGMOID_GROUP_TOPK}

# Entry points the header declares (checked by the CPU tests).
EXPORTS = ("moe_workspace_size", "moe_route", "moe_permute", "moe_experts", "moe_shared_expert",
           "moe_combine", "moe_layer_forward", "moe_layer_forward_noalloc", "moe_layer_forward_direct",
           "moe_rms_norm", "moe_layer_forward_norm",
           "moe_layer_stage", "moe_stream_read", "moe_mfma_rate", "moe_l2_read_rate", "moe_status_string", "moe_last_error")
STAGE_ROUTER_LOGITS, STAGE_GATE_UP, STAGE_DOWN, STAGE_GATE_UP_DIRECT, STAGE_DOWN_GROUPED, STAGE_DOWN_DIRECT = range(6)


class MoeConfig(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("family", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32)]


class MoeMatrix(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("min", ctypes.c_void_p)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("expert_bias", ctypes.c_void_p), ("gate", MoeMatrix),
                ("up", MoeMatrix), ("down", MoeMatrix), ("shared_gate", MoeMatrix), ("shared_up", MoeMatrix),
                ("shared_down", MoeMatrix), ("shared_gate_vec", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with python -m top_routing_grouped_amd.build")
        L = ctypes.CDLL(_LIB_PATH)
        P, S, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        cfg = ctypes.POINTER(MoeConfig)
        wts = ctypes.POINTER(MoeWeights)
        sig = {
            "moe_workspace_size": [cfg, ctypes.POINTER(ctypes.c_size_t)],
            "moe_route": [cfg, P, P, P, P, P, P, S, P],
            "moe_permute": [cfg, P, P, P, P, P, P, S, P],
            "moe_experts": [cfg, P, wts, P, P, P, P, P, P, P, S, P],
            "moe_shared_expert": [cfg, P, wts, P, P, S, P],
            "moe_combine": [cfg, P, P, P, P, P],
            "moe_layer_forward": [cfg, wts, P, P, P, P, P, P, S, P, P],
            "moe_layer_forward_noalloc": [cfg, wts, P, P, P, P, P, P],
            "moe_layer_forward_direct": [cfg, wts, P, P, P, P, P, P, S, P],
            "moe_rms_norm": [cfg, P, P, ctypes.c_float, P, P],
            "moe_layer_forward_norm": [cfg, wts, P, ctypes.c_float, P, P, P, P, P, P, S, P, P],
            "moe_layer_stage": [cfg, wts, P, I32, P, S, P],
            "moe_stream_read": [P, S, P, S, P],
            "moe_mfma_rate": [I32, I32, I32, P, S, P],
            "moe_l2_read_rate": [I32, I32, I32, P, S, P, S, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I32
        L.moe_status_string.argtypes = [I32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != MOE_OK:
        msg = lib().moe_last_error().decode()
        raise MoeError(status, where, f"{lib().moe_status_string(status).decode()} {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_config(n_tokens, d_model, n_experts, top_k, d_ff, d_ff_shared, family="softmax", n_group=1,
                topk_group=1, routed_scaling=1.0, act_dtype="bf16", router_dtype="bf16",
                expert_dtype="bf16") -> MoeConfig:
    return MoeConfig(n_tokens, d_model, n_experts, top_k, d_ff, d_ff_shared, _FAM[family], n_group, topk_group,
                     routed_scaling, _DT[act_dtype], _DT[router_dtype], _DT[expert_dtype])


def config_from_spec(spec, n_tokens: Optional[int] = None) -> MoeConfig:
    """Config from any object with LayerSpec's attribute names."""
    return make_config(spec.n_tokens if n_tokens is None else n_tokens, spec.d_model, spec.n_experts, spec.top_k,
                       spec.d_ff, spec.d_ff_shared, spec.family, spec.n_group, spec.topk_group, spec.routed_scaling,
                       spec.act_dtype, spec.router_dtype, spec.expert_dtype)


def _matrix(m) -> MoeMatrix:
    if m is None:
        return MoeMatrix(None, None, None)
    return MoeMatrix(m.w.data_ptr(), None if m.scale is None else m.scale.data_ptr(),
                     None if m.min is None else m.min.data_ptr())


def weights_struct(w) -> MoeWeights:
    """moe_weights from any object with LayerWeights' attribute names (matrices carry w/scale/min)."""
    return MoeWeights(w.router.data_ptr(), None if w.expert_bias is None else w.expert_bias.data_ptr(),
                      _matrix(w.gate), _matrix(w.up), _matrix(w.down), _matrix(w.shared_gate),
                      _matrix(w.shared_up), _matrix(w.shared_down),
                      None if w.shared_gate_vec is None else w.shared_gate_vec.data_ptr())


def workspace_size(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def alloc_workspace(cfg: MoeConfig, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(cfg), 256), dtype=torch.uint8, device=device)


def route(cfg, x, router, expert_bias, ids, weights, ws, stream=None):
    _check(lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(router), _ptr(expert_bias), _ptr(ids), _ptr(weights),
                           _ptr(ws), ws.numel(), _stream(stream)), "moe_route")


def permute(cfg, ids, offsets, active, n_active, sorted_pairs, ws=None, stream=None):
    _check(lib().moe_permute(ctypes.byref(cfg), _ptr(ids), _ptr(offsets), _ptr(active), _ptr(n_active),
                             _ptr(sorted_pairs), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "moe_permute")


def experts(cfg, x, wstruct: MoeWeights, offsets, active, n_active, sorted_pairs, topk_weights, slot_out, ws,
            stream=None):
    _check(lib().moe_experts(ctypes.byref(cfg), _ptr(x), ctypes.byref(wstruct), _ptr(offsets), _ptr(active),
                             _ptr(n_active), _ptr(sorted_pairs), _ptr(topk_weights), _ptr(slot_out), _ptr(ws),
                             ws.numel(), _stream(stream)), "moe_experts")


def shared_expert(cfg, x, wstruct: MoeWeights, shared_out, ws, stream=None):
    _check(lib().moe_shared_expert(ctypes.byref(cfg), _ptr(x), ctypes.byref(wstruct), _ptr(shared_out), _ptr(ws),
                                   ws.numel(), _stream(stream)), "moe_shared_expert")


def combine(cfg, slot_out, shared_out, residual, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(cfg), _ptr(slot_out), _ptr(shared_out), _ptr(residual), _ptr(out),
                             _stream(stream)), "moe_combine")


def layer_forward(cfg, wstruct: MoeWeights, x, residual, out, ids_out=None, weights_out=None, ws=None,
                  stream=None, aux_stream=None):
    _check(lib().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(wstruct), _ptr(x), _ptr(residual), _ptr(out),
                                   _ptr(ids_out), _ptr(weights_out), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(stream), None if aux_stream is None else _stream(aux_stream)),
           "moe_layer_forward")


def layer_forward_noalloc(cfg, wstruct: MoeWeights, x, residual, out, ids_out=None, weights_out=None, stream=None):
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(wstruct), _ptr(x), _ptr(residual),
                                           _ptr(out), _ptr(ids_out), _ptr(weights_out), _stream(stream)),
           "moe_layer_forward_noalloc")


def layer_forward_direct(cfg, wstruct: MoeWeights, x, residual, out, ids_out=None, weights_out=None, ws=None,
                         stream=None):
    _check(lib().moe_layer_forward_direct(ctypes.byref(cfg), ctypes.byref(wstruct), _ptr(x), _ptr(residual),
                                          _ptr(out), _ptr(ids_out), _ptr(weights_out), _ptr(ws),
                                          0 if ws is None else ws.numel(), _stream(stream)),
           "moe_layer_forward_direct")


def rms_norm(cfg, residual, norm_weight, eps: float, x, stream=None):
    _check(lib().moe_rms_norm(ctypes.byref(cfg), _ptr(residual), _ptr(norm_weight), eps, _ptr(x), _stream(stream)),
           "moe_rms_norm")


def layer_forward_norm(cfg, wstruct: MoeWeights, norm_weight, eps: float, residual, out, x_out=None, ids_out=None,
                       weights_out=None, ws=None, stream=None, aux_stream=None):
    _check(lib().moe_layer_forward_norm(ctypes.byref(cfg), ctypes.byref(wstruct), _ptr(norm_weight), eps,
                                        _ptr(residual), _ptr(x_out), _ptr(out), _ptr(ids_out), _ptr(weights_out),
                                        _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream),
                                        None if aux_stream is None else _stream(aux_stream)),
           "moe_layer_forward_norm")


def stream_read(buf, sink, stream=None):
    """One streaming read of the bytes of device tensor `buf` (measurement aid;
    sink: a uint32 device tensor of at least buf.nbytes / 1024 elements)."""
    _check(lib().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), sink.numel(),
                                 _stream(stream)), "moe_stream_read")


def mfma_rate(shape: int, workgroups: int, iterations: int, sink, stream=None):
    """One launch of the MFMA issue-rate loop (measurement aid; shape 0:
    16x16x32 bf16, 1: 32x32x16 bf16; sink: a float32 device tensor of at
    least 256 * workgroups elements)."""
    _check(lib().moe_mfma_rate(shape, workgroups, iterations, _ptr(sink), sink.numel(), _stream(stream)),
           "moe_mfma_rate")


def l2_read_rate(pattern: int, workgroups: int, iterations: int, buf, sink, stream=None):
    """One launch of the L2 read-rate loop (measurement aid; pattern 0: row
    segments, 1: MFMA operand order, 2: row quads; buf: a device tensor of at
    least 1 MiB; sink: an int32 device tensor of at least 256 * workgroups
    elements)."""
    _check(lib().moe_l2_read_rate(pattern, workgroups, iterations, _ptr(buf), buf.numel() * buf.element_size(),
                                  _ptr(sink), sink.numel(), _stream(stream)), "moe_l2_read_rate")


def layer_stage(cfg, wstruct: MoeWeights, x, stage: int, ws, stream=None):
    """Re-launch one kernel stage of the last layer_forward on `ws` (measurement aid)."""
    _check(lib().moe_layer_stage(ctypes.byref(cfg), ctypes.byref(wstruct), _ptr(x), stage, _ptr(ws), ws.numel(),
                                 _stream(stream)), "moe_layer_stage")
