"""ctypes binding of libmoe_mi355x.so: argument marshalling only.

Every function here has the name and argument order of the C entry point it wraps
(include/moe.h).  Tensors are torch tensors on the GPU; the binding passes their
data_ptr() and the current HIP stream and raises ``MoeError`` on a negative status.
All arithmetic happens in the library's HIP kernels.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_DEVICE = \
    -1, -2, -3, -4, -5
(MOE_FMT_FP32, MOE_FMT_INT8_ROW, MOE_FMT_INT4_G32, MOE_FMT_INT6_G32, MOE_FMT_INT3_G32,
 MOE_FMT_INT2_G32) = range(6)
MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_EXPERT_FFN, MOE_OP_LAYER_DECODE, MOE_OP_EXPERTS_DECODE = \
    0, 1, 2, 3, 4
MOE_OP_BLOCK_DECODE = 5

EXPORTED = ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
            "moe_layer_decode", "moe_layer_decode_noalloc", "moe_experts_decode",
            "moe_dequant_probe", "moe_rmsnorm", "moe_combine_gated", "moe_block_decode",
            "moe_workspace_size", "moe_check_device_error", "moe_status_string",
            "moe_last_error", "moe_version")


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (status %d)" % (msg, status))
        self.status = status


class moe_router(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("w", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class moe_norm(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("gate_w", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("gate_b", ctypes.c_float)]


class moe_experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


_lib = None


def lib():
    """Load the library; fail loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmoe_mi355x.so is not built (%s); run "
                              "`python -m quantized_sparse_moe_router_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "moe_route": [P, P, I32, I32, P, P, P, P, SZ, P],
            "moe_permute": [P, I32, I32, I32, P, P, P, P, SZ, P],
            "moe_expert_ffn": [P, P, I32, I32, P, P, P, P, P, SZ, P],
            "moe_combine": [P, P, P, P, P, I32, I32, I32, P, P],
            "moe_layer_decode": [P, P, P, P, I32, I32, P, P, P, P, P, SZ, P],
            "moe_experts_decode": [P, P, P, I32, I32, P, P, P, P, P, SZ, P],
            "moe_layer_decode_noalloc": [P, P, P, P, I32, I32, P, P, P, P, P],
            "moe_dequant_probe": [I32, I32, P, P, ctypes.c_int64, P, P],
            "moe_rmsnorm": [P, P, I32, I32, P, P, P],
            "moe_combine_gated": [P, P, P, P, P, P, I32, I32, I32, P, P],
            "moe_block_decode": [P, P, P, P, P, I32, I32, P, P, P, P, SZ, P],
            "moe_workspace_size": [I32, I32, I32, I32, I32, I32],
            "moe_check_device_error": [P],
            "moe_status_string": [I32],
            "moe_last_error": [],
            "moe_version": [],
        }
        res = {"moe_workspace_size": SZ, "moe_status_string": ctypes.c_char_p,
               "moe_last_error": ctypes.c_char_p, "moe_version": ctypes.c_char_p}
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res.get(name, ctypes.c_int32)
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st, name):
    if st != MOE_OK:
        raise MoeError(st, "%s: %s" % (name, lib().moe_last_error().decode()))


def router_desc(fmt, w, scale=None, bias=None):
    """moe_router for a router tensor set; keep the returned object alive while in use."""
    d = moe_router(int(fmt), int(w.shape[0]), int(w.shape[1]), 0, _ptr(w), _ptr(scale),
                   _ptr(bias))
    d._keep = (w, scale, bias)
    return d


def norm_desc(gamma, eps, gate_w=None, gate_b=0.0):
    """moe_norm for a norm / residual-gate tensor set; keep the returned object alive."""
    d = moe_norm(_ptr(gamma), _ptr(gate_w), float(eps), float(gate_b))
    d._keep = (gamma, gate_w)
    return d


def experts_desc(fmt, d_model, d_ff, w_gate, w_up, w_down, s_gate, s_up, s_down):
    """moe_experts for a set of experts; n_experts is the leading dim of w_gate."""
    d = moe_experts(int(fmt), int(w_gate.shape[0]), int(d_model), int(d_ff), _ptr(w_gate),
                    _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down))
    d._keep = (w_gate, w_up, w_down, s_gate, s_up, s_down)
    return d


def moe_workspace_size(op, T, k, E, d, d_ff):
    return int(lib().moe_workspace_size(op, T, k, E, d, d_ff))


def moe_route(router, x, T, k, ids, weights, logits=None, ws=None, stream=None):
    """ws: a zero-initialised workspace of moe_workspace_size(MOE_OP_ROUTE, ...) bytes."""
    st = lib().moe_route(ctypes.byref(router), _ptr(x), T, k, _ptr(ids), _ptr(weights),
                         _ptr(logits), _ptr(ws), 0 if ws is None else ws.numel() *
                         ws.element_size(), _stream(stream))
    _check(st, "moe_route")


def moe_permute(ids, T, k, E, offsets, sorted_pairs, pair_pos, ws=None, stream=None):
    st = lib().moe_permute(_ptr(ids), T, k, E, _ptr(offsets), _ptr(sorted_pairs),
                           _ptr(pair_pos), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_permute")


def moe_expert_ffn(experts, x, T, k, ids, offsets, sorted_pairs, y, ws, stream=None):
    st = lib().moe_expert_ffn(ctypes.byref(experts), _ptr(x), T, k, _ptr(ids), _ptr(offsets),
                              _ptr(sorted_pairs), _ptr(y), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream))
    _check(st, "moe_expert_ffn")


def moe_combine(y_pairs, pair_pos, weights, y_shared, residual, T, k, d, out, stream=None):
    st = lib().moe_combine(_ptr(y_pairs), _ptr(pair_pos), _ptr(weights), _ptr(y_shared),
                           _ptr(residual), T, k, d, _ptr(out), _stream(stream))
    _check(st, "moe_combine")


def moe_layer_decode(router, routed, shared, x, T, k, ids, weights, residual, out, ws,
                     stream=None):
    """ws: a zero-initialised workspace of moe_workspace_size(MOE_OP_LAYER_DECODE, ...)."""
    st = lib().moe_layer_decode(ctypes.byref(router), ctypes.byref(routed),
                                ctypes.byref(shared) if shared is not None else None,
                                _ptr(x), T, k, _ptr(ids), _ptr(weights), _ptr(residual),
                                _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream))
    _check(st, "moe_layer_decode")


def moe_layer_decode_noalloc(router, routed, shared, x, T, k, ids, weights, residual, out,
                             stream=None):
    st = lib().moe_layer_decode_noalloc(
        ctypes.byref(router), ctypes.byref(routed),
        ctypes.byref(shared) if shared is not None else None, _ptr(x), int(T), int(k),
        _ptr(ids), _ptr(weights), _ptr(residual), _ptr(out), _stream(stream))
    _check(st, "moe_layer_decode_noalloc")


def moe_experts_decode(routed, shared, x, T, k, ids, weights, residual, out, ws, stream=None):
    """ws: a zero-initialised workspace of moe_workspace_size(MOE_OP_EXPERTS_DECODE, ...)."""
    st = lib().moe_experts_decode(ctypes.byref(routed),
                                  ctypes.byref(shared) if shared is not None else None,
                                  _ptr(x), T, k, _ptr(ids), _ptr(weights), _ptr(residual),
                                  _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream))
    _check(st, "moe_experts_decode")


def moe_dequant_probe(fmt, form, w, s, n_groups, out, stream=None):
    st = lib().moe_dequant_probe(int(fmt), int(form), _ptr(w), _ptr(s), int(n_groups),
                                 _ptr(out), _stream(stream))
    _check(st, "moe_dequant_probe")


def moe_rmsnorm(norm, x, T, d, xn, z, stream=None):
    st = lib().moe_rmsnorm(ctypes.byref(norm), _ptr(x), int(T), int(d), _ptr(xn), _ptr(z),
                           _stream(stream))
    _check(st, "moe_rmsnorm")


def moe_combine_gated(y_pairs, pair_pos, weights, y_shared, z, residual, T, k, d, out,
                      stream=None):
    st = lib().moe_combine_gated(_ptr(y_pairs), _ptr(pair_pos), _ptr(weights), _ptr(y_shared),
                                 _ptr(z), _ptr(residual), int(T), int(k), int(d), _ptr(out),
                                 _stream(stream))
    _check(st, "moe_combine_gated")


def moe_block_decode(norm, router, routed, shared, x, T, k, ids, weights, out, ws,
                     stream=None):
    st = lib().moe_block_decode(ctypes.byref(norm), ctypes.byref(router), ctypes.byref(routed),
                                ctypes.byref(shared) if shared is not None else None, _ptr(x),
                                int(T), int(k), _ptr(ids), _ptr(weights), _ptr(out), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_block_decode")


def moe_check_device_error(stream=None):
    st = lib().moe_check_device_error(_stream(stream))
    _check(st, "moe_check_device_error")


def moe_status_string(st):
    return lib().moe_status_string(st).decode()


def moe_last_error():
    return lib().moe_last_error().decode()


def moe_version():
    return lib().moe_version().decode()
