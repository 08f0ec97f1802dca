"""Routed MoE layer (forward and local backward) for MI355X (gfx950): Python binding of libmoe.

The binding only marshals arguments: torch tensors give device pointers and
the current HIP stream, and every step runs in the HIP kernels of libmoe.so
(built by ``python -m mixture_experts_layer_09_amd.build``).  There is no
fallback: if the library is missing or a call fails, an exception is raised.

Function names and argument meanings follow include/moe.h.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

PREC = {"fp32": 0, "bf16": 1, "fp8": 2, "mxfp8": 3, "mxfp4": 4, "int8": 5}
SCORE = {"sigmoid": 0, "softmax": 1, "sqrt_softplus": 2}
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP", -5: "MOE_ERR_DEVICE_DATA",
          -6: "MOE_ERR_SCRATCH"}
NO_ALLOC_MAX_ASSIGNMENTS = 262144   # MOE_NO_ALLOC_MAX_ASSIGNMENTS
EXPORTED = ["moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
            "moe_forward", "moe_check_device_error", "moe_status_string",
            "moe_backward_workspace_size", "moe_backward", "moe_forward_train",
            "moe_backward_saved", "moe_permute_no_alloc"]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {moe_status_string(status)}")


class moe_shape(C.Structure):
    _fields_ = [("tokens", C.c_int32), ("hidden", C.c_int32), ("experts", C.c_int32),
                ("topk", C.c_int32), ("inter", C.c_int32), ("has_shared", C.c_int32),
                ("precision", C.c_int32)]


class moe_route_opts(C.Structure):
    _fields_ = [("score_fn", C.c_int32), ("renorm", C.c_int32), ("alpha", C.c_float),
                ("expert_bias", C.c_void_p), ("gate_bias", C.c_void_p),
                ("token_ids", C.c_void_p), ("tid2eid", C.c_void_p), ("vocab", C.c_int32)]


class moe_expert_weights(C.Structure):
    _fields_ = [("W1", C.c_void_p), ("w1_scale", C.c_void_p), ("W2", C.c_void_p),
                ("w2_scale", C.c_void_p), ("Ws1", C.c_void_p), ("ws1_scale", C.c_void_p),
                ("Ws2", C.c_void_p), ("ws2_scale", C.c_void_p)]


class moe_grads(C.Structure):
    _fields_ = [("dX", C.c_void_p), ("dW1", C.c_void_p), ("dW2", C.c_void_p), ("dWs1", C.c_void_p),
                ("dWs2", C.c_void_p), ("dWg", C.c_void_p), ("dgate_bias", C.c_void_p),
                ("dG", C.c_void_p)]


_lib = None


def lib():
    """The loaded libmoe.so; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_09_amd.build` (no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        vp, i32 = C.c_void_p, C.c_int
        S = C.POINTER(moe_shape)
        L.moe_workspace_size.restype = C.c_size_t
        L.moe_workspace_size.argtypes = [S]
        L.moe_route.restype = i32
        L.moe_route.argtypes = [S, C.POINTER(moe_route_opts), vp, vp, vp, vp, vp, vp, C.c_size_t,
                                vp]
        L.moe_permute.restype = i32
        L.moe_permute.argtypes = [S, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.moe_permute_no_alloc.restype = i32
        L.moe_permute_no_alloc.argtypes = [S, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn.restype = i32
        L.moe_expert_ffn.argtypes = [S, vp, vp, vp, vp, vp, C.POINTER(moe_expert_weights), vp, vp,
                                     vp, C.c_size_t, vp]
        L.moe_combine.restype = i32
        L.moe_combine.argtypes = [S, vp, vp, vp, vp, vp, vp]
        L.moe_forward.restype = i32
        L.moe_forward.argtypes = [S, C.POINTER(moe_route_opts), vp, vp,
                                  C.POINTER(moe_expert_weights), vp, vp, vp, vp, C.c_size_t, vp]
        L.moe_check_device_error.restype = i32
        L.moe_check_device_error.argtypes = [vp, C.c_size_t, vp]
        L.moe_backward_workspace_size.restype = C.c_size_t
        L.moe_backward_workspace_size.argtypes = [S]
        L.moe_backward.restype = i32
        L.moe_backward.argtypes = [S, C.POINTER(moe_route_opts), vp, vp,
                                   C.POINTER(moe_expert_weights), vp, vp, vp,
                                   C.POINTER(moe_grads), vp, C.c_size_t, vp]
        L.moe_forward_train.restype = i32
        L.moe_forward_train.argtypes = L.moe_forward.argtypes
        L.moe_backward_saved.restype = i32
        L.moe_backward_saved.argtypes = L.moe_backward.argtypes
        L.moe_status_string.restype = C.c_char_p
        L.moe_status_string.argtypes = [i32]
        _lib = L
    return _lib


# ------------------------------------------------------------------ marshalling
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(fn: str, st: int):
    if st != 0:
        raise MoeError(fn, st)


def make_shape(tokens, hidden, experts, topk, inter, has_shared=0, precision="bf16") -> moe_shape:
    p = PREC[precision] if isinstance(precision, str) else int(precision)
    return moe_shape(int(tokens), int(hidden), int(experts), int(topk), int(inter),
                     int(bool(has_shared)), p)


def make_route_opts(score="sigmoid", renorm=True, alpha=1.0, expert_bias=None, gate_bias=None,
                    token_ids=None, tid2eid=None) -> moe_route_opts:
    return moe_route_opts(SCORE[score] if isinstance(score, str) else int(score), int(bool(renorm)),
                          float(alpha), _ptr(expert_bias), _ptr(gate_bias), _ptr(token_ids),
                          _ptr(tid2eid), 0 if tid2eid is None else int(tid2eid.shape[0]))


def make_weights(W1, W2, w1_scale=None, w2_scale=None, Ws1=None, Ws2=None, ws1_scale=None,
                 ws2_scale=None) -> moe_expert_weights:
    return moe_expert_weights(_ptr(W1), _ptr(w1_scale), _ptr(W2), _ptr(w2_scale), _ptr(Ws1),
                              _ptr(ws1_scale), _ptr(Ws2), _ptr(ws2_scale))


def make_grads(dX, dW1, dW2, dWs1=None, dWs2=None, dWg=None, dgate_bias=None,
               dG=None) -> moe_grads:
    return moe_grads(_ptr(dX), _ptr(dW1), _ptr(dW2), _ptr(dWs1), _ptr(dWs2), _ptr(dWg),
                     _ptr(dgate_bias), _ptr(dG))


# ------------------------------------------------------------------ C ABI, same names
def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_workspace_size(shape: moe_shape) -> int:
    return int(lib().moe_workspace_size(C.byref(shape)))


def moe_route(shape, opts, X, Wg, expert_ids, gate_weights, keys_out, workspace, stream=None):
    _check("moe_route", lib().moe_route(C.byref(shape), C.byref(opts), _ptr(X), _ptr(Wg),
                                        _ptr(expert_ids), _ptr(gate_weights), _ptr(keys_out),
                                        _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_permute(shape, expert_ids, X, counts, offsets, dst_row, src_tok, Xp, xp_scale, Xq, x_scale,
                workspace, stream=None):
    _check("moe_permute", lib().moe_permute(
        C.byref(shape), _ptr(expert_ids), _ptr(X), _ptr(counts), _ptr(offsets), _ptr(dst_row),
        _ptr(src_tok), _ptr(Xp), _ptr(xp_scale), _ptr(Xq), _ptr(x_scale), _ptr(workspace),
        workspace.numel(), _stream(stream)))


def moe_permute_no_alloc(shape, expert_ids, X, counts, offsets, dst_row, src_tok, Xp, xp_scale,
                         Xq, x_scale, stream=None):
    """moe_permute with the library's static scratch instead of a workspace."""
    _check("moe_permute_no_alloc", lib().moe_permute_no_alloc(
        C.byref(shape), _ptr(expert_ids), _ptr(X), _ptr(counts), _ptr(offsets), _ptr(dst_row),
        _ptr(src_tok), _ptr(Xp), _ptr(xp_scale), _ptr(Xq), _ptr(x_scale), _stream(stream)))


def moe_expert_ffn(shape, Xp, xp_scale, offsets, Xs, xs_scale, weights, Yp, Ys, workspace,
                   stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        C.byref(shape), _ptr(Xp), _ptr(xp_scale), _ptr(offsets), _ptr(Xs), _ptr(xs_scale),
        C.byref(weights), _ptr(Yp), _ptr(Ys), _ptr(workspace), workspace.numel(),
        _stream(stream)))


def moe_combine(shape, Yp, dst_row, gate_weights, Ys, Y, stream=None):
    _check("moe_combine", lib().moe_combine(C.byref(shape), _ptr(Yp), _ptr(dst_row),
                                            _ptr(gate_weights), _ptr(Ys), _ptr(Y),
                                            _stream(stream)))


def moe_forward(shape, opts, X, Wg, weights, expert_ids, gate_weights, Y, workspace, stream=None):
    _check("moe_forward", lib().moe_forward(
        C.byref(shape), None if opts is None else C.byref(opts), _ptr(X), _ptr(Wg),
        C.byref(weights), _ptr(expert_ids), _ptr(gate_weights), _ptr(Y), _ptr(workspace),
        workspace.numel(), _stream(stream)))


def moe_backward_workspace_size(shape: moe_shape) -> int:
    return int(lib().moe_backward_workspace_size(C.byref(shape)))


def moe_backward(shape, opts, X, Wg, weights, expert_ids, gate_weights, dY, grads, workspace,
                 stream=None):
    _check("moe_backward", lib().moe_backward(
        C.byref(shape), None if opts is None else C.byref(opts), _ptr(X), _ptr(Wg),
        C.byref(weights), _ptr(expert_ids), _ptr(gate_weights), _ptr(dY), C.byref(grads),
        _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_forward_train(shape, opts, X, Wg, weights, expert_ids, gate_weights, Y, workspace,
                      stream=None):
    """moe_forward that keeps the activations moe_backward_saved reads, in a
    backward workspace (alloc_workspace(shape, backward=True))."""
    _check("moe_forward_train", lib().moe_forward_train(
        C.byref(shape), None if opts is None else C.byref(opts), _ptr(X), _ptr(Wg),
        C.byref(weights), _ptr(expert_ids), _ptr(gate_weights), _ptr(Y), _ptr(workspace),
        workspace.numel(), _stream(stream)))


def moe_backward_saved(shape, opts, X, Wg, weights, expert_ids, gate_weights, dY, grads,
                       workspace, stream=None):
    _check("moe_backward_saved", lib().moe_backward_saved(
        C.byref(shape), None if opts is None else C.byref(opts), _ptr(X), _ptr(Wg),
        C.byref(weights), _ptr(expert_ids), _ptr(gate_weights), _ptr(dY), C.byref(grads),
        _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_check_device_error(workspace, stream=None) -> int:
    """Returns the status (0 or MOE_ERR_DEVICE_DATA) of the most recent call on
    this workspace that can flag bad ids (each such call resets the flag);
    raises on other errors."""
    st = lib().moe_check_device_error(_ptr(workspace), workspace.numel(), _stream(stream))
    if st not in (0, -5):
        raise MoeError("moe_check_device_error", st)
    return st


def alloc_workspace(shape: moe_shape, device="cuda", backward=False) -> torch.Tensor:
    """A uint8 device tensor of moe_workspace_size (or, with backward,
    moe_backward_workspace_size) bytes; torch allocations are 256-byte
    aligned."""
    n = moe_backward_workspace_size(shape) if backward else moe_workspace_size(shape)
    if n == 0:
        raise MoeError("moe_workspace_size", -1)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws
