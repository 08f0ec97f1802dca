"""CPU oracle of the routed MoE layer forward pass (test infrastructure).

Only the tests, the GPU smoke check and the CPU-baseline leg of the benchmark
import this package.  The product library never does, and this package never
imports the product library: the two share no code.  The arithmetic lives in
``moe_oracle.c`` (plain C, fp64, OpenMP over tokens); this module only builds
it, loads it and marshals numpy arrays.

Element types are given as numpy arrays of raw bits:
  fp32  -> float32
  bf16  -> uint16 (the top 16 bits of an IEEE binary32)
  e4m3  -> uint8  (OCP e4m3fn codes)

Sources are cited in ``moe_oracle.c``: the CANN ``mega_moe`` operator page
(§计算公式, §计算过程: EP Dispatch, Expert Compute, Token Combine, A8W8 block),
the blog post "Megatron-LM 的 MoE 并行：以 DeepSeek-V4 为例" (§模型与入口,
§路由张量, §Hash 路由, §计数与重排, §ETP 里的矩阵) and "Megatron 分布式训练
全维度并行技术文档" (§4.1, §4.2).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_LIB points the loader at another build of moe_oracle.c (the
# sanitizer test builds one with AddressSanitizer and UBSan)
_LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

PRECISIONS = {"fp32": 0, "bf16": 1, "fp8": 2, "mxfp8": 3, "mxfp4": 4, "int8": 5}
MX_FORMATS = {"e4m3": 0, "e2m1": 1}
SCORES = {"sigmoid": 0, "softmax": 1, "sqrt_softplus": 2}


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layer(C.Structure):
    _fields_ = [
        ("T", C.c_int), ("hidden", C.c_int), ("E", C.c_int), ("k", C.c_int),
        ("inter", C.c_int), ("has_shared", C.c_int), ("precision", C.c_int),
        ("X", C.c_void_p), ("W1", C.c_void_p), ("W2", C.c_void_p),
        ("w1_scale", C.c_void_p), ("w2_scale", C.c_void_p),
        ("Ws1", C.c_void_p), ("Ws2", C.c_void_p),
        ("ws1_scale", C.c_void_p), ("ws2_scale", C.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = C.CDLL(_LIB_PATH)
        vp, i32, dbl = C.c_void_p, C.c_int, C.c_double
        L.oracle_set_threads.restype = i32
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_e2m1_decode.restype = dbl
        L.oracle_e2m1_decode.argtypes = [C.c_uint8]
        L.oracle_e2m1_encode.restype = C.c_uint8
        L.oracle_e2m1_encode.argtypes = [dbl]
        L.oracle_mx_scale_code.restype = C.c_uint8
        L.oracle_mx_scale_code.argtypes = [dbl, i32]
        L.oracle_mx_quantize.argtypes = [i32, vp, i32, vp, vp]
        L.oracle_mx_value.restype = dbl
        L.oracle_mx_value.argtypes = [C.c_uint8, C.c_uint8, i32]
        L.oracle_e4m3_decode.restype = dbl
        L.oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_e4m3_encode.argtypes = [dbl]
        L.oracle_quantize_row_f32.argtypes = [i32, vp, vp, vp]
        L.oracle_quantize_row_i8_f32.argtypes = [i32, vp, vp, vp]
        L.oracle_gate_logits.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_affinity.argtypes = [i32, i32, i32, vp, vp]
        L.oracle_topk.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_route.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32, dbl,
                                   vp, vp, vp, vp, vp, vp, vp]
        L.oracle_dispatch.restype = i32
        L.oracle_dispatch.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_layer_tokens.argtypes = [C.POINTER(_Layer), vp, vp, i32, vp, vp]
        L.oracle_expert_rows.argtypes = [C.POINTER(_Layer), vp, vp, i32, vp, vp]
        L.oracle_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_backward_tokens.restype = i32
        L.oracle_backward_tokens.argtypes = [C.POINTER(_Layer), vp, vp, vp, i32, vp, vp, vp]
        L.oracle_backward_weights.restype = i32
        L.oracle_backward_weights.argtypes = [C.POINTER(_Layer), vp, vp, vp, i32, vp, vp, vp]
        L.oracle_route_backward.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32, i32, dbl,
                                            vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _elem_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.uint8:
        return 2
    raise TypeError(f"unsupported element array dtype {a.dtype}")


# ---------------------------------------------------------------- formats
def e4m3_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    f = lib().oracle_e4m3_decode
    return np.array([f(int(c)) for c in codes.ravel()], dtype=np.float64).reshape(codes.shape)


def e4m3_encode(values) -> np.ndarray:
    values = np.asarray(values, dtype=np.float64)
    f = lib().oracle_e4m3_encode
    return np.array([f(float(v)) for v in values.ravel()], dtype=np.uint8).reshape(values.shape)


def quantize_rows_f32(X: np.ndarray):
    """Per-row e4m3 quantisation in fp32: returns (codes uint8, scale float32)."""
    X = _c(X, np.float32)
    T, h = X.shape
    q = np.empty((T, h), np.uint8)
    s = np.empty(T, np.float32)
    L = lib()
    for t in range(T):
        L.oracle_quantize_row_f32(h, _p(X[t]), _p(q[t]), C.c_void_p(s.ctypes.data + 4 * t))
    return q, s


def quantize_rows_i8_f32(X: np.ndarray):
    """Per-row INT8 quantisation of the A8W8 block (s = max|x|/127, codes
    rounded half away from zero), scale and quotient in fp32: returns
    (codes int8, scale float32)."""
    X = _c(X, np.float32)
    T, h = X.shape
    q = np.empty((T, h), np.int8)
    s = np.empty(T, np.float32)
    L = lib()
    for t in range(T):
        L.oracle_quantize_row_i8_f32(h, _p(X[t]), _p(q[t]), C.c_void_p(s.ctypes.data + 4 * t))
    return q, s


# ---------------------------------------------------------------- routing
def gate_logits(X, Wg, gate_bias=None) -> np.ndarray:
    X = np.ascontiguousarray(X)
    Wg = np.ascontiguousarray(Wg, dtype=X.dtype)
    T, h = X.shape
    E = Wg.shape[1]
    out = np.empty((T, E), np.float64)
    lib().oracle_gate_logits(T, h, E, _elem_code(X), _p(X), _p(Wg), _p(_c(gate_bias, np.float64)),
                             _p(out))
    return out


def affinity(logits, score="sigmoid") -> np.ndarray:
    logits = _c(logits, np.float64)
    T, E = logits.shape
    out = np.empty((T, E), np.float64)
    lib().oracle_affinity(T, E, SCORES[score], _p(logits), _p(out))
    return out


def topk(keys, k):
    """Top-k of keys (any float array, compared as fp64): (ids [T,k], margin [T])."""
    keys = _c(keys, np.float64)
    T, E = keys.shape
    ids = np.empty((T, k), np.int32)
    margin = np.empty(T, np.float64)
    lib().oracle_topk(T, E, k, _p(keys), _p(ids), _p(margin))
    return ids, margin


def route(X, Wg, k, *, gate_bias=None, beta=None, score="sigmoid", renorm=True, alpha=1.0,
          token_ids=None, tid2eid=None) -> dict:
    """Router of the layer.  Returns ids, G, logits, keys, margin (fp64 / int32)."""
    X = np.ascontiguousarray(X)
    Wg = np.ascontiguousarray(Wg, dtype=X.dtype)
    T, h = X.shape
    E = Wg.shape[1]
    ids = np.empty((T, k), np.int32)
    G = np.empty((T, k), np.float64)
    logits = np.empty((T, E), np.float64)
    keys = np.empty((T, E), np.float64)
    margin = np.empty(T, np.float64)
    lib().oracle_route(T, h, E, k, _elem_code(X), _p(X), _p(Wg), _p(_c(gate_bias, np.float64)),
                       _p(_c(beta, np.float64)), SCORES[score], int(bool(renorm)), float(alpha),
                       _p(_c(token_ids, np.int32)), _p(_c(tid2eid, np.int32)), _p(ids), _p(G),
                       _p(logits), _p(keys), _p(margin))
    return {"ids": ids, "G": G, "logits": logits, "keys": keys, "margin": margin}


def route_backward(X, Wg, ids, dG, *, gate_bias=None, score="sigmoid", renorm=True, alpha=1.0,
                   dX=None) -> dict:
    """Router backward for the chosen ids and dG [T,k]: dl [T,E], dWg
    [h,E], dgate_bias [E]; adds dl Wgᵀ into dX [T,h] (fp64) when given."""
    X = np.ascontiguousarray(X)
    Wg = np.ascontiguousarray(Wg, dtype=X.dtype)
    T, h = X.shape
    E = Wg.shape[1]
    ids = _c(ids, np.int32)
    k = ids.shape[1]
    dl = np.empty((T, E), np.float64)
    dWg = np.empty((h, E), np.float64)
    db = np.empty(E, np.float64)
    if dX is not None:
        assert dX.dtype == np.float64 and dX.flags.c_contiguous and dX.shape == (T, h)
    lib().oracle_route_backward(T, h, E, k, _elem_code(X), _p(X), _p(Wg),
                                _p(_c(gate_bias, np.float64)), SCORES[score], int(bool(renorm)),
                                float(alpha), _p(ids), _p(_c(dG, np.float64)), _p(dl), _p(dWg),
                                _p(db), _p(dX))
    return {"dl": dl, "dWg": dWg, "dgate_bias": db}


def e2m1_decode(code: int) -> float:
    return float(lib().oracle_e2m1_decode(int(code) & 0xF))


def e2m1_encode(v: float) -> int:
    return int(lib().oracle_e2m1_encode(float(v)))


def mx_scale_code(amax: float, fmt: str) -> int:
    """E8M0 code of a group's shared scale (OCP MX rule; see moe_oracle.c)."""
    return int(lib().oracle_mx_scale_code(float(amax), MX_FORMATS[fmt]))


def mx_quantize(x, fmt: str):
    """MX quantisation along the last axis (a multiple of 32) in groups of 32:
    returns (element codes, one per value, uint8; E8M0 scale codes, uint8)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % 32 == 0
    flat = np.ascontiguousarray(x.reshape(-1, n))
    q = np.empty(flat.shape, np.uint8)
    sc = np.empty((flat.shape[0], n // 32), np.uint8)
    for r in range(flat.shape[0]):
        lib().oracle_mx_quantize(n, _p(flat[r]), MX_FORMATS[fmt], _p(q[r]), _p(sc[r]))
    return q.reshape(x.shape), sc.reshape(x.shape[:-1] + (n // 32,))


def mx_value(code: int, scale: int, fmt: str) -> float:
    return float(lib().oracle_mx_value(int(code), int(scale), MX_FORMATS[fmt]))


def set_threads(n: int) -> int:
    """OpenMP threads of the oracle's parallel loops (n < 1: default); returns
    the count now in effect.  No effect on results."""
    return int(lib().oracle_set_threads(int(n)))


# ---------------------------------------------------------------- dispatch
def dispatch(ids, E) -> dict:
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    dst = np.empty(T * k, np.int32)
    src = np.full(T * k, -1, np.int32)
    bad = lib().oracle_dispatch(T, k, E, _p(ids), _p(counts), _p(offsets), _p(dst), _p(src))
    return {"counts": counts, "offsets": offsets, "dst_row": dst, "src_tok": src, "bad": bad}


def combine(Yp, dst_row, G, Ys=None) -> np.ndarray:
    Yp = _c(Yp, np.float64)
    G = _c(G, np.float64)
    T, k = G.shape
    h = Yp.shape[1]
    Y = np.empty((T, h), np.float64)
    lib().oracle_combine(T, k, h, _p(Yp), _p(_c(dst_row, np.int32)), _p(G), _p(_c(Ys, np.float64)),
                         _p(Y))
    return Y


# ---------------------------------------------------------------- experts
class Layer:
    """The expert side of one layer: X, W1, W2 (+ scales, + shared expert).

    precision 'fp32': X, W float32.  'bf16': X, W uint16 bits.  'fp8': X uint16
    (bf16 bits, quantised per token inside the layer), W uint8 e4m3 codes with
    float32 per-output-channel scales.  'int8': as 'fp8' with int8 weights
    (the INT8 A8W8 block).  'mxfp8' / 'mxfp4': X uint16 (bf16
    bits, MX-quantised inside the layer).  mxfp8: W uint8 e4m3 codes [E,K,N],
    scales uint8 E8M0 [E,K/32,N].  mxfp4: W K-contiguous e2m1 code pairs
    [E,N,K/2] (element 2i in the low nibble), scales [E,N,K/32].
    """

    def __init__(self, precision, X, W1, W2, *, w1_scale=None, w2_scale=None, Ws1=None, Ws2=None,
                 ws1_scale=None, ws2_scale=None, k=1):
        self.precision = precision
        mx = precision.startswith("mx")
        wdt = {"fp32": np.float32, "bf16": np.uint16, "int8": np.int8}.get(precision, np.uint8)
        sdt = np.uint8 if mx else np.float32
        xdt = np.float32 if precision == "fp32" else np.uint16
        self.X = _c(X, xdt)
        self.W1 = _c(W1, wdt)
        self.W2 = _c(W2, wdt)
        self.w1_scale = _c(w1_scale, sdt)
        self.w2_scale = _c(w2_scale, sdt)
        self.Ws1 = _c(Ws1, wdt)
        self.Ws2 = _c(Ws2, wdt)
        self.ws1_scale = _c(ws1_scale, sdt)
        self.ws2_scale = _c(ws2_scale, sdt)
        T, h = self.X.shape
        if precision == "mxfp4":   # K-contiguous [E, 2f, h/2]: two e2m1 codes per byte
            E, f2, hb = self.W1.shape
            h2 = 2 * hb
        else:
            E, h2, f2 = self.W1.shape
        assert h2 == h and f2 % 2 == 0
        self.T, self.hidden, self.E, self.inter, self.k = T, h, E, f2 // 2, int(k)
        if precision == "mxfp8":
            assert h % 32 == 0 and self.inter % 32 == 0
            assert self.w1_scale.shape == (E, h // 32, f2)
            assert self.w2_scale.shape == (E, self.inter // 32, h)
        if precision == "mxfp4":
            assert h % 32 == 0 and self.inter % 32 == 0
            assert self.W2.shape == (E, h, self.inter // 2)
            assert self.w1_scale.shape == (E, f2, h // 32)
            assert self.w2_scale.shape == (E, h, self.inter // 32)
        if precision in ("fp8", "int8", "mxfp8", "mxfp4"):
            assert self.w1_scale is not None and self.w2_scale is not None
        self._s = _Layer(T, h, E, self.k, self.inter, int(self.Ws1 is not None),
                         PRECISIONS[precision], _p(self.X), _p(self.W1), _p(self.W2),
                         _p(self.w1_scale), _p(self.w2_scale), _p(self.Ws1), _p(self.Ws2),
                         _p(self.ws1_scale), _p(self.ws2_scale))

    def tokens(self, ids, G, tokens=None) -> np.ndarray:
        """y_t = F_s(x_t) + sum_j G[t,j] F_{ids[t,j]}(x_t) for the listed tokens."""
        ids = _c(ids, np.int32)
        G = _c(G, np.float64)
        assert ids.shape == (self.T, self.k) and G.shape == ids.shape
        tok = None if tokens is None else _c(tokens, np.int32)
        n = self.T if tok is None else len(tok)
        Y = np.empty((n, self.hidden), np.float64)
        lib().oracle_layer_tokens(C.byref(self._s), _p(ids), _p(G), n, _p(tok), _p(Y))
        return Y

    def backward_tokens(self, ids, G, dY, tokens=None):
        """(dX [n,h], dG [n,k]) of the experts' side for the listed tokens."""
        ids = _c(ids, np.int32)
        G = _c(G, np.float64)
        dY = _c(dY, np.float64)
        assert dY.shape == (self.T, self.hidden)
        tok = None if tokens is None else _c(tokens, np.int32)
        n = self.T if tok is None else len(tok)
        dX = np.empty((n, self.hidden), np.float64)
        dG = np.empty((n, self.k), np.float64)
        st = lib().oracle_backward_tokens(C.byref(self._s), _p(ids), _p(G), _p(dY), n, _p(tok),
                                          _p(dX), _p(dG))
        assert st == 0, "backward needs an fp32 or bf16 layer"
        return dX, dG

    def backward_weights(self, ids, G, dY, experts):
        """(dW1 [n,h,2f], dW2 [n,f,h]) of the listed experts (E = shared)."""
        ids = _c(ids, np.int32)
        G = _c(G, np.float64)
        dY = _c(dY, np.float64)
        ex = _c(np.atleast_1d(experts), np.int32)
        n = len(ex)
        dW1 = np.empty((n, self.hidden, 2 * self.inter), np.float64)
        dW2 = np.empty((n, self.inter, self.hidden), np.float64)
        st = lib().oracle_backward_weights(C.byref(self._s), _p(ids), _p(G), _p(dY), n, _p(ex),
                                           _p(dW1), _p(dW2))
        assert st == 0, "backward needs an fp32 or bf16 layer"
        return dW1, dW2

    def expert_rows(self, offsets, src_tok, rows=None) -> np.ndarray:
        """Yp[r] = F_e(x_{src_tok[r]}) for dispatched rows r (r >= T*k: shared)."""
        rr = None if rows is None else _c(rows, np.int32)
        n = self.T * self.k if rr is None else len(rr)
        Yp = np.empty((n, self.hidden), np.float64)
        lib().oracle_expert_rows(C.byref(self._s), _p(_c(offsets, np.int32)),
                                 _p(_c(src_tok, np.int32)), n, _p(rr), _p(Yp))
        return Yp
