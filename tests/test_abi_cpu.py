"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects out-of-contract arguments on the host, before
any launch (none of these calls reaches the HIP runtime)."""
from __future__ import annotations

import ctypes as C
import os
import re
import subprocess

import pytest

import mixture_experts_layer_09_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -3
FAKE_WS = 1 << 20  # an aligned, never-dereferenced address


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def _lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return moe.lib()


def test_header_declares_the_five_steps_and_helpers():
    names = _declared()
    for n in ["moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
              "moe_workspace_size", "moe_check_device_error", "moe_status_string"]:
        assert n in names
    assert sorted(moe.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for n in _declared():
        assert n in exported, n
        assert hasattr(moe.lib(), n)


def test_status_strings():
    _lib()
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert moe.moe_status_string(st) != "unknown status"
    assert moe.moe_status_string(7) == "unknown status"


def _shape(**kw):
    """Raw struct (no normalisation of out-of-range fields)."""
    d = dict(tokens=64, hidden=128, experts=8, topk=2, inter=64, has_shared=0, precision="bf16")
    d.update(kw)
    p = d["precision"]
    d["precision"] = moe.PREC[p] if isinstance(p, str) else p
    return moe.moe_shape(d["tokens"], d["hidden"], d["experts"], d["topk"], d["inter"],
                         d["has_shared"], d["precision"])


@pytest.mark.parametrize("kw,expect", [
    (dict(tokens=0), INVALID), (dict(topk=0), INVALID), (dict(topk=9), INVALID),
    (dict(experts=40, topk=17), INVALID), (dict(has_shared=2), INVALID),
    (dict(precision=6), INVALID), (dict(precision=-1), INVALID), (dict(hidden=96), UNSUPPORTED),
    (dict(inter=96), UNSUPPORTED), (dict(inter=192, precision="fp8"), UNSUPPORTED),
    (dict(hidden=384, inter=128, precision="fp8"), UNSUPPORTED),
    (dict(hidden=384, inter=128, precision="mxfp8"), UNSUPPORTED),
    (dict(hidden=384, inter=128, precision="mxfp4"), UNSUPPORTED),
    (dict(hidden=384, inter=128, precision="int8"), UNSUPPORTED),
    (dict(hidden=256, inter=192, precision="int8"), UNSUPPORTED),
    (dict(experts=600, topk=2), UNSUPPORTED),
])
def test_bad_shapes_rejected(kw, expect):
    L = _lib()
    s = _shape(**kw)
    assert L.moe_workspace_size(C.byref(s)) == 0
    ws = FAKE_WS
    opts = moe.make_route_opts()
    assert L.moe_route(C.byref(s), C.byref(opts), 16, 16, 16, 16, None, ws, 1 << 40, None) == expect
    assert L.moe_combine(C.byref(s), 16, 16, 16, None, 16, None) == expect


def test_workspace_size_grows_with_the_problem():
    _lib()
    a = moe.moe_workspace_size(_shape())
    b = moe.moe_workspace_size(_shape(tokens=128))
    c = moe.moe_workspace_size(_shape(tokens=128, has_shared=1))
    d = moe.moe_workspace_size(_shape(tokens=128, has_shared=1, precision="fp8", inter=128,
                                      hidden=256))
    e = moe.moe_workspace_size(_shape(tokens=128, has_shared=1, precision="mxfp8", inter=128,
                                      hidden=256))
    assert 0 < a < b < c and d > 0 and e > 0 and a % 256 == 0
    # MX keeps no fp32 copy of the SwiGLU output, so it needs less than A8W8
    assert e < d


def test_null_pointers_and_workspace_rejected():
    L = _lib()
    s = _shape()
    n = moe.moe_workspace_size(s)
    opts = moe.make_route_opts()
    # null X / outputs
    assert L.moe_route(C.byref(s), C.byref(opts), None, 16, 16, 16, None, FAKE_WS, n, None) == INVALID
    assert L.moe_route(C.byref(s), C.byref(opts), 16, 16, None, 16, None, FAKE_WS, n, None) == INVALID
    # workspace: null, misaligned, too small
    assert L.moe_route(C.byref(s), C.byref(opts), 16, 16, 16, 16, None, None, n, None) == WORKSPACE
    assert L.moe_route(C.byref(s), C.byref(opts), 16, 16, 16, 16, None, FAKE_WS + 8, n,
                       None) == WORKSPACE
    assert L.moe_route(C.byref(s), C.byref(opts), 16, 16, 16, 16, None, FAKE_WS, n - 1,
                       None) == WORKSPACE
    # permute: null outputs, fp8 without scales
    assert L.moe_permute(C.byref(s), 16, 16, None, 16, 16, 16, 16, None, None, None, FAKE_WS, n,
                         None) == INVALID
    s8 = _shape(precision="fp8", inter=128, hidden=256)
    n8 = moe.moe_workspace_size(s8)
    assert L.moe_permute(C.byref(s8), 16, 16, 16, 16, 16, 16, 16, None, None, None, FAKE_WS, n8,
                         None) == INVALID
    # expert ffn: missing weights, shared expert without its weights, fp8 without scales
    w = moe.moe_expert_weights(16, None, None, None, None, None, None, None)
    assert L.moe_expert_ffn(C.byref(s), 16, None, 16, None, None, C.byref(w), 16, None, FAKE_WS, n,
                            None) == INVALID
    sh = _shape(has_shared=1)
    nsh = moe.moe_workspace_size(sh)
    w = moe.moe_expert_weights(16, None, 16, None, None, None, None, None)
    assert L.moe_expert_ffn(C.byref(sh), 16, None, 16, 16, None, C.byref(w), 16, 16, FAKE_WS, nsh,
                            None) == INVALID
    w8 = moe.moe_expert_weights(16, None, 16, None, None, None, None, None)
    assert L.moe_expert_ffn(C.byref(s8), 16, 16, 16, None, None, C.byref(w8), 16, None, FAKE_WS,
                            n8, None) == INVALID
    # forward: router options without a gate weight
    w = moe.moe_expert_weights(16, None, 16, None, None, None, None, None)
    assert L.moe_forward(C.byref(s), C.byref(opts), 16, None, C.byref(w), 16, 16, 16, FAKE_WS, n,
                         None) == INVALID
    # device arrays that are not 16-byte aligned
    assert L.moe_route(C.byref(s), C.byref(opts), 24, 16, 16, 16, None, FAKE_WS, n, None) == INVALID
    assert L.moe_permute(C.byref(s), 16, 16, 16, 16, 16, 16, 40, None, None, None, FAKE_WS, n,
                         None) == INVALID
    w = moe.moe_expert_weights(16, None, 20, None, None, None, None, None)
    assert L.moe_expert_ffn(C.byref(s), 16, None, 16, None, None, C.byref(w), 16, None, FAKE_WS, n,
                            None) == INVALID
    assert L.moe_combine(C.byref(s), 16, 16, 16, None, 8, None) == INVALID
    w = moe.moe_expert_weights(16, None, 16, None, None, None, None, None)
    assert L.moe_forward(C.byref(s), None, 16, None, C.byref(w), 16, 16, 36, FAKE_WS, n,
                         None) == INVALID
    # check_device_error with no workspace
    assert L.moe_check_device_error(None, 0, None) == WORKSPACE


def test_route_options_rejected():
    L = _lib()
    s = _shape()
    n = moe.moe_workspace_size(s)
    for bad in [moe.moe_route_opts(5, 1, 1.0, None, None, None, None, 0),
                moe.moe_route_opts(0, 2, 1.0, None, None, None, None, 0),
                moe.moe_route_opts(0, 1, 1.0, None, None, 16, None, 10),   # ids without a table
                moe.moe_route_opts(0, 1, 1.0, None, None, 16, 16, 0)]:     # table of 0 rows
        assert L.moe_route(C.byref(s), C.byref(bad), 16, 16, 16, 16, None, FAKE_WS, n,
                           None) == INVALID


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        moe.lib()


@pytest.mark.parametrize("entry", ["moe_backward", "moe_backward_saved"])
def test_backward_rejects_out_of_contract_arguments(entry):
    L = _lib()
    fn = getattr(L, entry)
    s = _shape(hidden=256, inter=128, experts=64, topk=2, has_shared=1)
    n = moe.moe_backward_workspace_size(s)
    assert n > moe.moe_workspace_size(s)
    opts = moe.make_route_opts()
    w = moe.moe_expert_weights(16, None, 16, None, 16, None, 16, None)
    g = moe.moe_grads(16, 16, 16, 16, 16, 16, 16, 16)
    args = lambda shape, o=C.byref(opts), grads=C.byref(g), ws=FAKE_WS, nb=n: (  # noqa: E731
        C.byref(shape), o, 16, 16, C.byref(w), 16, 16, 16, grads, ws, nb, None)
    # precision other than bf16, and shapes off the backward tiles
    for bad in (_shape(hidden=256, inter=128, experts=64, precision="fp8"),
                _shape(hidden=256, inter=128, experts=64, precision="fp32"),
                _shape(hidden=128, inter=128, experts=64), _shape(hidden=256, inter=64, experts=64)):
        assert fn(*args(bad)) == UNSUPPORTED
    # router gradients need experts in multiples of 64; without options they are not asked for
    s40 = _shape(hidden=256, inter=128, experts=40, topk=2, has_shared=1)
    n40 = moe.moe_backward_workspace_size(s40)
    assert fn(*args(s40, nb=n40)) == UNSUPPORTED
    # missing gradient outputs, shared-expert gradients missing, misaligned arrays
    assert fn(*args(s, grads=None)) == INVALID
    g2 = moe.moe_grads(16, 16, 16, None, 16, 16, 16, 16)
    assert fn(*args(s, grads=C.byref(g2))) == INVALID
    g3 = moe.moe_grads(16, 24, 16, 16, 16, 16, 16, 16)
    assert fn(*args(s, grads=C.byref(g3))) == INVALID
    # workspace: misaligned or smaller than moe_backward_workspace_size
    assert fn(*args(s, ws=FAKE_WS + 8)) == WORKSPACE
    assert fn(*args(s, nb=n - 1)) == WORKSPACE
    assert fn(*args(s, nb=moe.moe_workspace_size(s))) == WORKSPACE


def test_training_forward_rejects_out_of_contract_arguments():
    L = _lib()
    s = _shape(hidden=256, inter=128, experts=64, topk=2, has_shared=1)
    n = moe.moe_backward_workspace_size(s)
    opts = moe.make_route_opts()
    w = moe.moe_expert_weights(16, None, 16, None, 16, None, 16, None)
    args = lambda shape, o=C.byref(opts), Y=16, ws=FAKE_WS, nb=n: (  # noqa: E731
        C.byref(shape), o, 16, 16, C.byref(w), 16, 16, Y, ws, nb, None)
    # the layers and shapes the backward takes
    for bad in (_shape(hidden=256, inter=128, experts=64, precision="fp8"),
                _shape(hidden=128, inter=128, experts=64), _shape(hidden=256, inter=64, experts=64)):
        assert L.moe_forward_train(*args(bad)) == UNSUPPORTED
    s40 = _shape(hidden=256, inter=128, experts=40, topk=2, has_shared=1)
    assert L.moe_forward_train(*args(s40, nb=moe.moe_backward_workspace_size(s40))) == UNSUPPORTED
    assert L.moe_forward_train(*args(s, Y=None)) == INVALID
    assert L.moe_forward_train(*args(s, Y=24)) == INVALID
    # a forward-sized workspace does not hold the saved activations
    assert L.moe_forward_train(*args(s, nb=moe.moe_workspace_size(s))) == WORKSPACE
    assert L.moe_forward_train(*args(s, ws=FAKE_WS + 8)) == WORKSPACE


def test_permute_no_alloc_host_checks():
    """moe_permute_no_alloc rejects out-of-contract arguments and calls larger
    than its static scratch on the host, before any launch."""
    L = _lib()
    vp = C.c_void_p
    a = vp(FAKE_WS)
    s = _shape()
    args = [a] * 10 + [None]
    # NULL ids
    assert L.moe_permute_no_alloc(C.byref(s), None, *args[1:]) == INVALID
    # misaligned X
    assert L.moe_permute_no_alloc(C.byref(s), a, vp(FAKE_WS + 2), *args[2:]) == INVALID
    # fp8 without the scale and code arrays
    s8 = _shape(hidden=256, inter=128, precision="fp8")
    assert L.moe_permute_no_alloc(C.byref(s8), a, a, a, a, a, a, a, None, None, None,
                                  None) == INVALID
    # more assignments than the scratch holds
    big = _shape(tokens=moe.NO_ALLOC_MAX_ASSIGNMENTS // 2 + 1, topk=2)
    assert L.moe_permute_no_alloc(C.byref(big), *args) == -6
    assert "scratch" in moe.moe_status_string(-6)
