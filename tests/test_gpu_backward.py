"""GPU parity of the local backward (moe_backward) against the oracle.

Routing comes from the GPU router (moe_route), the upstream gradient dY is a
seeded bf16 tensor; the oracle differentiates the same layer (bf16 values) at
the same routing in fp64: dX (experts' part plus, with router options, the
router's), dG, the weight gradients of every expert and of the shared expert,
and the router's dWg and gating-bias gradient.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_09_amd as moe
import oracle
import synth
from tests.gpu_layer import to_device
from tests.helpers import bits, f64, row_rel_err

pytestmark = pytest.mark.gpu

# The GPU chain rounds four intermediates to bf16 (dYp, H1, A, dH1; 2^-9
# relative each) and its outputs; the weight gradients are sums over an
# expert's rows, with cancellation, compared per row against the row's
# largest magnitude.  Measured: 0.4e-2 .. 1.5e-2.
TOL = 3e-2

CASES = {
    "v4pro_bwd": ("v4pro_bf16", dict(T=256, hidden=512, experts=64, inter=256), True),
    "v4pro_bwd_given_routing": ("v4pro_bf16", dict(T=256, hidden=512, experts=64, inter=256), False),
    "llama_bwd_softmax": ("llama_bf16", dict(T=200, hidden=256, experts=64, inter=128), True),
    "sqrt_softplus_bwd": ("v4pro_bf16", dict(T=150, hidden=256, experts=64, inter=128,
                                             score="sqrt_softplus"), True),
    "hash_bwd": ("decode_hash_bf16", dict(T=40, hidden=512, experts=64, inter=256), True),
}


def _log(msg):
    print(msg, flush=True)


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_case(name):
    base, kw, with_router = CASES[name]
    cpu = synth.make_inputs(base, **kw)
    wl = cpu["workload"]
    gpu = to_device(cpu)
    T, h, E, k, f = wl.T, wl.hidden, wl.experts, wl.topk, wl.inter
    shape = moe.make_shape(T, h, E, k, f, wl.shared, "bf16")
    opts = moe.make_route_opts(wl.score, wl.renorm, wl.alpha, gpu["beta"], gpu["gate_bias"],
                               gpu["token_ids"], gpu["tid2eid"])
    weights = moe.make_weights(gpu["W1"], gpu["W2"], None, None, gpu["Ws1"], gpu["Ws2"])
    ws = moe.alloc_workspace(shape)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    G = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(shape, opts, gpu["X"], gpu["Wg"], ids, G, None, ws)
    gen = torch.Generator().manual_seed(1234)
    dY = torch.randn((T, h), generator=gen).to(torch.bfloat16)
    dYg = dY.cuda()
    bf = dict(dtype=torch.bfloat16, device="cuda")
    g = dict(dX=torch.empty((T, h), **bf), dW1=torch.empty((E, h, 2 * f), **bf),
             dW2=torch.empty((E, f, h), **bf),
             dWs1=torch.empty((h, 2 * f), **bf) if wl.shared else None,
             dWs2=torch.empty((f, h), **bf) if wl.shared else None,
             dWg=torch.empty((h, E), **bf) if with_router else None,
             dgate_bias=torch.empty(E, dtype=torch.float32, device="cuda") if with_router else None,
             dG=torch.empty((T, k), dtype=torch.float32, device="cuda"))
    grads = moe.make_grads(**g)
    wsb = moe.alloc_workspace(shape, backward=True)
    _log(f"[backward] {name}: moe_backward T={T} h={h} E={E} k={k} f={f} router={with_router}")
    moe.moe_backward(shape, opts if with_router else None, gpu["X"], gpu["Wg"], weights, ids, G,
                     dYg, grads, wsb)
    torch.cuda.synchronize()
    assert moe.moe_check_device_error(wsb) == 0
    return cpu, wl, ids.cpu().numpy(), G.cpu().double().numpy(), dY.double().numpy(), g, with_router


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    _need_gpu()
    cpu, wl, ids, G, dY, g, with_router = run_case(name)
    L = oracle.Layer("bf16", bits(cpu["X"]), bits(cpu["W1"]), bits(cpu["W2"]), Ws1=bits(cpu["Ws1"]),
                     Ws2=bits(cpu["Ws2"]), k=wl.topk)
    dX, dG = L.backward_tokens(ids, G, dY)
    err = {}
    # dG[t,j] is a dot product over hidden (k values per token, which can all
    # be small by cancellation): normalised by its largest magnitude
    err["dG"] = float(np.abs(f64(g["dG"]) - dG).max() / np.abs(dG).max())
    if with_router:
        b = oracle.route_backward(bits(cpu["X"]), bits(cpu["Wg"]), ids, dG,
                                  gate_bias=f64(cpu["gate_bias"]), score=wl.score,
                                  renorm=wl.renorm, alpha=wl.alpha, dX=dX)
        err["dWg"] = row_rel_err(f64(g["dWg"]), b["dWg"])
        db = g["dgate_bias"].cpu().double().numpy()
        err["dgate_bias"] = float(np.abs(db - b["dgate_bias"]).max() / np.abs(b["dgate_bias"]).max())
    err["dX"] = row_rel_err(f64(g["dX"]), dX)
    experts = list(range(wl.experts)) + ([wl.experts] if wl.shared else [])
    dW1, dW2 = L.backward_weights(ids, G, dY, experts)
    gw1 = f64(g["dW1"])
    gw2 = f64(g["dW2"])
    if wl.shared:
        gw1 = np.concatenate([gw1, f64(g["dWs1"])[None]])
        gw2 = np.concatenate([gw2, f64(g["dWs2"])[None]])
    used = np.zeros(len(experts), bool)
    used[np.unique(ids)] = True
    if wl.shared:
        used[-1] = True
    assert not gw1[~used].any() and not gw2[~used].any()   # experts without rows: zeros
    err["dW1"] = row_rel_err(gw1[used].reshape(-1, gw1.shape[-1]), dW1[used].reshape(-1, dW1.shape[-1]))
    err["dW2"] = row_rel_err(gw2[used].reshape(-1, gw2.shape[-1]), dW2[used].reshape(-1, dW2.shape[-1]))
    _log(f"[backward] {name}: " + ", ".join(f"{k} {v:.3e}" for k, v in err.items()))
    for k, v in err.items():
        assert v <= TOL, (k, v)
