"""Pins of the oracle's local backward (CPU only).

Checked against things other than the backward code itself: central finite
differences of the oracle's own fp64 forward (an fp32 layer, loss = sum of
dY * y for a fixed upstream gradient dY), and a torch autograd restatement of
the layer in fp64 (independent code).  The gradients of the chain follow
the blog "Megatron-LM 的 MoE 并行" (反向的通信: unpermute backward, expert
dgrad / wgrad with dX = Ȳ Wᵀ and dW = Xᵀ Ȳ, permute backward summing the k
copies) and the SwiGLU backward of "Megatron 分布式训练全维度并行技术文档"
§1.8.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

T, H, F, E, K = 6, 16, 8, 4, 2


def _layer(rng, shared=True):
    X = rng.standard_normal((T, H)).astype(np.float32)
    W1 = (rng.standard_normal((E, H, 2 * F)) / 4).astype(np.float32)
    W2 = (rng.standard_normal((E, F, H)) / 3).astype(np.float32)
    Ws1 = (rng.standard_normal((H, 2 * F)) / 4).astype(np.float32) if shared else None
    Ws2 = (rng.standard_normal((F, H)) / 3).astype(np.float32) if shared else None
    return dict(X=X, W1=W1, W2=W2, Ws1=Ws1, Ws2=Ws2)


def _mk(p):
    return oracle.Layer("fp32", p["X"], p["W1"], p["W2"], Ws1=p["Ws1"], Ws2=p["Ws2"], k=K)


def _ids(rng):
    return np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)


def _loss(p, ids, G, dY):
    return float((_mk(p).tokens(ids, G) * dY).sum())


def _fd(p, name, idx, ids, G, dY, rel=1e-3):
    """Central difference of the loss in parameter p[name][idx] (fp32 steps)."""
    w = float(p[name][idx])
    eps = rel * max(1.0, abs(w))
    hi, lo = dict(p), dict(p)
    hi[name] = p[name].copy()
    lo[name] = p[name].copy()
    hi[name][idx] = np.float32(w + eps)
    lo[name][idx] = np.float32(w - eps)
    d = float(hi[name][idx]) - float(lo[name][idx])
    return (_loss(hi, ids, G, dY) - _loss(lo, ids, G, dY)) / d


def _pick(rng, shape, n=8):
    return [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(n)]


def test_expert_gradients_match_finite_differences():
    rng = np.random.default_rng(40)
    p = _layer(rng)
    ids = _ids(rng)
    G = rng.uniform(0.2, 1.0, (T, K))
    dY = rng.standard_normal((T, H))
    L = _mk(p)
    dX, dG = L.backward_tokens(ids, G, dY)
    used = sorted(set(ids.ravel().tolist()))
    dW1, dW2 = L.backward_weights(ids, G, dY, used + [E])
    for idx in _pick(rng, (T, H)):
        assert _fd(p, "X", idx, ids, G, dY) == pytest.approx(dX[idx], rel=1e-5, abs=1e-6)
    for q, e in enumerate(used[:2]):
        for c, n in _pick(rng, (H, 2 * F), 5):
            fd = _fd(p, "W1", (e, c, n), ids, G, dY)
            assert fd == pytest.approx(dW1[q, c, n], rel=1e-5, abs=1e-6)
        for n, o in _pick(rng, (F, H), 5):
            fd = _fd(p, "W2", (e, n, o), ids, G, dY)
            assert fd == pytest.approx(dW2[q, n, o], rel=1e-5, abs=1e-6)
    for c, n in _pick(rng, (H, 2 * F), 5):
        assert _fd(p, "Ws1", (c, n), ids, G, dY) == pytest.approx(dW1[-1, c, n], rel=1e-5, abs=1e-6)
    for n, o in _pick(rng, (F, H), 5):
        assert _fd(p, "Ws2", (n, o), ids, G, dY) == pytest.approx(dW2[-1, n, o], rel=1e-5, abs=1e-6)
    # dG: the loss is linear in G, so the difference is exact up to rounding
    for t, j in _pick(rng, (T, K)):
        Gp, Gm = G.copy(), G.copy()
        Gp[t, j] += 1e-3
        Gm[t, j] -= 1e-3
        fd = (_loss(p, ids, Gp, dY) - _loss(p, ids, Gm, dY)) / 2e-3
        assert fd == pytest.approx(dG[t, j], rel=1e-7, abs=1e-9)
    # an expert that received no row has zero weight gradients
    unused = [e for e in range(E) if e not in used]
    if unused:
        z1, z2 = L.backward_weights(ids, G, dY, unused)
        assert not z1.any() and not z2.any()


def _router_loss(p, Wg, gb, dY, score, renorm, alpha, ids_ref):
    r = oracle.route(p["X"], Wg, K, gate_bias=gb, score=score, renorm=renorm, alpha=alpha)
    assert np.array_equal(r["ids"], ids_ref), "a step changed the selection"
    return float((_mk(p).tokens(r["ids"], r["G"]) * dY).sum())


@pytest.mark.parametrize("score,renorm,alpha", [("sigmoid", True, 2.5), ("softmax", False, 1.0),
                                                ("sqrt_softplus", True, 1.5),
                                                ("sigmoid", False, 1.0)])
def test_router_and_full_input_gradients_match_finite_differences(score, renorm, alpha):
    rng = np.random.default_rng(41)
    p = _layer(rng)
    Wg = (rng.standard_normal((H, E)) / 2).astype(np.float32)
    gb = rng.uniform(-0.3, 0.3, E)
    dY = rng.standard_normal((T, H))
    r = oracle.route(p["X"], Wg, K, gate_bias=gb, score=score, renorm=renorm, alpha=alpha)
    assert r["margin"].min() > 1e-3   # steps below keep the selection
    ids, G = r["ids"], r["G"]
    L = _mk(p)
    dX, dG = L.backward_tokens(ids, G, dY)
    b = oracle.route_backward(p["X"], Wg, ids, dG, gate_bias=gb, score=score, renorm=renorm,
                              alpha=alpha, dX=dX)
    eps = 2e-4
    for c, e in _pick(rng, (H, E), 6):
        hi, lo = Wg.copy(), Wg.copy()
        hi[c, e] = np.float32(Wg[c, e] + eps)
        lo[c, e] = np.float32(Wg[c, e] - eps)
        d = float(hi[c, e]) - float(lo[c, e])
        fd = (_router_loss(p, hi, gb, dY, score, renorm, alpha, ids) -
              _router_loss(p, lo, gb, dY, score, renorm, alpha, ids)) / d
        assert fd == pytest.approx(b["dWg"][c, e], rel=1e-4, abs=1e-6)
    for e in range(E):
        hi, lo = gb.copy(), gb.copy()
        hi[e] += 1e-5
        lo[e] -= 1e-5
        fd = (_router_loss(p, Wg, hi, dY, score, renorm, alpha, ids) -
              _router_loss(p, Wg, lo, dY, score, renorm, alpha, ids)) / 2e-5
        assert fd == pytest.approx(b["dgate_bias"][e], rel=1e-5, abs=1e-7)
    # dX now holds the whole input gradient: experts' part + router part
    for t, c in _pick(rng, (T, H), 6):
        hi, lo = dict(p), dict(p)
        hi["X"], lo["X"] = p["X"].copy(), p["X"].copy()
        x = float(p["X"][t, c])
        hi["X"][t, c] = np.float32(x + 2e-4)
        lo["X"][t, c] = np.float32(x - 2e-4)
        d = float(hi["X"][t, c]) - float(lo["X"][t, c])
        fd = (_router_loss(hi, Wg, gb, dY, score, renorm, alpha, ids) -
              _router_loss(lo, Wg, gb, dY, score, renorm, alpha, ids)) / d
        assert fd == pytest.approx(dX[t, c], rel=1e-4, abs=1e-6)
    if score != "softmax":   # sigmoid / sqrt(softplus): only chosen experts get a logit gradient
        mask = np.zeros((T, E), bool)
        np.put_along_axis(mask, ids.astype(np.int64), True, axis=1)
        assert not b["dl"][~mask].any()


def test_backward_matches_torch_autograd_restatement():
    """The same layer written with torch ops in fp64 (gating linear, sigmoid,
    renormalised top-k weights over the oracle's ids, SwiGLU experts, shared
    expert), differentiated by autograd."""
    rng = np.random.default_rng(42)
    p = _layer(rng)
    Wg = (rng.standard_normal((H, E)) / 2).astype(np.float32)
    gb = rng.uniform(-0.3, 0.3, E)
    dY = rng.standard_normal((T, H))
    alpha = 2.5
    r = oracle.route(p["X"], Wg, K, gate_bias=gb, score="sigmoid", renorm=True, alpha=alpha)
    ids = r["ids"]
    L = _mk(p)
    dX, dG = L.backward_tokens(ids, r["G"], dY)
    b = oracle.route_backward(p["X"], Wg, ids, dG, gate_bias=gb, score="sigmoid", renorm=True,
                              alpha=alpha, dX=dX)
    dW1, dW2 = L.backward_weights(ids, r["G"], dY, list(range(E)) + [E])

    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True)
         for k, v in dict(X=p["X"], Wg=Wg, gb=gb, W1=p["W1"], W2=p["W2"], Ws1=p["Ws1"],
                          Ws2=p["Ws2"]).items()}
    a = torch.sigmoid(t["X"] @ t["Wg"] + t["gb"])
    idx = torch.from_numpy(ids.astype(np.int64))
    sel = torch.gather(a, 1, idx)
    Gt = alpha * sel / sel.sum(1, keepdim=True)

    def ffn(x, w1, w2):
        hh = x @ w1
        return (torch.nn.functional.silu(hh[:, :F]) * hh[:, F:]) @ w2

    y = ffn(t["X"], t["Ws1"], t["Ws2"])
    for j in range(K):
        rows = [ffn(t["X"][i:i + 1], t["W1"][ids[i, j]], t["W2"][ids[i, j]]) for i in range(T)]
        y = y + Gt[:, j:j + 1] * torch.cat(rows)
    (y * torch.from_numpy(dY)).sum().backward()
    np.testing.assert_allclose(dX, t["X"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dWg"], t["Wg"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dgate_bias"], t["gb"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dW1[:E], t["W1"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dW2[:E], t["W2"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dW1[E], t["Ws1"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dW2[E], t["Ws2"].grad.numpy(), rtol=1e-10, atol=1e-12)


def test_bf16_layer_backward_equals_fp32_layer_on_the_same_values():
    """A bf16 layer reads the same numbers as an fp32 layer holding the
    bf16-rounded values; its gradients must be those of the fp32 layer."""
    rng = np.random.default_rng(43)
    p = _layer(rng)
    q = {k: (None if v is None else torch.from_numpy(v).to(torch.bfloat16)) for k, v in p.items()}
    bits = {k: (None if v is None else v.view(torch.int16).numpy().view(np.uint16))
            for k, v in q.items()}
    f32 = {k: (None if v is None else v.float().numpy()) for k, v in q.items()}
    ids = _ids(rng)
    G = rng.uniform(0.2, 1.0, (T, K))
    dY = rng.standard_normal((T, H))
    Lb = oracle.Layer("bf16", bits["X"], bits["W1"], bits["W2"], Ws1=bits["Ws1"], Ws2=bits["Ws2"],
                      k=K)
    Lf = _mk(f32)
    for a, b in zip(Lb.backward_tokens(ids, G, dY), Lf.backward_tokens(ids, G, dY)):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(Lb.backward_weights(ids, G, dY, [0, E]), Lf.backward_weights(ids, G, dY, [0, E])):
        np.testing.assert_array_equal(a, b)
