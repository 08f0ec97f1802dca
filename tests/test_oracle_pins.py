"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on a page, a closed form, a library routine (numpy / scipy /
torch's float8 cast), a brute-force dense formulation, or an invariant of the
definition.  The planted-mistake test at the end shows that a plausible slip
in the oracle is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from tests import test_oracle_backward_pins as bwd
from tests.helpers import bits, oracle_layer, oracle_route

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers
def _np_swiglu(x, W1, W2):
    """Dense SwiGLU FFN with numpy fp64 matmuls (x [n,h], W1 [h,2f], W2 [f,h])."""
    f = W1.shape[1] // 2
    H = x @ W1
    g, u = H[:, :f], H[:, f:]
    return (g / (1.0 + np.exp(-g)) * u) @ W2


def _rand_ids(rng, T, k, E):
    """k distinct expert ids per token."""
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


# ------------------------------------------------------------------ dispatch
def test_four_token_split_example():
    """The worked split of §计数与重排 (DeepSeek-V4 blog post)."""
    g = json.load(open(os.path.join(GOLDEN, "four_token_split.json")))
    E, k, L = g["experts"], g["topk"], g["experts_per_rank"]
    names = list(g["tokens"])
    ids = np.array([g["tokens"][n] for n in names], np.int32)
    d = oracle.dispatch(ids, E)
    assert d["counts"].tolist() == g["expected"]["global_counts"]
    splits = []
    for toks in g["rank_tokens"]:
        local = np.array([g["tokens"][n] for n in toks], np.int32)
        cnt = oracle.dispatch(local, E)["counts"]
        splits.append([int(cnt[j * L:(j + 1) * L].sum()) for j in range(E // L)])
        assert sum(splits[-1]) == len(toks) * k
    assert splits == g["expected"]["input_splits"]
    out = [[splits[src][dst] for src in range(len(splits))] for dst in range(len(splits))]
    assert out == g["expected"]["output_splits"]
    assert [sum(o) for o in out] == g["expected"]["received_rows"]


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (7, 2, 8), (64, 6, 384), (333, 4, 17), (0, 2, 4)])
def test_dispatch_invariants(T, k, E):
    rng = np.random.default_rng(T * 131 + k * 7 + E)
    ids = _rand_ids(rng, T, k, E) if T else np.zeros((0, k), np.int32)
    d = oracle.dispatch(ids, E)
    counts, offs, dst, src = d["counts"], d["offsets"], d["dst_row"], d["src_tok"]
    # counts sum to T*k and agree with numpy's bincount
    assert counts.sum() == T * k
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert offs[0] == 0 and np.array_equal(np.diff(offs), counts)
    # dst_row is a bijection onto [0, T*k) and lands in the expert's block
    assert np.array_equal(np.sort(dst), np.arange(T * k))
    e_of = ids.ravel()
    assert np.all(dst >= offs[e_of]) and np.all(dst < offs[e_of + 1])
    # the source token of each row is the token of the assignment
    assert np.array_equal(src[dst], np.arange(T * k) // max(k, 1))
    # stable: within an expert block, rows follow ascending flat index
    for e in range(E):
        flat = np.nonzero(e_of == e)[0]
        assert np.array_equal(dst[flat], offs[e] + np.arange(len(flat)))


def test_dispatch_flags_bad_ids():
    ids = np.array([[0, 5], [1, -1]], np.int32)
    d = oracle.dispatch(ids, 4)
    assert d["bad"] == 2
    assert d["dst_row"][1] == -1 and d["dst_row"][3] == -1
    assert d["counts"].tolist() == [1, 1, 0, 0]


def test_permute_then_unpermute_is_identity():
    rng = np.random.default_rng(3)
    T, k, E, h = 50, 3, 9, 16
    X = rng.standard_normal((T, h))
    ids = _rand_ids(rng, T, k, E)
    d = oracle.dispatch(ids, E)
    Xp = X[d["src_tok"]]                       # permute (with duplication)
    back = Xp[d["dst_row"]].reshape(T, k, h)   # unpermute each copy
    for j in range(k):
        assert np.array_equal(back[:, j], X)


def test_identity_experts_combine_gives_weight_sum_times_x():
    rng = np.random.default_rng(4)
    T, k, E, h = 40, 4, 11, 24
    X = rng.standard_normal((T, h))
    ids = _rand_ids(rng, T, k, E)
    G = rng.random((T, k))
    d = oracle.dispatch(ids, E)
    Y = oracle.combine(X[d["src_tok"]], d["dst_row"], G)
    np.testing.assert_allclose(Y, G.sum(1, keepdims=True) * X, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ routing
def test_affinity_closed_forms_and_library():
    l = np.array([[-30.0, -2.5, -1e-3, 0.0, 1e-3, 0.7, 3.0, 40.0]])
    np.testing.assert_allclose(oracle.affinity(l, "sigmoid"), scipy.special.expit(l), rtol=1e-15)
    assert oracle.affinity(np.zeros((1, 1)), "sigmoid")[0, 0] == 0.5
    np.testing.assert_allclose(oracle.affinity(l, "sqrt_softplus"),
                               np.sqrt(np.logaddexp(0.0, l)), rtol=1e-14)
    assert math.isclose(oracle.affinity(np.zeros((1, 1)), "sqrt_softplus")[0, 0],
                        math.sqrt(math.log(2.0)), rel_tol=1e-15)
    np.testing.assert_allclose(oracle.affinity(l, "softmax"), scipy.special.softmax(l, axis=1),
                               rtol=1e-13)


def test_topk_matches_stable_argsort_and_ties_go_to_lower_id():
    rng = np.random.default_rng(5)
    keys = rng.integers(0, 6, size=(200, 13)).astype(np.float64)   # many exact ties
    for k in (1, 3, 13):
        ids, margin = oracle.topk(keys, k)
        ref = np.argsort(-keys, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        if k < 13:
            srt = -np.sort(-keys, axis=1)
            np.testing.assert_array_equal(margin, srt[:, k - 1] - srt[:, k])


def test_zero_gate_weight_selects_first_k_with_uniform_weights():
    T, h, E, k = 5, 16, 10, 4
    X = _bf16(np.random.default_rng(6).standard_normal((T, h)))
    Wg = _bf16(np.zeros((h, E)))
    r = oracle.route(bits(X), bits(Wg), k, score="sigmoid", renorm=True, alpha=2.5)
    assert np.array_equal(r["ids"], np.tile(np.arange(k), (T, 1)))
    np.testing.assert_allclose(r["G"], 2.5 / k, rtol=1e-15)
    r = oracle.route(bits(X), bits(Wg), k, score="softmax", renorm=False)
    np.testing.assert_allclose(r["G"], 1.0 / E, rtol=1e-15)


def test_selection_uses_bias_but_weights_use_raw_affinity():
    rng = np.random.default_rng(7)
    T, h, E, k = 32, 64, 16, 3
    X = rng.standard_normal((T, h)).astype(np.float32)
    Wg = (rng.standard_normal((h, E)) * 0.3).astype(np.float32)
    beta = np.zeros(E)
    beta[5] = 10.0
    r = oracle.route(X, Wg, k, beta=beta, score="sigmoid", renorm=True, alpha=1.7)
    assert np.all(r["ids"][:, 0] == 5)          # beta dominates the selection
    a = scipy.special.expit(X.astype(np.float64) @ Wg.astype(np.float64))
    sel = np.take_along_axis(a, r["ids"].astype(np.int64), axis=1)
    np.testing.assert_allclose(r["G"], 1.7 * sel / sel.sum(1, keepdims=True), rtol=1e-12)
    # the biased key would give a visibly different weight for expert 5
    biased = sel.copy()
    biased[:, 0] += 10.0
    assert np.abs(1.7 * biased / biased.sum(1, keepdims=True) - r["G"]).max() > 0.1
    # without the bias, the selection is the top-k of the raw affinity
    r0 = oracle.route(X, Wg, k, score="sigmoid")
    assert np.array_equal(r0["ids"], np.argsort(-a, axis=1, kind="stable")[:, :k])


def test_softmax_router_raw_weights():
    rng = np.random.default_rng(8)
    T, h, E, k = 20, 32, 8, 2
    X = rng.standard_normal((T, h)).astype(np.float32)
    Wg = (rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32)
    r = oracle.route(X, Wg, k, score="softmax", renorm=False, alpha=1.0)
    p = scipy.special.softmax(X.astype(np.float64) @ Wg.astype(np.float64), axis=1)
    np.testing.assert_allclose(r["G"], np.take_along_axis(p, r["ids"].astype(np.int64), 1),
                               rtol=1e-12)
    full = oracle.route(X, Wg, E, score="softmax", renorm=False)
    np.testing.assert_allclose(full["G"].sum(1), 1.0, rtol=1e-13)


def test_gate_bias_shifts_logits():
    rng = np.random.default_rng(9)
    X = rng.standard_normal((6, 8)).astype(np.float32)
    Wg = rng.standard_normal((8, 5)).astype(np.float32)
    b = rng.standard_normal(5)
    np.testing.assert_allclose(oracle.gate_logits(X, Wg, b),
                               X.astype(np.float64) @ Wg.astype(np.float64) + b, rtol=1e-12)


def test_hash_routing_is_a_table_lookup():
    rng = np.random.default_rng(10)
    T, h, E, k, V = 30, 16, 12, 3, 50
    X = rng.standard_normal((T, h)).astype(np.float32)
    Wg = rng.standard_normal((h, E)).astype(np.float32)
    tab = _rand_ids(rng, V, k, E)
    tok = rng.integers(0, V, T).astype(np.int32)
    beta = rng.standard_normal(E) * 5
    r = oracle.route(X, Wg, k, beta=beta, token_ids=tok, tid2eid=tab, alpha=2.0)
    assert np.array_equal(r["ids"], tab[tok])
    a = scipy.special.expit(X.astype(np.float64) @ Wg.astype(np.float64))
    sel = np.take_along_axis(a, r["ids"].astype(np.int64), 1)
    np.testing.assert_allclose(r["G"], 2.0 * sel / sel.sum(1, keepdims=True), rtol=1e-12)


# ------------------------------------------------------------------ experts
def test_single_expert_top1_is_dense_swiglu_plus_shared():
    rng = np.random.default_rng(11)
    T, h, f = 9, 32, 16
    X = rng.standard_normal((T, h)).astype(np.float32)
    W1 = (rng.standard_normal((1, h, 2 * f)) / math.sqrt(h)).astype(np.float32)
    W2 = (rng.standard_normal((1, f, h)) / math.sqrt(f)).astype(np.float32)
    Ws1 = (rng.standard_normal((h, 2 * f)) / math.sqrt(h)).astype(np.float32)
    Ws2 = (rng.standard_normal((f, h)) / math.sqrt(f)).astype(np.float32)
    Wg = rng.standard_normal((h, 1)).astype(np.float32)
    r = oracle.route(X, Wg, 1, alpha=1.0)            # G = a / a = 1
    np.testing.assert_allclose(r["G"], 1.0, rtol=1e-15)
    L = oracle.Layer("fp32", X, W1, W2, k=1)
    x64 = X.astype(np.float64)
    np.testing.assert_allclose(L.tokens(r["ids"], r["G"]),
                               _np_swiglu(x64, W1[0].astype(np.float64), W2[0].astype(np.float64)),
                               rtol=1e-11, atol=1e-12)
    Ls = oracle.Layer("fp32", X, W1, W2, Ws1=Ws1, Ws2=Ws2, k=1)
    ref = (_np_swiglu(x64, W1[0].astype(np.float64), W2[0].astype(np.float64))
           + _np_swiglu(x64, Ws1.astype(np.float64), Ws2.astype(np.float64)))
    np.testing.assert_allclose(Ls.tokens(r["ids"], r["G"]), ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("score,renorm", [("sigmoid", True), ("softmax", False),
                                          ("sqrt_softplus", True)])
def test_k_equals_E_is_the_dense_mixture(score, renorm):
    """With k = E every expert is selected: the layer is the dense mixture
    sum_e g_e F_e(x), computed here with numpy matmuls over all experts."""
    rng = np.random.default_rng(12)
    T, h, E, f = 12, 24, 5, 8
    X = rng.standard_normal((T, h)).astype(np.float32)
    Wg = (rng.standard_normal((h, E)) / math.sqrt(h)).astype(np.float32)
    W1 = (rng.standard_normal((E, h, 2 * f)) / math.sqrt(h)).astype(np.float32)
    W2 = (rng.standard_normal((E, f, h)) / math.sqrt(f)).astype(np.float32)
    alpha = 1.3
    r = oracle.route(X, Wg, E, score=score, renorm=renorm, alpha=alpha)
    y = oracle.Layer("fp32", X, W1, W2, k=E).tokens(r["ids"], r["G"])
    x64 = X.astype(np.float64)
    logits = x64 @ Wg.astype(np.float64)
    a = {"sigmoid": scipy.special.expit(logits), "softmax": scipy.special.softmax(logits, 1),
         "sqrt_softplus": np.sqrt(np.logaddexp(0, logits))}[score]
    g = alpha * a / a.sum(1, keepdims=True) if renorm else alpha * a
    dense = sum(g[:, e:e + 1] * _np_swiglu(x64, W1[e].astype(np.float64), W2[e].astype(np.float64))
                for e in range(E))
    np.testing.assert_allclose(y, dense, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny_fp32", "v4pro_bf16", "v4pro_fp8", "v4pro_int8",
                                  "decode_hash_bf16"])
def test_token_loop_equals_staged_dispatch_experts_combine(name):
    """The per-token layer equation (blog §模型与入口) and the staged
    dispatch / expert / combine definition (mega_moe §计算过程) agree."""
    inp = synth.make_inputs(name, T=24, hidden=64, inter=32, experts=16 if name != "tiny_fp32" else 8,
                            zipf=False)
    wl = inp["workload"]
    r = oracle_route(inp)
    L = oracle_layer(inp)
    d = oracle.dispatch(r["ids"], wl.experts)
    y_tok = L.tokens(r["ids"], r["G"])
    Yp = L.expert_rows(d["offsets"], d["src_tok"])
    Ys = None
    if wl.shared:
        Ys = L.expert_rows(d["offsets"], d["src_tok"], rows=np.arange(wl.T * wl.topk,
                                                                      wl.T * wl.topk + wl.T))
    y_stg = oracle.combine(Yp, d["dst_row"], r["G"], Ys)
    np.testing.assert_allclose(y_tok, y_stg, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ fp8
def test_e4m3_decode_all_codes_match_torch_and_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[finite], ref[finite])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and np.isnan(ours).sum() == 2
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9
    assert ours[0x38] == 1.0 and ours[0xB8] == -1.0


def test_e4m3_encode_roundtrip_ties_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)
    # ties go to the even mantissa: 1.0625 between 1.0 (0x38) and 1.125 (0x39)
    assert oracle.e4m3_encode(np.array([1.0625, 1.1875, -1.0625]))[()].tolist() == [0x38, 0x3A, 0xB8]
    assert oracle.e4m3_encode(np.array([448.0, 463.99, 500.0, 1e30, -1e30])).tolist() == \
        [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    # random values: nearest-even agrees with torch's float8_e4m3fn cast
    rng = np.random.default_rng(13)
    v = np.concatenate([rng.standard_normal(4000) * 50, rng.standard_normal(2000) * 1e-2,
                        rng.uniform(-448, 448, 2000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), ref)


def test_quantize_rows_f32_matches_torch_cast():
    rng = np.random.default_rng(14)
    X = (rng.standard_normal((16, 300)) * rng.uniform(0.01, 100, (16, 1))).astype(np.float32)
    X[3] = 0.0
    q, s = oracle.quantize_rows_f32(X)
    amax = np.abs(X).max(1)
    s_ref = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(s, s_ref)
    q_ref = torch.from_numpy(X / s_ref[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, q_ref)
    assert np.all(q[3] == 0) and s[3] == 1.0


def test_fp8_expert_is_exact_when_every_quantisation_is_lossless():
    """inter = 1 makes the SwiGLU output one value per row, whose requantised
    code is exactly +-448; with X rows holding e4m3 values and max|x| = 448,
    the activation scale is 1.  The fp8 layer then equals the exact SwiGLU
    with dequantised weights (code * per-channel scale)."""
    rng = np.random.default_rng(15)
    T, h, f, E = 6, 32, 1, 3
    grid = oracle.e4m3_decode(np.arange(0x30, 0x50, dtype=np.uint8))  # 0.25 .. 8
    X = rng.choice(grid, size=(T, h)) * rng.choice([-1, 1], size=(T, h))
    X[:, 0] = 448.0
    Xb = _bf16(X)
    assert np.array_equal(Xb.float().numpy(), X.astype(np.float32))  # exact in bf16
    W1q = rng.integers(0, 0x7E, size=(E, h, 2 * f)).astype(np.uint8) | \
        (rng.integers(0, 2, size=(E, h, 2 * f)).astype(np.uint8) << 7)
    W2q = rng.integers(0, 0x7E, size=(E, f, h)).astype(np.uint8)
    s1 = rng.uniform(1e-4, 1e-3, (E, 2 * f)).astype(np.float32)
    s2 = rng.uniform(1e-3, 1e-2, (E, h)).astype(np.float32)
    ids = np.array([[t % E] for t in range(T)], np.int32)
    G = np.ones((T, 1))
    L = oracle.Layer("fp8", bits(Xb), W1q, W2q, w1_scale=s1, w2_scale=s2, k=1)
    y = L.tokens(ids, G)
    dq1 = oracle.e4m3_decode(W1q) * s1[:, None, :].astype(np.float64)
    dq2 = oracle.e4m3_decode(W2q) * s2[:, None, :].astype(np.float64)
    for t in range(T):
        e = ids[t, 0]
        ref = _np_swiglu(X[t:t + 1].astype(np.float64), dq1[e], dq2[e])
        np.testing.assert_allclose(y[t:t + 1], ref, rtol=1e-12)


def test_fp8_layer_within_quantisation_error_of_exact_layer():
    inp = synth.make_inputs("v4pro_fp8", T=16, hidden=256, inter=128, experts=8, zipf=False)
    wl = inp["workload"]
    r = oracle_route(inp)
    y8 = oracle_layer(inp).tokens(r["ids"], r["G"])
    dq = dict(inp)
    dq["workload"] = wl.replace(precision="fp32")
    dq["X"] = inp["X"].float()
    for w, s in (("W1", "w1_scale"), ("W2", "w2_scale"), ("Ws1", "ws1_scale"), ("Ws2", "ws2_scale")):
        dq[w] = inp[w].float() * inp[s].unsqueeze(-2)
        dq[s] = None
    y = oracle_layer(dq).tokens(r["ids"], r["G"])
    rel = np.abs(y8 - y).max(1) / np.abs(y).max(1)
    assert rel.max() < 0.1 and rel.max() > 1e-4   # lossy, but only by the fp8 rounding


# ------------------------------------------------------------------ INT8 A8W8
def _i8_quant_rows(v, dtype):
    """The mega_moe page's INT8 rule restated with numpy: per row s = max|v| /
    127 (1 for a zero row), codes = v / s rounded half away from zero, in
    [-127, 127]; scale and quotient in `dtype`, the rounding exact."""
    v = np.asarray(v, dtype)
    amax = np.abs(v).max(1)
    s = np.where(amax > 0, amax / dtype(127.0), dtype(1.0)).astype(dtype)
    r = (v / s[:, None]).astype(np.float64)
    q = np.clip(np.trunc(r + np.copysign(0.5, r)), -127, 127)
    return q.astype(np.int8), s


def _i8_weights(rng, E, K, N):
    """Per-output-channel INT8 weights: codes [E,K,N], fp32 scales [E,N] and
    the dequantised fp64 matrices."""
    W = rng.standard_normal((E, K, N)) / np.sqrt(K)
    amax = np.abs(W).max(1)
    s = (amax / 127.0).astype(np.float32)
    r = W / s[:, None, :].astype(np.float64)
    q = np.clip(np.trunc(r + np.copysign(0.5, r)), -127, 127).astype(np.int8)
    return q, s, q.astype(np.float64) * s[:, None, :].astype(np.float64)


def test_quantize_rows_i8_rounds_half_away_from_zero():
    # scale 1 (max 127): halves go away from zero, as ⌊z⌉ of the page's §约定 reads
    x = np.array([[127.0, 63.5, -63.5, 0.5, -0.5, 2.5, -2.5, 1.49, -126.5, 0.0]], np.float32)
    q, s = oracle.quantize_rows_i8_f32(x)
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 64, -64, 1, -1, 3, -3, 1, -127, 0]
    rng = np.random.default_rng(30)
    X = (rng.standard_normal((16, 300)) * rng.uniform(0.01, 100, (16, 1))).astype(np.float32)
    X[3] = 0.0
    q, s = oracle.quantize_rows_i8_f32(X)
    q_ref, s_ref = _i8_quant_rows(X, np.float32)
    assert np.array_equal(s, s_ref) and np.array_equal(q, q_ref)
    assert np.all(q[3] == 0) and s[3] == 1.0
    assert np.all(np.abs(q).max(1)[np.arange(16) != 3] == 127)


def test_int8_expert_is_exact_when_every_quantisation_is_lossless():
    """Integer X rows with max 127 quantise with scale 1 to themselves, and
    inter = 1 makes the SwiGLU output one value per row, requantised to
    +-127 exactly: the INT8 layer then equals the exact SwiGLU with
    dequantised weights (code * per-channel scale)."""
    rng = np.random.default_rng(31)
    T, h, f, E = 6, 32, 1, 3
    X = rng.integers(-127, 128, size=(T, h)).astype(np.float64)
    X[:, 0] = 127.0
    Xb = _bf16(X)
    assert np.array_equal(Xb.float().numpy(), X.astype(np.float32))  # exact in bf16
    W1q = rng.integers(-127, 128, size=(E, h, 2 * f)).astype(np.int8)
    W2q = rng.integers(-127, 128, size=(E, f, h)).astype(np.int8)
    s1 = rng.uniform(1e-4, 1e-3, (E, 2 * f)).astype(np.float32)
    s2 = rng.uniform(1e-3, 1e-2, (E, h)).astype(np.float32)
    ids = np.array([[t % E] for t in range(T)], np.int32)
    L = oracle.Layer("int8", bits(Xb), W1q, W2q, w1_scale=s1, w2_scale=s2, k=1)
    y = L.tokens(ids, np.ones((T, 1)))
    dq1 = W1q.astype(np.float64) * s1[:, None, :].astype(np.float64)
    dq2 = W2q.astype(np.float64) * s2[:, None, :].astype(np.float64)
    for t in range(T):
        e = ids[t, 0]
        ref = _np_swiglu(X[t:t + 1], dq1[e], dq2[e])
        np.testing.assert_allclose(y[t:t + 1], ref, rtol=1e-12)


def test_int8_layer_is_the_dense_swiglu_of_dequantised_operands():
    """Routed and shared experts: Q8(x) -> DQ . DQ(W1) -> SwiGLU -> Q8 -> DQ
    . DQ(W2), rebuilt with numpy matmuls and the numpy restatement of the
    rounding rule above."""
    rng = np.random.default_rng(32)
    T, h, f, E, k = 5, 64, 48, 3, 2
    Xb = _bf16(rng.standard_normal((T, h)))
    W1, s1, dq1 = _i8_weights(rng, E, h, 2 * f)
    W2, s2, dq2 = _i8_weights(rng, E, f, h)
    Ws1, ss1, dqs1 = _i8_weights(rng, 1, h, 2 * f)
    Ws2, ss2, dqs2 = _i8_weights(rng, 1, f, h)
    ids = np.array([[t % E, (t + 1) % E] for t in range(T)], np.int32)
    G = rng.uniform(0.1, 1.0, (T, k))
    L = oracle.Layer("int8", bits(Xb), W1, W2, w1_scale=s1, w2_scale=s2, Ws1=Ws1[0], Ws2=Ws2[0],
                     ws1_scale=ss1[0], ws2_scale=ss2[0], k=k)
    y = L.tokens(ids, G)
    xq, xs = _i8_quant_rows(Xb.float().numpy(), np.float32)
    xd = xq.astype(np.float64) * xs[:, None].astype(np.float64)

    def expert(x, d1, d2):
        hh = x @ d1
        u = hh[:, :f] / (1.0 + np.exp(-hh[:, :f])) * hh[:, f:]
        uq, us = _i8_quant_rows(u, np.float64)
        return (uq.astype(np.float64) * us[:, None]) @ d2

    for t in range(T):
        ref = expert(xd[t:t + 1], dqs1[0], dqs2[0])
        for j in range(k):
            ref = ref + G[t, j] * expert(xd[t:t + 1], dq1[ids[t, j]], dq2[ids[t, j]])
        np.testing.assert_allclose(y[t:t + 1], ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_int8_layer_within_quantisation_error_of_exact_layer():
    inp = synth.make_inputs("v4pro_int8", T=16, hidden=256, inter=128, experts=8, zipf=False)
    wl = inp["workload"]
    r = oracle_route(inp)
    y8 = oracle_layer(inp).tokens(r["ids"], r["G"])
    dq = dict(inp)
    dq["workload"] = wl.replace(precision="fp32")
    dq["X"] = inp["X"].float()
    for w, s in (("W1", "w1_scale"), ("W2", "w2_scale"), ("Ws1", "ws1_scale"), ("Ws2", "ws2_scale")):
        dq[w] = inp[w].float() * inp[s].unsqueeze(-2)
        dq[s] = None
    y = oracle_layer(dq).tokens(r["ids"], r["G"])
    rel = np.abs(y8 - y).max(1) / np.abs(y).max(1)
    assert rel.max() < 0.1 and rel.max() > 1e-4   # lossy, but only by the INT8 rounding


# ------------------------------------------------------------------ MX (group-32, E8M0)
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP FP4 e2m1, codes 0..7
EMAX = {"e4m3": 8, "e2m1": 2}                                # exponent of the largest normal


def _e2m1_nearest_even(v):
    """Brute force: the e2m1 code nearest to v, ties to the even code, |v| >= 6 -> 6."""
    out = []
    for x in np.asarray(v, np.float64).ravel():
        a = min(abs(x), 6.0)
        d = [abs(a - m) for m in E2M1_MAGNITUDES]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        out.append(c | (8 if (x < 0 or (x == 0 and math.copysign(1, x) < 0)) else 0))
    return np.array(out, np.uint8).reshape(np.shape(v))


def _mx_dequant(codes, scales, fmt):
    """Independent MX dequantisation: element values from torch (e4m3) or the
    OCP table (e2m1), times 2^(scale - 127) per group of 32 along the last axis."""
    codes = np.asarray(codes, np.uint8)
    if fmt == "e4m3":
        v = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    else:
        mag = np.array(E2M1_MAGNITUDES)[codes & 7]
        v = np.where(codes & 8, -mag, mag)
    sc = np.repeat(np.asarray(scales, np.int64), 32, axis=-1)
    return np.ldexp(v, sc - 127)


def test_e2m1_codes_are_the_ocp_table():
    vals = [oracle.e2m1_decode(c) for c in range(16)]
    assert vals[:8] == E2M1_MAGNITUDES
    assert vals[8:] == [-m for m in E2M1_MAGNITUDES]
    assert all(oracle.e2m1_encode(vals[c]) == c for c in range(16))
    # ties go to the even code; beyond 6 saturates
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 7.0, 1e9]
    assert [oracle.e2m1_encode(v) for v in ties] == [0, 2, 2, 4, 4, 6, 6, 14, 7, 7]


def test_e2m1_encode_matches_brute_force():
    rng = np.random.default_rng(21)
    v = np.concatenate([rng.standard_normal(3000) * 3, rng.uniform(-8, 8, 3000),
                        np.arange(-28, 29) / 4.0])
    ours = np.array([oracle.e2m1_encode(x) for x in v], np.uint8)
    assert np.array_equal(ours, _e2m1_nearest_even(v))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_mx_scale_code_is_floor_log2_minus_emax(fmt):
    rng = np.random.default_rng(22)
    amax = np.concatenate([np.exp(rng.uniform(-60, 60, 2000)), 2.0 ** np.arange(-20, 21)])
    ref = np.clip(np.floor(np.log2(amax)).astype(np.int64) - EMAX[fmt] + 127, 0, 254)
    assert [oracle.mx_scale_code(a, fmt) for a in amax] == ref.tolist()
    assert oracle.mx_scale_code(0.0, fmt) == 0
    assert oracle.mx_scale_code(1.0, fmt) == 127 - EMAX[fmt]


def test_mx_quantize_e4m3_matches_torch_cast_and_error_bound():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((40, 256)) * np.exp(rng.uniform(-8, 8, (40, 1)))
    x[3] = 0.0
    x[5, :32] = 1.0          # one value, scale 2^-8, element 256
    x[6, :32] = 500.0        # scale 2^0: 500 saturates to 448
    q, sc = oracle.mx_quantize(x, "e4m3")
    assert sc.shape == (40, 8) and np.all(sc[3] == 0) and np.all(q[3] == 0)
    assert sc[5, 0] == 119 and np.all(q[5, :32] == 0x78)
    assert sc[6, 0] == 127 and np.all(q[6, :32] == 0x7E)
    # element codes: the torch e4m3fn cast of the scaled, clamped values
    scaled = np.ldexp(x, 127 - np.repeat(sc.astype(np.int64), 32, axis=1))
    ref = torch.from_numpy(np.clip(scaled, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    # round trip: relative error at most 2^-4 where the scaled value is a normal e4m3
    dq = _mx_dequant(q, sc, "e4m3")
    normal = (np.abs(scaled) >= 2.0 ** -6) & (np.abs(scaled) <= 448)
    assert np.all(np.abs(dq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])


def test_mx_quantize_e2m1_matches_brute_force():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((12, 128)) * np.exp(rng.uniform(-4, 4, (12, 1)))
    x[2] = 0.0
    q, sc = oracle.mx_quantize(x, "e2m1")
    amax = np.abs(x.reshape(12, 4, 32)).max(-1)
    ref_sc = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 2 + 127, 0)
    assert np.array_equal(sc, ref_sc.astype(np.uint8))
    scaled = np.ldexp(x, 127 - np.repeat(sc.astype(np.int64), 32, axis=1))
    assert np.array_equal(q, _e2m1_nearest_even(scaled))


def _mx_weights(rng, E, K, N, fmt):
    """Random MX weights of K x N matrices.  e4m3: codes [E,K,N], E8M0 scales
    [E,K/32,N].  e2m1 (K-contiguous, as the MXFP4 layer stores them): code
    pairs [E,N,K/2] (element 2i in the low nibble), scales [E,N,K/32].
    Returns (stored codes, stored scales, dequantised [E,K,N])."""
    scales_nk = rng.integers(112, 124, size=(E, N, K // 32)).astype(np.uint8)
    if fmt == "e4m3":
        codes_nk = rng.integers(0, 0x7E, size=(E, N, K)).astype(np.uint8) | \
            (rng.integers(0, 2, size=(E, N, K)).astype(np.uint8) << 7)
        stored = np.ascontiguousarray(np.swapaxes(codes_nk, 1, 2))
        stored_sc = np.ascontiguousarray(np.swapaxes(scales_nk, 1, 2))
    else:
        codes_nk = rng.integers(0, 16, size=(E, N, K)).astype(np.uint8)
        stored = (codes_nk[..., 0::2] | (codes_nk[..., 1::2] << 4)).astype(np.uint8)
        stored_sc = scales_nk
    # dequantised: the scale of W[e, k, n] belongs to group k // 32 of column n
    deq = _mx_dequant(codes_nk, scales_nk, fmt)
    return stored, stored_sc, np.ascontiguousarray(np.swapaxes(deq, 1, 2))


@pytest.mark.parametrize("prec,fmt", [("mxfp8", "e4m3"), ("mxfp4", "e2m1")])
def test_mx_layer_is_the_dense_swiglu_of_dequantised_operands(prec, fmt):
    """Each routed and the shared expert: Q_MX(x) -> DQ . DQ(W1) -> SwiGLU ->
    Q_MX -> DQ . DQ(W2), rebuilt here with numpy matmuls and the independent
    dequantisation above (the quantisation steps themselves are pinned by
    the tests before)."""
    rng = np.random.default_rng(25)
    T, h, f, E, k = 5, 64, 64, 3, 2
    X = rng.standard_normal((T, h))
    Xb = _bf16(X)
    W1, s1, dq1 = _mx_weights(rng, E, h, 2 * f, fmt)
    W2, s2, dq2 = _mx_weights(rng, E, f, h, fmt)
    Ws1, ss1, dqs1 = _mx_weights(rng, 1, h, 2 * f, fmt)
    Ws2, ss2, dqs2 = _mx_weights(rng, 1, f, h, fmt)
    ids = np.array([[t % E, (t + 1) % E] for t in range(T)], np.int32)
    G = rng.uniform(0.1, 1.0, (T, k))
    L = oracle.Layer(prec, bits(Xb), W1, W2, w1_scale=s1, w2_scale=s2, Ws1=Ws1[0], Ws2=Ws2[0],
                     ws1_scale=ss1[0], ws2_scale=ss2[0], k=k)
    y = L.tokens(ids, G)
    xq, xs = oracle.mx_quantize(Xb.double().numpy(), fmt)
    xd = _mx_dequant(xq, xs, fmt)

    def expert(x, d1, d2):
        hh = x @ d1
        u = hh[:, :f] / (1.0 + np.exp(-hh[:, :f])) * hh[:, f:]
        uq, us = oracle.mx_quantize(u, fmt)
        return _mx_dequant(uq, us, fmt) @ d2

    for t in range(T):
        ref = expert(xd[t:t + 1], dqs1[0], dqs2[0])
        for j in range(k):
            ref = ref + G[t, j] * expert(xd[t:t + 1], dq1[ids[t, j]], dq2[ids[t, j]])
        np.testing.assert_allclose(y[t:t + 1], ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


# ------------------------------------------------------------------ shapes
def test_workload_shapes_match_the_pages_arithmetic():
    v4 = synth.WORKLOADS["v4pro_bf16"]
    assert v4.params_per_expert == 66_060_288          # 3hf, blog §模型与入口
    ep = synth.WORKLOADS["ep_share_bf16"]
    assert ep.T * ep.topk == 24_576 and ep.experts == 6  # 6 experts x 4096 rows per EP64 rank


def test_zipf_fixture_gives_skewed_load():
    """Realised load on a fresh batch follows the Zipf target roughly."""
    inp = synth.make_inputs("v4pro_bf16", T=1024, hidden=512, experts=64, inter=8)
    r = oracle_route(inp)
    cnt = np.sort(np.bincount(r["ids"].ravel(), minlength=64))[::-1]
    assert cnt[0] > 8 * max(cnt[-1], 1)
    assert cnt[0] > 0.5 * 1024 and cnt.sum() == 6 * 1024


# ------------------------------------------------------------------ planted mistake
PLANTED = {
    # SwiGLU halves swapped in the bf16/fp32 expert
    "swiglu": ("h1[n] = silu(h1[n]) * h1[f + n];", "h1[n] = silu(h1[f + n]) * h1[n];",
               lambda: test_single_expert_top1_is_dense_swiglu_plus_shared()),
    # e2m1 weight pairs read high nibble first
    "nibble": ("(W[i / 2] >> (4 * (i & 1)))", "(W[i / 2] >> (4 * (1 - (i & 1))))",
               lambda: test_mx_layer_is_the_dense_swiglu_of_dequantised_operands("mxfp4", "e2m1")),
    # INT8 codes rounded half to even instead of half away from zero
    "i8round": ("return round(v);", "return rint(v);",
                lambda: test_quantize_rows_i8_rounds_half_away_from_zero()),
    # INT8 Linear1 dequantised without the per-token activation scale
    "i8scale": ("h1[n] = (double)acc[n] * (double)s_w1[n] * sx;",
                "h1[n] = (double)acc[n] * (double)s_w1[n];",
                lambda: test_int8_layer_is_the_dense_swiglu_of_dequantised_operands()),
    # SwiGLU backward without the A (1 - sigma(G)) term of SiLU's derivative
    "swiglu_bwd": ("dh1[n] = dA * (sg + act * (1.0 - sg));", "dh1[n] = dA * sg;",
                   lambda: bwd.test_expert_gradients_match_finite_differences()),
    # renormalised gate weights differentiated as if the sum were constant
    "renorm_bwd": ("da[e] += renorm ? alpha * (g / S - dGa / (S * S)) : alpha * g;",
                   "da[e] += renorm ? alpha * (g / S) : alpha * g;",
                   lambda: bwd.test_router_and_full_input_gradients_match_finite_differences(
                       "sigmoid", True, 2.5)),
    # permute backward keeping one copy's gradient instead of summing the k copies
    "permute_bwd": ("for (int c = 0; c < h; ++c) dxt[c] += dx[c];",
                    "for (int c = 0; c < h; ++c) dxt[c] = dx[c];",
                    lambda: bwd.test_expert_gradients_match_finite_differences()),
    # MX weight scale taken from the wrong group
    "mxscale": ("mx_pow2_table[S[(size_t)(c / 32) * N + n]]",
                "mx_pow2_table[S[(size_t)((c + 32) / 32 % (c / 32 + 1)) * N + n]]",
                lambda: test_mx_layer_is_the_dense_swiglu_of_dequantised_operands("mxfp8", "e4m3")),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_pins_catch_a_planted_mistake(tmp_path, name):
    """Build a copy of the oracle with a plausible slip planted and check that
    the pin for that part rejects it."""
    import ctypes
    import subprocess
    src = open(os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")).read()
    good, slip, pin = PLANTED[name]
    bad = src.replace(good, slip, 1)
    assert bad != src
    c = tmp_path / "bad.c"
    c.write_text(bad)
    so = tmp_path / "libbad.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"])
    saved = oracle._lib
    try:
        oracle._lib = None
        real = oracle._LIB_PATH
        oracle._LIB_PATH = str(so)
        with pytest.raises(AssertionError):
            pin()
    finally:
        oracle._LIB_PATH = real
        oracle._lib = saved
    del ctypes
