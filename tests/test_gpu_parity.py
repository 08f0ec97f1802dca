"""GPU parity: every entry point of the C ABI against the CPU oracle.

Cases are the workloads at sizes the oracle finishes in seconds that still
span several tiles in M, N and K and leave ragged tails (a hot expert with
more than one 128-row tile, experts with 0-3 rows, the shared segment).

Bars:
  - integers (expert ids, counts, offsets, row maps) and copies (Xp, the
    e4m3 codes of X and their scales): bit-exact;
  - expert ids from the router: exact at every token whose oracle top-k
    margin is >= 1e-5, and at every token equal to the oracle's selection
    re-run on the kernel's own fp32 keys (pure comparisons);
  - floating outputs: max over rows of ||y - y_ref||_inf / ||y_ref||_inf
    <= 1e-4 (fp32), 2e-2 (bf16), 5e-2 (A8W8 e4m3, against the oracle that
    applies the same quantisation steps).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import bits, f64, oracle_layer, oracle_route, row_rel_err

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2, "fp8": 5e-2, "int8": 2e-2, "mxfp8": 5e-2, "mxfp4": 5e-2}
DELTA = 1e-5

CASES = {
    "tiny_fp32": ("tiny_fp32", {}),
    "llama_small": ("llama_bf16", dict(T=512, hidden=256, experts=16, inter=128)),
    "v4pro_small": ("v4pro_bf16", dict(T=256, hidden=512, experts=64, inter=256)),
    "v4pro_fp8_small": ("v4pro_fp8", dict(T=256, hidden=512, experts=64, inter=256)),
    "v4pro_int8_small": ("v4pro_int8", dict(T=256, hidden=512, experts=64, inter=256)),
    "v4pro_mxfp8_small": ("v4pro_mxfp8", dict(T=256, hidden=512, experts=64, inter=256)),
    "v4pro_mxfp4_small": ("v4pro_mxfp4", dict(T=256, hidden=512, experts=64, inter=256)),
    # K = 1024 and 512: the MXFP4 kernels' 512-value scale windows, several per row
    "v4pro_mxfp4_k1024": ("v4pro_mxfp4", dict(T=200, hidden=1024, experts=64, inter=512)),
    "decode_hash_small": ("decode_hash_bf16", dict(T=16, hidden=512, experts=64, inter=256)),
    "decode_score_small": ("decode_score_bf16", dict(T=16, hidden=512, experts=64, inter=256)),
    "ep_share_small": ("ep_share_bf16", dict(T=600, hidden=256, inter=128)),
    # the DeepSeek-V4 affinity sqrt(softplus(l)) with the V4-Pro router
    "v4pro_sqrt_softplus_small": ("v4pro_bf16", dict(T=256, hidden=512, experts=64, inter=256,
                                                     score="sqrt_softplus")),
    # expert counts that take the DMA gate GEMM and the 16-lane top-k kernel
    # (E a multiple of 128): ragged token tiles, one and several K-splits,
    # every score function and hash routing
    "route_dma_e384": ("v4pro_bf16", dict(T=300, hidden=512, experts=384, inter=128)),
    "route_dma_e128_softmax": ("llama_bf16", dict(T=260, hidden=1024, experts=128, inter=128)),
    "route_dma_e256_sqrt_softplus": ("v4pro_bf16", dict(T=130, hidden=256, experts=256, inter=128,
                                                        zipf=False, score="sqrt_softplus")),
    "route_dma_e512": ("v4pro_bf16", dict(T=70, hidden=768, experts=512, topk=8, inter=128,
                                          zipf=False)),
    "decode_hash_e384": ("decode_hash_bf16", dict(T=20, hidden=512, experts=384, inter=128)),
    # 128-token gate blocks (T >= 4096), a ragged last block
    "route_dma_bm128": ("v4pro_bf16", dict(T=4100, hidden=256, experts=128, inter=128,
                                           zipf=False)),
    # the shape limits: top-16 (the most the ABI takes) over 512 experts on
    # the DMA router (32 experts per lane, a 32-bit taken mask), over 64
    # experts on the other router, and by hash
    "max_topk16_e512": ("v4pro_bf16", dict(T=96, hidden=512, experts=512, topk=16, inter=128,
                                           zipf=False)),
    "max_topk16_e64_softmax": ("llama_bf16", dict(T=128, hidden=256, experts=64, topk=16,
                                                  inter=128)),
    "max_topk16_hash": ("decode_hash_bf16", dict(T=24, hidden=512, experts=64, topk=16,
                                                 inter=128)),
}


def _log(msg):
    print(msg, flush=True)


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_cache = {}


def case(name):
    """(cpu inputs, gpu inputs, GpuLayer) of a named case, built once."""
    if name not in _cache:
        from tests.gpu_layer import GpuLayer, to_device
        wl, kw = CASES[name]
        cpu = synth.make_inputs(wl, **kw)
        gpu = to_device(cpu)
        _cache[name] = (cpu, gpu, GpuLayer(gpu))
    return _cache[name]


def check_route(cpu, ids_g, G_g, keys_g):
    wl = cpu["workload"]
    r = oracle_route(cpu)
    ids_g = ids_g.cpu().numpy()
    G_g = G_g.cpu().numpy()
    keys_g = keys_g.cpu().numpy()
    sure = r["margin"] >= DELTA
    assert np.array_equal(ids_g[sure], r["ids"][sure]), "selection differs at a clear margin"
    np.testing.assert_allclose(keys_g, r["keys"], atol=1e-5, rtol=0)
    if not wl.hash:
        ids_k, _ = oracle.topk(keys_g.astype(np.float64), wl.topk)
        assert np.array_equal(ids_g, ids_k), "selection is not the top-k of the kernel's keys"
    same = (ids_g == r["ids"]).all(axis=1)
    np.testing.assert_allclose(G_g[same], r["G"][same], atol=1e-5 * max(1.0, wl.alpha), rtol=1e-5)
    return r, int((~sure).sum())


@pytest.mark.parametrize("name", list(CASES))
def test_route(name):
    _need_gpu()
    cpu, gpu, L = case(name)
    _log(f"[route] {name} {cpu['workload']}")
    ids, G, keys = L.route()
    torch.cuda.synchronize()
    assert L.device_error() == 0
    _, near = check_route(cpu, ids, G, keys)
    _log(f"[route] {name}: near-tie tokens {near}")


@pytest.mark.parametrize("name", list(CASES))
def test_permute_bit_exact(name):
    _need_gpu()
    cpu, gpu, L = case(name)
    wl = cpu["workload"]
    r = oracle_route(cpu)
    _log(f"[permute] {name}")
    p = L.permute(torch.from_numpy(r["ids"]).cuda())
    torch.cuda.synchronize()
    assert L.device_error() == 0
    d = oracle.dispatch(r["ids"], wl.experts)
    for k in ("counts", "offsets", "dst_row", "src_tok"):
        assert np.array_equal(p[k].cpu().numpy(), d[k]), k
    if wl.precision == "mxfp4":
        q, s = oracle.mx_quantize(cpu["X"].double().numpy(), "e2m1")
        q = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)   # two codes per byte
        assert np.array_equal(bits(p["x_scale"]), s)
        assert np.array_equal(bits(p["Xq"]), q)
        assert np.array_equal(bits(p["Xp"]), q[d["src_tok"]])
        assert np.array_equal(bits(p["xp_scale"]), s[d["src_tok"]])
    elif wl.precision == "mxfp8":
        # bf16 inputs make the MX decision exact in any precision
        q, s = oracle.mx_quantize(cpu["X"].double().numpy(), "e4m3")
        assert np.array_equal(bits(p["x_scale"]), s)
        assert np.array_equal(bits(p["Xq"]), q)
        assert np.array_equal(bits(p["Xp"]), q[d["src_tok"]])
        assert np.array_equal(bits(p["xp_scale"]), s[d["src_tok"]])
    elif wl.precision in ("fp8", "int8"):
        quant = oracle.quantize_rows_f32 if wl.precision == "fp8" else oracle.quantize_rows_i8_f32
        q, s = quant(cpu["X"].float().numpy())
        assert np.array_equal(bits(p["x_scale"]), s)
        assert np.array_equal(bits(p["Xq"]), q)
        assert np.array_equal(bits(p["Xp"]), q[d["src_tok"]])
        assert np.array_equal(bits(p["xp_scale"]), s[d["src_tok"]])
    else:
        assert np.array_equal(bits(p["Xp"]), bits(cpu["X"])[d["src_tok"]])


@pytest.mark.parametrize("name", list(CASES))
def test_expert_ffn(name):
    _need_gpu()
    cpu, gpu, L = case(name)
    wl = cpu["workload"]
    r = oracle_route(cpu)
    _log(f"[expert_ffn] {name}")
    p = L.permute(torch.from_numpy(r["ids"]).cuda())
    Yp, Ys = L.expert_ffn(p)
    torch.cuda.synchronize()
    d = oracle.dispatch(r["ids"], wl.experts)
    OL = oracle_layer(cpu)
    ref = OL.expert_rows(d["offsets"], d["src_tok"])
    err = row_rel_err(f64(Yp), ref)
    _log(f"[expert_ffn] {name}: routed rel err {err:.3e}")
    assert err <= TOL[wl.precision]
    if wl.shared:
        n = wl.T * wl.topk
        ref_s = OL.expert_rows(d["offsets"], d["src_tok"], rows=np.arange(n, n + wl.T))
        err_s = row_rel_err(f64(Ys), ref_s)
        _log(f"[expert_ffn] {name}: shared rel err {err_s:.3e}")
        assert err_s <= TOL[wl.precision]


@pytest.mark.parametrize("name", list(CASES))
def test_combine(name):
    """Combine on the kernel's own Yp/Ys: against the oracle's combine of the
    same values (only the fp32 accumulation and the final rounding differ)."""
    _need_gpu()
    cpu, gpu, L = case(name)
    wl = cpu["workload"]
    r = oracle_route(cpu)
    _log(f"[combine] {name}")
    ids = torch.from_numpy(r["ids"]).cuda()
    G = torch.from_numpy(r["G"].astype(np.float32)).cuda()
    p = L.permute(ids)
    Yp, Ys = L.expert_ffn(p)
    Y = L.combine(Yp, p["dst_row"], G, Ys)
    torch.cuda.synchronize()
    ref = oracle.combine(f64(Yp), p["dst_row"].cpu().numpy(), r["G"].astype(np.float32),
                         f64(Ys) if Ys is not None else None)
    tol = 1e-5 if wl.precision == "fp32" else 8e-3  # one bf16 rounding of the sum
    assert row_rel_err(f64(Y), ref) <= tol


@pytest.mark.parametrize("name", list(CASES))
def test_forward(name):
    _need_gpu()
    cpu, gpu, L = case(name)
    wl = cpu["workload"]
    _log(f"[forward] {name}")
    Y, ids, G = L.forward()
    Y2, ids2, G2 = L.forward()
    torch.cuda.synchronize()
    assert L.device_error() == 0
    # deterministic: bit-identical on a second call
    assert torch.equal(ids, ids2) and torch.equal(G, G2)
    assert torch.equal(Y.view(torch.uint8), Y2.view(torch.uint8))
    r = oracle_route(cpu)
    ids_n = ids.cpu().numpy()
    same = (ids_n == r["ids"]).all(axis=1)
    assert same[r["margin"] >= DELTA].all()
    ref = oracle_layer(cpu).tokens(r["ids"], r["G"])
    err = row_rel_err(f64(Y)[same], ref[same])
    _log(f"[forward] {name}: rel err {err:.3e} over {same.sum()} tokens")
    assert err <= TOL[wl.precision]


@pytest.mark.parametrize("name", list(CASES))
def test_forward_matches_the_four_entry_points(name):
    """moe_forward against moe_route -> moe_permute -> moe_expert_ffn ->
    moe_combine on the same inputs: bit-identical.  Where the shape allows it
    (bf16 on the DMA GEMM), moe_forward writes no permuted rows and Linear1
    reads the token rows of X through the row -> token map instead, which
    must change no bit."""
    _need_gpu()
    cpu, gpu, L = case(name)
    _log(f"[forward vs staged] {name}")
    ids, G, _ = L.route()
    p = L.permute(ids)
    Yp, Ys = L.expert_ffn(p)
    Y_staged = L.combine(Yp, p["dst_row"], G, Ys)
    Y, ids_f, G_f = L.forward()
    torch.cuda.synchronize()
    assert L.device_error() == 0
    assert torch.equal(ids_f, ids) and torch.equal(G_f, G)
    assert torch.equal(Y.view(torch.uint8), Y_staged.view(torch.uint8))


@pytest.mark.parametrize("name", ["v4pro_small", "tiny_fp32", "v4pro_fp8_small",
                                  "v4pro_int8_small", "v4pro_mxfp8_small", "v4pro_mxfp4_small"])
def test_forward_with_given_routing(name):
    """The mega_moe form: expert ids and weights are inputs (no router)."""
    _need_gpu()
    cpu, gpu, L = case(name)
    wl = cpu["workload"]
    rng = np.random.default_rng(21)
    ids = np.stack([rng.choice(wl.experts, wl.topk, replace=False)
                    for _ in range(wl.T)]).astype(np.int32)
    G = rng.random((wl.T, wl.topk)).astype(np.float32)
    _log(f"[forward given routing] {name}")
    Y, _, _ = L.forward(torch.from_numpy(ids).cuda(), torch.from_numpy(G).cuda(), route=False)
    torch.cuda.synchronize()
    ref = oracle_layer(cpu).tokens(ids, G.astype(np.float64))
    assert row_rel_err(f64(Y), ref) <= TOL[wl.precision]


# ------------------------------------------------------------------ edge cases
def _edge(base, ids=None, **kw):
    from tests.gpu_layer import GpuLayer, to_device
    cpu = synth.make_inputs(base, **kw)
    gpu = to_device(cpu)
    return cpu, GpuLayer(gpu)


@pytest.mark.parametrize("kind", ["one_token", "all_to_one_expert", "k_equals_E", "single_expert",
                                  "fp8_all_to_one", "int8_all_to_one", "int8_decode",
                                  "mxfp8_all_to_one", "mxfp8_decode",
                                  "mxfp4_all_to_one", "mxfp4_decode",
                                  "decode_one_token", "bf16_wide_tiles", "fp8_wide_tiles",
                                  "int8_wide_tiles", "mxfp8_wide_tiles"])
def test_edge_cases(kind):
    _need_gpu()
    spec = {
        "one_token": ("v4pro_bf16", dict(T=1, hidden=256, experts=64, inter=128)),
        "all_to_one_expert": ("v4pro_bf16", dict(T=300, hidden=256, experts=64, inter=128, topk=1,
                                                  zipf=False)),
        "k_equals_E": ("tiny_fp32", dict(T=40, experts=4, topk=4)),
        "single_expert": ("llama_bf16", dict(T=200, hidden=128, experts=1, topk=1, inter=64)),
        "fp8_all_to_one": ("v4pro_fp8", dict(T=300, hidden=256, experts=64, inter=128, topk=1,
                                              zipf=False)),
        "int8_all_to_one": ("v4pro_int8", dict(T=300, hidden=256, experts=64, inter=128, topk=1,
                                                zipf=False)),
        "int8_decode": ("v4pro_int8", dict(T=3, hidden=512, experts=64, inter=256)),
        "mxfp8_all_to_one": ("v4pro_mxfp8", dict(T=300, hidden=256, experts=64, inter=128,
                                                  topk=1, zipf=False)),
        "mxfp8_decode": ("v4pro_mxfp8", dict(T=3, hidden=512, experts=64, inter=256)),
        "mxfp4_all_to_one": ("v4pro_mxfp4", dict(T=300, hidden=256, experts=64, inter=128,
                                                  topk=1, zipf=False)),
        "mxfp4_decode": ("v4pro_mxfp4", dict(T=3, hidden=512, experts=64, inter=256)),
        "decode_one_token": ("decode_hash_bf16", dict(T=1, hidden=256, experts=64, inter=128)),
        # 128 x 512 tiles: two n-tiles per linear, K of 1024 and 512, Zipf load
        # (the hottest expert holds 4 m-tiles, the last one ragged)
        "bf16_wide_tiles": ("v4pro_bf16", dict(T=512, hidden=1024, experts=64, inter=512)),
        "fp8_wide_tiles": ("v4pro_fp8", dict(T=512, hidden=1024, experts=64, inter=512)),
        "int8_wide_tiles": ("v4pro_int8", dict(T=512, hidden=1024, experts=64, inter=512)),
        "mxfp8_wide_tiles": ("v4pro_mxfp8", dict(T=512, hidden=1024, experts=64, inter=512)),
    }[kind]
    cpu, L = _edge(spec[0], **spec[1])
    wl = cpu["workload"]
    _log(f"[edge] {kind} {wl}")
    if kind in ("all_to_one_expert", "fp8_all_to_one", "int8_all_to_one", "mxfp8_all_to_one",
                "mxfp4_all_to_one"):
        ids = np.full((wl.T, 1), 37, np.int32)       # 300 rows: 3 tiles, ragged
        G = np.full((wl.T, 1), 0.75, np.float32)
        Y, _, _ = L.forward(torch.from_numpy(ids).cuda(), torch.from_numpy(G).cuda(), route=False)
        torch.cuda.synchronize()
        ref = oracle_layer(cpu).tokens(ids, G.astype(np.float64))
    else:
        Y, ids_g, G_g = L.forward()
        torch.cuda.synchronize()
        r = oracle_route(cpu)
        assert np.array_equal(ids_g.cpu().numpy()[r["margin"] >= DELTA],
                              r["ids"][r["margin"] >= DELTA])
        ref = oracle_layer(cpu).tokens(r["ids"], r["G"])
    assert L.device_error() == 0
    assert row_rel_err(f64(Y), ref) <= TOL[wl.precision]


def test_bad_expert_ids_are_flagged_and_skipped():
    _need_gpu()
    cpu, gpu, L = case("v4pro_small")
    wl = cpu["workload"]
    ids = oracle_route(cpu)["ids"].copy()
    ids[3, 1] = wl.experts      # out of range
    ids[7, 0] = -2
    _log("[bad ids] permute with two invalid ids")
    p = L.permute(torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    assert L.device_error() == -5
    assert L.device_error() == 0          # the check clears the flag
    d = oracle.dispatch(ids, wl.experts)
    assert d["bad"] == 2
    for k in ("counts", "offsets", "dst_row"):
        assert np.array_equal(p[k].cpu().numpy(), d[k]), k
    n_ok = wl.T * wl.topk - 2
    assert np.array_equal(p["src_tok"].cpu().numpy()[:n_ok], d["src_tok"][:n_ok])


def test_bad_token_ids_are_flagged():
    _need_gpu()
    cpu, gpu, L = case("decode_hash_small")
    tok = gpu["token_ids"].clone()
    tok[2] = synth.VOCAB + 5
    import mixture_experts_layer_09_amd as moe
    wl = cpu["workload"]
    opts = moe.make_route_opts(wl.score, wl.renorm, wl.alpha, None, None, tok, gpu["tid2eid"])
    ids = torch.empty((wl.T, wl.topk), dtype=torch.int32, device="cuda")
    G = torch.empty((wl.T, wl.topk), dtype=torch.float32, device="cuda")
    _log("[bad token id] hash route")
    moe.moe_route(L.shape, opts, gpu["X"], gpu["Wg"], ids, G, None, L.ws)
    torch.cuda.synchronize()
    assert L.device_error() == -5
    assert (ids[2] == -1).all() and (G[2] == 0).all()
    assert (ids[3] >= 0).all()
    # moe_forward reports its router's bad token id too (it covers all its
    # steps), and a clean call afterwards clears the flag again
    Y = torch.empty((wl.T, wl.hidden), dtype=torch.bfloat16, device="cuda")
    _log("[bad token id] hash forward")
    moe.moe_forward(L.shape, opts, gpu["X"], gpu["Wg"], L.weights, ids, G, Y, L.ws)
    torch.cuda.synchronize()
    assert L.device_error() == -5
    moe.moe_route(L.shape, L.opts, gpu["X"], gpu["Wg"], ids, G, None, L.ws)
    torch.cuda.synchronize()
    assert L.device_error() == 0
