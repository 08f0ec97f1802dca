"""moe_permute_no_alloc (the dispatch with the library's static scratch
instead of a workspace) against moe_permute, through the C ABI.

Two calls in a row on one GPU, the second with fewer tokens and fewer
per-block count rows than the first, in bf16 and in the quantised e4m3
layout: every output (counts, offsets, row maps, the copied or quantised
rows and their scales) bit-identical to moe_permute's on the same ids, and
both equal to the oracle's dispatch; the same at exactly the scratch's limit
(over 512 experts).  A call larger than the scratch is refused on the host.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_09_amd as moe
import oracle
import synth
from tests.gpu_layer import GpuLayer, to_device
from tests.helpers import bits

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _outputs(L, like):
    return {k: (torch.empty_like(v) if v is not None else None) for k, v in like.items()}


@pytest.mark.parametrize("base", ["v4pro_bf16", "v4pro_fp8"])
def test_no_alloc_permute_equals_moe_permute(base):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call: 3000 tokens x 6 = 18000 assignments (9 count blocks); the
    # second: 100 tokens (one block), so stale rows of the first would show
    for T in (3000, 100):
        cpu = synth.make_inputs(base, T=T, hidden=512, experts=64, inter=256)
        wl = cpu["workload"]
        L = GpuLayer(to_device(cpu))
        ids_np = oracle.route(bits(cpu["X"]), bits(cpu["Wg"]), wl.topk,
                              gate_bias=cpu["gate_bias"].double().numpy(),
                              beta=cpu["beta"].double().numpy(), score=wl.score,
                              renorm=wl.renorm, alpha=wl.alpha)["ids"].copy()
        ids_np[5, 2] = wl.experts       # one id out of range: skipped by both
        ids = torch.from_numpy(ids_np).cuda()
        _log(f"[no-alloc] {base} T={T}: moe_permute, then moe_permute_no_alloc")
        ref = L.permute(ids)
        out = _outputs(L, ref)
        moe.moe_permute_no_alloc(L.shape, ids, L.inp["X"], out["counts"], out["offsets"],
                                 out["dst_row"], out["src_tok"], out["Xp"], out["xp_scale"],
                                 out["Xq"], out["x_scale"])
        torch.cuda.synchronize()
        n = int(ref["offsets"][-1].item())   # valid rows: the skipped id writes none
        assert n == T * wl.topk - 1
        for k, v in ref.items():
            if v is None:
                continue
            if k in ("src_tok", "Xp", "xp_scale"):   # per dispatched row
                assert torch.equal(out[k][:n].view(torch.uint8), v[:n].view(torch.uint8)), k
                continue
            assert torch.equal(out[k].view(torch.uint8), v.view(torch.uint8)), k
        d = oracle.dispatch(ids_np, wl.experts)
        for k in ("counts", "offsets", "dst_row"):
            assert np.array_equal(out[k].cpu().numpy(), d[k]), k
        assert L.device_error() == -5      # moe_permute's workspace saw the bad id


def test_no_alloc_permute_at_its_limit():
    """Exactly MOE_NO_ALLOC_MAX_ASSIGNMENTS assignments over the most experts
    the ABI takes (512): the scratch's per-block count table and rank array
    are full."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    k, E, h = 8, 512, 128
    T = moe.NO_ALLOC_MAX_ASSIGNMENTS // k
    assert T * k == moe.NO_ALLOC_MAX_ASSIGNMENTS
    g = torch.Generator().manual_seed(20260)
    ids_cpu = torch.randint(0, E, (T, k), generator=g, dtype=torch.int32)
    X = torch.randn((T, h), generator=g).to(torch.bfloat16).cuda()
    ids = ids_cpu.cuda()
    shape = moe.make_shape(T, h, E, k, 64, 0, "bf16")
    ws = moe.alloc_workspace(shape)
    n = T * k

    def bufs():
        i32 = dict(dtype=torch.int32, device="cuda")
        return dict(counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                    dst_row=torch.empty(n, **i32), src_tok=torch.empty(n, **i32),
                    Xp=torch.empty((n, h), dtype=torch.bfloat16, device="cuda"))

    _log(f"[no-alloc] at the limit: T={T} k={k} E={E}: moe_permute, then moe_permute_no_alloc")
    ref, out = bufs(), bufs()
    moe.moe_permute(shape, ids, X, ref["counts"], ref["offsets"], ref["dst_row"], ref["src_tok"],
                    ref["Xp"], None, None, None, ws)
    moe.moe_permute_no_alloc(shape, ids, X, out["counts"], out["offsets"], out["dst_row"],
                             out["src_tok"], out["Xp"], None, None, None)
    torch.cuda.synchronize()
    for key in ref:
        assert torch.equal(out[key].view(torch.uint8), ref[key].view(torch.uint8)), key
    d = oracle.dispatch(ids_cpu.numpy(), E)
    for key in ("counts", "offsets", "dst_row", "src_tok"):
        assert np.array_equal(out[key].cpu().numpy(), d[key]), key
    assert moe.moe_check_device_error(ws) == 0


def test_no_alloc_permute_refuses_more_than_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T = moe.NO_ALLOC_MAX_ASSIGNMENTS // 4 + 1
    shape = moe.make_shape(T, 128, 8, 4, 64, 0, "bf16")
    fake = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_permute_no_alloc(shape, fake, fake, fake, fake, fake, fake, fake, None, None,
                                 None)
    assert e.value.status == -6
