"""Small test helpers: torch tensors <-> the oracle's raw-bits numpy arrays."""
from __future__ import annotations

import numpy as np
import torch


def bits(t: torch.Tensor | None) -> np.ndarray | None:
    """Host numpy array of a tensor's raw elements (bf16 -> uint16, fp8 -> uint8)."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def f64(t: torch.Tensor | None) -> np.ndarray | None:
    if t is None:
        return None
    return t.detach().cpu().to(torch.float64).numpy()


def oracle_layer(inp: dict):
    """oracle.Layer of a synth input dict."""
    import oracle
    wl = inp["workload"]
    return oracle.Layer(wl.precision, bits(inp["X"]), bits(inp["W1"]), bits(inp["W2"]),
                        w1_scale=bits(inp["w1_scale"]), w2_scale=bits(inp["w2_scale"]),
                        Ws1=bits(inp["Ws1"]), Ws2=bits(inp["Ws2"]),
                        ws1_scale=bits(inp["ws1_scale"]), ws2_scale=bits(inp["ws2_scale"]),
                        k=wl.topk)


def oracle_route(inp: dict, **kw) -> dict:
    import oracle
    wl = inp["workload"]
    return oracle.route(bits(inp["X"]), bits(inp["Wg"]), wl.topk, gate_bias=f64(inp["gate_bias"]),
                        beta=f64(inp["beta"]), score=wl.score, renorm=wl.renorm, alpha=wl.alpha,
                        token_ids=bits(inp["token_ids"]), tid2eid=bits(inp["tid2eid"]), **kw)


def row_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max_t ||y[t] - ref[t]||_inf / max(||ref[t]||_inf, 1e-30)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(y - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max()) if len(num) else 0.0
