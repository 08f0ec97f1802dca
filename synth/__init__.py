"""Seeded synthetic inputs for the routed MoE layer.

This module only draws random tensors of the shapes and distributions of the
workloads; it computes none of the layer's arithmetic.  Both the HIP path and
the CPU oracle take their inputs from here (the oracle through host copies of
the same tensors).

Workloads (T tokens, hidden h, E routed experts, top-k, inter f, shared S):
  tiny_fp32          64, 128, 8, 2, 64, 0      fp32, sigmoid, renorm, alpha 1
  llama_bf16         8192, 8192, 64, 2, 4096, 0  bf16, softmax top-2, raw weights
  v4pro_bf16         8192, 7168, 384, 6, 3072, 1 bf16, sigmoid + beta, alpha 2.5,
                                                 Zipf(0.8) expert load
  v4pro_fp8          as v4pro_bf16, A8W8 e4m3 experts, bf16 output
  v4pro_int8         as v4pro_bf16, A8W8 INT8 experts (the page's INT8 block)
  v4pro_mxfp8        as v4pro_bf16, MXFP8 experts (e4m3, group-32 E8M0 scales)
  v4pro_mxfp4        as v4pro_bf16, MXFP4 experts (e2m1, group-32 E8M0 scales)
  decode_hash_bf16   128, 7168, 384, 6, 3072, 1  token-id hash routing
  decode_score_bf16  128, v4pro router
  ep_share_bf16      4096, 7168, 6, 6, 3072, 0   one GPU's expert-parallel share
                                                 (6 experts x 4096 rows)

Distributions: X ~ N(0,1); gate weight N(0, std) with the std each workload
names (0.02 for tiny, else 1/sqrt(h)); W1 ~ N(0, 1/sqrt(h)), W2 ~ N(0,
1/sqrt(f)); expert bias beta ~ U(-0.1, 0.1) where used.  The Zipf load of the
V4-Pro workloads comes from an ordinary per-expert gating bias read from a
fixture under tests/golden (written by a script that runs the CPU oracle's
router on a calibration batch).  bf16 values are drawn in fp32 and rounded to
nearest even by torch.  fp8 expert weights are quantised offline per output
channel: scale = max|W[:, n]| / 448, codes = torch's float8_e4m3fn cast of
W / scale; INT8 ones the same way with 127 and W / scale rounded half away
from zero.  MXFP8 expert weights are quantised offline in groups of 32 rows
(K) per column: E8M0 scale code = floor(log2 max|W|) - 8 + 127 (0 for a zero
group), codes = torch's float8_e4m3fn cast of W * 2^(127 - code) clamped to
+-448.  MXFP4 weights the same way with exponent floor(log2 max|W|) - 2 and
e2m1 codes (nearest even, saturating at 6), stored K-contiguous: codes
[N, K/2] (element 2i of a row in the low nibble), scales [N, K/32].  Hash
tables hold k distinct expert ids per token id.
"""
from __future__ import annotations

import dataclasses
import math
import os
import zlib

import numpy as np
import torch

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(_ROOT, "tests", "golden")
VOCAB = 129280
BASE_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    hidden: int
    experts: int
    topk: int
    inter: int
    shared: int
    precision: str          # fp32 | bf16 | fp8 | int8 | mxfp8 | mxfp4
    score: str = "sigmoid"  # sigmoid | softmax | sqrt_softplus
    renorm: bool = True
    alpha: float = 1.0
    gate_std: float | None = None   # None: 1/sqrt(hidden)
    beta_range: float = 0.0         # beta ~ U(-r, r); 0: no expert bias
    zipf: bool = False              # gating bias from the Zipf fixture
    hash: bool = False              # token-id table routing
    family: str = ""                # workloads of one family share seeds (weights)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def params_per_expert(self) -> int:
        return 3 * self.hidden * self.inter


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 64, 128, 8, 2, 64, 0, "fp32", gate_std=0.02),
        Workload("llama_bf16", 8192, 8192, 64, 2, 4096, 0, "bf16", score="softmax",
                 renorm=False),
        Workload("v4pro_bf16", 8192, 7168, 384, 6, 3072, 1, "bf16", alpha=2.5, beta_range=0.1,
                 zipf=True, family="v4pro"),
        Workload("v4pro_fp8", 8192, 7168, 384, 6, 3072, 1, "fp8", alpha=2.5, beta_range=0.1,
                 zipf=True, family="v4pro"),
        Workload("v4pro_int8", 8192, 7168, 384, 6, 3072, 1, "int8", alpha=2.5, beta_range=0.1,
                 zipf=True, family="v4pro"),
        Workload("v4pro_mxfp8", 8192, 7168, 384, 6, 3072, 1, "mxfp8", alpha=2.5,
                 beta_range=0.1, zipf=True, family="v4pro"),
        Workload("v4pro_mxfp4", 8192, 7168, 384, 6, 3072, 1, "mxfp4", alpha=2.5,
                 beta_range=0.1, zipf=True, family="v4pro"),
        Workload("decode_hash_bf16", 128, 7168, 384, 6, 3072, 1, "bf16", alpha=2.5, hash=True,
                 family="v4pro"),
        Workload("decode_score_bf16", 128, 7168, 384, 6, 3072, 1, "bf16", alpha=2.5,
                 beta_range=0.1, zipf=True, family="v4pro"),
        Workload("ep_share_bf16", 4096, 7168, 6, 6, 3072, 0, "bf16", alpha=1.0),
    ]
}


def zipf_fixture_path(experts: int, topk: int) -> str:
    return os.path.join(GOLDEN, f"zipf_gate_bias_E{experts}_k{topk}.txt")


def load_zipf_gate_bias(experts: int, topk: int) -> np.ndarray:
    """Per-expert gating bias that gives Zipf(0.8) expert load (fixture)."""
    path = zipf_fixture_path(experts, topk)
    lines = [ln.strip() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    arr = np.array([float(v) for v in lines], dtype=np.float32)
    assert arr.shape == (experts,), (path, arr.shape)
    return arr


def workload_seed(wl: Workload) -> int:
    """Seed of a workload: one per family (so the V4-Pro workloads share their
    router and expert weights), else one per workload name."""
    key = wl.family or wl.name
    return BASE_SEED + zlib.crc32(key.encode()) % 100000


def _seed(seed: int, name: str) -> int:
    return (seed * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFFFFFF


def _gen(device, seed, name):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, name))
    return g


def normal(shape, std, *, seed, name, device="cpu", dtype=torch.float32):
    g = _gen(device, seed, name)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(dtype)


def uniform(shape, lo, hi, *, seed, name, device="cpu"):
    g = _gen(device, seed, name)
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def quantize_weight_e4m3(W: torch.Tensor):
    """Offline per-output-channel e4m3 quantisation of a [.., K, N] weight.

    scale[.., n] = max_k |W[.., k, n]| / 448 (1 where the column is zero);
    codes = float8_e4m3fn cast of W / scale (torch's conversion)."""
    Wf = W.float()
    amax = Wf.abs().amax(dim=-2)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (Wf / scale.unsqueeze(-2)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q, scale.float()


def quantize_weight_i8(W: torch.Tensor):
    """Offline per-output-channel INT8 quantisation of a [.., K, N] weight.

    scale[.., n] = max_k |W[.., k, n]| / 127 (1 where the column is zero);
    codes = W / scale rounded half away from zero (in fp64), int8 in
    [-127, 127]."""
    Wf = W.double()
    amax = Wf.abs().amax(dim=-2)
    scale = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax))
    v = Wf / scale.unsqueeze(-2)
    q = torch.trunc(v + torch.copysign(torch.full_like(v, 0.5), v)).clamp_(-127, 127)
    return q.to(torch.int8), scale.float()


def quantize_weight_mx_e4m3(W: torch.Tensor):
    """Offline MXFP8 quantisation of a [K, N] weight (K a multiple of 32):
    codes [K, N] e4m3fn and E8M0 scale codes [K/32, N] uint8 (see the module
    docstring)."""
    Wf = W.float()
    K, N = Wf.shape
    g = Wf.reshape(K // 32, 32, N)
    amax = g.abs().amax(dim=1)
    _, ex = torch.frexp(amax)                        # amax = m * 2^ex, m in [0.5, 1)
    code = torch.where(amax > 0, (ex - 1 - 8 + 127).clamp(0, 254), torch.zeros_like(ex))
    q = torch.ldexp(g, (127 - code).unsqueeze(1).to(torch.float32))
    q = q.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).reshape(K, N)
    return q, code.to(torch.uint8)


_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def quantize_weight_mx_e2m1(W: torch.Tensor):
    """Offline MXFP4 quantisation of a [K, N] weight (K a multiple of 32),
    stored K-contiguous: code pairs [N, K/2] uint8 and E8M0 scale codes
    [N, K/32] uint8 (see the module docstring)."""
    Wt = W.float().t().contiguous()                  # [N, K]
    N, K = Wt.shape
    g = Wt.reshape(N, K // 32, 32)
    amax = g.abs().amax(dim=2)
    _, ex = torch.frexp(amax)
    code = torch.where(amax > 0, (ex - 1 - 2 + 127).clamp(0, 254), torch.zeros_like(ex))
    v = torch.ldexp(g, (127 - code).unsqueeze(2).to(torch.float32)).reshape(N, K)
    a = v.abs()
    mag = torch.zeros_like(a, dtype=torch.uint8)
    # nearest of 0, .5, 1, 1.5, 2, 3, 4, 6; midpoints go to the even code
    for i, m in enumerate(_E2M1_MIDPOINTS):
        up = (a > m) if i % 2 == 0 else (a >= m)
        mag += up.to(torch.uint8)
    nib = mag | (torch.signbit(v).to(torch.uint8) << 3)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).to(torch.uint8)
    return packed, code.to(torch.uint8)


def _expert_weights(wl: Workload, seed, device, act_dtype):
    """W1 [E,h,2f], W2 [E,f,h] (bf16/fp32), generated one expert at a time."""
    E, h, f = wl.experts, wl.hidden, wl.inter
    fp8 = wl.precision == "fp8"
    i8 = wl.precision == "int8"
    mx = wl.precision == "mxfp8"
    mx4 = wl.precision == "mxfp4"
    wdt = torch.float8_e4m3fn if (fp8 or mx) else (torch.int8 if i8 else act_dtype)
    if mx4:   # K-contiguous e2m1 pairs
        W1 = torch.empty((E, 2 * f, h // 2), dtype=torch.uint8, device=device)
        W2 = torch.empty((E, h, f // 2), dtype=torch.uint8, device=device)
    else:
        W1 = torch.empty((E, h, 2 * f), dtype=wdt, device=device)
        W2 = torch.empty((E, f, h), dtype=wdt, device=device)
    s1 = s2 = None
    if mx4:
        s1 = torch.empty((E, 2 * f, h // 32), dtype=torch.uint8, device=device)
        s2 = torch.empty((E, h, f // 32), dtype=torch.uint8, device=device)
    if fp8 or i8:
        s1 = torch.empty((E, 2 * f), dtype=torch.float32, device=device)
        s2 = torch.empty((E, h), dtype=torch.float32, device=device)
    if mx:
        s1 = torch.empty((E, h // 32, 2 * f), dtype=torch.uint8, device=device)
        s2 = torch.empty((E, f // 32, h), dtype=torch.uint8, device=device)
    for e in range(E):
        w1 = normal((h, 2 * f), 1.0 / math.sqrt(h), seed=seed, name=f"W1.{e}", device=device,
                    dtype=act_dtype)
        w2 = normal((f, h), 1.0 / math.sqrt(f), seed=seed, name=f"W2.{e}", device=device,
                    dtype=act_dtype)
        if mx4:
            W1[e], s1[e] = quantize_weight_mx_e2m1(w1)
            W2[e], s2[e] = quantize_weight_mx_e2m1(w2)
        elif mx:
            W1[e], s1[e] = quantize_weight_mx_e4m3(w1)
            W2[e], s2[e] = quantize_weight_mx_e4m3(w2)
        elif fp8:
            W1[e], s1[e] = quantize_weight_e4m3(w1)
            W2[e], s2[e] = quantize_weight_e4m3(w2)
        elif i8:
            W1[e], s1[e] = quantize_weight_i8(w1)
            W2[e], s2[e] = quantize_weight_i8(w2)
        else:
            W1[e] = w1
            W2[e] = w2
    return W1, W2, s1, s2


def make_inputs(wl: Workload | str, *, device="cpu", seed: int | None = None, **override) -> dict:
    """All inputs of one layer invocation, as torch tensors on `device`.

    Small per-expert/per-token vectors (beta, gating bias, token ids, hash
    table, gate weight, X) are drawn on the CPU so that they do not depend on
    the device; the expert weights are drawn on `device`.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if override:
        wl = wl.replace(**override)
    if seed is None:
        seed = workload_seed(wl)
    act_dtype = torch.float32 if wl.precision == "fp32" else torch.bfloat16
    T, h, E, k, f = wl.T, wl.hidden, wl.experts, wl.topk, wl.inter
    gate_std = wl.gate_std if wl.gate_std is not None else 1.0 / math.sqrt(h)
    out = {"workload": wl, "seed": seed}
    out["X"] = normal((T, h), 1.0, seed=seed, name="X", dtype=act_dtype).to(device)
    out["Wg"] = normal((h, E), gate_std, seed=seed, name="Wg", dtype=act_dtype).to(device)
    out["beta"] = (uniform((E,), -wl.beta_range, wl.beta_range, seed=seed, name="beta").to(device)
                   if wl.beta_range > 0 else None)
    out["gate_bias"] = (torch.from_numpy(load_zipf_gate_bias(E, k)).to(device)
                        if wl.zipf else None)
    if wl.hash:
        g = _gen("cpu", seed, "tid2eid")
        tab = torch.multinomial(torch.ones(VOCAB, E), k, replacement=False, generator=g)
        out["tid2eid"] = tab.to(torch.int32).to(device)
        g = _gen("cpu", seed, "token_ids")
        out["token_ids"] = torch.randint(0, VOCAB, (T,), generator=g, dtype=torch.int32).to(device)
    else:
        out["tid2eid"] = None
        out["token_ids"] = None
    W1, W2, s1, s2 = _expert_weights(wl, seed, device, act_dtype)
    out.update(W1=W1, W2=W2, w1_scale=s1, w2_scale=s2)
    if wl.shared:
        sh = wl.replace(experts=1)
        Ws1, Ws2, ss1, ss2 = _expert_weights(sh, seed + 7919, device, act_dtype)
        out.update(Ws1=Ws1[0], Ws2=Ws2[0], ws1_scale=None if ss1 is None else ss1[0],
                   ws2_scale=None if ss2 is None else ss2[0])
    else:
        out.update(Ws1=None, Ws2=None, ws1_scale=None, ws2_scale=None)
    return out
