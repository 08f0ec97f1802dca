"""Write the per-expert gating-bias fixtures that give Zipf(0.8) expert load.

The pages name no load distribution for the skewed V4-Pro workload; the
benchmark asks for expert frequencies that follow Zipf(s = 0.8).  The skew is
made with an ordinary bias of the gating linear (distinct from the
selection-only expert bias beta, as the DeepSeek-V4 blog post's §路由张量
separates the two).  The bias is found here, once, by a fixed damped
iteration on a seeded calibration batch:

    b <- b + 0.5 * (ln p_target - ln p_observed)

where p_observed[e] is the fraction of tokens whose top-k (by the CPU
oracle's router: sigmoid affinity, + beta, top-k) contains e, and p_target is
k * r^-0.8 / sum_r r^-0.8 over a seeded permutation of expert ranks r.

Only the CPU oracle computes routing here.  Run from the repository root:
    python tests/golden/make_zipf_gate_bias.py
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

S = 0.8
STEPS = 50
CAL_TOKENS = 8192


def _bits(t: torch.Tensor) -> np.ndarray:
    """A CPU tensor as the oracle's raw-bits numpy form."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def calibrate(wl: synth.Workload, cal_tokens: int = CAL_TOKENS, steps: int = STEPS):
    seed = synth.workload_seed(wl)
    E, k, h = wl.experts, wl.topk, wl.hidden
    dt = torch.float32 if wl.precision == "fp32" else torch.bfloat16
    # gate weight and beta exactly as the workload draws them (CPU, seeded)
    Wg = synth.normal((h, E), 1.0 / np.sqrt(h), seed=seed, name="Wg", dtype=dt)
    beta = synth.uniform((E,), -wl.beta_range, wl.beta_range, seed=seed, name="beta").numpy()
    Xc = synth.normal((cal_tokens, h), 1.0, seed=seed, name="Xcal", dtype=dt)
    z = oracle.gate_logits(_bits(Xc), _bits(Wg))
    rng = np.random.default_rng(seed)
    rank = rng.permutation(E) + 1
    w = rank.astype(np.float64) ** -S
    p_target = k * w / w.sum()
    b = np.zeros(E)
    for _ in range(steps):
        a = oracle.affinity(z + b[None, :], wl.score)
        ids, _ = oracle.topk(a + beta[None, :], k)
        cnt = np.bincount(ids.ravel(), minlength=E)
        p_obs = (cnt + 0.5) / cal_tokens
        b = b + 0.5 * (np.log(p_target) - np.log(p_obs))
    a = oracle.affinity(z + b[None, :], wl.score)
    ids, _ = oracle.topk(a + beta[None, :], k)
    cnt = np.bincount(ids.ravel(), minlength=E)
    return b.astype(np.float32), cnt, p_target * cal_tokens


def main():
    jobs = [synth.WORKLOADS["v4pro_bf16"],
            synth.WORKLOADS["v4pro_bf16"].replace(hidden=512, experts=64, inter=256)]
    for wl in jobs:
        b, cnt, tgt = calibrate(wl)
        path = synth.zipf_fixture_path(wl.experts, wl.topk)
        order = np.argsort(-tgt)
        with open(path, "w") as fh:
            fh.write(f"# gating bias for Zipf({S}) load, E={wl.experts} k={wl.topk} "
                     f"hidden={wl.hidden}; written by make_zipf_gate_bias.py\n")
            fh.write(f"# calibration batch of {CAL_TOKENS} tokens: max count {cnt.max()} "
                     f"(target {tgt.max():.0f}), min count {cnt.min()} (target {tgt.min():.0f})\n")
            for v in b:
                fh.write(f"{v:.7g}\n")
        print(path, "max", cnt.max(), "min", cnt.min(), "top5", cnt[order[:5]],
              "tgt", np.round(tgt[order[:5]]))


if __name__ == "__main__":
    main()
