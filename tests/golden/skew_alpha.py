"""Writes skew_alpha.json: the skew strength alpha of the skewed-routing workload for each
routing configuration of the workloads.

The workload (aiter MI308 decoding PR, Performance, "Skewed routing") adds a fixed per-expert
bias -alpha * log(1 + rank) to the router scores (moe_harness.workloads.skew_bias), with alpha
chosen so that over many tokens the most popular expert receives twice the mean load.  This
script finds that alpha by bisection: seeded N(0,1) gating for many tokens, the oracle's
routing (oracle.route) of the skewed scores, the largest expert load over the mean load.  A
routing whose own load is already above twice the mean at alpha = 0 (sigmoid scores with an
N(0, 0.1^2) correction bias) gets alpha 0 and its ratio is recorded.

Test infrastructure: calls only oracle/ and the input generators.
    python tests/golden/skew_alpha.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from moe_harness.workloads import CONFIGS, make_inputs, skew_bias  # noqa: E402

TOKENS = 32768
SEED = 7
TARGET = 2.0
OUT = os.path.join(HERE, "skew_alpha.json")


def routing_key(cfg):
    return "%s E=%d k=%d groups=%d/%d bias=%d" % (cfg.scoring, cfg.E, cfg.k, cfg.num_expert_group,
                                                  cfg.topk_group, int(cfg.bias))


def load_ratio(cfg, gating, bias, alpha):
    g = gating + skew_bias(cfg.E, alpha).numpy()          # float64 sum
    g = g.astype(np.float32)                              # rounded to f32 once
    ids, _ = oracle.route(g, bias, cfg.k, cfg.scoring, cfg.renormalize, cfg.num_expert_group,
                          cfg.topk_group, float(np.float32(cfg.rsf)))
    load = np.bincount(ids.ravel(), minlength=cfg.E)
    return float(load.max() / load.mean())


def main():
    table = {}
    for name in ("qwen3-30b-decode", "qwen3-235b-batch", "ds-v3-grouped-prefill",
                 "kimi-k2-shared"):
        cfg = CONFIGS[name]
        key = routing_key(cfg)
        if key in table:
            table[key]["workloads"].append(name)
            continue
        d = make_inputs(cfg, "cpu", seed=SEED, weights=False, num_tokens=TOKENS)
        gating = d["gating_output"].numpy().astype(np.float64)
        bias = None if d["correction_bias"] is None else d["correction_bias"].numpy()
        r0 = load_ratio(cfg, gating, bias, 0.0)
        if r0 >= TARGET:
            alpha, ratio = 0.0, r0
        else:
            lo, hi = 0.0, 1.0
            for _ in range(24):
                mid = 0.5 * (lo + hi)
                if load_ratio(cfg, gating, bias, mid) < TARGET:
                    lo = mid
                else:
                    hi = mid
            alpha = round(hi, 4)
            ratio = load_ratio(cfg, gating, bias, alpha)
        table[key] = {"alpha": alpha, "max_over_mean_load": round(ratio, 4),
                      "ratio_at_alpha_0": round(r0, 4), "tokens": TOKENS, "seed": SEED,
                      "workloads": [name]}
        print(key, table[key], flush=True)
    with open(OUT, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
