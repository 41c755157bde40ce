"""GPU parity of moe_route (top-k / grouped top-k routing) against the oracle: topk_ids
bit-exact, topk_weights within 1e-6 absolute."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe
from moe_harness.workloads import CONFIGS, make_inputs
from parity import WEIGHT_ATOL, oracle_route

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(cfg, d):
    ids, w = moe.moe_route(d["gating_output"], cfg.k, d.get("correction_bias"), cfg.scoring,
                           cfg.renormalize, cfg.num_expert_group, cfg.topk_group, cfg.rsf)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _compare(cfg, d, what):
    ids, w = _run(cfg, d)
    rid, rw = oracle_route(d, cfg)
    bad = np.nonzero(np.any(ids != rid, axis=1))[0]
    assert bad.size == 0, "%s: ids differ at tokens %s" % (what, bad[:5])
    err = np.max(np.abs(w.astype(np.float64) - rw)) if w.size else 0.0
    assert err <= WEIGHT_ATOL, "%s: weight error %.3e" % (what, err)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_route_full_size(name):
    cfg = CONFIGS[name]
    print("route", name, cfg.T, flush=True)
    _compare(cfg, make_inputs(cfg, DEV, weights=False), name)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 7, 33, 257, 1000])
@pytest.mark.parametrize("name", ["qwen3-30b-decode", "ds-v3-grouped-prefill", "kimi-k2-shared"])
def test_route_token_sweep(name, T):
    cfg = CONFIGS[name]
    _compare(cfg, make_inputs(cfg, DEV, seed=T, weights=False, num_tokens=T), "%s T=%d" % (name, T))


@pytest.mark.parametrize("variant", [
    dict(E=64, k=4, scoring="sigmoid", bias=True, num_expert_group=64, topk_group=7),
    dict(E=1024, k=32, scoring="softmax"),
    dict(E=1000, k=6, scoring="sigmoid", bias=True, num_expert_group=8, topk_group=3),
    dict(E=96, k=5, scoring="softmax", renormalize=False, rsf=1.5),
    dict(E=256, k=8, scoring="sigmoid", bias=False, renormalize=False),
    dict(E=32, k=32, scoring="softmax", renormalize=False),
    dict(E=48, k=3, scoring="sigmoid", bias=True, num_expert_group=2, topk_group=1, rsf=3.0),
    # group sizes that are powers of two (group scores by a butterfly over the group's lanes):
    # 16, 32 with 12 groups, 64
    dict(E=128, k=6, scoring="sigmoid", bias=True, num_expert_group=8, topk_group=3),
    dict(E=384, k=8, scoring="sigmoid", bias=True, num_expert_group=12, topk_group=5, rsf=2.0),
    dict(E=512, k=8, scoring="sigmoid", bias=True, num_expert_group=8, topk_group=4),
])
def test_route_variants(variant):
    cfg = replace(CONFIGS["tiny"], T=300, **variant)
    _compare(cfg, make_inputs(cfg, DEV, seed=5, weights=False), str(variant))


def test_route_exact_ties():
    """All-equal logits: ties go to the lower index at both levels."""
    cfg = replace(CONFIGS["tiny"], T=5, E=16, k=4, scoring="sigmoid", bias=False,
                  num_expert_group=4, topk_group=2)
    d = {"gating_output": torch.zeros((5, 16), dtype=torch.float32, device=DEV),
         "correction_bias": None}
    _compare(cfg, d, "ties")
    ids, _ = _run(cfg, d)
    assert np.all(ids == np.array([0, 1, 2, 3]))
    cfg2 = replace(cfg, scoring="softmax", num_expert_group=1, topk_group=1)
    g = torch.zeros((3, 16), dtype=torch.float32, device=DEV)
    g[1, 5] = -0.0
    _compare(cfg2, {"gating_output": g, "correction_bias": None}, "signed zero ties")
