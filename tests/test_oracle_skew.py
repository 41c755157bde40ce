"""The skewed-routing workload (aiter MI308 decoding PR, Performance, "Skewed routing": a fixed
per-expert bias -alpha * log(1 + rank) on the router scores, alpha chosen so the most popular
expert receives twice the mean load) is what its recipe says: the bias values, their ranking,
and the recorded alpha reproducing the 2x load on a fresh token sample through the oracle's
routing."""
import math

import numpy as np
import pytest
import torch

import oracle
from moe_harness.workloads import CONFIGS, make_inputs, skew_alpha, skew_bias, skew_gating


def test_skew_bias_is_minus_alpha_log1p_rank():
    E, a = 128, 0.1
    b = skew_bias(E, a).numpy()
    # the values are -a*log(1 + r) for r = 0..E-1, each once
    assert np.allclose(np.sort(b)[::-1], -a * np.log1p(np.arange(E)), rtol=0, atol=1e-15)
    assert np.count_nonzero(b == 0.0) == 1
    # fixed ranking: the same seed gives the same permutation, another seed another one
    assert np.array_equal(b, skew_bias(E, a).numpy())
    assert not np.array_equal(b, skew_bias(E, a, seed=43).numpy())
    # alpha scales the bias linearly
    assert np.allclose(skew_bias(E, 2 * a).numpy(), 2 * b, rtol=0, atol=1e-15)


def test_skew_gating_rounds_the_sum_once():
    g = torch.randn(6, 16, generator=torch.Generator().manual_seed(1), dtype=torch.float32)
    assert torch.equal(skew_gating(g, 0.0), g)
    got = skew_gating(g, 0.09)
    want = (g.double() + skew_bias(16, 0.09)).float()
    assert torch.equal(got, want)


def _ratio(cfg, alpha, tokens, seed):
    d = make_inputs(cfg, "cpu", seed=seed, weights=False, num_tokens=tokens)
    g = skew_gating(d["gating_output"], alpha).numpy()
    b = None if d["correction_bias"] is None else d["correction_bias"].numpy()
    ids, _ = oracle.route(g, b, cfg.k, cfg.scoring, cfg.renormalize, cfg.num_expert_group,
                          cfg.topk_group, float(np.float32(cfg.rsf)))
    load = np.bincount(ids.ravel(), minlength=cfg.E)
    return load.max() / load.mean(), int(np.argmax(load))


@pytest.mark.parametrize("name", ["qwen3-30b-decode", "qwen3-235b-batch"])
def test_recorded_alpha_gives_twice_the_mean_load(name):
    cfg = CONFIGS[name]
    a = skew_alpha(cfg)
    assert 0.05 < a < 0.15
    # a fresh sample (another seed than the one alpha was fitted on)
    r, top = _ratio(cfg, a, 16384, seed=11)
    assert abs(r - 2.0) < 0.1, r
    # the most loaded expert is the rank-0 expert (bias 0)
    assert skew_bias(cfg.E, a).numpy()[top] == 0.0
    # unskewed softmax routing of N(0,1) logits is near uniform
    r0, _ = _ratio(cfg, 0.0, 16384, seed=11)
    assert r0 < 1.2, r0


@pytest.mark.parametrize("name", ["ds-v3-grouped-prefill", "kimi-k2-shared"])
def test_biased_sigmoid_routing_is_already_beyond_twice(name):
    cfg = CONFIGS[name]
    assert skew_alpha(cfg) == 0.0
    r, _ = _ratio(cfg, 0.0, 8192, seed=11)
    assert r > 2.0 * 2, r
