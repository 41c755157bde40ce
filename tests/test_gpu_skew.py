"""GPU parity of the whole pass, routing included, under the skewed-routing workload of the
aiter MI308 decoding PR (Performance, "Skewed routing"): the router scores carry a fixed
per-expert bias -alpha * log(1 + rank), alpha recorded so that the most popular expert gets
twice the mean load.  Qwen3-30B decode (every token) and Qwen3-235B batch (sampled tokens, every
token's routing) dimensions, and the DeepSeek-V3 grouped routing with the page's largest alpha on
top of its own bias."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from moe_harness.workloads import CONFIGS, make_inputs, skew_alpha, skew_gating
from parity import sample_tokens
from test_gpu_fused import _check_pass

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("name,T,path,n_sample", [
    ("qwen3-30b-decode", 32, "auto", None),
    ("qwen3-30b-decode", 32, "sorted", None),
    ("qwen3-30b-decode", 256, "sorted", None),
    ("qwen3-235b-batch", 512, "auto", 24),
])
def test_skewed_router_scores(name, T, path, n_sample):
    cfg = replace(CONFIGS[name], T=T)
    a = skew_alpha(cfg)
    assert a > 0.0
    d = make_inputs(cfg, DEV, seed=21, num_tokens=T)
    d["gating_output"] = skew_gating(d["gating_output"], a)
    tokens = None if n_sample is None else sample_tokens(T, n_sample)
    _check_pass(cfg, d, path, tokens, "%s T=%d skew %.4f %s" % (name, T, a, path))


def test_skewed_grouped_routing_small():
    """DeepSeek-V3 routing (sigmoid, correction bias, 8 groups / top-4, scaling 2.5) at
    alpha 0.09 on reduced expert dimensions: the row-tiled path, hundreds of rows on the
    hottest experts."""
    cfg = replace(CONFIGS["ds-v3-grouped-prefill"], T=512, H=256, F=128)
    d = make_inputs(cfg, DEV, seed=22)
    d["gating_output"] = skew_gating(d["gating_output"], 0.09)
    _check_pass(cfg, d, "auto", sample_tokens(cfg.T, 64), "ds-v3 routing skew 0.09")
