"""GPU parity of the fused pass with FP8 expert weights (fused_moe_fp8_fwd) against the oracle's
FP8 pass (oracle.fp8_forward, the same steps in double with the pinned quantiser and GEMMs).
The routed x rows are quantised bit-exactly on both sides; gate/up and h can differ by float
rounding (f32 MFMA sums and SiLU vs double), which can move an h code by one step: the bf16
pass's tolerance (tests/parity.py) covers it."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe
import oracle
from moe_harness.workloads import CONFIGS, make_fp8_weights, make_inputs, to_u16
from parity import WEIGHT_ATOL, assert_output_close, oracle_route, sample_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(cfg, d, fw, tokens=None, what=""):
    out, ids, w = moe.fused_moe_fp8_fwd(
        d["hidden_states"], d["gating_output"], fw["w_gate_up"], fw["w_gate_up_scale"],
        fw["w_down"], fw["w_down_scale"], cfg.k, d.get("correction_bias"), cfg.scoring,
        cfg.renormalize, cfg.num_expert_group, cfg.topk_group, cfg.rsf, return_routing=True)
    torch.cuda.synchronize()
    rid, rw = oracle_route(d, cfg)
    assert np.array_equal(ids.cpu().numpy(), rid), "%s: routing ids differ" % what
    assert np.max(np.abs(w.cpu().numpy().astype(np.float64) - rw)) <= WEIGHT_ATOL
    tokens = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    b = None if d.get("correction_bias") is None else d["correction_bias"].cpu().numpy()
    h = {k: v.cpu().numpy() for k, v in fw.items()}
    _, _, ref = oracle.fp8_forward(to_u16(d["hidden_states"]), d["gating_output"].cpu().numpy(),
                                   h["w_gate_up"], h["w_gate_up_scale"], h["w_down"],
                                   h["w_down_scale"], b, cfg.k, cfg.scoring, cfg.renormalize,
                                   cfg.num_expert_group, cfg.topk_group,
                                   float(np.float32(cfg.rsf)), tokens=tokens)
    rel = assert_output_close(out[torch.as_tensor(tokens, device=DEV)], ref, what)
    print("%s: rel-L2 %.2e" % (what, rel), flush=True)


@pytest.mark.parametrize("T,E,k", [(4, 8, 2), (33, 8, 2), (64, 4, 2), (1, 8, 2)])
def test_fp8_pass_small(T, E, k):
    cfg = replace(CONFIGS["tiny"], T=T, H=256, E=E, F=256, k=k)
    d = make_inputs(cfg, DEV, seed=T + E, weights=False)
    fw = make_fp8_weights(cfg, DEV, seed=T)
    _check(cfg, d, fw, what="fp8 pass T=%d E=%d" % (T, E))


def test_fp8_pass_grouped_sigmoid():
    cfg = replace(CONFIGS["ds-v3-grouped-prefill"], T=48, H=256, E=32, F=128)
    d = make_inputs(cfg, DEV, seed=4, weights=False)
    fw = make_fp8_weights(cfg, DEV, seed=4)
    _check(cfg, d, fw, what="fp8 pass grouped sigmoid")


def test_fp8_pass_qwen3_30b_decode_sampled():
    cfg = CONFIGS["qwen3-30b-decode"]
    d = make_inputs(cfg, DEV, weights=False)
    fw = make_fp8_weights(cfg, DEV)
    _check(cfg, d, fw, sample_tokens(cfg.T, 3), "fp8 pass qwen3-30b decode")
