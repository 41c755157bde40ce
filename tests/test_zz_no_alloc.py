"""fused_moe_fwd_noalloc (the library's fixed scratch array instead of a caller workspace) gives
the same bits as fused_moe_fwd, through the C ABI, on two calls in a row with the second one
smaller (so the array holds the first call's larger contents when the second starts), then
the first shape again."""
from dataclasses import replace

import pytest
import torch

import mixture_experts_forward_amd as moe
from moe_harness.workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _pair(cfg, d, path="auto"):
    args = (d["hidden_states"], d["gating_output"], d["w_gate_up"], d["w_down"], cfg.k,
            d.get("correction_bias"), cfg.scoring, cfg.renormalize, cfg.num_expert_group,
            cfg.topk_group, cfg.rsf)
    ref, ids_r, w_r = moe.fused_moe_fwd(*args, path=path, return_routing=True)
    ids = torch.full_like(ids_r, -7)
    w = torch.full_like(w_r, float("nan"))
    out = torch.full_like(ref, float("nan"))
    moe.fused_moe_fwd_noalloc(*args, path=path, out=out, topk_ids_out=ids, topk_weights_out=w)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_r), "%s: routing ids differ" % cfg.name
    assert torch.equal(w, w_r), "%s: route weights differ" % cfg.name
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "%s: output bits differ" % \
        cfg.name


def test_noalloc_equals_fused_two_calls_shrinking():
    big = CONFIGS["qwen3-235b-batch"]                      # 512 tokens: 68 MB of scratch
    small = replace(CONFIGS["qwen3-30b-decode"], T=20)     # direct path, 1 MB
    grouped = replace(CONFIGS["ds-v3-grouped-prefill"], T=256, H=512, F=256)  # 256 x 256 tiles
    d_big = make_inputs(big, DEV, seed=5)
    _pair(big, d_big)
    d_small = make_inputs(small, DEV, seed=6, num_tokens=small.T)
    _pair(small, d_small)
    _pair(small, d_small, path="sorted")
    _pair(big, d_big)
    d_g = make_inputs(grouped, DEV, seed=7)
    _pair(grouped, d_g)


def test_noalloc_rejects_a_workspace_beyond_its_array():
    cfg = CONFIGS["ds-v3-grouped-prefill"]                 # 832 MB of workspace
    p = moe.make_params(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, cfg.scoring)
    assert moe.workspace_bytes(p) > moe.NOALLOC_SCRATCH_BYTES
    fake = moe.ctypes.c_void_p(1 << 20)
    st = moe.lib().fused_moe_fwd_noalloc(fake, fake, fake, fake, fake, moe.ctypes.byref(p), fake,
                                         None, None, None)
    assert st == -4
