"""The fused pass captured in a HIP graph: every replay equals the eager call bit for bit.

The library only enqueues kernels on the caller's stream (no allocation, no memset, no host
synchronisation), so a captured call replays the same kernels.  Replays are interleaved with
eager calls on other inputs and synchronisations, and each replay is checked."""
from dataclasses import replace

import pytest
import torch

import mixture_experts_forward_amd as moe
from moe_harness.workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _call(cfg, d, out, ws):
    if cfg.S > 0:
        return moe.fused_moe_shared_fwd(d["hidden_states"], d["gating_output"], d["w_gate_up"],
                                        d["w_down"], d["shared_w_gate_up"], d["shared_w_down"],
                                        cfg.k, d["correction_bias"], cfg.scoring,
                                        cfg.renormalize, cfg.num_expert_group, cfg.topk_group,
                                        cfg.rsf, out=out, workspace=ws)
    return moe.fused_moe_fwd(d["hidden_states"], d["gating_output"], d["w_gate_up"],
                             d["w_down"], cfg.k, d["correction_bias"], cfg.scoring,
                             cfg.renormalize, cfg.num_expert_group, cfg.topk_group, cfg.rsf,
                             out=out, workspace=ws)


# reduced dimensions that keep each workload's kernel choice: the weight-streaming kernel
# (decode), the row-tiled kernel (batch), and the 256 x 256 kernel on the sorted layout with
# its per-XCD tile counters and, with a shared expert, its K-split dense tiles
_DIMS = {"kimi-k2-shared": dict(H=1024, E=64, F=256, S=512),
         "ds-v3-grouped-prefill": dict(H=512, E=16, F=256, num_expert_group=4, topk_group=2),
         "kimi-k2-wide": dict(H=512, E=16, F=256, S=640)}


@pytest.mark.parametrize("name,T", [("qwen3-30b-decode", 32), ("qwen3-30b-decode", 4),
                                    ("qwen3-235b-batch", 160),
                                    ("kimi-k2-shared", 40),
                                    ("ds-v3-grouped-prefill", 512),
                                    ("kimi-k2-wide", 300)])
def test_graph_replays_match_eager(name, T):
    base = CONFIGS["kimi-k2-shared" if name == "kimi-k2-wide" else name]
    cfg = replace(base, T=T, **_DIMS.get(name, {}))
    d = make_inputs(cfg, DEV, num_tokens=T)
    other = make_inputs(cfg, DEV, num_tokens=T, seed=7)
    p = moe.make_params(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, cfg.scoring, cfg.renormalize,
                        cfg.num_expert_group, cfg.topk_group, cfg.rsf)
    ws = torch.empty(max(256, moe.workspace_bytes(p, cfg.S)), dtype=torch.uint8, device=DEV)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    eager = _call(cfg, d, torch.empty_like(out), ws).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(cfg, d, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(cfg, d, out, ws)
    for rep in range(4):
        out.fill_(0)
        other_out = _call(cfg, other, None, ws)   # eager work on the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager call" % rep
        assert not torch.equal(other_out, eager)
