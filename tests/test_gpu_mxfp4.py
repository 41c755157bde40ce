"""GPU parity of the fused pass with MXFP4 expert weights (fused_moe_mxfp4_fwd: e2m1 codes with
E8M0 scales per 32 elements, bf16 activations) against the oracle: the routed experts'
computation on the dequantised weights (exact in bf16 at these scales), with the bf16 pass's
tolerance (tests/parity.py).  Covers the direct path (route and scan workgroups), the sorted
path with 16-row passes (a few rows per expert), with 64-row tiles (tens of rows per expert: the
row-tiled form) and with 256 x 256 tiles (more than 64 rows per expert), full qwen3-30b decode
and qwen3-235b batch dimensions and DeepSeek-V3 dimensions on sampled tokens."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe
import oracle
from moe_harness.workloads import CONFIGS, make_inputs, make_mxfp4_weights, to_u16
from parity import (WEIGHT_ATOL, assert_output_close, oracle_route, routing_tokens,
                    sample_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle_mx(d, mx, ids, w, tokens):
    """oracle output for `tokens` from the dequantised weights of the experts they use"""
    E = mx["w_gate_up_q"].shape[0]
    sub = ids[tokens]
    used = np.unique(sub[(sub >= 0) & (sub < E)])
    remap = np.full(E, -1, np.int64)
    remap[used] = np.arange(used.size)
    local = np.where((sub >= 0) & (sub < E), remap[np.clip(sub, 0, E - 1)], -1).astype(np.int32)
    sel = torch.as_tensor(used, device=DEV, dtype=torch.long)
    host = {k: v.index_select(0, sel).cpu().numpy() for k, v in mx.items()}
    wgu = oracle.mxfp4_to_bf16(host["w_gate_up_q"], host["w_gate_up_scale"])
    wd = oracle.mxfp4_to_bf16(host["w_down_q"], host["w_down_scale"])
    x = to_u16(d["hidden_states"][torch.as_tensor(tokens, device=DEV)])
    return oracle.experts(x, wgu, wd, local, np.asarray(w, np.float32)[tokens])


def _check(cfg, d, mx, path, tokens=None, what=""):
    out, ids, w = moe.fused_moe_mxfp4_fwd(
        d["hidden_states"], d["gating_output"], mx["w_gate_up_q"], mx["w_gate_up_scale"],
        mx["w_down_q"], mx["w_down_scale"], cfg.k, d.get("correction_bias"), cfg.scoring,
        cfg.renormalize, cfg.num_expert_group, cfg.topk_group, cfg.rsf, path=path,
        return_routing=True)
    torch.cuda.synchronize()
    rid, rw = oracle_route(d, cfg)
    assert np.array_equal(ids.cpu().numpy(), rid), "%s: routing ids differ" % what
    assert np.max(np.abs(w.cpu().numpy().astype(np.float64) - rw)) <= WEIGHT_ATOL
    tokens = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    _, ref = _oracle_mx(d, mx, rid, rw, tokens)
    rel = assert_output_close(out[torch.as_tensor(tokens, device=DEV)], ref, what)
    print("%s: rel-L2 %.2e" % (what, rel), flush=True)


@pytest.mark.parametrize("T,path", [(4, "auto"), (4, "direct"), (4, "sorted"), (40, "direct"),
                                    (40, "sorted"), (1, "direct")])
def test_mxfp4_small(T, path):
    cfg = replace(CONFIGS["tiny"], T=T, H=256, E=8, F=128, k=2)
    d = make_inputs(cfg, DEV, seed=T, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=T)
    _check(cfg, d, mx, path, what="mxfp4 T=%d %s" % (T, path))


def test_mxfp4_several_tiles_per_expert():
    # about 64 rows per expert (H and F multiples of 256): the 256 x 256 tile, some experts
    # past 64 rows
    cfg = replace(CONFIGS["tiny"], T=128, H=256, E=4, F=256, k=2)
    d = make_inputs(cfg, DEV, seed=5, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=5)
    _check(cfg, d, mx, "sorted", what="mxfp4 multi-pass")


@pytest.mark.parametrize("T,path", [(1, "direct"), (32, "direct"), (32, "sorted")])
def test_mxfp4_qwen3_30b_decode_sampled(T, path):
    cfg = replace(CONFIGS["qwen3-30b-decode"], T=T)
    d = make_inputs(cfg, DEV, seed=300 + T, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=7)
    _check(cfg, d, mx, path, sample_tokens(T, 3), "mxfp4 qwen3-30b T=%d %s" % (T, path))


def test_mxfp4_grouped_sigmoid_routing():
    cfg = replace(CONFIGS["ds-v3-grouped-prefill"], T=24, H=256, E=32, F=128)
    d = make_inputs(cfg, DEV, seed=9, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=9)
    _check(cfg, d, mx, "auto", what="mxfp4 grouped sigmoid")


@pytest.mark.parametrize("T,E,k,H,F", [
    (300, 8, 4, 384, 256),     # ~150 rows per expert, H not a multiple of 256: 64-row tiles,
                               # three per expert, a ragged last one
    (70, 16, 8, 384, 128),     # ~35 rows per expert: one partial tile each, 3 k-steps
    (96, 4, 2, 256, 256),      # ~48 rows per expert, H and F multiples of 256: 64-row tiles
    (128, 4, 2, 256, 256),     # 64 rows, ungrouped routing: still 64-row tiles (the 256 x 256
                               # tile takes over above 64, above 48 with grouped routing)
    (33, 4, 2, 128, 128),      # 16-17 rows: one 16-row MFMA tile and a one-row one
])
def test_mxfp4_row_tiled_sizes(T, E, k, H, F):
    cfg = replace(CONFIGS["tiny"], T=T, E=E, k=k, H=H, F=F)
    d = make_inputs(cfg, DEV, seed=T + 1, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=T + 1)
    _check(cfg, d, mx, "auto", what="mxfp4 tiled T=%d E=%d" % (T, E))


@pytest.mark.parametrize("T,E,k,H,F", [
    (300, 8, 4, 256, 256),     # ~150 rows per expert: one 256-row tile each; K 256 for both
                               # GEMMs (4 k-steps: one scale group)
    (512, 4, 2, 512, 256),     # ~256 rows: experts past 256 rows split evenly over two tiles;
                               # gate-up K 512 (two scale groups, rotated start)
    (200, 4, 2, 768, 512),     # ~100 rows; K 768 and 512 (three and two groups)
])
def test_mxfp4_wide_sizes(T, E, k, H, F):
    """More than 64 routed rows per expert with H and F multiples of 256: the 256 x 256 tile
    with the codes and scales brought in by DMA and dequantised into its bf16 LDS stage."""
    cfg = replace(CONFIGS["tiny"], T=T, E=E, k=k, H=H, F=F)
    d = make_inputs(cfg, DEV, seed=T + 2, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=T + 2)
    _check(cfg, d, mx, "auto", what="mxfp4 wide T=%d E=%d H=%d" % (T, E, H))


def test_mxfp4_wide_ds_v3_dims_sampled():
    """DeepSeek-V3 dimensions and routing with 32 experts at 512 tokens (128 routed rows per
    expert, as at 4096 tokens of 256): the 256 x 256 MXFP4 tile over 112 and 32 k-steps, tokens
    chosen from the realized routing (the heaviest expert's last tile, every eighth of the
    sorted routes)."""
    cfg = replace(CONFIGS["ds-v3-grouped-prefill"], T=512, E=32)
    d = make_inputs(cfg, DEV, seed=13, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=13)
    rid, _ = oracle_route(d, cfg)
    _check(cfg, d, mx, "auto", routing_tokens(rid, cfg.E, 256, n=16), "mxfp4 wide ds-v3 dims")


def test_mxfp4_qwen3_235b_batch_sampled():
    """Qwen3-235B batch (512 tokens, 32 routed rows per expert on average): row-tiled.  Every
    token's routing is compared; the outputs of 3 tokens (the oracle dequantises each expert
    they use on the host, about a second per expert at these dimensions)."""
    cfg = CONFIGS["qwen3-235b-batch"]
    d = make_inputs(cfg, DEV, seed=11, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=11)
    _check(cfg, d, mx, "auto", sample_tokens(cfg.T, 3), "mxfp4 qwen3-235b batch")


def test_mxfp4_skewed_grouped_routing():
    """DeepSeek-V3 routing on reduced dimensions: hundreds of rows on the hottest experts,
    a few on the coldest, one 64-row tile to many per expert."""
    cfg = replace(CONFIGS["ds-v3-grouped-prefill"], T=1024, H=256, F=128)
    d = make_inputs(cfg, DEV, seed=12, weights=False)
    mx = make_mxfp4_weights(cfg, DEV, seed=12)
    _check(cfg, d, mx, "auto", sample_tokens(cfg.T, 96), "mxfp4 ds-v3 routing")
