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
from parity import (WEIGHT_ATOL, assert_output_close, oracle_route, routing_tokens,
                    sample_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(cfg, d, fw, path):
    return moe.fused_moe_fp8_fwd(
        d["hidden_states"], d["gating_output"], fw["w_gate_up"], fw["w_gate_up_scale"],
        fw["w_down"], fw["w_down_scale"], cfg.k, d.get("correction_bias"), cfg.scoring,
        cfg.renormalize, cfg.num_expert_group, cfg.topk_group, cfg.rsf, return_routing=True,
        path=path)


def _check(cfg, d, fw, tokens=None, what="", path="auto"):
    out, ids, w = _run(cfg, d, fw, path)
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


@pytest.mark.parametrize("path", ["sorted", "direct"])
@pytest.mark.parametrize("T,E,k", [(4, 8, 2), (32, 8, 2), (64, 4, 1), (1, 8, 2)])
def test_fp8_pass_small(T, E, k, path):
    cfg = replace(CONFIGS["tiny"], T=T, H=256, E=E, F=256, k=k)
    d = make_inputs(cfg, DEV, seed=T + E, weights=False)
    fw = make_fp8_weights(cfg, DEV, seed=T)
    _check(cfg, d, fw, what="fp8 pass T=%d E=%d %s" % (T, E, path), path=path)


def test_fp8_pass_sorted_past_direct_limit():
    cfg = replace(CONFIGS["tiny"], T=33, H=256, E=8, F=256, k=2)
    d = make_inputs(cfg, DEV, seed=41, weights=False)
    fw = make_fp8_weights(cfg, DEV, seed=33)
    _check(cfg, d, fw, what="fp8 pass T=33 (66 routes) sorted")
    with pytest.raises(moe.MoEError):
        _run(cfg, d, fw, "direct")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_fp8_direct_qwen3_30b_decode(T):
    """The direct form at Qwen3-30B-A3B dimensions (H 2048: two-k-step weight segments; F 768:
    K split over two waves), every token against the oracle."""
    cfg = replace(CONFIGS["qwen3-30b-decode-b1"], T=T)
    d = make_inputs(cfg, DEV, seed=100 + T, weights=False)
    fw = make_fp8_weights(cfg, DEV, seed=7)
    _check(cfg, d, fw, what="fp8 direct qwen3-30b T=%d" % T, path="direct")


@pytest.mark.parametrize("T", [1, 2, 8])
def test_fp8_direct_ds_v3_dims(T):
    """DeepSeek-V3 dimensions (H 7168: one-k-step segments over 124 KB of LDS; F 2048) and
    routing (sigmoid, 8 groups, bias, scaling 2.5) with 32 experts, so that T = 8 puts several
    routes on one expert (the 16-row pass of the direct form gathers them)."""
    cfg = replace(CONFIGS["ds-v3-grouped-prefill"], T=T, E=32)
    d = make_inputs(cfg, DEV, seed=200 + T, weights=False)
    fw = make_fp8_weights(cfg, DEV, seed=9)
    _check(cfg, d, fw, what="fp8 direct ds-v3 dims T=%d" % T, path="direct")


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


def _stages(cfg, d, fw, ids, w, path):
    p = moe.make_params(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, path=path)
    ws = torch.empty(max(256, moe.fp8_workspace_bytes(p)), dtype=torch.uint8, device=DEV)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    for s in (moe.STAGE_ALIGN, moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_COMBINE):
        moe.fused_moe_fp8_stage(s, p, d["hidden_states"], fw, ids, w, out, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T,k,E,pattern", [
    (2, 8, 8, "one-expert"),      # 16 routes on expert 0: 8 passes of 2 rows on the direct path
    (3, 4, 6, "repeats"),         # repeated ids within a token, some routes padded (-1)
    (16, 4, 64, "repeats"),       # 64 routes, up to 16 rows per pass
    (5, 2, 4, "all-padded"),      # every id out of range: the output is zero
])
def test_fp8_stages_given_routing(T, k, E, pattern):
    """The four stages of the FP8 pass with caller-given ids that break the rows-per-expert bound
    of distinct top-k ids (so the direct form takes several passes), on both paths, against the
    oracle's expert part with the same ids and weights."""
    cfg = replace(CONFIGS["tiny"], T=T, H=256, E=E, F=256, k=k)
    d = make_inputs(cfg, DEV, seed=T * 31 + E, weights=False)
    fw = make_fp8_weights(cfg, DEV, seed=E)
    r = np.random.default_rng(T + 7 * E)
    if pattern == "one-expert":
        ids = np.zeros((T, k), np.int32)
    elif pattern == "all-padded":
        ids = np.full((T, k), -1, np.int32)
        ids[0, 0] = E
    else:
        ids = r.integers(0, E, (T, k)).astype(np.int32)
        ids[r.random((T, k)) < 0.15] = -1
    w = r.random((T, k)).astype(np.float32)
    h = {kk: v.cpu().numpy() for kk, v in fw.items()}
    ref = oracle.fp8_experts(to_u16(d["hidden_states"]), h["w_gate_up"], h["w_gate_up_scale"],
                             h["w_down"], h["w_down_scale"], ids, w)
    for path in ("direct", "sorted"):
        out = _stages(cfg, d, fw, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                      path)
        if pattern == "all-padded":
            assert not out.float().abs().max().item(), path
            continue
        rel = assert_output_close(out, ref, "fp8 stages %s %s" % (pattern, path))
        print("fp8 stages %s %s: rel-L2 %.2e" % (pattern, path, rel), flush=True)


def _oracle_fp8_sampled(cfg, d, fw, ids, w, tokens):
    """The oracle's FP8 expert part for ``tokens``, with only the experts those tokens touch
    copied to the host."""
    sub = np.asarray(ids)[tokens]
    ok = (sub >= 0) & (sub < cfg.E)
    used = np.unique(sub[ok])
    remap = np.full(cfg.E, -1, np.int64)
    remap[used] = np.arange(used.size)
    local = np.where(ok, remap[np.clip(sub, 0, cfg.E - 1)], -1).astype(np.int32)
    sel = torch.as_tensor(used, device=DEV, dtype=torch.long)
    h = {kk: v.index_select(0, sel).cpu().numpy() for kk, v in fw.items()}
    x = to_u16(d["hidden_states"][torch.as_tensor(tokens, device=DEV)])
    return oracle.fp8_experts(x, h["w_gate_up"], h["w_gate_up_scale"], h["w_down"],
                              h["w_down_scale"], local, np.asarray(w, np.float32)[tokens])


@pytest.mark.slow
@pytest.mark.parametrize("name,E,T", [
    ("qwen3-235b-prefill", None, None),      # full size: 256 routes per expert on average
    ("ds-v3-grouped-prefill", 64, 1024),     # DeepSeek-V3 dimensions and routing, 128 routes
                                             # per expert on average as at 4096 tokens of 256
])
def test_fp8_prefill_sampled(name, E, T):
    """The 256-row FP8 tile (k_fp8_wide) in the pass's launch configuration: both stage forms
    (tiles of at most 128 rows take three stages), evenly split experts, the route-to-token row
    map; tokens chosen from the realized routing (the heaviest expert's last tile, every
    eighth of the expert-sorted routes) against the oracle."""
    cfg = CONFIGS[name] if E is None else replace(CONFIGS[name], E=E, T=T)
    d = make_inputs(cfg, DEV, seed=11, weights=False)
    fw = make_fp8_weights(cfg, DEV, seed=12)
    out, ids, w = _run(cfg, d, fw, "auto")
    torch.cuda.synchronize()
    rid, rw = oracle_route(d, cfg)
    assert np.array_equal(ids.cpu().numpy(), rid), "routing ids differ"
    tokens = routing_tokens(rid, cfg.E, 256, n=40)
    ref = _oracle_fp8_sampled(cfg, d, fw, rid, rw, tokens)
    rel = assert_output_close(out[torch.as_tensor(tokens, device=DEV)], ref, "fp8 " + name)
    print("fp8 %s E=%d T=%d: rel-L2 %.2e over %d tokens" % (name, cfg.E, cfg.T, rel, len(tokens)),
          flush=True)
    del d, fw
    torch.cuda.empty_cache()
