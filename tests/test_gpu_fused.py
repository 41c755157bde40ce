"""GPU parity of the whole pass (fused_moe_fwd / fused_moe_shared_fwd / fused_moe_experts_fwd)
against the oracle, on both the direct and the sorted path.

Tolerance (see parity.py): rel-L2 <= 2e-2 and |got - ref| <= 5e-2 + 2e-2|ref| per element on the
bf16 output; routing bit-exact / 1e-6.  Full-size configurations compare sampled tokens (the
first, the last and random ones) that the oracle evaluates one by one."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe
import oracle
from moe_harness.workloads import CONFIGS, make_inputs, random_topk_ids, random_topk_weights, to_u16
from parity import (WEIGHT_ATOL, assert_output_close, oracle_experts_sampled, oracle_route,
                    routing_tokens, sample_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _fused(cfg, d, path="auto", **kw):
    fn = moe.fused_moe_shared_fwd if cfg.S > 0 else moe.fused_moe_fwd
    args = [d["hidden_states"], d["gating_output"], d["w_gate_up"], d["w_down"]]
    if cfg.S > 0:
        args += [d["shared_w_gate_up"], d["shared_w_down"]]
    out, ids, w = fn(*args, cfg.k, d.get("correction_bias"), cfg.scoring, cfg.renormalize,
                     cfg.num_expert_group, cfg.topk_group, cfg.rsf, path=path,
                     return_routing=True, **kw)
    torch.cuda.synchronize()
    return out, ids.cpu().numpy(), w.cpu().numpy()


def _check_pass(cfg, d, path, tokens=None, what=""):
    """tokens: None (every token), an array, or a function of the realized routing ids."""
    out, ids, w = _fused(cfg, d, path)
    rid, rw = oracle_route(d, cfg)
    assert np.array_equal(ids, rid), "%s: routing ids differ" % what
    assert np.max(np.abs(w.astype(np.float64) - rw)) <= WEIGHT_ATOL
    if tokens is None:
        tokens = np.arange(cfg.T)
    elif callable(tokens):
        tokens = tokens(rid)
    _, ref = oracle_experts_sampled(d, rid, rw, tokens, with_shared=cfg.S > 0)
    rel = assert_output_close(out[torch.as_tensor(tokens, device=DEV)], ref, what)
    print("%s: rel-L2 %.2e" % (what, rel), flush=True)
    return out


@pytest.mark.parametrize("path", ["auto", "direct", "sorted"])
def test_tiny_all_tokens(path):
    cfg = CONFIGS["tiny"]
    _check_pass(cfg, make_inputs(cfg, DEV), path, what="tiny/" + path)


def test_qwen3_30b_decode_all_tokens():
    cfg = CONFIGS["qwen3-30b-decode"]
    _check_pass(cfg, make_inputs(cfg, DEV), "auto", what=cfg.name)


# odd and boundary token counts from 1 to 256 (the aiter decoding PR's served counts include
# 3, 5-7 and 9-15); both paths where the direct path applies
@pytest.mark.parametrize("T", [1, 2, 3, 5, 6, 7, 8, 9, 11, 13, 15, 17, 31, 33, 63, 65, 100, 127,
                               129, 255, 256])
def test_decode_token_sweep(T):
    cfg = CONFIGS["qwen3-30b-decode"]
    d = make_inputs(cfg, DEV, seed=100 + T, num_tokens=T)
    c = replace(cfg, T=T)
    paths = ["sorted"] + (["direct"] if T * cfg.k <= moe.DIRECT_MAX_ROUTES else [])
    for p in paths:
        _check_pass(c, d, p, what="T=%d %s" % (T, p))


@pytest.mark.parametrize("T", [24, 100])
def test_qwen3_235b_dims_decode(T):
    """8 KB gate-up weight rows on the weight-streaming kernel (two-k-step row segments): the
    direct path (24 tokens) and the sorted path at ~6 rows per expert (100 tokens)."""
    cfg = replace(CONFIGS["qwen3-235b-batch"], T=T)
    d = make_inputs(cfg, DEV, seed=300 + T, num_tokens=T)
    paths = ["sorted"] + (["direct"] if T * cfg.k <= moe.DIRECT_MAX_ROUTES else [])
    for p in paths:
        _check_pass(cfg, d, p, sample_tokens(T, 10), "qwen3-235b dims T=%d %s" % (T, p))


def test_qwen3_235b_batch_all_tokens():
    cfg = CONFIGS["qwen3-235b-batch"]
    d = make_inputs(cfg, DEV)
    _check_pass(cfg, d, "auto", None, cfg.name)


@pytest.mark.slow
def test_ds_v3_grouped_prefill_sampled():
    """The benchmark's launch configuration at full size: 64+ tokens chosen from the realized
    routing (the heaviest expert's ragged last 256-row tile, every eighth of the sorted route
    order, i.e. every XCD's tile range)."""
    cfg = CONFIGS["ds-v3-grouped-prefill"]
    d = make_inputs(cfg, DEV)
    _check_pass(cfg, d, "auto", lambda ids: routing_tokens(ids, cfg.E, 256, n=64), cfg.name)
    del d
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_ds_v3_prefill_16k_sampled():
    cfg = CONFIGS["ds-v3-prefill-16k"]
    d = make_inputs(cfg, DEV)
    _check_pass(cfg, d, "auto", lambda ids: routing_tokens(ids, cfg.E, 256, n=32), cfg.name)
    del d
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_kimi_k2_shared_sampled():
    cfg = CONFIGS["kimi-k2-shared"]
    d = make_inputs(cfg, DEV)
    _check_pass(cfg, d, "auto", lambda ids: routing_tokens(ids, cfg.E, 64, n=96), cfg.name)
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,path", [(4, "direct"), (4, "sorted"), (40, "sorted")])
def test_shared_expert_small(T, path):
    cfg = replace(CONFIGS["kimi-k2-shared"], T=T, H=256, E=24, F=128, S=192, k=4)
    _check_pass(cfg, make_inputs(cfg, DEV, seed=9), path, what="shared T=%d %s" % (T, path))


@pytest.mark.parametrize("T,E,k,H,F", [
    (37, 16, 4, 256, 128),    # ~9 rows per expert: 64-row tiles, ragged tiles and tail
    (300, 8, 4, 128, 192),    # ~150 rows per expert: 256 x 256 tiles, part-full row groups
    (129, 4, 2, 192, 64),     # ~65 rows per expert: 256 x 256 tiles, F one partial column block
    (70, 16, 8, 320, 64),     # ~35 rows per expert: 64-row tiles, F a single column block
])
def test_row_tiled_sizes(T, E, k, H, F):
    cfg = replace(CONFIGS["tiny"], T=T, E=E, k=k, H=H, F=F)
    _check_pass(cfg, make_inputs(cfg, DEV, seed=T), "sorted", what="tiled T=%d E=%d" % (T, E))


@pytest.mark.parametrize("T", [1, 31, 200])
def test_shared_expert_rows(T):
    """Dense shared-expert GEMMs (256 x 256 tiles, K-split tail) over 1, a ragged 31 and 200
    tokens."""
    cfg = replace(CONFIGS["kimi-k2-shared"], T=T, H=192, E=16, F=64, S=320, k=2)
    _check_pass(cfg, make_inputs(cfg, DEV, seed=T + 1), "auto", what="shared rows T=%d" % T)


@pytest.mark.parametrize("T,path", [(7, "direct"), (7, "sorted"), (20, "direct"),
                                    (20, "sorted"), (64, "direct"), (200, "sorted"),
                                    (600, "sorted")])
def test_experts_given_routing_with_padding_and_repeats(T, path):
    """fused_moe_experts_fwd with -1 routes, repeated ids of one token, and NaN weights in every
    expert no route selects: a kernel that reads expert -1, an unselected expert or a skipped row
    produces NaN and fails the check.  T=7 takes the route-major direct path, T=20 and T=64 the
    expert-major scan (160 and 512 routes); T=200 and T=600 (1600 and 4800 routes, ~100 and
    ~300 rows per expert) the chunked align and the 256-row tile GEMM."""
    cfg = replace(CONFIGS["tiny"], T=T, E=16, k=8, H=128, F=64)
    d = make_inputs(cfg, DEV, seed=11)
    ids = random_topk_ids(cfg.T, cfg.k, cfg.E, seed=3, pad_fraction=0.2, allow_repeats=True)
    ids[0, :] = -1                                # a token with no route at all
    ids[1, 0] = ids[1, 1] = 5                     # a repeated id
    ids = ids.to(DEV)
    w = random_topk_weights(cfg.T, cfg.k, seed=3).to(DEV)
    used = torch.unique(ids[ids >= 0]).cpu()
    for e in range(cfg.E):
        if e not in used:
            d["w_gate_up"][e].fill_(float("nan"))
            d["w_down"][e].fill_(float("nan"))
    P = cfg.T * cfg.k
    if path == "direct":
        assert P <= moe.DIRECT_MAX_ROUTES
    p = moe.make_params(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, path=path)
    ws = torch.full((moe.workspace_bytes(p),), 0xFF, dtype=torch.uint8, device=DEV)  # NaN fill
    out = moe.fused_moe_experts_fwd(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w,
                                    path=path, workspace=ws)
    torch.cuda.synchronize()
    _, ref = oracle.experts(to_u16(d["hidden_states"]), to_u16(d["w_gate_up"]),
                            to_u16(d["w_down"]), ids.cpu().numpy(), w.cpu().numpy())
    assert_output_close(out, ref, "padding/repeats " + path)
    assert torch.all(out[0] == 0)


@pytest.mark.parametrize("T,E,k,H,F,skew", [
    (700, 16, 4, 128, 128, 1.5),   # ~1000 rows on the hottest expert: four 256-row tiles
    (64, 32, 8, 256, 64, 2.0),     # 512 routes, ~16 per expert on average: 64-row tiles
    (150, 128, 4, 128, 64, 1.2),   # 600 routes, ~5 per expert: weight-streaming, chunked align
])
def test_skewed_routing_sorted(T, E, k, H, F, skew):
    """Given Zipf-like routing ids (experts drawn with probability proportional to
    (1 + rank)^-skew: a few very hot experts, a long tail of cold or unused ones) through the
    sorted path, every token compared with the oracle.  This stresses hot experts harder than
    the router-score skew of tests/test_gpu_skew.py."""
    cfg = replace(CONFIGS["tiny"], T=T, E=E, k=k, H=H, F=F)
    d = make_inputs(cfg, DEV, seed=T + E)
    ids = random_topk_ids(T, k, E, seed=5, skew=skew).to(DEV)
    w = random_topk_weights(T, k, seed=5).to(DEV)
    out = moe.fused_moe_experts_fwd(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w,
                                    path="sorted")
    torch.cuda.synchronize()
    _, ref = oracle.experts(to_u16(d["hidden_states"]), to_u16(d["w_gate_up"]),
                            to_u16(d["w_down"]), ids.cpu().numpy(), w.cpu().numpy())
    rel = assert_output_close(out, ref, "skewed T=%d E=%d" % (T, E))
    print("skewed T=%d E=%d: max expert load %d, rel-L2 %.2e" % (
        T, E, int(torch.bincount(ids.flatten().long().cpu()).max()), rel), flush=True)


def test_empty_tokens_is_a_no_op():
    cfg = CONFIGS["tiny"]
    d = make_inputs(cfg, DEV, num_tokens=0)
    out = moe.fused_moe_fwd(d["hidden_states"], d["gating_output"], d["w_gate_up"], d["w_down"],
                            cfg.k)
    assert out.shape == (0, cfg.H)


@pytest.mark.parametrize("name,T", [("qwen3-30b-decode", 32), ("qwen3-30b-decode", 5),
                                    ("qwen3-235b-batch", 512)])
def test_bitwise_deterministic_repeats(name, T):
    """Three calls on identical inputs give identical bits (no float atomics anywhere)."""
    cfg = replace(CONFIGS[name], T=T)
    d = make_inputs(cfg, DEV, num_tokens=T)
    outs = [_fused(cfg, d)[0].clone() for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("T", [40, 512])
def test_shared_fused_equals_stages(T):
    """fused_moe_shared_fwd runs the shared expert on a second stream beside the routed GEMMs;
    the stages run the same kernels in order on one stream: the same bits.  Kimi-K2 expert and
    shared-expert dimensions (S = 18432) with 32 routed experts."""
    cfg = replace(CONFIGS["kimi-k2-shared"], T=T, E=32)
    d = make_inputs(cfg, DEV, seed=900 + T)
    out, ids, w = moe.fused_moe_shared_fwd(
        d["hidden_states"], d["gating_output"], d["w_gate_up"], d["w_down"],
        d["shared_w_gate_up"], d["shared_w_down"], cfg.k, d["correction_bias"], cfg.scoring,
        cfg.renormalize, cfg.num_expert_group, cfg.topk_group, cfg.rsf, return_routing=True)
    p = moe.make_params(T, cfg.H, cfg.E, cfg.F, cfg.k)
    ws = torch.empty(moe.workspace_bytes(p, cfg.S), dtype=torch.uint8, device=DEV)
    staged = torch.full_like(out, float("nan"))
    for s in (moe.STAGE_ALIGN, moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_SHARED,
              moe.STAGE_COMBINE):
        moe.fused_moe_experts_stage(s, p, d["hidden_states"], d["w_gate_up"], d["w_down"], ids,
                                    w, staged, ws, d["shared_w_gate_up"], d["shared_w_down"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), staged.view(torch.int16))
    rid, rw = oracle_route(d, cfg)
    tokens = sample_tokens(T, 6)
    _, ref = oracle_experts_sampled(d, rid, rw, tokens, with_shared=True)
    assert_output_close(out[torch.as_tensor(tokens, device=DEV)], ref, "shared T=%d" % T)


def test_shared_fused_concurrent_host_threads():
    """Two host threads call fused_moe_shared_fwd at once, each on its own stream and
    workspace: the per-device side stream and its fork/join events are shared (guarded by the
    library), and every result equals the single-threaded one bit for bit."""
    import threading
    cfg = replace(CONFIGS["kimi-k2-shared"], T=64, E=16, S=1024)
    inputs = [make_inputs(cfg, DEV, seed=950 + i) for i in range(2)]

    def run(d, stream, out):
        with torch.cuda.stream(stream):
            out.copy_(moe.fused_moe_shared_fwd(
                d["hidden_states"], d["gating_output"], d["w_gate_up"], d["w_down"],
                d["shared_w_gate_up"], d["shared_w_down"], cfg.k, d["correction_bias"],
                cfg.scoring, cfg.renormalize, cfg.num_expert_group, cfg.topk_group, cfg.rsf))

    refs = []
    for d in inputs:
        o = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
        run(d, torch.cuda.current_stream(), o)
        refs.append(o)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [[torch.empty_like(refs[0]) for _ in range(6)] for _ in range(2)]

    def worker(i):
        for j in range(6):
            run(inputs[i], streams[i], outs[i][j])

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(2):
        for j in range(6):
            assert torch.equal(outs[i][j], refs[i]), "thread %d call %d differs" % (i, j)
