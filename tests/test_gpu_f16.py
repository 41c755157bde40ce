"""GPU parity of the f16 pass (moe_params_t.dtype = MOE_DTYPE_F16; the TileOPs "MoE" page runs
FusedMoEFwd qwen3-235b-decode in both bf16 and f16) against the oracle's f16 evaluation, on
every GEMM kernel family: the weight-streaming decode kernel (direct and sorted), the row-tiled
kernel (tens of rows per expert), the 256 x 256 tile kernel (hundreds), and the shared expert's
dense kernels.  Tolerance as for bf16 (tests/parity.py)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe
from moe_harness.workloads import CONFIGS, make_inputs, random_topk_ids, random_topk_weights
from parity import (WEIGHT_ATOL, assert_output_close, oracle_experts_sampled, oracle_route,
                    sample_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F16 = torch.float16


def _check_pass(cfg, d, path, tokens=None, what=""):
    fn = moe.fused_moe_shared_fwd if cfg.S > 0 else moe.fused_moe_fwd
    args = [d["hidden_states"], d["gating_output"], d["w_gate_up"], d["w_down"]]
    if cfg.S > 0:
        args += [d["shared_w_gate_up"], d["shared_w_down"]]
    out, ids, w = fn(*args, cfg.k, d.get("correction_bias"), cfg.scoring, cfg.renormalize,
                     cfg.num_expert_group, cfg.topk_group, cfg.rsf, path=path,
                     return_routing=True)
    torch.cuda.synchronize()
    assert out.dtype == F16
    rid, rw = oracle_route(d, cfg)
    assert np.array_equal(ids.cpu().numpy(), rid), "%s: routing ids differ" % what
    assert np.max(np.abs(w.cpu().numpy().astype(np.float64) - rw)) <= WEIGHT_ATOL
    tokens = np.arange(cfg.T) if tokens is None else tokens
    _, ref = oracle_experts_sampled(d, rid, rw, tokens, with_shared=cfg.S > 0)
    rel = assert_output_close(out[torch.as_tensor(tokens, device=DEV)], ref, what)
    print("%s: rel-L2 %.2e" % (what, rel), flush=True)


@pytest.mark.parametrize("path", ["auto", "direct", "sorted"])
def test_f16_tiny(path):
    cfg = CONFIGS["tiny"]
    _check_pass(cfg, make_inputs(cfg, DEV, dtype=F16), path, what="tiny f16 " + path)


@pytest.mark.parametrize("T", [1, 7, 32, 100])
def test_f16_decode_tokens(T):
    cfg = replace(CONFIGS["qwen3-30b-decode"], T=T)
    d = make_inputs(cfg, DEV, seed=200 + T, dtype=F16)
    for p in ["sorted"] + (["direct"] if T * cfg.k <= moe.DIRECT_MAX_ROUTES else []):
        _check_pass(cfg, d, p, what="qwen3-30b T=%d f16 %s" % (T, p))


def test_f16_qwen3_235b_decode_sampled():
    # the page's f16 workload: T=512, H=4096, E=128, F=1536, top-8 (row-tiled kernel)
    cfg = CONFIGS["qwen3-235b-batch"]
    d = make_inputs(cfg, DEV, dtype=F16)
    _check_pass(cfg, d, "auto", sample_tokens(cfg.T, 12), "qwen3-235b T=512 f16")


def test_f16_wide_tiles_and_shared_expert():
    # hundreds of rows per expert (the 256 x 256 tile kernel) plus a shared expert (dense
    # 256 x 256 tiles for gate-up and down)
    cfg = replace(CONFIGS["kimi-k2-shared"], T=384, H=256, E=4, F=128, S=192, k=2)
    d = make_inputs(cfg, DEV, seed=7, dtype=F16)
    _check_pass(cfg, d, "sorted", sample_tokens(cfg.T, 48), "wide + shared f16")


def test_f16_experts_given_routing():
    cfg = replace(CONFIGS["tiny"], T=40, E=16, k=4, H=192, F=128)
    d = make_inputs(cfg, DEV, seed=11, dtype=F16)
    ids = random_topk_ids(cfg.T, cfg.k, cfg.E, seed=3, pad_fraction=0.1).to(DEV)
    w = random_topk_weights(cfg.T, cfg.k, seed=3).to(DEV)
    for path in ("direct", "sorted"):
        out = moe.fused_moe_experts_fwd(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w,
                                        path=path)
        torch.cuda.synchronize()
        _, ref = oracle_experts_sampled(d, ids.cpu().numpy(), w.cpu().numpy(),
                                        np.arange(cfg.T))
        assert_output_close(out, ref, "experts f16 " + path)
