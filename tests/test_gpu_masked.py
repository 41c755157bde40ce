"""GPU parity of the masked layout (fused_moe_masked_fwd) and of expert-parallel shards.

Masked layout: every row in use is compared with the oracle (same tolerance as the routed pass);
rows past masked_m must keep the caller's bytes.  Shards: the routed pass on a shard's local
experts (ids of other shards mapped to -1) equals the oracle on that shard, and the shards of a
split sum to the unsharded pass."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe
import oracle
from moe_harness.workloads import (CONFIGS, MASKED_CONFIGS, make_inputs, make_masked_inputs,
                                   to_u16)
from parity import assert_output_close, oracle_experts_sampled, oracle_route, routing_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = 0x7FC1   # a bf16 NaN: a row the kernels must not write keeps it


def _weights(E, H, F, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    a = lambda shape, std: (torch.randn(shape, generator=g, device=DEV) * std).to(torch.bfloat16)
    return a((E, 2 * F, H), H ** -0.5), a((E, H, F), F ** -0.5), g


@pytest.mark.parametrize("E,max_m,H,F,counts", [
    (4, 37, 128, 64, [0, 37, 5, 20]),           # ragged, an empty and a full expert
    (8, 128, 256, 128, "random"),               # 256-row tile kernel
    (16, 8, 128, 64, "random"),                 # weight-streaming kernel
    (12, 48, 192, 128, "random"),               # 64-row tile kernel
    (2, 1, 64, 64, [1, 0]),                     # one-row blocks
    (3, 300, 128, 64, [300, 299, 257]),         # several 256-row tiles per expert
    (5, 16, 128, 64, [-4, 99, 16, 0, 3]),       # out-of-range counts are clamped
])
def test_masked_matches_oracle(E, max_m, H, F, counts):
    w_gu, w_d, g = _weights(E, H, F, seed=E * 1000 + max_m)
    a = torch.randn((E, max_m, H), generator=g, device=DEV).to(torch.bfloat16)
    if counts == "random":
        counts = torch.randint(0, max_m + 1, (E,), generator=g, device=DEV).cpu().tolist()
    m = torch.tensor(counts, dtype=torch.int32, device=DEV)
    out = torch.full((E, max_m, H), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.fused_moe_masked_fwd(a, m, w_gu, w_d, out=out)
    torch.cuda.synchronize()
    _, ref = oracle.masked_mlp(to_u16(a), np.asarray(counts, dtype=np.int32), to_u16(w_gu),
                               to_u16(w_d))
    got = to_u16(out)
    used = np.arange(max_m)[None, :] < np.clip(np.asarray(counts), 0, max_m)[:, None]
    assert np.all(got[~used] == SENTINEL), "a row past masked_m was written"
    if used.any():
        rel = assert_output_close(out[torch.from_numpy(used).to(DEV)], ref[used],
                                  "masked E=%d max_m=%d" % (E, max_m))
        print("masked E=%d max_m=%d: rel-L2 %.2e" % (E, max_m, rel), flush=True)


def test_masked_stages_equal_fused_call():
    E, max_m, H, F = 6, 96, 256, 128
    w_gu, w_d, g = _weights(E, H, F, seed=5)
    a = torch.randn((E, max_m, H), generator=g, device=DEV).to(torch.bfloat16)
    m = torch.tensor([96, 0, 17, 80, 1, 64], dtype=torch.int32, device=DEV)
    fused = moe.fused_moe_masked_fwd(a, m, w_gu, w_d)
    ws = torch.empty(moe.masked_workspace_bytes(E, max_m, H, F), dtype=torch.uint8, device=DEV)
    staged = torch.zeros_like(fused)
    for st in (moe.STAGE_ALIGN, moe.STAGE_GATE_UP, moe.STAGE_DOWN):
        moe.fused_moe_masked_stage(st, a, m, w_gu, w_d, staged, ws)
    torch.cuda.synchronize()
    assert torch.equal(fused, staged)


def _local_ids(ids, shard, n_local):
    lo = shard * n_local
    loc = ids - lo
    return torch.where((ids >= lo) & (ids < lo + n_local), loc, torch.full_like(ids, -1))


def test_ep_shards_sum_to_unsharded_pass():
    """DeepSeek-V3-style routing (sigmoid + bias, 8 groups / top-4, rsf 2.5) over 64 experts split
    into 8 shards of 8: each shard runs the routed pass on its local experts with the other
    shards' routes mapped to -1, matches the oracle on its own, and the 8 shard outputs add up
    to the unsharded pass."""
    cfg = replace(CONFIGS["ds-v3-grouped-prefill"], T=100, H=256, E=64, F=128)
    d = make_inputs(cfg, DEV, num_tokens=cfg.T)
    ids, w = oracle_route(d, cfg)
    ids_t = torch.from_numpy(ids).to(DEV)
    w_t = torch.from_numpy(w).to(DEV)
    full = moe.fused_moe_experts_fwd(d["hidden_states"], d["w_gate_up"], d["w_down"], ids_t, w_t)
    n_local = 8
    total = torch.zeros((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    for shard in range(cfg.E // n_local):
        sl = slice(shard * n_local, (shard + 1) * n_local)
        wgu, wd = d["w_gate_up"][sl].contiguous(), d["w_down"][sl].contiguous()
        loc = _local_ids(ids_t, shard, n_local).to(torch.int32).contiguous()
        out = moe.fused_moe_experts_fwd(d["hidden_states"], wgu, wd, loc, w_t)
        torch.cuda.synchronize()
        _, ref = oracle.experts(to_u16(d["hidden_states"]), to_u16(wgu), to_u16(wd),
                                loc.cpu().numpy(), w)
        assert_output_close(out, ref, "shard %d" % shard)
        total += out.float()
    torch.cuda.synchronize()
    rel = float(torch.linalg.norm(total - full.float()) / torch.linalg.norm(full.float()))
    assert rel < 2e-2, rel


@pytest.mark.slow
def test_ep8_shard_masked_real_shape():
    """One EP8 shard of DeepSeek-V3 at its real shape (32 local experts, H 7168, F 2048, row
    blocks of 128 with 64..128 rows in use; the benchmark's ds-v3-ep8-masked): every row of six
    experts -- the fullest, the emptiest and four others -- against the oracle, and rows past
    masked_m untouched."""
    cfg = MASKED_CONFIGS["ds-v3-ep8-masked"]
    d = make_masked_inputs(cfg, DEV)
    out = torch.full((cfg.E, cfg.max_m, cfg.H), SENTINEL, dtype=torch.int16,
                     device=DEV).view(torch.bfloat16)
    moe.fused_moe_masked_fwd(d["a"], d["masked_m"], d["w_gate_up"], d["w_down"], out=out)
    torch.cuda.synchronize()
    counts = d["masked_m"].cpu().numpy()
    r = np.random.default_rng(1)
    pick = {int(np.argmax(counts)), int(np.argmin(counts))}
    while len(pick) < 6:
        pick.add(int(r.integers(cfg.E)))
    pick = np.array(sorted(pick))
    sel = torch.as_tensor(pick, device=DEV)
    _, ref = oracle.masked_mlp(to_u16(d["a"].index_select(0, sel)), counts[pick],
                               to_u16(d["w_gate_up"].index_select(0, sel)),
                               to_u16(d["w_down"].index_select(0, sel)))
    got = out.index_select(0, sel)
    used = np.arange(cfg.max_m)[None, :] < counts[pick][:, None]
    assert np.all(to_u16(got)[~used] == SENTINEL), "a row past masked_m was written"
    rel = assert_output_close(got[torch.from_numpy(used).to(DEV)], ref[used], "ep8 masked")
    print("ep8 masked experts %s: rel-L2 %.2e" % (pick.tolist(), rel), flush=True)


@pytest.mark.slow
def test_ep8_shard_routed_real_shape():
    """The routed pass on shard 0 of 8 at DeepSeek-V3's real shape: 4096 tokens routed over all
    256 experts (sigmoid + bias, 8 groups / top-4, rsf 2.5), the 32 local experts' weights only,
    the other shards' routes -1; 64+ tokens chosen from the local routing compared with the
    oracle on the same local ids."""
    cfg = CONFIGS["ds-v3-grouped-prefill"]
    d = make_inputs(cfg, DEV, weights=False)
    ids, w = oracle_route(d, cfg)
    n_local = 32
    loc = np.where((ids >= 0) & (ids < n_local), ids, -1).astype(np.int32)
    local = replace(cfg, E=n_local)
    dl = make_inputs(local, DEV)                 # 32 experts of the real shape
    dl["hidden_states"] = d["hidden_states"]
    out = moe.fused_moe_experts_fwd(dl["hidden_states"], dl["w_gate_up"], dl["w_down"],
                                    torch.from_numpy(loc).to(DEV), torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    tokens = routing_tokens(loc, n_local, 256, n=64)
    _, ref = oracle_experts_sampled(dl, loc, w, tokens)
    rel = assert_output_close(out[torch.as_tensor(tokens, device=DEV)], ref, "ep8 routed shard")
    print("ep8 routed shard: %d local routes, rel-L2 %.2e" % (int((loc >= 0).sum()), rel),
          flush=True)
