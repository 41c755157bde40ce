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
from moe_harness.workloads import CONFIGS, make_inputs, to_u16
from parity import assert_output_close, oracle_route

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
