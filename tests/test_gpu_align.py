"""GPU parity of moe_align_sort against the oracle: every output bit-exact."""
import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ids(T, k, E, seed, pad=0.0, repeats=False, skew=False):
    r = np.random.default_rng(seed)
    if repeats:
        ids = r.integers(0, E, (T, k))
    elif skew:
        ids = np.minimum(r.geometric(0.3, (T, k)) - 1, E - 1)
    else:
        ids = np.array([r.permutation(E)[:k] for _ in range(T)]).reshape(T, k)
    if pad > 0:
        ids[r.random((T, k)) < pad] = -1
    return ids.astype(np.int32)


@pytest.mark.parametrize("T,k,E,bm,pad,repeats,skew", [
    (4, 2, 8, 16, 0.0, False, False),
    (32, 8, 128, 16, 0.0, False, False),
    (512, 8, 128, 16, 0.0, False, False),
    (4096, 8, 256, 128, 0.0, False, False),
    (4096, 8, 256, 256, 0.0, False, True),  # DeepSeek-V3 prefill size, chunked, skewed
    (1025, 1, 16, 16, 0.0, False, False),    # two chunks, the second holding one route
    (4096, 8, 256, 16, 0.05, False, False),
    (512, 8, 384, 16, 0.0, False, False),
    (1000, 6, 1024, 1, 0.1, True, False),
    (777, 3, 40, 64, 0.0, False, True),     # heavy skew: one expert holds most routes
    (3, 8, 1024, 32, 0.2, False, False),
    (1, 1, 1, 1024, 0.0, False, False),
    (50, 4, 7, 5, 0.3, True, False),
])
def test_align_sort_matches_oracle(T, k, E, bm, pad, repeats, skew):
    ids = _ids(T, k, E, seed=T + E, pad=pad, repeats=repeats, skew=skew)
    ids[0, 0] = E + 3 if T * k > 1 else ids[0, 0]          # out-of-range id: skipped
    ref = oracle.align_sort(ids, E, bm)
    got = moe.moe_align_sort(torch.from_numpy(ids).to(DEV), E, bm)
    torch.cuda.synchronize()
    for key in ("sorted_route_ids", "expert_offsets", "tile_expert", "inverse_pos"):
        g = got[key].cpu().numpy()
        assert np.array_equal(g, ref[key]), key
    assert int(got["n_tiles"].item()) == ref["n_tiles"]


def test_align_sort_overwrites_poisoned_outputs():
    ids = _ids(64, 8, 32, seed=3, pad=0.1)
    got = moe.moe_align_sort(torch.from_numpy(ids).to(DEV), 32, 16)
    for v in got.values():
        v.fill_(0x7abcdef0 & 0x7fffffff)
    # the call writes every element of every output again
    ids_dev = torch.from_numpy(ids).to(DEV)
    st = moe.lib().moe_align_sort(
        moe._ptr(ids_dev), 64, 8, 32, 16,
        moe._ptr(got["sorted_route_ids"]), moe._ptr(got["expert_offsets"]),
        moe._ptr(got["tile_expert"]), moe._ptr(got["inverse_pos"]), moe._ptr(got["n_tiles"]),
        None, 0, moe._stream(torch.device(DEV)))
    assert st == 0
    torch.cuda.synchronize()
    ref = oracle.align_sort(ids, 32, 16)
    for key in ("sorted_route_ids", "expert_offsets", "tile_expert", "inverse_pos"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key


def test_align_sort_chunked_poisoned_workspace():
    """32768 routes through the public call with a workspace that holds stale values: the
    chunked form writes every count it reads, and every output matches the oracle."""
    ids = _ids(4096, 8, 256, seed=11, pad=0.02)
    need = moe.moe_align_sort_workspace_bytes(4096, 8, 256, 256)
    ws = torch.full((need // 4,), 0x3c3c3c3c, dtype=torch.int32, device=DEV).view(torch.uint8)
    ref = oracle.align_sort(ids, 256, 256)
    for _ in range(2):
        got = moe.moe_align_sort(torch.from_numpy(ids).to(DEV), 256, 256, workspace=ws)
        torch.cuda.synchronize()
        for key in ("sorted_route_ids", "expert_offsets", "tile_expert", "inverse_pos"):
            assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
        assert int(got["n_tiles"].item()) == ref["n_tiles"]
