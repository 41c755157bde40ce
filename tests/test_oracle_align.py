"""Pins of the oracle's align/sort (a stable counting sort of routes by expert, each expert's
segment padded to block_m; TileOPs "MoE" page, MoEPermuteAlignFwd) against numpy's stable
argsort and bincount, and against the invariants the layout must satisfy."""
import numpy as np
import pytest

import oracle


def _numpy_reference(ids, E, bm):
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    padded = -(-counts // bm) * bm
    offsets = np.concatenate([[0], np.cumsum(padded)])
    routes = np.nonzero(valid)[0]
    order = routes[np.argsort(flat[routes], kind="stable")]
    return counts, offsets, order


@pytest.mark.parametrize("T,k,E,bm,pad,rep", [
    (4, 2, 8, 1, 0.0, False), (32, 8, 128, 16, 0.0, False), (57, 8, 64, 32, 0.1, False),
    (300, 6, 40, 64, 0.05, True), (5, 8, 256, 128, 0.2, False), (1, 1, 1, 4, 0.0, False),
    (0, 8, 16, 16, 0.0, False),
])
def test_align_matches_stable_argsort(T, k, E, bm, pad, rep):
    r = np.random.default_rng(T * 31 + E)
    if rep:
        ids = r.integers(0, E, (T, k)).astype(np.int32)
    else:
        ids = np.array([r.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    if pad > 0:
        ids[r.random((T, k)) < pad] = -1
    out = oracle.align_sort(ids, E, bm)
    counts, offsets, order = _numpy_reference(ids, E, bm)
    assert np.array_equal(out["expert_offsets"], offsets)
    assert out["n_tiles"] == int(np.sum(-(-counts // bm)))
    srt = out["sorted_route_ids"]
    assert srt.size == T * k + E * (bm - 1)
    # each expert's segment: its routes in increasing route order, then -1 padding
    got = []
    for e in range(E):
        seg = srt[offsets[e]:offsets[e + 1]]
        c = counts[e]
        assert np.all(seg[c:] == -1)
        assert np.all(np.diff(seg[:c]) > 0)              # stable: increasing route index
        assert np.all(ids.ravel()[seg[:c]] == e)
        got.extend(seg[:c].tolist())
    assert got == order.tolist()
    assert np.all(srt[offsets[E]:] == -1)
    assert np.all(offsets % bm == 0)
    inv = out["inverse_pos"]
    flat = ids.ravel()
    for rr in range(T * k):
        if 0 <= flat[rr] < E:
            assert srt[inv[rr]] == rr
        else:
            assert inv[rr] == -1
    te = out["tile_expert"]
    for i in range(out["n_tiles"]):
        e = te[i]
        assert offsets[e] <= i * bm < offsets[e + 1]
    assert np.all(te[out["n_tiles"]:] == -1)


def test_out_of_range_ids_are_skipped_like_padding():
    ids = np.array([[0, 9], [-1, 3], [-7, 3]], np.int32)
    out = oracle.align_sort(ids, 4, 2)
    assert list(out["inverse_pos"]) == [0, -1, -1, 2, -1, 3]
    assert list(out["expert_offsets"]) == [0, 2, 2, 2, 4]


def test_page_example_padding_arithmetic():
    """FlashInfer BF16-activation PR, "Why 4096 remains bandwidth-sensitive": 3715 routes over
    32 experts padded to 128-row tiles give 40 tiles = 5120 slots, 72.56% useful.  Build a
    routing with those totals and check the slot count and the useful-row share."""
    counts = [116] * 31 + [3715 - 116 * 31]          # 31*116 + 119 = 3715
    assert sum(counts) == 3715
    # 116 rows -> 1 tile each; 119 -> 1 tile: 32 tiles.  Move rows so that 8 experts need 2 tiles
    counts = [100] * 24 + [164] * 8
    counts[0] += 3715 - sum(counts)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    out = oracle.align_sort(ids.reshape(-1, 1), 32, 128)
    assert out["n_tiles"] == 40
    assert out["expert_offsets"][-1] == 5120
    assert round(3715 / 5120 * 100, 2) == 72.56
