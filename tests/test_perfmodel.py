"""The FLOP/byte model used for roofline reporting, pinned by numbers the pages print."""
import os

import pytest

from moe_harness import perfmodel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tileops_moe_tflops.txt")


def _rows():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, T, H, E, F, k, S, ms, tf = line.split()
        rows.append((name, int(T), int(H), int(E), int(F), int(k), int(S), float(ms), float(tf)))
    return rows


@pytest.mark.parametrize("row", _rows(), ids=lambda r: r[0])
def test_flops_reproduce_tileops_tflops_column(row):
    """The page's TFLOP/s column = 2*T*k*3*H*F (+ 2*T*3*H*S) / device time.  The printed
    values carry three significant digits."""
    name, T, H, E, F, k, S, ms, tf = row
    got = perfmodel.flops(T, k, H, F, S) / (ms * 1e-3) / 1e12
    assert abs(got - tf) / tf < 0.006, (name, got, tf)


def test_unique_weight_bytes_match_flashinfer_ep8_example():
    """FlashInfer BF16-activation PR, "Why 4096 remains bandwidth-sensitive": the 32 local
    DeepSeek-V3 experts (H=7168, I=2048) hold 2.819 GB of bf16 weights, and useful FLOPs per
    unique weight byte equal the routed rows per expert, 3715/32 = 116.09."""
    w = 32 * perfmodel.expert_weight_bytes(7168, 2048)
    assert round(w / 1e9, 3) == 2.819
    fl = perfmodel.routed_flops(3715, 1, 7168, 2048)
    assert round(fl / w, 2) == 116.09


def test_algorithmic_bytes_terms():
    b = perfmodel.algorithmic_bytes(T=32, H=2048, E=128, F=768, k=8, touched=100)
    assert b == 100 * 6 * 2048 * 768 + 4 * 32 * 2048 + 4 * 32 * 128 + 8 * 32 * 8
    b2 = perfmodel.algorithmic_bytes(T=1, H=16, E=4, F=8, k=2, touched=2, S=32, bias=True)
    assert b2 == 2 * 6 * 16 * 8 + 6 * 16 * 32 + 4 * 16 + 4 * 4 + 4 * 4 + 16


def test_load_stats():
    import numpy as np
    ids = np.array([[0, 1], [1, 3], [-1, 1]])
    s = perfmodel.load_stats(ids, 4)
    assert s == {"touched": 3, "min": 1, "max": 3, "median": 1.0}
    assert perfmodel.touched_experts(ids, 4) == 3
