"""Pin of the oracle's FP8 pass (oracle.fp8_forward) against a numpy chain of the same steps:
dequantised operands (codes x block scales) multiplied with float64 matmuls, one token and one
route at a time.  The block scales factor out of the block sums exactly, so the two agree to
the last bit except where a bf16 rounding of gate/up falls within float64 noise of a tie; a
wrong expert, route order, scale index or weighting would show as a large difference."""
import numpy as np

import oracle


def _codes(rng, shape):
    return ((rng.integers(0, 2, shape) << 7) | (rng.integers(3, 12, shape) << 3) |
            rng.integers(0, 8, shape)).astype(np.uint8)


def _deq(q, s):
    """e4m3 codes [N, K] with scales [N/128, K/128] -> float64"""
    N, K = q.shape
    return oracle.fp8_e4m3_decode(q) * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128,
                                                 1)[:N, :K]


def _bf16(v):
    return oracle.bf16_bits_to_float(oracle.double_to_bf16(v)).astype(np.float64)


def test_fp8_pass_matches_numpy_chain():
    rng = np.random.default_rng(8)
    T, H, E, F, k = 6, 256, 3, 128, 2
    x = oracle.double_to_bf16(rng.standard_normal((T, H)))
    gating = rng.standard_normal((T, E)).astype(np.float32)
    wgu = _codes(rng, (E, 2 * F, H))
    wd = _codes(rng, (E, H, F))
    sgu = ((rng.random((E, 2 * F // 128, H // 128)) + 0.5) * 2.0 ** -9).astype(np.float32)
    sd = ((rng.random((E, H // 128, F // 128)) + 0.5) * 2.0 ** -9).astype(np.float32)
    ids, w, out = oracle.fp8_forward(x, gating, wgu, sgu, wd, sd, k=k)
    ref = np.zeros((T, H))
    for t in range(T):
        xq, xs = oracle.quant_fp8_1x128(x[t:t + 1])
        xd = oracle.fp8_e4m3_decode(xq[0]) * np.repeat(xs[0].astype(np.float64), 128)
        for j in range(k):
            e = ids[t, j]
            gu = _bf16(_deq(wgu[e], sgu[e]) @ xd)
            g, u = gu[:F], gu[F:]
            h = oracle.double_to_bf16(g / (1 + np.exp(-g)) * u)
            hq, hs = oracle.quant_fp8_1x128(h[None, :])
            hd = oracle.fp8_e4m3_decode(hq[0]) * np.repeat(hs[0].astype(np.float64), 128)
            ref[t] += float(w[t, j]) * (_deq(wd[e], sd[e]) @ hd)
    got = oracle.bf16_bits_to_float(out).astype(np.float64)
    want = _bf16(ref)
    assert np.mean(got == want) > 0.99
    assert np.linalg.norm(got - want) <= 1e-3 * np.linalg.norm(want)


def test_fp8_pass_token_subset_and_skipped_experts():
    # rows of a token subset equal the same rows of the whole pass
    rng = np.random.default_rng(9)
    T, H, E, F, k = 5, 128, 4, 128, 2
    x = oracle.double_to_bf16(rng.standard_normal((T, H)))
    gating = rng.standard_normal((T, E)).astype(np.float32)
    wgu, wd = _codes(rng, (E, 2 * F, H)), _codes(rng, (E, H, F))
    sgu = np.full((E, 2, 1), 2.0 ** -8, np.float32)
    sd = np.full((E, 1, 1), 2.0 ** -8, np.float32)
    _, _, whole = oracle.fp8_forward(x, gating, wgu, sgu, wd, sd, k=k)
    _, _, part = oracle.fp8_forward(x, gating, wgu, sgu, wd, sd, k=k, tokens=[3, 0])
    assert np.array_equal(part, whole[[3, 0]])
