"""Pins of the oracle's f16 element type: the binary16 rounding against numpy's float16
conversion (IEEE round to nearest even, a library routine), and the f16 expert evaluation
against the bf16 one on inputs exact in both types (their double sums are then identical, so
the two results differ only in the final rounding)."""
import numpy as np

import oracle


def test_double_to_f16_matches_numpy():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 5, 4000),   # subnormal .. 1e4
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, -1e9, 2.0 ** -24,
                  2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]),
    ])
    got = oracle.double_to_f16(vals)
    with np.errstate(over="ignore"):  # 65520 and above round to infinity on purpose
        want = vals.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "differs at %s" % vals[bad[:5]]


def test_f16_decode_through_experts_matches_numpy():
    # E = 1, k = 1 with identity-like weights: out equals the dense MLP, computed here with numpy
    # from numpy's own float16 decoding of the same bits
    rng = np.random.default_rng(2)
    H, F = 64, 64
    x = (rng.standard_normal((3, H)) * 0.5).astype(np.float16)
    wgu = (rng.standard_normal((1, 2 * F, H)) / 8).astype(np.float16)
    wd = (rng.standard_normal((1, H, F)) / 8).astype(np.float16)
    ids = np.zeros((3, 1), np.int32)
    w = np.ones((3, 1), np.float32)
    acc, out = oracle.experts(x.view(np.uint16), wgu.view(np.uint16), wd.view(np.uint16), ids, w,
                              dtype="f16")
    xd, g, u, d = (x.astype(np.float64), wgu[0, :F].astype(np.float64),
                   wgu[0, F:].astype(np.float64), wd[0].astype(np.float64))
    gate, up = xd @ g.T, xd @ u.T
    ref = (gate / (1 + np.exp(-gate)) * up) @ d.T
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out, ref.astype(np.float16).view(np.uint16))


def test_f16_and_bf16_agree_on_shared_values():
    # values with few significant bits and moderate exponents are exact in both types
    rng = np.random.default_rng(3)
    T, H, E, F, k = 5, 128, 4, 64, 2

    def vals(shape, scale):
        return (rng.integers(-15, 16, shape) * scale).astype(np.float32)

    x, wgu, wd = vals((T, H), 2.0 ** -3), vals((E, 2 * F, H), 2.0 ** -6), vals((E, H, F), 2.0 ** -6)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = np.full((T, k), 0.5, np.float32)
    as_bf16 = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    as_f16 = lambda a: a.astype(np.float16).view(np.uint16)
    acc_b, out_b = oracle.experts(as_bf16(x), as_bf16(wgu), as_bf16(wd), ids, w)
    acc_h, out_h = oracle.experts(as_f16(x), as_f16(wgu), as_f16(wd), ids, w, dtype="f16")
    assert np.array_equal(acc_b, acc_h)
    assert np.array_equal(out_b, oracle.double_to_bf16(acc_b))
    assert np.array_equal(out_h, oracle.double_to_f16(acc_h))
