"""Pins of oracle.masked_mlp (the masked-layout expert MLPs) against an independent numpy
evaluation: for every expert and every row in use, bf16 operands widened to float64, gate and
up projections, z*sigmoid(z)*up, down projection, one rounding to bf16 at the end."""
import numpy as np

import oracle


def _bf16(rng, shape, scale):
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return oracle.double_to_bf16(v.astype(np.float64))


def _widen(bits):
    return oracle.bf16_bits_to_float(bits).astype(np.float64)


def _brute(a, masked_m, w_gu, w_d):
    E, max_m, H = a.shape
    F = w_d.shape[2]
    out = np.zeros((E, max_m, H), dtype=np.float64)
    for e in range(E):
        m = min(max(int(masked_m[e]), 0), max_m)
        x = _widen(a[e, :m])
        g = x @ _widen(w_gu[e, :F]).T
        u = x @ _widen(w_gu[e, F:]).T
        h = g / (1.0 + np.exp(-g)) * u
        out[e, :m] = h @ _widen(w_d[e]).T
    return out


def _case(E, max_m, H, F, masked_m, seed):
    rng = np.random.default_rng(seed)
    a = _bf16(rng, (E, max_m, H), 1.0)
    w_gu = _bf16(rng, (E, 2 * F, H), H ** -0.5)
    w_d = _bf16(rng, (E, H, F), F ** -0.5)
    acc, out = oracle.masked_mlp(a, np.asarray(masked_m, dtype=np.int32), w_gu, w_d)
    ref = _brute(a, masked_m, w_gu, w_d)
    return acc, out, ref


def test_masked_mlp_matches_brute_force():
    acc, out, ref = _case(3, 5, 64, 64, [0, 5, 2], seed=1)
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)
    # one rounding from double: equal bits, up to a last-place tie flip from summation order
    want = oracle.double_to_bf16(ref)
    assert np.max(np.abs(out.astype(np.int32) - want.astype(np.int32))) <= 1
    assert np.all(out[0] == 0) and np.all(out[2, 2:] == 0)


def test_masked_mlp_clamps_counts_and_permutes_with_experts():
    acc, out, ref = _case(4, 6, 64, 128, [-3, 9, 6, 1], seed=2)
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)
    assert np.all(out[0] == 0)                     # negative count: no rows
    assert np.any(out[1, 5] != 0)                  # count past max_m: every row
    # swapping two experts (rows, counts and weights together) swaps their outputs
    rng = np.random.default_rng(3)
    a = _bf16(rng, (2, 4, 64), 1.0)
    w_gu = _bf16(rng, (2, 128, 64), 0.125)
    w_d = _bf16(rng, (2, 64, 64), 0.125)
    m = np.array([3, 1], dtype=np.int32)
    _, o1 = oracle.masked_mlp(a, m, w_gu, w_d)
    _, o2 = oracle.masked_mlp(a[::-1].copy(), m[::-1].copy(), w_gu[::-1].copy(), w_d[::-1].copy())
    assert np.array_equal(o1, o2[::-1])
