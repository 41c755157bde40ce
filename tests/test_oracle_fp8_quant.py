"""Pins of the oracle's e4m3 encoder, 1 x 128 activation quantiser and contiguous-layout FP8
grouped GEMM against what the OCP e4m3 format and plain arithmetic fix.

The encoder is the nearest finite e4m3 value with ties to the even code (the format's
round-to-nearest-even), saturating at 448; the quantiser's rule (group scale amax / 448, codes
of x / scale, both divisions in f32) is a reading of the TileOPs "MoE" page's a_scale tensor,
whose shape [.., ceil_div(K, 128)] f32 is all the page gives."""
import numpy as np
import pytest

import oracle


def _bf16(values):
    """float32 values exactly representable in bf16 -> uint16 bits"""
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "not a bf16 value"
    return (bits >> 16).astype(np.uint16)


def test_encode_known_codes():
    # values and codes fixed by the format: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    # exponent 0 is subnormal m/8 * 2^-6
    cases = {1.0: 0x38, 0.5: 0x30, 2.0: 0x40, 1.125: 0x39, 448.0: 0x7E, 240.0: 0x77,
             2.0 ** -6: 0x08, 2.0 ** -9: 0x01, 7 * 2.0 ** -9: 0x07, -1.0: 0xB8, 0.0: 0x00}
    for v, code in cases.items():
        assert oracle.fp8_e4m3_encode([v])[0] == code, v


def test_encode_ties_go_to_even_codes():
    # halfway between 2^-9 (code 1) and 2^-8 (code 2) -> 2; between 0 and 2^-9 -> 0;
    # between 1 (0x38) and 1.125 (0x39) -> 0x38; between 1.125 and 1.25 (0x3A) -> 0x3A
    assert oracle.fp8_e4m3_encode([1.5 * 2.0 ** -9])[0] == 0x02
    assert oracle.fp8_e4m3_encode([2.0 ** -10])[0] == 0x00
    assert oracle.fp8_e4m3_encode([1.0625])[0] == 0x38
    assert oracle.fp8_e4m3_encode([1.1875])[0] == 0x3A


def test_encode_saturates_and_keeps_sign():
    assert list(oracle.fp8_e4m3_encode([460.0, 464.0, 1e9, -500.0])) == [0x7E, 0x7E, 0x7E, 0xFE]
    assert oracle.fp8_e4m3_encode([-0.0])[0] == 0x80


def test_encode_decode_round_trip_and_midpoints():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = oracle.fp8_e4m3_decode(codes)
    assert np.array_equal(oracle.fp8_e4m3_encode(vals), codes)
    pos = np.arange(0x00, 0x7F, dtype=np.uint8)     # 0 .. 448, ascending values
    pv = oracle.fp8_e4m3_decode(pos)
    assert np.all(np.diff(pv) > 0)
    mid = (pv[:-1] + pv[1:]) / 2
    below = oracle.fp8_e4m3_encode(np.nextafter(mid, 0))
    above = oracle.fp8_e4m3_encode(np.nextafter(mid, np.inf))
    at = oracle.fp8_e4m3_encode(mid)
    assert np.array_equal(below, pos[:-1]) and np.array_equal(above, pos[1:])
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(at, even)


def test_quant_group_scale_amax_and_bound():
    rng = np.random.default_rng(5)
    M, K = 6, 384 + 64                              # three full groups and a partial one
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[2, 128:256] *= 1e-3                           # a small-magnitude group
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)   # bf16 values
    q, s = oracle.quant_fp8_1x128(_bf16(x))
    assert q.shape == (M, K) and s.shape == (M, 4)
    dq = oracle.fp8_e4m3_decode(q)
    for r in range(M):
        for g in range(4):
            k0, k1 = 128 * g, min(K, 128 * g + 128)
            xs = x[r, k0:k1]
            amax = np.float32(np.max(np.abs(xs)))
            assert s[r, g] == np.float32(amax / np.float32(448.0))
            # the amax element lands on +-448
            i = int(np.argmax(np.abs(xs)))
            assert abs(dq[r, k0 + i]) == 448.0
            # every code is within half an e4m3 spacing of its f32 quotient
            t = (xs / s[r, g]).astype(np.float32).astype(np.float64)
            err = np.abs(dq[r, k0:k1] - t)
            spacing = np.where(np.abs(t) < 2.0 ** -6, 2.0 ** -9,
                               2.0 ** (np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -6))) - 3))
            assert np.all(err <= spacing / 2 + 1e-12)


def test_quant_zero_group_and_exact_values():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, :128] = 0.0
    x[1, 128] = 448.0                               # scale exactly 1: codes are the values' own
    x[1, 129] = 1.0
    x[1, 130] = -0.5
    x[1, 131] = 2.0 ** -9
    q, s = oracle.quant_fp8_1x128(_bf16(x))
    assert np.all(s[0] == 1.0) and np.all(q[0] == 0) and s[1, 0] == 1.0 and np.all(q[1, :128] == 0)
    assert s[1, 1] == 1.0
    assert list(q[1, 128:132]) == [0x7E, 0x38, 0xB0, 0x01]


def _brute_contig(a, sa, b, sb, off):
    """numpy: dequantise each 1 x 128 / 128 x 128 block and multiply, in float64"""
    P, K = a.shape
    E, N = b.shape[:2]
    da = oracle.fp8_e4m3_decode(a)
    db = oracle.fp8_e4m3_decode(b)
    out = np.zeros((P, N))
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        for kb in range((K + 127) // 128):
            ks = slice(128 * kb, min(K, 128 * kb + 128))
            part = da[r0:r1, ks] @ db[e, :, ks].T
            colscale = np.repeat(sb[e, :, kb].astype(np.float64), 128)[:N]
            out[r0:r1] += part * sa[r0:r1, kb:kb + 1].astype(np.float64) * colscale[None, :]
    return out


@pytest.mark.parametrize("counts", [[3, 0, 5, 1], [0, 0, 0, 9], [4, 4, 4, 4]])
def test_contiguous_gemm_matches_brute_force(counts):
    rng = np.random.default_rng(11)
    E, N, K = 4, 192, 256 + 40
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    P = int(off[-1]) + 2                            # two rows outside every expert
    exp_field = rng.integers(3, 12, size=(P, K))
    a = ((rng.integers(0, 2, (P, K)) << 7) | (exp_field << 3) | rng.integers(0, 8, (P, K)))
    b = ((rng.integers(0, 2, (E, N, K)) << 7) | (rng.integers(3, 12, (E, N, K)) << 3) |
         rng.integers(0, 8, (E, N, K)))
    a, b = a.astype(np.uint8), b.astype(np.uint8)
    sa = (rng.random((P, 3)) + 0.5).astype(np.float32) * 2.0 ** -7
    sb = (rng.random((E, 2, 3)) + 0.5).astype(np.float32) * 2.0 ** -9
    acc, out = oracle.grouped_gemm_fp8_contiguous(a, sa, b, sb, off)
    ref = _brute_contig(a, sa, b, sb, off)
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)
    assert np.all(out[P - 2:] == 0) and np.all(acc[P - 2:] == 0)
    assert np.array_equal(out, oracle.double_to_bf16(acc))
