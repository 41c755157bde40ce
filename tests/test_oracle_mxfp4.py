"""Pins of the oracle's MXFP4 weight decoding against the OCP MX definitions: e2m1 values
(sign, 2 exponent bits with bias 1, 1 mantissa bit; exponent 0 subnormal), E8M0 scales
2^(s-127) with 255 = NaN, 32-element blocks along K, element 2i in the low nibble of byte i
(the packing reading, the order gfx950's fp4 conversion takes), and exactness in bf16."""
import numpy as np

import oracle


def test_e2m1_table():
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    lib = oracle._load()
    for c in range(16):
        v = lib.oracle_e2m1_to_double(c)
        assert v == (-1 if c & 8 else 1) * want[c & 7], c
    assert np.signbit(lib.oracle_e2m1_to_double(8))     # -0


def test_e8m0_scales():
    lib = oracle._load()
    assert lib.oracle_e8m0_to_double(127) == 1.0
    assert lib.oracle_e8m0_to_double(128) == 2.0
    assert lib.oracle_e8m0_to_double(120) == 2.0 ** -7
    assert lib.oracle_e8m0_to_double(0) == 2.0 ** -127
    assert lib.oracle_e8m0_to_double(254) == 2.0 ** 127
    assert np.isnan(lib.oracle_e8m0_to_double(255))


def test_packing_and_blocks():
    K = 64
    q = np.zeros((1, K // 2), np.uint8)
    q[0, 0] = 0x21            # element 0: code 1 (0.5), element 1: code 2 (1.0)
    q[0, 15] = 0xF7           # element 30: code 7 (6.0), element 31: code 15 (-6.0)
    q[0, 16] = 0x0B           # element 32: code 11 (-1.5), element 33: 0
    s = np.array([[128, 125]], np.uint8)     # x2 for elements 0..31, x1/4 for 32..63
    w = oracle.mxfp4_dequant(q, s)
    assert list(w[0, :2]) == [1.0, 2.0]
    assert list(w[0, 30:34]) == [12.0, -12.0, -0.375, 0.0]
    assert np.count_nonzero(w) == 5


def test_dequant_is_exact_in_bf16():
    rng = np.random.default_rng(4)
    q = rng.integers(0, 256, (8, 64), dtype=np.uint8)
    s = rng.integers(0, 253, (8, 4), dtype=np.uint8)  # scales up to 2^125: 6 * 2^125 < bf16 max
    w = oracle.mxfp4_dequant(q, s)
    back = oracle.bf16_bits_to_float(oracle.mxfp4_to_bf16(q, s)).astype(np.float64)
    assert np.array_equal(w, back)
    # from scale 253 up the largest codes overflow bf16 (6 * 2^126 = 1.5 * 2^128)
    big = oracle.mxfp4_to_bf16(np.array([[0x77] * 16], np.uint8), np.array([[253]], np.uint8))
    assert np.all(np.isinf(oracle.bf16_bits_to_float(big)))
