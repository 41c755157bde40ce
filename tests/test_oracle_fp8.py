"""Pins of the oracle's FP8 pieces.

The e4m3 decoder is checked code by code against torch's float8_e4m3fn conversion (a library
routine) and against values the OCP format fixes; the block-scaled grouped GEMM against a numpy
evaluation that decodes through torch, and against closed forms (all-ones operands, a zero
scale block, a swapped pair of experts)."""
import numpy as np
import torch

import oracle


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]


def test_e4m3_fixed_values():
    vals = dict(zip([0x00, 0x80, 0x38, 0xB8, 0x40, 0x30, 0x7E, 0xFE, 0x01, 0x08, 0x07],
                    oracle.fp8_e4m3_decode(np.array([0x00, 0x80, 0x38, 0xB8, 0x40, 0x30, 0x7E,
                                                     0xFE, 0x01, 0x08, 0x07], np.uint8))))
    assert vals[0x00] == 0.0 and vals[0x80] == 0.0 and np.signbit(vals[0x80])
    assert vals[0x38] == 1.0 and vals[0xB8] == -1.0 and vals[0x40] == 2.0 and vals[0x30] == 0.5
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0          # largest finite
    assert vals[0x01] == 2.0 ** -9                                # smallest subnormal
    assert vals[0x08] == 2.0 ** -6 and vals[0x07] == 7 * 2.0 ** -9  # normal / subnormal edge


def _inputs(E, max_m, N, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (E, max_m, K), dtype=np.uint8)
    b = rng.integers(0, 256, (E, N, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x3C     # no NaN codes
    b[(b & 0x7F) == 0x7F] = 0x44
    sa = rng.uniform(0.5, 1.5, (E, max_m, (K + 127) // 128)).astype(np.float32)
    sb = rng.uniform(0.5, 1.5, (E, (N + 127) // 128, (K + 127) // 128)).astype(np.float32)
    return a, sa, b, sb


def _numpy_ref(a, sa, b, sb, masked_m):
    E, max_m, K = a.shape
    N = b.shape[1]
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    A, B = dec(a), dec(b)
    out = np.zeros((E, max_m, N))
    for e in range(E):
        m = min(max(int(masked_m[e]), 0), max_m)
        for kb in range((K + 127) // 128):
            ks = slice(kb * 128, min(K, kb * 128 + 128))
            part = A[e, :m, ks] @ B[e, :, ks].T                       # [m, N]
            scale = (sa[e, :m, kb].astype(np.float64)[:, None]
                     * np.repeat(sb[e, :, kb].astype(np.float64), 128)[:N][None, :])
            out[e, :m] += scale * part
    return out


def test_grouped_gemm_fp8_matches_numpy():
    a, sa, b, sb = _inputs(3, 5, 256 + 64, 384, seed=1)     # ragged last N block of 64
    m = np.array([5, 0, 3], dtype=np.int32)
    acc, out = oracle.grouped_gemm_fp8(a, sa, b, sb, m)
    ref = _numpy_ref(a, sa, b, sb, m)
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
    want = oracle.double_to_bf16(ref)
    assert np.max(np.abs(out.astype(np.int32) - want.astype(np.int32))) <= 1
    assert np.all(out[1] == 0) and np.all(out[2, 3:] == 0)


def test_grouped_gemm_fp8_closed_forms():
    E, max_m, N, K = 2, 4, 128, 256
    a = np.full((E, max_m, K), 0x38, np.uint8)                     # 1.0
    b = np.full((E, N, K), 0x40, np.uint8)                         # 2.0
    sa = np.ones((E, max_m, 2), np.float32)
    sb = np.ones((E, 1, 2), np.float32)
    sb[1, 0, 1] = 0.0                                              # expert 1: second block off
    sa[0, 2, 0] = 0.25
    acc, _ = oracle.grouped_gemm_fp8(a, sa, b, sb, np.array([4, 4], np.int32))
    assert np.all(acc[0, [0, 1, 3]] == 2.0 * K)
    assert np.all(acc[0, 2] == 2.0 * 128 * 0.25 + 2.0 * 128)
    assert np.all(acc[1] == 2.0 * 128)
    # swapping the experts (operands, scales and counts together) swaps the outputs
    a, sa, b, sb = _inputs(2, 3, 128, 128, seed=4)
    m = np.array([3, 1], np.int32)
    _, o1 = oracle.grouped_gemm_fp8(a, sa, b, sb, m)
    _, o2 = oracle.grouped_gemm_fp8(a[::-1], sa[::-1], b[::-1], sb[::-1], m[::-1])
    assert np.array_equal(o1, o2[::-1])
