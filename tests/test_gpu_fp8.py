"""GPU parity of the block-scaled FP8 grouped GEMM (moe_grouped_gemm_fp8) against the oracle.

Bound per element: one bf16 step of the result plus the accumulation error,
|got - ref| <= 2^-7 |ref| + 2^-12 A, where A = sum_kb sa*sb*sum_k |a_k b_k| (the oracle on
sign-stripped codes).  The products of e4m3 codes are exact and the K/128 block sums are added
in f32, but the 16x16x128 FP8 MFMA sums a block's 128 products with less than f32 precision:
on MI355X, errors of ~3e-5 A show up where the sum cancels (f32 alone would stay below
(128 + K/128) 2^-24 A ~ 8e-6 A at K = 384).  2^-12 A leaves 8x room over that.
Rows past masked_m must keep the caller's bytes.  Full-size decode shapes compare two experts on
the first and last 256 output columns, which the oracle evaluates directly."""
import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe
import oracle
from moe_harness.workloads import FP8_CONFIGS, Fp8Config, make_fp8_inputs, to_u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = 0x7FC1


def _abs_sum(a, sa, b, sb, m):
    """sum_kb sa*sb*sum_k |a_k b_k| from the oracle on sign-stripped codes."""
    acc, _ = oracle.grouped_gemm_fp8(a & 0x7F, sa, b & 0x7F, sb, m)
    return acc


def _close(got_bits, ref_bits, abs_sum, what):
    g = oracle.bf16_bits_to_float(got_bits).astype(np.float64)
    r = oracle.bf16_bits_to_float(ref_bits).astype(np.float64)
    assert np.all(np.isfinite(g)), "%s: non-finite output" % what
    bound = 2.0 ** -7 * np.abs(r) + 2.0 ** -12 * abs_sum
    worst = np.max(np.abs(g - r) - bound) if g.size else -1.0
    assert worst <= 0, "%s: an element exceeds one bf16 step by %.3e" % (what, worst)


def _run(d, out=None):
    out = moe.moe_grouped_gemm_fp8(d["a"], d["a_scale"], d["b"], d["b_scale"], d["masked_m"],
                                   out=out)
    torch.cuda.synchronize()
    return out


def _host(d):
    return {k: v.cpu().numpy() for k, v in d.items()}


@pytest.mark.parametrize("E,max_m,N,K,counts", [
    (3, 37, 192, 384, [37, 0, 20]),           # ragged rows, an empty expert, N past 128
    (4, 64, 256, 512, None),                   # one 64-row tile per expert
    (2, 130, 128, 256, [130, 65]),             # three row tiles, a partial last one
    (5, 16, 64, 128, [-1, 99, 16, 0, 3]),      # one k-block; counts clamped to [0, max_m]
    (3, 200, 256, 1024, [200, 7, 130]),        # 256-row form, 128 columns per workgroup
    (512, 65, 256, 512, None),                 # 256-row form, 256 columns per workgroup
])
def test_fp8_small_matches_oracle(E, max_m, N, K, counts):
    d = make_fp8_inputs(Fp8Config("t", E, max_m, N, K, 0), DEV, seed=E + max_m)
    if counts is not None:
        d["masked_m"] = torch.tensor(counts, dtype=torch.int32, device=DEV)
    out = torch.full((E, max_m, N), SENTINEL, dtype=torch.int16,
                     device=DEV).view(torch.bfloat16)
    _run(d, out)
    h = _host(d)
    args = (h["a"], h["a_scale"], h["b"], h["b_scale"], h["masked_m"])
    _, ref = oracle.grouped_gemm_fp8(*args)
    A = _abs_sum(*args)
    got = to_u16(out)
    used = np.arange(max_m)[None, :] < np.clip(h["masked_m"], 0, max_m)[:, None]
    assert np.all(got[~used] == SENTINEL), "a row past masked_m was written"
    _close(got[used], ref[used], A[used], "fp8 E=%d max_m=%d N=%d K=%d" % (E, max_m, N, K))


@pytest.mark.parametrize("name", ["ds-v3-dec-b64-up", "ds-v3-dec-b64-down"])
def test_fp8_decode_shapes_sampled(name):
    cfg = FP8_CONFIGS[name]
    d = make_fp8_inputs(cfg, DEV)
    got = to_u16(_run(d))
    h = _host(d)
    for e in (0, cfg.E - 1):
        for cols in (slice(0, 256), slice(cfg.N - 256, cfg.N)):
            nb = slice(cols.start // 128, cols.stop // 128)
            args = (h["a"][e:e + 1], h["a_scale"][e:e + 1], h["b"][e:e + 1, cols],
                    h["b_scale"][e:e + 1, nb], h["masked_m"][e:e + 1])
            _, ref = oracle.grouped_gemm_fp8(*args)
            A = _abs_sum(*args)
            m = int(h["masked_m"][e])
            _close(got[e, :m, cols], ref[0, :m], A[0, :m],
                   "%s expert %d cols %s" % (name, e, cols))


def test_fp8_nan_code_poisons_only_its_row():
    cfg = Fp8Config("t", 2, 32, 128, 256, 32)
    d = make_fp8_inputs(cfg, DEV, seed=3)
    d["a"][1, 7, 200] = 0x7F                   # NaN code in expert 1, row 7
    out = _run(d).float()
    assert torch.all(torch.isnan(out[1, 7]))
    out[1, 7] = 0
    assert torch.all(torch.isfinite(out))
