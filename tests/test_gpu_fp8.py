"""GPU parity of the block-scaled FP8 grouped GEMMs (moe_grouped_gemm_fp8 on the masked layout,
moe_grouped_gemm_fp8_contiguous on the contiguous one) and of the 1 x 128 activation quantiser
(moe_quant_fp8, bit-exact codes and scales) against the oracle.

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
    (4, 16, 256, 2048, [16, 0, 1, 9]),         # weight-streaming form (decode): 4-way K split
    (3, 12, 192, 384, [12, 5, 0]),             # weight-streaming form: 2-way K split, N % 32
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


def _contig_inputs(E, counts, N, K, seed, extra_rows=3):
    """a [P,K] e4m3 rows (the experts' rows stacked, then extra rows of no expert), offsets."""
    g = torch.Generator().manual_seed(seed)
    off = torch.zeros(E + 1, dtype=torch.int32)
    off[1:] = torch.cumsum(torch.tensor(counts, dtype=torch.int32), 0)
    P = int(off[-1]) + extra_rows
    d = make_fp8_inputs(Fp8Config("c", E, 1, N, K, 0), DEV, seed=seed)
    from moe_harness.workloads import random_e4m3_codes
    d["a"] = random_e4m3_codes((P, K), g, DEV)
    d["a_scale"] = ((torch.rand((P, (K + 127) // 128), generator=g) + 0.5) * 2.0 ** -7).to(DEV)
    d["offsets"] = off.to(DEV)
    del d["masked_m"]
    return d, P


@pytest.mark.parametrize("E,counts,N,K", [
    (4, [5, 0, 37, 64], 192, 384),            # 64-row form: ragged, an empty expert
    (3, [130, 1, 64], 128, 256),              # 64-row form: several row tiles of one expert
    (3, [300, 77, 256], 256, 1024),           # 256-row form (mean rows > 64), partial tiles
    (2, [130, 90], 256, 9216),                # 256-row form past 64 k-blocks (a wave's weight
                                              # scales span two registers)
    (6, [1, 0, 3, 17, 2, 5], 192, 384),       # weight-streaming form (mean rows <= 8): a
                                              # 17-row expert takes two 16-row passes
    (8, [2, 1, 0, 4, 3, 1, 2, 2], 256, 2048),  # weight-streaming form, 4-way K split
    (2, [0, 0], 64, 128),                     # no rows at all
])
def test_fp8_contiguous_matches_oracle(E, counts, N, K):
    d, P = _contig_inputs(E, counts, N, K, seed=E * 7 + N)
    out = torch.full((P, N), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.moe_grouped_gemm_fp8_contiguous(d["a"], d["a_scale"], d["b"], d["b_scale"],
                                        d["offsets"], out=out)
    torch.cuda.synchronize()
    h = _host(d)
    args = (h["a"], h["a_scale"], h["b"], h["b_scale"], h["offsets"])
    _, ref = oracle.grouped_gemm_fp8_contiguous(*args)
    A, _ = oracle.grouped_gemm_fp8_contiguous(h["a"] & 0x7F, h["a_scale"], h["b"] & 0x7F,
                                              h["b_scale"], h["offsets"])
    got = to_u16(out)
    used = np.arange(P) < int(h["offsets"][-1])
    assert np.all(got[~used] == SENTINEL), "a row of no expert was written"
    _close(got[used], ref[used], A[used], "fp8 contiguous E=%d N=%d K=%d" % (E, N, K))


def test_fp8_contiguous_equals_masked_layout():
    """The same rows through both layouts give the same bits (both pick the 256-row form here:
    max_m 96 and mean rows 82 are above 64; same expert order, same sums per row)."""
    E, max_m, N, K = 3, 96, 256, 512
    counts = [96, 80, 70]
    d = make_fp8_inputs(Fp8Config("t", E, max_m, N, K, 0), DEV, seed=3)
    d["masked_m"] = torch.tensor(counts, dtype=torch.int32, device=DEV)
    masked = to_u16(_run(d))
    rows = torch.cat([d["a"][e, :c] for e, c in enumerate(counts)])
    srows = torch.cat([d["a_scale"][e, :c] for e, c in enumerate(counts)])
    off = torch.tensor([0, 96, 176, 246], dtype=torch.int32, device=DEV)
    got = to_u16(moe.moe_grouped_gemm_fp8_contiguous(rows, srows, d["b"], d["b_scale"], off))
    want = np.concatenate([masked[e, :c] for e, c in enumerate(counts)])
    assert np.array_equal(got, want)


def _bf16_rows(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[1] = 0.0                                          # an all-zero row
    x[2] *= 2.0 ** -12                                  # codes in the subnormal range
    x[3, :64] *= 1e4                                    # one large value per group dominates
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("M,K", [(5, 128), (7, 200), (33, 7168), (4, 2048 + 8)])
def test_quant_fp8_bit_exact(M, K):
    x = _bf16_rows(M, K, seed=M + K)
    q, s = moe.moe_quant_fp8(x.to(DEV))
    torch.cuda.synchronize()
    rq, rs = oracle.quant_fp8_1x128(to_u16(x))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "scales differ"
    got = q.cpu().numpy()
    bad = np.argwhere(got != rq)
    assert bad.size == 0, "codes differ at %s: got %s want %s" % (
        bad[:4].tolist(), got[tuple(bad[:4].T)], rq[tuple(bad[:4].T)])


def test_quant_then_contiguous_gemm_matches_oracle_chain():
    """bf16 rows -> quantiser -> contiguous GEMM, against the oracle's quantiser and GEMM."""
    E, counts, N, K = 3, [40, 0, 90], 128, 512
    P = sum(counts)
    x = _bf16_rows(P, K, seed=9)
    d, _ = _contig_inputs(E, counts, N, K, seed=5, extra_rows=0)
    q, s = moe.moe_quant_fp8(x.to(DEV))
    got = to_u16(moe.moe_grouped_gemm_fp8_contiguous(q, s, d["b"], d["b_scale"], d["offsets"]))
    torch.cuda.synchronize()
    rq, rs = oracle.quant_fp8_1x128(to_u16(x))
    h = _host(d)
    _, ref = oracle.grouped_gemm_fp8_contiguous(rq, rs, h["b"], h["b_scale"], h["offsets"])
    A, _ = oracle.grouped_gemm_fp8_contiguous(rq & 0x7F, rs, h["b"] & 0x7F, h["b_scale"],
                                              h["offsets"])
    _close(got, ref, A, "quant + contiguous fp8")

