"""Workload shapes and seeded synthetic inputs for the fused MoE forward pass.

This module holds no arithmetic of the method.  It only fixes shapes, value distributions and a
seeded generator, and it is the one module that both the GPU path's tests and the CPU oracle
receive their inputs from.

Shapes follow the model-shaped workloads of the TileOPs "MoE" benchmark page (FusedMoEFwd and
FusedMoESharedExpertFwd tables): Qwen3-30B decode, Qwen3-235B batch, DeepSeek-V3 grouped
prefill and Kimi-K2 with a shared expert, plus a tiny case.  The pages' workloads are themselves
synthetic tensors of these shapes; no dataset is involved.

Distributions: hidden_states ~ N(0,1) rounded to bf16; gating_output ~ N(0,1) f32;
correction_bias ~ N(0, 0.1^2) f32; every weight ~ N(0, 1/fan_in) (std 1/sqrt(fan_in)) rounded
to bf16, fan_in = H for w_gate_up and shared_w_gate_up, F for w_down, S for shared_w_down.
Rounding to bf16 is torch's f32 -> bf16 conversion (nearest-even).

Seeding: seed 42 by default; each tensor draws from its own torch generator seeded with
``seed * 1000 + stream`` (streams: hidden 1, gating 2, bias 3, w_gate_up 4, w_down 5,
shared_w_gate_up 6, shared_w_down 7), filled one expert slice at a time on the target device.
The same (seed, device type, shape) always gives the same bytes; CPU and GPU generators give
different streams, so a test draws once and hands the same bytes to both sides.
"""
from dataclasses import dataclass, replace
from typing import Optional

import json
import math
import os

import torch

STREAM_HIDDEN = 1
STREAM_GATING = 2
STREAM_BIAS = 3
STREAM_W_GATE_UP = 4
STREAM_W_DOWN = 5
STREAM_SHARED_GATE_UP = 6
STREAM_SHARED_DOWN = 7
STREAM_SKEW = 8
STREAM_MASKED_COUNTS = 11
STREAM_FP8 = 12
STREAM_MXFP4 = 13


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size
    E: int            # experts
    F: int            # expert intermediate size
    k: int            # top_k
    scoring: str = "softmax"       # "softmax" | "sigmoid"
    renormalize: bool = True
    num_expert_group: int = 1
    topk_group: int = 1
    rsf: float = 1.0               # routed_scaling_factor
    bias: bool = False             # correction_bias present
    S: int = 0                     # shared expert intermediate size (0 = none)

    def with_tokens(self, T: int) -> "MoEConfig":
        return replace(self, T=T)


CONFIGS = {
    "tiny": MoEConfig("tiny", T=4, H=128, E=8, F=64, k=2),
    "qwen3-30b-decode": MoEConfig("qwen3-30b-decode", T=32, H=2048, E=128, F=768, k=8),
    "qwen3-235b-batch": MoEConfig("qwen3-235b-batch", T=512, H=4096, E=128, F=1536, k=8),
    "ds-v3-grouped-prefill": MoEConfig("ds-v3-grouped-prefill", T=4096, H=7168, E=256, F=2048,
                                       k=8, scoring="sigmoid", num_expert_group=8,
                                       topk_group=4, rsf=2.5, bias=True),
    "kimi-k2-shared": MoEConfig("kimi-k2-shared", T=512, H=7168, E=384, F=2048, k=8,
                                scoring="sigmoid", rsf=2.827, bias=True, S=18432),
    # further TileOPs FusedMoEFwd rows (the page's Kimi-K2 rows without the shared expert list
    # E = 256)
    "qwen3-30b-decode-b1": MoEConfig("qwen3-30b-decode-b1", T=1, H=2048, E=128, F=768, k=8),
    "qwen3-235b-prefill": MoEConfig("qwen3-235b-prefill", T=4096, H=4096, E=128, F=1536, k=8),
    "ds-v3-grouped-decode": MoEConfig("ds-v3-grouped-decode", T=512, H=7168, E=256, F=2048,
                                      k=8, scoring="sigmoid", num_expert_group=8,
                                      topk_group=4, rsf=2.5, bias=True),
    "kimi-k2-decode": MoEConfig("kimi-k2-decode", T=512, H=7168, E=256, F=2048, k=8,
                                scoring="sigmoid", rsf=2.827, bias=True),
    "kimi-k2-prefill": MoEConfig("kimi-k2-prefill", T=4096, H=7168, E=256, F=2048, k=8,
                                 scoring="sigmoid", rsf=2.827, bias=True),
    # DeepSeek-V3 routing and dimensions at 16384 tokens: about 500 routed rows per expert, so
    # about 500 FLOP per weight byte, above the MI355X ridge (2.5 PFLOP/s / 8 TB/s = 312): the
    # expert GEMMs are MFMA-bound here, unlike at 4096 tokens
    "ds-v3-prefill-16k": MoEConfig("ds-v3-prefill-16k", T=16384, H=7168, E=256, F=2048, k=8,
                                   scoring="sigmoid", num_expert_group=8, topk_group=4,
                                   rsf=2.5, bias=True),
}


@dataclass(frozen=True)
class MaskedConfig:
    """Masked-layout workload of one expert-parallel shard: E local experts, row blocks of
    max_m, rows in use per expert drawn uniformly from [lo, max_m]."""
    name: str
    E: int
    max_m: int
    H: int
    F: int
    lo: int


# TileOPs "MoE" page, MoEGroupedGemmFwd ds-v3-ep8-masked: a [32, 128, 7168], b [32, 4096, 7168];
# its TFLOP/s figure implies about 96 rows in use per expert, the mean of counts in [64, 128]
MASKED_CONFIGS = {
    "ds-v3-ep8-masked": MaskedConfig("ds-v3-ep8-masked", E=32, max_m=128, H=7168, F=2048, lo=64),
}


def make_masked_inputs(cfg: MaskedConfig, device="cpu", seed: int = 42) -> dict:
    """a [E,max_m,H] bf16, masked_m [E] int32, w_gate_up [E,2F,H] and w_down [E,H,F] bf16."""
    E, m, H, F = cfg.E, cfg.max_m, cfg.H, cfg.F
    g = _gen("cpu", seed, STREAM_MASKED_COUNTS)
    counts = torch.randint(cfg.lo, m + 1, (E,), generator=g, dtype=torch.int32)
    return {
        "a": _normal((E, m, H), 1.0, torch.bfloat16, device, seed, STREAM_HIDDEN),
        "masked_m": counts.to(device),
        "w_gate_up": _normal((E, 2 * F, H), H ** -0.5, torch.bfloat16, device, seed,
                             STREAM_W_GATE_UP),
        "w_down": _normal((E, H, F), F ** -0.5, torch.bfloat16, device, seed, STREAM_W_DOWN),
    }


def random_e4m3_codes(shape, generator, device="cpu") -> torch.Tensor:
    """Seeded OCP e4m3 codes (uint8): random sign, exponent field 3..11 (magnitudes 2^-4 to
    ~2^4.9, as block-quantised values occupy), random mantissa; never a NaN code."""
    sign = torch.randint(0, 2, shape, generator=generator, dtype=torch.int32)
    exp = torch.randint(3, 12, shape, generator=generator, dtype=torch.int32)
    man = torch.randint(0, 8, shape, generator=generator, dtype=torch.int32)
    return ((sign << 7) | (exp << 3) | man).to(torch.uint8).to(device)


@dataclass(frozen=True)
class Fp8Config:
    """Masked-layout FP8 grouped GEMM workload: E experts, row blocks of max_m (rows in use
    drawn from [lo, max_m]), N output columns, K reduction."""
    name: str
    E: int
    max_m: int
    N: int
    K: int
    lo: int


# TileOPs "MoE" page, MoEGroupedGemmFP8Fwd workloads (T = tokens of the step)
FP8_CONFIGS = {
    "ds-v3-dec-b64-up": Fp8Config("ds-v3-dec-b64-up", E=32, max_m=64, N=4096, K=7168, lo=64),
    "ds-v3-dec-b64-down": Fp8Config("ds-v3-dec-b64-down", E=32, max_m=64, N=7168, K=2048,
                                    lo=64),
    "ds-v3-dec-b256-up": Fp8Config("ds-v3-dec-b256-up", E=32, max_m=256, N=4096, K=7168,
                                   lo=256),
    "ds-v3-e8-up-masked": Fp8Config("ds-v3-e8-up-masked", E=8, max_m=128, N=4096, K=7168,
                                    lo=96),
}


def make_fp8_inputs(cfg: Fp8Config, device="cpu", seed: int = 42) -> dict:
    """a [E,max_m,K] / b [E,N,K] e4m3 codes (uint8), a_scale [E,max_m,K/128] and
    b_scale [E,ceil(N/128),K/128] f32 (positive, 2^-7 and 2^-9 times U[0.5, 1.5]),
    masked_m [E] int32 in [lo, max_m]."""
    E, m, N, K = cfg.E, cfg.max_m, cfg.N, cfg.K
    g = _gen("cpu", seed, STREAM_FP8)
    KB, NB = (K + 127) // 128, (N + 127) // 128
    return {
        "a": random_e4m3_codes((E, m, K), g, device),
        "a_scale": ((torch.rand((E, m, KB), generator=g) + 0.5) * 2.0 ** -7).to(device),
        "b": random_e4m3_codes((E, N, K), g, device),
        "b_scale": ((torch.rand((E, NB, KB), generator=g) + 0.5) * 2.0 ** -9).to(device),
        "masked_m": torch.randint(cfg.lo, m + 1, (E,), generator=g,
                                  dtype=torch.int32).to(device),
    }


# the configuration the benchmark times by default: the DeepSeek-V3-style grouped prefill
# (4096 tokens, 256 experts of 7168 x 2048), the largest of the single-GPU workloads
BENCH_CONFIG = "ds-v3-grouped-prefill"


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(stream))
    return g


def _normal(shape, std: float, dtype, device, seed: int, stream: int) -> torch.Tensor:
    """N(0, std^2) samples, drawn as f32, scaled, converted to ``dtype``; filled slice by slice
    along dim 0 so large weight tensors never need a full f32 copy."""
    g = _gen(device, seed, stream)
    out = torch.empty(shape, dtype=dtype, device=device)
    if len(shape) == 0 or shape[0] == 0:
        return out
    rows = shape[0]
    per = 1
    for s in shape[1:]:
        per *= s
    chunk = max(1, (1 << 26) // max(per, 1))  # about 64M values per draw
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        v = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        out[r0:r1].copy_(v.to(dtype))
        del v
    return out


def make_inputs(cfg: MoEConfig, device="cpu", seed: int = 42, weights: bool = True,
                num_tokens: Optional[int] = None, dtype=torch.bfloat16) -> dict:
    """Seeded synthetic tensors for ``cfg`` on ``device``.

    Returns a dict with hidden_states [T,H] bf16, gating_output [T,E] f32, correction_bias [E]
    f32 or None, w_gate_up [E,2F,H] bf16, w_down [E,H,F] bf16 and, for S > 0,
    shared_w_gate_up [2S,H] / shared_w_down [H,S] bf16.  ``num_tokens`` overrides T (token
    sweeps); weights do not depend on it.  ``weights=False`` skips the weight tensors.
    ``dtype`` (bf16 or f16) is the element type of the activations and weights; the same f32
    draws are rounded to it."""
    T = cfg.T if num_tokens is None else int(num_tokens)
    H, E, F, S = cfg.H, cfg.E, cfg.F, cfg.S
    d = {
        "hidden_states": _normal((T, H), 1.0, dtype, device, seed, STREAM_HIDDEN),
        "gating_output": _normal((T, E), 1.0, torch.float32, device, seed, STREAM_GATING),
        "correction_bias": (_normal((E,), 0.1, torch.float32, device, seed, STREAM_BIAS)
                            if cfg.bias else None),
    }
    if weights:
        d["w_gate_up"] = _normal((E, 2 * F, H), H ** -0.5, dtype, device, seed,
                                 STREAM_W_GATE_UP)
        d["w_down"] = _normal((E, H, F), F ** -0.5, dtype, device, seed, STREAM_W_DOWN)
        if S > 0:
            d["shared_w_gate_up"] = _normal((2 * S, H), H ** -0.5, dtype, device, seed,
                                            STREAM_SHARED_GATE_UP)
            d["shared_w_down"] = _normal((H, S), S ** -0.5, dtype, device, seed,
                                         STREAM_SHARED_DOWN)
    return d


def skew_bias(E: int, alpha: float, seed: int = 42) -> torch.Tensor:
    """Per-expert router-score bias of the skewed-routing workload (aiter MI308 decoding PR,
    Performance, "Skewed routing"): -alpha * log(1 + rank[e]), the ranks a fixed seeded random
    permutation of the experts (rank 0 the most popular).  float64 [E] on the host."""
    g = _gen("cpu", seed, STREAM_SKEW)
    rank = torch.empty(E, dtype=torch.float64)
    rank[torch.randperm(E, generator=g)] = torch.arange(E, dtype=torch.float64)
    return -float(alpha) * torch.log1p(rank)


def skew_gating(gating: torch.Tensor, alpha: float, seed: int = 42) -> torch.Tensor:
    """gating_output [T,E] f32 with the skew bias added to every token's scores (the sum in
    float64, rounded to f32 once), on gating's device."""
    if alpha == 0.0:
        return gating.clone()
    b = skew_bias(gating.shape[1], alpha, seed).to(gating.device)
    return (gating.double() + b).to(torch.float32)


SKEW_ALPHA_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                               "tests", "golden", "skew_alpha.json")


def skew_alpha(cfg: MoEConfig) -> float:
    """The skew strength that gives cfg's routing a most popular expert at twice the mean load
    (tests/golden/skew_alpha.json, written by tests/golden/skew_alpha.py with the oracle's
    routing); 0 for routings already above that."""
    with open(SKEW_ALPHA_FILE) as f:
        table = json.load(f)
    for entry in table.values():
        if cfg.name in entry["workloads"]:
            return float(entry["alpha"])
    raise KeyError("no skew alpha recorded for workload %s" % cfg.name)


def random_topk_ids(T: int, k: int, E: int, seed: int = 42, device="cpu",
                    pad_fraction: float = 0.0, allow_repeats: bool = False,
                    skew: float = 0.0) -> torch.Tensor:
    """Seeded synthetic topk_ids [T,k] int32 for the routing-given entry points: k distinct
    experts per token (or independent draws with ``allow_repeats``), a fraction of entries
    replaced by -1 padding routes.  ``skew`` > 0 draws the k distinct experts with probability
    proportional to (1 + popularity rank)^-skew, the ranks a seeded permutation of the experts
    (a few hot experts and a long tail, as real routers produce)."""
    g = _gen("cpu", seed, 9)
    if allow_repeats:
        ids = torch.randint(0, E, (T, k), generator=g, dtype=torch.int64)
    elif skew > 0.0:
        probs = torch.empty(E, dtype=torch.float64)
        probs[torch.randperm(E, generator=g)] = (1.0 + torch.arange(E, dtype=torch.float64)) ** -skew
        ids = torch.multinomial(probs.expand(T, E), k, replacement=False, generator=g)
    else:
        ids = torch.argsort(torch.rand((T, E), generator=g), dim=1)[:, :k]
    if pad_fraction > 0.0:
        mask = torch.rand((T, k), generator=g) < pad_fraction
        ids = torch.where(mask, torch.full_like(ids, -1), ids)
    return ids.to(torch.int32).to(device)


def random_topk_weights(T: int, k: int, seed: int = 42, device="cpu") -> torch.Tensor:
    """Seeded positive route weights [T,k] f32 in [0.05, 1)."""
    g = _gen("cpu", seed, 10)
    return (torch.rand((T, k), generator=g) * 0.95 + 0.05).to(torch.float32).to(device)


def to_u16(t: torch.Tensor):
    """bf16 tensor (any device) -> numpy uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def mxfp4_scale_byte(fan_in: int) -> int:
    """E8M0 scale byte that gives MXFP4 weights of uniformly random e2m1 codes (RMS magnitude
    sqrt(68.5/8) ~ 2.93) a standard deviation of about 1/sqrt(fan_in), like the bf16 weights."""
    return int(round(127 + math.log2(1.0 / (math.sqrt(fan_in) * math.sqrt(68.5 / 8)))))


def make_mxfp4_weights(cfg: MoEConfig, device="cpu", seed: int = 42) -> dict:
    """MXFP4 expert weights of cfg's shape: w_gate_up_q [E,2F,H/2] and w_down_q [E,H,F/2] uint8
    (two uniformly random e2m1 codes per byte), w_gate_up_scale [E,2F,H/32] and w_down_scale
    [E,H,F/32] uint8 E8M0 scales drawn from {s0-1, s0, s0+1}, s0 = mxfp4_scale_byte(fan_in)."""
    E, H, F = cfg.E, cfg.H, cfg.F
    g = _gen(device, seed, STREAM_MXFP4)

    def codes(shape):
        return torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.int32).to(
            torch.uint8)

    def scales(shape, fan_in):
        s0 = mxfp4_scale_byte(fan_in)
        return torch.randint(s0 - 1, s0 + 2, shape, generator=g, device=device,
                             dtype=torch.int32).to(torch.uint8)

    return {
        "w_gate_up_q": codes((E, 2 * F, H // 2)),
        "w_gate_up_scale": scales((E, 2 * F, H // 32), H),
        "w_down_q": codes((E, H, F // 2)),
        "w_down_scale": scales((E, H, F // 32), F),
    }


def make_fp8_weights(cfg: MoEConfig, device="cpu", seed: int = 42) -> dict:
    """FP8 expert weights of cfg's shape: w_gate_up [E,2F,H] and w_down [E,H,F] e4m3 codes
    (uint8; random_e4m3_codes) with f32 scales per 128 x 128 block [E,2F/128,H/128] and
    [E,H/128,F/128], chosen so the dequantised weights have a standard deviation of about
    1/sqrt(fan_in) (the codes' RMS magnitude is about 9): 1/(9 sqrt(fan_in)) x U[0.5, 1.5]."""
    E, H, F = cfg.E, cfg.H, cfg.F
    g = _gen("cpu", seed, STREAM_FP8 + 100)

    def scales(shape, fan_in):
        return ((torch.rand(shape, generator=g) + 0.5) / (9.0 * math.sqrt(fan_in))).to(device)

    return {
        "w_gate_up": random_e4m3_codes((E, 2 * F, H), g, device),
        "w_gate_up_scale": scales((E, 2 * F // 128, H // 128), H),
        "w_down": random_e4m3_codes((E, H, F), g, device),
        "w_down_scale": scales((E, H // 128, F // 128), F),
    }

