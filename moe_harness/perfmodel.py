"""FLOP and byte model of the fused MoE forward pass, for roofline reporting.

FLOPs: 2*T*k*3*H*F for the routed experts (gate, up and down projections of every route) plus
2*T*3*H*S for a shared expert.  This is the count behind the TFLOP/s column of the TileOPs "MoE"
benchmark page (FusedMoEFwd and FusedMoESharedExpertFwd tables); the tests recompute that
column from the printed device times.

Algorithmic HBM bytes: every touched expert's weights once (6*H*F bytes in bf16: 2F*H gate/up
plus H*F down), the shared expert's 6*H*S, the activations in and out (2*T*H each, bf16), the
f32 gating logits (4*T*E), the f32 bias (4*E) and the route ids and weights (8*T*k).
Intermediates (h, route rows) and padding are overhead, not algorithmic bytes.  The weight term
is the "unique weights" count of the FlashInfer BF16-activation MoE PR ("Why 4096 remains
bandwidth-sensitive": 32 DeepSeek-V3 experts -> 2.819 GB, and FLOP/byte = routed rows per
expert, 116.09 for 3715 routes over 32 experts).

MI355X peaks (AMD public specifications): HBM3E 8.0 TB/s; dense bf16 MFMA 2.5 PFLOP/s.
"""

HBM_PEAK_BYTES_PER_S = 8.0e12
BF16_MFMA_PEAK_FLOP_PER_S = 2.5e15


def routed_flops(T: int, k: int, H: int, F: int) -> float:
    return 2.0 * T * k * 3.0 * H * F


def shared_flops(T: int, H: int, S: int) -> float:
    return 2.0 * T * 3.0 * H * S


def flops(T: int, k: int, H: int, F: int, S: int = 0) -> float:
    return routed_flops(T, k, H, F) + shared_flops(T, H, S)


def expert_weight_bytes(H: int, F: int) -> float:
    """bf16 bytes of one expert: w_gate_up [2F,H] + w_down [H,F]."""
    return 6.0 * H * F


def algorithmic_bytes(T: int, H: int, E: int, F: int, k: int, touched: int, S: int = 0,
                      bias: bool = False) -> float:
    b = touched * expert_weight_bytes(H, F)
    b += 6.0 * H * S
    b += 2.0 * T * H * 2          # hidden_states in, output out (bf16)
    b += 4.0 * T * E              # gating_output f32
    b += 4.0 * E if bias else 0.0
    b += 8.0 * T * k              # topk ids (i32) + weights (f32)
    return b


def touched_experts(topk_ids, E: int) -> int:
    """Number of distinct experts in [0, E) that at least one route selects."""
    import numpy as np
    ids = np.asarray(topk_ids).ravel()
    ids = ids[(ids >= 0) & (ids < E)]
    return int(np.unique(ids).size)


def load_stats(topk_ids, E: int) -> dict:
    """Rows per touched expert: min / max / median, plus the touched count."""
    import numpy as np
    ids = np.asarray(topk_ids).ravel()
    ids = ids[(ids >= 0) & (ids < E)]
    c = np.bincount(ids, minlength=E)
    c = c[c > 0]
    if c.size == 0:
        return {"touched": 0, "min": 0, "max": 0, "median": 0.0}
    return {"touched": int(c.size), "min": int(c.min()), "max": int(c.max()),
            "median": float(np.median(c))}
