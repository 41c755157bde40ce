"""Shared helpers of the GPU parity tests: oracle calls on bytes copied from the device, and
the output tolerance.

Output tolerance (bf16 output of a pass whose GPU side rounds h and the expert output rows to
bf16 and accumulates in f32): relative L2 error <= 2e-2 over the compared elements, and every
element within 5e-2 + 2e-2 * |ref| of the oracle's bf16 output.  The f16 pass keeps the same
bound (its roundings of h and the rows are 8x finer).  Route weights: 1e-6 absolute.
Route ids, sort results: bit-exact."""
import numpy as np
import torch

import oracle
from moe_harness.workloads import to_u16

REL_L2 = 2e-2
ATOL = 5e-2
RTOL = 2e-2
WEIGHT_ATOL = 1e-6


def bf16_to_np(t):
    return oracle.bf16_bits_to_float(to_u16(t)).astype(np.float64)


def bits_to_np(bits, dtype="bf16"):
    """16-bit patterns -> float64 values of type dtype ("bf16" or "f16")"""
    if dtype == "f16":
        return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)
    return oracle.bf16_bits_to_float(bits).astype(np.float64)


def oracle_dtype(t):
    """the oracle's name of a torch tensor's 16-bit element type"""
    return "f16" if t.dtype == torch.float16 else "bf16"


def assert_output_close(got_bf16, ref_bits, what="", dtype=None):
    """got: GPU bf16 or f16 tensor [n,H] (or numpy float64); ref_bits: oracle uint16 [n,H] of
    the same type (dtype: "bf16"/"f16", default the tensor's own)."""
    if dtype is None:
        dtype = "bf16" if isinstance(got_bf16, np.ndarray) else oracle_dtype(got_bf16)
    g = got_bf16 if isinstance(got_bf16, np.ndarray) else bits_to_np(to_u16(got_bf16), dtype)
    r = bits_to_np(ref_bits, dtype)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite output" % what
    err = g - r
    denom = np.linalg.norm(r)
    rel = np.linalg.norm(err) / denom if denom > 0 else np.linalg.norm(err)
    worst = np.max(np.abs(err) - (ATOL + RTOL * np.abs(r))) if err.size else -1.0
    assert rel <= REL_L2, "%s: relative L2 error %.3e > %.1e" % (what, rel, REL_L2)
    assert worst <= 0, "%s: an element exceeds 5e-2 + 2e-2|ref| by %.3e" % (what, worst)
    return rel


def oracle_route(d, cfg, k=None, rsf=None):
    g = d["gating_output"].cpu().numpy()
    b = None if d.get("correction_bias") is None else d["correction_bias"].cpu().numpy()
    # the library receives the scaling factor as f32; hand the oracle that same value
    r = float(np.float32(cfg.rsf if rsf is None else rsf))
    return oracle.route(g, b, cfg.k if k is None else k, cfg.scoring, cfg.renormalize,
                        cfg.num_expert_group, cfg.topk_group, r)


def oracle_experts_sampled(d, ids, w, tokens, with_shared=False):
    """Oracle output for ``tokens`` using only the experts those tokens touch (copied from
    the device once), so full-size weights never need to be on the host."""
    ids = np.asarray(ids)
    w = np.asarray(w, np.float32)
    tokens = np.asarray(tokens, np.int64)
    E = d["w_gate_up"].shape[0]
    sub_ids = ids[tokens]
    used = np.unique(sub_ids[(sub_ids >= 0) & (sub_ids < E)])
    remap = np.full(E, -1, np.int64)
    remap[used] = np.arange(used.size)
    local_ids = np.where((sub_ids >= 0) & (sub_ids < E), remap[np.clip(sub_ids, 0, E - 1)],
                         -1).astype(np.int32)
    sel = torch.as_tensor(used, device=d["w_gate_up"].device, dtype=torch.long)
    wgu = to_u16(d["w_gate_up"].index_select(0, sel)) if used.size else \
        np.zeros((1,) + tuple(d["w_gate_up"].shape[1:]), np.uint16)
    wd = to_u16(d["w_down"].index_select(0, sel)) if used.size else \
        np.zeros((1,) + tuple(d["w_down"].shape[1:]), np.uint16)
    x = to_u16(d["hidden_states"][torch.as_tensor(tokens, device=d["hidden_states"].device)])
    sgu = sd = None
    if with_shared:
        sgu = to_u16(d["shared_w_gate_up"])
        sd = to_u16(d["shared_w_down"])
    return oracle.experts(x, wgu, wd, local_ids, w[tokens], sgu, sd,
                          dtype=oracle_dtype(d["hidden_states"]))


def sample_tokens(T, n, seed=0):
    """n distinct tokens including the first and the last one."""
    if T <= n:
        return np.arange(T)
    r = np.random.default_rng(seed)
    mid = r.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))


def routing_tokens(ids, E, block_m, n=64, seed=0):
    """At least n distinct tokens (if T allows) chosen from the realized routing ids [T,k] so
    that the compared outputs cover the tiles the sorted path forms: tokens of the heaviest
    expert's first route, its last route and up to 8 routes of its last (ragged) block_m-row
    tile; an equal share of tokens from each eighth of the expert-sorted route order (the
    tiles are numbered expert by expert, and the 8 XCDs take contiguous ranges of them); the
    first and the last token; random tokens to make up n."""
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.ravel()
    routes = np.nonzero((flat >= 0) & (flat < E))[0]
    rng = np.random.default_rng(seed)
    pick = {0, T - 1}
    if routes.size:
        order = routes[np.argsort(flat[routes], kind="stable")]
        counts = np.bincount(flat[routes], minlength=E)
        heavy = routes[flat[routes] == int(np.argmax(counts))]     # route order
        tail = heavy[(heavy.size - 1) // block_m * block_m:]
        pick.update(int(r) // k for r in rng.choice(tail, size=min(8, tail.size), replace=False))
        pick.update((int(heavy[0]) // k, int(heavy[-1]) // k))
        per = max(1, (n - len(pick)) // 8)
        for p in range(8):
            seg = order[p * order.size // 8:(p + 1) * order.size // 8]
            if seg.size:
                pick.update(int(r) // k for r in rng.choice(seg, size=min(per, seg.size),
                                                           replace=False))
    while len(pick) < min(n, T):
        pick.add(int(rng.integers(T)))
    return np.array(sorted(pick))
