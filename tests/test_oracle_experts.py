"""Pins of the oracle's expert evaluation and combine.

The references here are independent of the oracle: a dense numpy evaluation of every expert
on every token (brute force, library matmuls), the dense SwiGLU MLP that the method reduces to
for one expert, exact algebraic invariants, and torch's own f32 -> bf16 rounding."""
import numpy as np
import pytest
import torch

import oracle
from moe_harness.workloads import CONFIGS, make_inputs, to_u16


def _f(bits):
    return oracle.bf16_bits_to_float(bits).astype(np.float64)


def _dense_mlp(x, wgu, wd):
    """silu(x Wg^T) * (x Wu^T) @ Wd^T with Wg = rows [0,F), Wu = rows [F,2F) of wgu."""
    F = wgu.shape[0] // 2
    u = x @ wgu[:F].T
    v = x @ wgu[F:].T
    a = u / (1.0 + np.exp(-u)) * v
    return a @ wd.T


def _tiny_inputs(seed=42, cfg="tiny", T=None, E=None):
    c = CONFIGS[cfg]
    if E is not None:
        from dataclasses import replace
        c = replace(c, E=E)
    d = make_inputs(c, "cpu", seed=seed, num_tokens=T)
    return c, {k: (to_u16(v) if v is not None and v.dtype == torch.bfloat16 else
                   (v.numpy() if v is not None else None)) for k, v in d.items()}


def test_bf16_rounding_matches_torch_on_f32_values():
    r = np.random.default_rng(0)
    vals = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-38).astype(np.float32),        # subnormal range
        np.clip(r.standard_normal(2000) * 1e38, -3.39e38, 3.39e38).astype(np.float32),
        # exact ties between two bf16 neighbours: odd and even lower neighbours
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130 * 1.5,
                  3.3895e38, -3.3895e38, 0.0, -0.0], np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.double_to_bf16(vals.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rounding_is_single_rounding_from_double():
    """1 + 2^-8 + 2^-40 lies just above the midpoint of 1 and 1 + 2^-7: one rounding gives
    1 + 2^-7 (0x3F81); rounding through f32 first would lose the 2^-40 and tie to 1.0."""
    assert oracle.double_to_bf16(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81
    assert oracle.double_to_bf16(np.array([1 + 2 ** -8]))[0] == 0x3F80
    assert oracle.double_to_bf16(np.array([-(1 + 2 ** -8 + 2 ** -40)]))[0] == 0xBF81


def _brute_force(x, wgu, wd, ids, w, sgu=None, sd=None):
    """Every expert on every token (dense), masked by a dense [T,E] route-weight matrix."""
    T, H = x.shape
    E = wgu.shape[0]
    xf = _f(x)
    dense_w = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            if 0 <= ids[t, j] < E:
                dense_w[t, ids[t, j]] += float(w[t, j])
    out = np.zeros((T, H))
    for e in range(E):
        out += dense_w[:, e:e + 1] * _dense_mlp(xf, _f(wgu[e]), _f(wd[e]))
    if sgu is not None:
        out += _dense_mlp(xf, _f(sgu), _f(sd))
    return out


def test_experts_match_dense_brute_force():
    c, d = _tiny_inputs()
    ids, w = oracle.route(d["gating_output"], None, c.k, "softmax", True)
    acc, out = oracle.experts(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w)
    ref = _brute_force(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w)
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out, oracle.double_to_bf16(ref))


def test_experts_with_shared_and_padding_match_brute_force():
    from dataclasses import replace
    c = replace(CONFIGS["tiny"], S=96, T=9, k=3)
    d = make_inputs(c, "cpu", seed=7)
    u = {k: to_u16(v) if v is not None and v.dtype == torch.bfloat16 else v
         for k, v in d.items()}
    g = d["gating_output"].numpy()
    ids, w = oracle.route(g, None, 3, "softmax", True)
    ids[2, 1] = -1
    ids[5, 0] = -1
    acc, _ = oracle.experts(u["hidden_states"], u["w_gate_up"], u["w_down"], ids, w,
                            u["shared_w_gate_up"], u["shared_w_down"])
    ref = _brute_force(u["hidden_states"], u["w_gate_up"], u["w_down"], ids, w,
                       u["shared_w_gate_up"], u["shared_w_down"])
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)


def test_one_expert_reduces_to_dense_swiglu():
    """E = 1, k = 1, softmax, renormalize: the weight is exactly 1 and the pass is the dense
    SwiGLU MLP."""
    c, d = _tiny_inputs(E=1)
    ids, w = oracle.route(d["gating_output"], None, 1, "softmax", True)
    assert np.all(ids == 0) and np.all(w == 1.0)
    acc, _ = oracle.experts(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w)
    ref = _dense_mlp(_f(d["hidden_states"]), _f(d["w_gate_up"][0]), _f(d["w_down"][0]))
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-13)


def test_identical_experts_give_rsf_times_mlp():
    c, d = _tiny_inputs(T=16)
    wgu = np.repeat(d["w_gate_up"][:1], c.E, axis=0)
    wd = np.repeat(d["w_down"][:1], c.E, axis=0)
    ids, w = oracle.route(d["gating_output"], None, 3, "softmax", True, rsf=2.5)
    acc, _ = oracle.experts(d["hidden_states"], wgu, wd, ids, w)
    ref = 2.5 * _dense_mlp(_f(d["hidden_states"]), _f(wgu[0]), _f(wd[0]))
    assert np.allclose(acc, ref, rtol=1e-6, atol=1e-9)   # f32 route weights sum to 2.5 +- 1ulp


def test_scaling_down_weights_scales_output_exactly():
    c, d = _tiny_inputs(T=8)
    ids, w = oracle.route(d["gating_output"], None, c.k, "softmax", True)
    acc1, _ = oracle.experts(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w)
    wd2 = to_u16(torch.from_numpy(d["w_down"].view(np.int16)).view(torch.bfloat16) * 2)
    acc2, _ = oracle.experts(d["hidden_states"], d["w_gate_up"], wd2, ids, w)
    assert np.array_equal(acc2, 2.0 * acc1)


def test_swapping_two_experts_with_their_gating_columns():
    c, d = _tiny_inputs(T=12)
    a, b = 1, 6
    g = d["gating_output"].copy()
    ids, w = oracle.route(g, None, c.k, "softmax", True)
    acc, _ = oracle.experts(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w)
    g2 = g.copy(); g2[:, [a, b]] = g2[:, [b, a]]
    wgu = d["w_gate_up"].copy(); wgu[[a, b]] = wgu[[b, a]]
    wd = d["w_down"].copy(); wd[[a, b]] = wd[[b, a]]
    ids2, w2 = oracle.route(g2, None, c.k, "softmax", True)
    acc2, _ = oracle.experts(d["hidden_states"], wgu, wd, ids2, w2)
    assert np.array_equal(acc, acc2)


def test_skipped_route_equals_zero_weight():
    c, d = _tiny_inputs(T=6)
    ids, w = oracle.route(d["gating_output"], None, c.k, "softmax", True)
    ids2 = ids.copy(); ids2[3, 1] = -1
    w2 = w.copy(); w2[3, 1] = 0.0
    a, _ = oracle.experts(d["hidden_states"], d["w_gate_up"], d["w_down"], ids2, w)
    b, _ = oracle.experts(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w2)
    assert np.array_equal(a, b)


def test_token_subset_and_thread_count_do_not_change_rows():
    c, d = _tiny_inputs(T=20)
    ids, w = oracle.route(d["gating_output"], None, c.k, "softmax", True)
    full, _ = oracle.experts(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w,
                             num_threads=1)
    sub, _ = oracle.experts(d["hidden_states"], d["w_gate_up"], d["w_down"], ids, w,
                            tokens=[17, 3, 3, 0], num_threads=4)
    assert np.array_equal(sub, full[[17, 3, 3, 0]])


def test_forward_routes_then_combines():
    c, d = _tiny_inputs()
    r = oracle.forward(d["hidden_states"], d["gating_output"], d["w_gate_up"], d["w_down"],
                       k=c.k)
    ref = _brute_force(d["hidden_states"], d["w_gate_up"], d["w_down"], r["topk_ids"],
                       r["topk_weights"])
    assert np.allclose(r["acc"], ref, rtol=1e-12, atol=1e-12)
