"""CPU oracle of the fused MoE forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use
this package.  It wraps ``moe_oracle.c`` (plain C11 + OpenMP, double precision) with ctypes and
numpy; it imports nothing from the GPU package and the GPU package imports nothing from it.

Arrays are numpy.  bf16 tensors travel as ``uint16`` bit patterns.

Functions (each follows the passage cited in ``moe_oracle.c``):
  route(gating, bias, k, scoring, renormalize, num_expert_group, topk_group, rsf)
      -> (topk_ids int32 [T,k], topk_weights float32 [T,k])
  align_sort(topk_ids, num_experts, block_m) -> dict of int32 arrays
  experts(x, w_gate_up, w_down, topk_ids, topk_weights, shared_w_gate_up=None,
          shared_w_down=None, tokens=None, num_threads=0, dtype="bf16")
      -> (acc float64 [n,H], out uint16 [n,H]); dtype "bf16" or "f16" (IEEE binary16)
  forward(...) = route + experts, the whole pass
  masked_mlp(a, masked_m, w_gate_up, w_down) -> (acc float64 [E,max_m,H], out uint16 [E,max_m,H])
  fp8_e4m3_decode(codes) -> float64 values of OCP e4m3 codes
  fp8_e4m3_encode(values) -> uint8 codes (nearest, ties to even, saturating at 448)
  quant_fp8_1x128(x) -> (codes uint8 [M,K], scales float32 [M,ceil(K/128)])
  grouped_gemm_fp8(a, a_scale, b, b_scale, masked_m) -> (acc float64 [E,max_m,N], out uint16)
  grouped_gemm_fp8_contiguous(a, a_scale, b, b_scale, offsets) -> (acc [P,N], out uint16 [P,N])
  double_to_bf16(values) -> uint16 (one rounding, nearest-even)
  double_to_f16(values) -> uint16 binary16 bits (one rounding, nearest-even)
  fp8_forward(x, gating, w_gate_up, w_gate_up_scale, w_down, w_down_scale, ...)
      -> the FP8 pass (1 x 128 activation groups, 128 x 128 weight blocks) for ``tokens``
  fp8_experts(x, w_gate_up, w_gate_up_scale, w_down, w_down_scale, topk_ids, topk_weights)
      -> its expert part with the routing given
  mxfp4_dequant(q, scale) -> float64 weights of MXFP4 codes and E8M0 block scales
  mxfp4_to_bf16(q, scale) -> the same values as bf16 bits (exact)
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

SOFTMAX = 0
SIGMOID = 1

_P = ctypes.c_void_p
_I = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_route.argtypes = [_P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_double, _P, _P]
    lib.oracle_route.restype = _I
    lib.oracle_align_sort.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
    lib.oracle_align_sort.restype = _I
    lib.oracle_experts_dt.argtypes = [_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I,
                                      _P, _P, _I]
    lib.oracle_mxfp4_dequant.argtypes = [_P, _P, _I, _I, _P]
    lib.oracle_e2m1_to_double.restype = ctypes.c_double
    lib.oracle_e2m1_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_to_double.restype = ctypes.c_double
    lib.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_double_to_f16.restype = ctypes.c_uint16
    lib.oracle_double_to_f16.argtypes = [ctypes.c_double]
    lib.oracle_experts.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I,
                                   _P, _P, _I]
    lib.oracle_experts.restype = _I
    lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    for name in ("oracle_double_to_bf16_n", "oracle_double_to_f16_n"):
        getattr(lib, name).argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        getattr(lib, name).restype = None
    lib.oracle_fp8_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_grouped_gemm_fp8.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]
    lib.oracle_fp8_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_fp8_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_quant_fp8_1x128.argtypes = [_P, _I, _I, _P, _P]
    lib.oracle_grouped_gemm_fp8_contig.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]
    lib.oracle_grouped_gemm_fp8.restype = _I
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = _I
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _scoring_code(scoring):
    if isinstance(scoring, str):
        return {"softmax": SOFTMAX, "sigmoid": SIGMOID}[scoring]
    return int(scoring)


def route(gating, bias=None, k=2, scoring="softmax", renormalize=True, num_expert_group=1,
          topk_group=1, rsf=1.0):
    g = _c(gating, np.float32)
    T, E = g.shape
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    st = _load().oracle_route(_ptr(g), _ptr(b), T, E, k, _scoring_code(scoring),
                              int(bool(renormalize)), num_expert_group, topk_group, float(rsf),
                              _ptr(ids), _ptr(w))
    if st != 0:
        raise ValueError("oracle_route rejected its arguments (status %d)" % st)
    return ids, w


def align_sort(topk_ids, num_experts, block_m):
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    P = T * k
    sorted_ids = np.empty(P + num_experts * (block_m - 1), np.int32)
    offsets = np.empty(num_experts + 1, np.int32)
    tile_expert = np.empty(P // block_m + num_experts, np.int32)
    inverse = np.empty(P, np.int32)
    n_tiles = np.empty(1, np.int32)
    st = _load().oracle_align_sort(_ptr(ids), T, k, num_experts, block_m, _ptr(sorted_ids),
                                   _ptr(offsets), _ptr(tile_expert), _ptr(inverse), _ptr(n_tiles))
    if st != 0:
        raise ValueError("oracle_align_sort rejected its arguments (status %d)" % st)
    return {"sorted_route_ids": sorted_ids, "expert_offsets": offsets,
            "tile_expert": tile_expert, "inverse_pos": inverse, "n_tiles": int(n_tiles[0])}


DTYPE_CODES = {"bf16": 0, "f16": 1}


def experts(x, w_gate_up, w_down, topk_ids, topk_weights, shared_w_gate_up=None,
            shared_w_down=None, tokens=None, num_threads=0, dtype="bf16"):
    """x [T,H] u16; w_gate_up [E,2F,H] u16; w_down [E,H,F] u16; ids/weights [T,k].  The 16-bit
    patterns are bf16 or IEEE f16 (dtype "bf16" / "f16"); the output is in the same type.

    tokens: optional list of token indices to evaluate (rows of the result follow it).
    Returns (acc float64 [n,H] before rounding, out uint16 [n,H] bits)."""
    x = _c(x, np.uint16)
    w_gate_up = _c(w_gate_up, np.uint16)
    w_down = _c(w_down, np.uint16)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_weights, np.float32)
    T, H = x.shape
    E, F2, H2 = w_gate_up.shape
    F = F2 // 2
    assert H2 == H and F2 == 2 * F and w_down.shape == (E, H, F), "weight shapes"
    k = ids.shape[1]
    assert ids.shape == (T, k) and w.shape == (T, k)
    S = 0
    sgu = sd = None
    if shared_w_gate_up is not None:
        sgu = _c(shared_w_gate_up, np.uint16)
        sd = _c(shared_w_down, np.uint16)
        S = sgu.shape[0] // 2
        assert sgu.shape == (2 * S, H) and sd.shape == (H, S), "shared weight shapes"
    if tokens is None:
        tok = None
        n = T
    else:
        tok = _c(tokens, np.int32)
        assert tok.ndim == 1 and (tok.size == 0 or (tok.min() >= 0 and tok.max() < T))
        n = tok.size
    acc = np.empty((n, H), np.float64)
    out = np.empty((n, H), np.uint16)
    st = _load().oracle_experts_dt(DTYPE_CODES[dtype], _ptr(x), _ptr(w_gate_up), _ptr(w_down),
                                   _ptr(ids), _ptr(w), _ptr(sgu), _ptr(sd), S, H, E, F, k,
                                   _ptr(tok), n, _ptr(acc), _ptr(out), int(num_threads))
    if st != 0:
        raise ValueError("oracle_experts failed (status %d)" % st)
    return acc, out


def forward(x, gating, w_gate_up, w_down, bias=None, k=2, scoring="softmax", renormalize=True,
            num_expert_group=1, topk_group=1, rsf=1.0, shared_w_gate_up=None,
            shared_w_down=None, tokens=None, num_threads=0, dtype="bf16"):
    """The whole pass: route every token, then evaluate the experts for ``tokens``."""
    ids, w = route(gating, bias, k, scoring, renormalize, num_expert_group, topk_group, rsf)
    acc, out = experts(x, w_gate_up, w_down, ids, w, shared_w_gate_up, shared_w_down, tokens,
                       num_threads, dtype)
    return {"topk_ids": ids, "topk_weights": w, "acc": acc, "out": out}


def masked_mlp(a, masked_m, w_gate_up, w_down, num_threads=0):
    """The expert MLPs of the masked layout (TileOPs "MoE" page, MoEGroupedGemmFwd with
    a: [E, layout.max_m, K] and layout_metadata [E]): row i of expert e, for
    i < clamp(masked_m[e], 0, max_m), is that expert's SwiGLU MLP of a[e, i]; other rows are 0.
    It is the routed experts' computation with every row a token routed to its block's expert
    with weight 1 (and -1, no route, for rows past masked_m)."""
    a = np.asarray(a)
    E, max_m, H = a.shape
    m = np.clip(np.asarray(masked_m, dtype=np.int64), 0, max_m)
    ids = np.where(np.arange(max_m)[None, :] < m[:, None],
                   np.arange(E)[:, None], -1).astype(np.int32).reshape(E * max_m, 1)
    w = np.ones((E * max_m, 1), dtype=np.float32)
    acc, out = experts(a.reshape(E * max_m, H), w_gate_up, w_down, ids, w,
                       num_threads=num_threads)
    return acc.reshape(E, max_m, H), out.reshape(E, max_m, H)


def fp8_e4m3_decode(codes):
    """OCP e4m3 codes (uint8 array) -> float64 values, one call per code into the C decoder."""
    c = np.asarray(codes, dtype=np.uint8)
    f = _load().oracle_fp8_e4m3_to_double
    return np.array([f(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def grouped_gemm_fp8(a, a_scale, b, b_scale, masked_m):
    """MoEGroupedGemmFP8Fwd on the masked layout: a uint8 [E,max_m,K] e4m3, a_scale float32
    [E,max_m,K/128], b uint8 [E,N,K] e4m3, b_scale float32 [E,N/128,K/128], masked_m int32 [E].
    Rows past masked_m are 0 in the result."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(a_scale, np.float32)
    sb = _c(b_scale, np.float32)
    m = _c(masked_m, np.int32)
    E, max_m, K = a.shape
    N = b.shape[1]
    out = np.zeros((E, max_m, N), dtype=np.uint16)
    acc = np.zeros((E, max_m, N), dtype=np.float64)
    rc = _load().oracle_grouped_gemm_fp8(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(m), E,
                                         max_m, N, K, _ptr(out), _ptr(acc))
    if rc != 0:
        raise ValueError("oracle_grouped_gemm_fp8 rejected its arguments (%d)" % rc)
    return acc, out


def fp8_e4m3_encode(values):
    """float values -> OCP e4m3 codes (uint8): nearest finite value, ties to the even code,
    saturating at +-448; one call per value into the C encoder."""
    v = np.asarray(values, dtype=np.float64)
    f = _load().oracle_fp8_e4m3_encode
    return np.array([f(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


def quant_fp8_1x128(x):
    """bf16 activations (uint16 bits [M,K]) -> (e4m3 codes uint8 [M,K], f32 scales
    [M,ceil(K/128)]): per 1 x 128 group s = fl32(amax / 448) (1 for an all-zero group), code =
    the e4m3 nearest to fl32(x / s)."""
    x = _c(x, np.uint16)
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros((M, (K + 127) // 128), dtype=np.float32)
    rc = _load().oracle_quant_fp8_1x128(_ptr(x), M, K, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_quant_fp8_1x128 rejected its arguments (%d)" % rc)
    return q, s


def grouped_gemm_fp8_contiguous(a, a_scale, b, b_scale, offsets):
    """The block-scaled FP8 grouped GEMM on the contiguous layout: a uint8 [P,K] e4m3 with
    a_scale float32 [P,K/128]; b uint8 [E,N,K] e4m3 with b_scale float32 [E,N/128,K/128];
    offsets int32 [E+1], expert e owning rows [offsets[e], offsets[e+1]).  Rows outside every
    range are 0 in the result."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(a_scale, np.float32)
    sb = _c(b_scale, np.float32)
    off = _c(offsets, np.int32)
    P, K = a.shape
    E, N = b.shape[0], b.shape[1]
    out = np.zeros((P, N), dtype=np.uint16)
    acc = np.zeros((P, N), dtype=np.float64)
    rc = _load().oracle_grouped_gemm_fp8_contig(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(off),
                                                E, P, N, K, _ptr(out), _ptr(acc))
    if rc != 0:
        raise ValueError("oracle_grouped_gemm_fp8_contig rejected its arguments (%d)" % rc)
    return acc, out


def fp8_forward(x, gating, w_gate_up, w_gate_up_scale, w_down, w_down_scale, bias=None, k=2,
                scoring="softmax", renormalize=True, num_expert_group=1, topk_group=1, rsf=1.0,
                tokens=None):
    """The MoE pass with FP8 expert weights (e4m3 codes with f32 scales per 128 x 128 block),
    step by step: route, then fp8_experts.  x [T,H] bf16 bits; returns (topk_ids, topk_weights,
    out [n,H] bf16 bits) for ``tokens`` (default all)."""
    ids, w = route(gating, bias, k, scoring, renormalize, num_expert_group, topk_group, rsf)
    return ids, w, fp8_experts(x, w_gate_up, w_gate_up_scale, w_down, w_down_scale, ids, w,
                               tokens)


def fp8_experts(x, w_gate_up, w_gate_up_scale, w_down, w_down_scale, topk_ids, topk_weights,
                tokens=None):
    """The expert part of the FP8 pass with the routing given (topk_ids [T,k] int32, ids outside
    [0,E) skipped, repeats allowed; topk_weights [T,k] f32): each routed x row quantised per
    1 x 128 group (quant_fp8_1x128); per expert the gate-up block-scaled GEMM
    (grouped_gemm_fp8_contiguous), rounded to bf16; h = bf16(SiLU(gate) * up) (reading: h is
    stored in bf16 before it is quantised, as the 16-bit passes store it) quantised the same
    way; the down GEMM; out[t] = bf16(sum_j w_j y_j) from the unrounded down sums.  Returns out
    [n,H] bf16 bits for ``tokens`` (default all)."""
    x = _c(x, np.uint16)
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_weights)
    T, H = x.shape
    k = ids.shape[1]
    E, F2 = w_gate_up.shape[0], w_gate_up.shape[1]
    F = F2 // 2
    tok = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    routes = [(int(t), j) for t in tok for j in range(k) if 0 <= ids[t, j] < E]
    order = sorted(range(len(routes)), key=lambda i: (ids[routes[i][0], routes[i][1]], i))
    routes = [routes[i] for i in order]
    counts = np.bincount([ids[t, j] for t, j in routes], minlength=E) if routes else \
        np.zeros(E, np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = np.array([x[t] for t, j in routes], np.uint16).reshape(len(routes), H)
    xq, xs = quant_fp8_1x128(rows) if routes else (np.zeros((0, H), np.uint8),
                                                     np.zeros((0, H // 128), np.float32))
    _, gu = grouped_gemm_fp8_contiguous(xq, xs, w_gate_up, w_gate_up_scale, offsets)
    g = bf16_bits_to_float(gu[:, :F]).astype(np.float64)
    u = bf16_bits_to_float(gu[:, F:]).astype(np.float64)
    h = double_to_bf16(g / (1.0 + np.exp(-g)) * u) if routes else np.zeros((0, F), np.uint16)
    hq, hs = quant_fp8_1x128(h) if routes else (np.zeros((0, F), np.uint8),
                                                  np.zeros((0, F // 128), np.float32))
    y, _ = grouped_gemm_fp8_contiguous(hq, hs, w_down, w_down_scale, offsets)
    acc = np.zeros((len(tok), H))
    row_of = {(t, j): r for r, (t, j) in enumerate(routes)}  # the sum runs in route order j
    for i, t in enumerate(tok.tolist()):
        for j in range(k):
            if (t, j) in row_of:
                acc[i] += float(w[t, j]) * y[row_of[(t, j)]]
    return double_to_bf16(acc)


def mxfp4_dequant(q, scale):
    """MXFP4 weights -> float64: q uint8 [..., K/2] (two e2m1 codes per byte, element 2i in the
    low nibble), scale uint8 [..., K/32] (E8M0) -> [..., K]."""
    q = _c(q, np.uint8)
    s = _c(scale, np.uint8)
    K = q.shape[-1] * 2
    rows = int(np.prod(q.shape[:-1])) if q.ndim > 1 else 1
    out = np.empty(q.shape[:-1] + (K,), dtype=np.float64)
    rc = _load().oracle_mxfp4_dequant(_ptr(q), _ptr(s), rows, K, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_mxfp4_dequant rejected its arguments (%d)" % rc)
    return out


def mxfp4_to_bf16(q, scale):
    """MXFP4 weights -> the bf16 bit patterns of the same values: exact for scales up to 252
    (an e2m1 value has at most two significant bits; 6 * 2^125 is below the bf16 maximum), the
    largest codes overflowing to infinity from scale 253 up."""
    return double_to_bf16(mxfp4_dequant(q, scale))


def double_to_f16(values):
    """float64 values -> IEEE binary16 bit patterns (uint16), one rounding to nearest even,
    overflow to infinity."""
    v = np.ascontiguousarray(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_double_to_f16_n(_ptr(v), v.size, _ptr(out))
    return out


def double_to_bf16(values):
    v = np.ascontiguousarray(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_double_to_bf16_n(_ptr(v), v.size, _ptr(out))
    return out


def bf16_bits_to_float(bits):
    """uint16 bf16 patterns -> float32 values (exact widening)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
