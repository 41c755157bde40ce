"""MI355X-native fused mixture-of-experts forward pass.

Python binding over ``libmoe_mi355x.so`` (the HIP kernels for gfx950 behind the C ABI of
``include/moe.h``).  This module only marshals arguments: it checks tensor shapes, dtypes and
devices, allocates outputs and the workspace with torch, and passes raw device pointers and the
current HIP stream to the library.  Every step of the pass runs in the library's kernels; if
the library is missing, importing a function raises instead of falling back to anything else.

Entry points (same names as the C ABI):
  moe_route(gating_output, top_k, ...)                        -> (topk_ids, topk_weights)
  moe_align_sort(topk_ids, num_experts, block_m[, workspace]) -> dict of int32 tensors
  moe_align_sort_workspace_bytes(T, k, num_experts, block_m) -> bytes
  fused_moe_fwd(hidden_states, gating_output, w_gate_up, w_down, top_k, ...) -> out
  fused_moe_fwd_noalloc(same as fused_moe_fwd, no workspace)  -> out (library-held scratch)
  fused_moe_shared_fwd(..., shared_w_gate_up, shared_w_down)  -> out
  fused_moe_experts_fwd(hidden_states, w_gate_up, w_down, topk_ids, topk_weights) -> out
  fused_moe_masked_fwd(a, masked_m, w_gate_up, w_down)        -> out [E, max_m, H]
  moe_grouped_gemm_fp8(a, a_scale, b, b_scale, masked_m)      -> out [E, max_m, N] bf16
  moe_grouped_gemm_fp8_contiguous(a, a_scale, b, b_scale, expert_offsets) -> out [P, N] bf16
  moe_quant_fp8(x)                                            -> (q [M, K] e4m3, scale [M, K/128])
  fused_moe_mxfp4_fwd(hidden, gating, w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale,
                      top_k, ...)                             -> out [T, H] bf16 (MXFP4 weights)
  fused_moe_fp8_fwd(hidden, gating, w_gate_up, w_gate_up_scale, w_down, w_down_scale, top_k, ...)
                                                              -> out [T, H] bf16 (FP8 weights)
  moe_stream_read(buf)                                        -> sink (measurement: one HBM
                                                                 streaming read of buf)
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK = 0
SCORING = {"softmax": 0, "sigmoid": 1}
PATHS = {"auto": 0, "direct": 1, "sorted": 2}
DIRECT_MAX_ROUTES = 512


class MoEError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


class MoEParams(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("num_expert_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("path", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

# symbol -> (restype, argtypes); every function declared in include/moe.h
SIGNATURES = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_check_params": (ctypes.c_int, [_P, ctypes.c_int, _I32]),
    "moe_route": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "moe_align_sort": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ,
                                      _P]),
    "moe_align_sort_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "fused_moe_workspace_bytes": (_SZ, [_P, _I32]),
    "fused_moe_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fused_moe_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "fused_moe_mxfp4_workspace_bytes": (_SZ, [_P]),
    "fused_moe_fp8_workspace_bytes": (_SZ, [_P]),
    "fused_moe_fp8_stage": (ctypes.c_int, [_I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                           _P]),
    "fused_moe_fp8_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                         _P]),
    "fused_moe_mxfp4_stage": (ctypes.c_int, [_I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                             _P]),
    "fused_moe_mxfp4_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _SZ, _P]),
    "fused_moe_shared_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P,
                                            _P, _SZ, _P]),
    "fused_moe_experts_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fused_moe_experts_stage": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I32,
                                               _P, _P, _P, _SZ, _P]),
    "fused_moe_masked_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "fused_moe_masked_fwd": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ,
                                            _P]),
    "fused_moe_masked_stage": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _P, _I32, _I32, _I32,
                                              _I32, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P,
                                            _P]),
    "moe_grouped_gemm_fp8_contiguous": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                       _I32, _P, _P]),
    "moe_quant_fp8": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P]),
    "moe_stream_read_sink_words": (ctypes.c_int, []),
    "moe_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
}

# stages of fused_moe_experts_stage, in the order fused_moe_experts_fwd runs them
STAGE_ALIGN, STAGE_GATE_UP, STAGE_DOWN, STAGE_SHARED, STAGE_COMBINE = 1, 2, 3, 4, 5
STAGE_NAMES = {1: "align", 2: "gate_up", 3: "down", 4: "shared", 5: "combine"}


def lib():
    """The loaded library.  Raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("%s is not built; run `python -m mixture_experts_forward_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status):
    return lib().moe_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, shape, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


# element type of the pass (MOE_DTYPE_*): torch dtype -> code
DTYPES = {torch.bfloat16: 0, torch.float16: 1}


def make_params(T, H, E, F, k, scoring="softmax", renormalize=True, num_expert_group=1,
                topk_group=1, routed_scaling_factor=1.0, path="auto", dtype=torch.bfloat16):
    return MoEParams(int(T), int(H), int(E), int(F), int(k), SCORING[scoring],
                     int(bool(renormalize)), int(num_expert_group), int(topk_group),
                     float(routed_scaling_factor), PATHS[path], DTYPES[dtype])


def _pass_dtype(hidden_states):
    """the pass's element type, taken from hidden_states (bf16 or f16)"""
    if hidden_states.dtype not in DTYPES:
        raise ValueError("hidden_states must be bfloat16 or float16, got %s" % hidden_states.dtype)
    return hidden_states.dtype


def workspace_bytes(params, shared_inter=0):
    return int(lib().fused_moe_workspace_bytes(ctypes.byref(params), int(shared_inter)))


def _workspace(params, shared_inter, device, workspace):
    n = workspace_bytes(params, shared_inter)
    if workspace is None:
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device), n
    if workspace.dtype != torch.uint8 or workspace.device != device or workspace.numel() < n:
        raise ValueError("workspace must be a uint8 tensor on %s with >= %d bytes" % (device, n))
    return workspace, workspace.numel()


def moe_route(gating_output, top_k, correction_bias=None, scoring="softmax", renormalize=True,
              num_expert_group=1, topk_group=1, routed_scaling_factor=1.0):
    T, E = gating_output.shape
    dev = gating_output.device
    _check(gating_output, "gating_output", torch.float32, (T, E))
    if correction_bias is not None:
        _check(correction_bias, "correction_bias", torch.float32, (E,), dev)
    p = make_params(T, 64, E, 64, top_k, scoring, renormalize, num_expert_group, topk_group,
                    routed_scaling_factor)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        st = lib().moe_route(_ptr(gating_output), _ptr(correction_bias), ctypes.byref(p),
                             _ptr(ids), _ptr(w), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "moe_route")
    return ids, w


def moe_align_sort(topk_ids, num_experts, block_m, workspace=None):
    """Sorted layout of the routes (dict of int32 tensors).  workspace: a uint8 device tensor of
    at least moe_align_sort_workspace_bytes bytes, or None to allocate one."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    _check(topk_ids, "topk_ids", torch.int32, (T, k))
    P = T * k
    E = int(num_experts)
    out = {
        "sorted_route_ids": torch.empty(P + E * (block_m - 1), dtype=torch.int32, device=dev),
        "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "tile_expert": torch.empty(P // block_m + E, dtype=torch.int32, device=dev),
        "inverse_pos": torch.empty(P, dtype=torch.int32, device=dev),
        "n_tiles": torch.empty(1, dtype=torch.int32, device=dev),
    }
    need = lib().moe_align_sort_workspace_bytes(T, k, E, int(block_m))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib().moe_align_sort(_ptr(topk_ids), T, k, E, int(block_m),
                                  _ptr(out["sorted_route_ids"]), _ptr(out["expert_offsets"]),
                                  _ptr(out["tile_expert"]), _ptr(out["inverse_pos"]),
                                  _ptr(out["n_tiles"]), _ptr(workspace), workspace.numel(),
                                  _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "moe_align_sort")
    return out


def moe_align_sort_workspace_bytes(T, k, num_experts, block_m):
    return int(lib().moe_align_sort_workspace_bytes(int(T), int(k), int(num_experts),
                                                    int(block_m)))


def _fused(hidden_states, gating_output, w_gate_up, w_down, top_k, correction_bias, scoring,
           renormalize, num_expert_group, topk_group, routed_scaling_factor,
           shared_w_gate_up, shared_w_down, path, out, workspace, return_routing):
    T, H = hidden_states.shape
    E, F2, _ = w_gate_up.shape
    F = F2 // 2
    dev = hidden_states.device
    dt = _pass_dtype(hidden_states)
    _check(hidden_states, "hidden_states", dt, (T, H))
    _check(gating_output, "gating_output", torch.float32, (T, E), dev)
    _check(w_gate_up, "w_gate_up", dt, (E, 2 * F, H), dev)
    _check(w_down, "w_down", dt, (E, H, F), dev)
    if correction_bias is not None:
        _check(correction_bias, "correction_bias", torch.float32, (E,), dev)
    S = 0
    if shared_w_gate_up is not None:
        S = shared_w_gate_up.shape[0] // 2
        _check(shared_w_gate_up, "shared_w_gate_up", dt, (2 * S, H), dev)
        _check(shared_w_down, "shared_w_down", dt, (H, S), dev)
    p = make_params(T, H, E, F, top_k, scoring, renormalize, num_expert_group, topk_group,
                    routed_scaling_factor, path, dt)
    if out is None:
        out = torch.empty((T, H), dtype=dt, device=dev)
    _check(out, "out", dt, (T, H), dev)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev) if return_routing else None
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev) if return_routing else None
    with torch.cuda.device(dev):
        ws, nbytes = _workspace(p, S, dev, workspace)
        if S > 0:
            st = lib().fused_moe_shared_fwd(
                _ptr(hidden_states), _ptr(gating_output), _ptr(w_gate_up), _ptr(w_down),
                _ptr(correction_bias), _ptr(shared_w_gate_up), _ptr(shared_w_down), S,
                ctypes.byref(p), _ptr(out), _ptr(ids), _ptr(w), _ptr(ws), nbytes, _stream(dev))
            where = "fused_moe_shared_fwd"
        else:
            st = lib().fused_moe_fwd(
                _ptr(hidden_states), _ptr(gating_output), _ptr(w_gate_up), _ptr(w_down),
                _ptr(correction_bias), ctypes.byref(p), _ptr(out), _ptr(ids), _ptr(w),
                _ptr(ws), nbytes, _stream(dev))
            where = "fused_moe_fwd"
    if st != MOE_OK:
        raise MoEError(st, where)
    if return_routing:
        return out, ids, w
    return out


def fused_moe_fwd(hidden_states, gating_output, w_gate_up, w_down, top_k, correction_bias=None,
                  scoring="softmax", renormalize=True, num_expert_group=1, topk_group=1,
                  routed_scaling_factor=1.0, path="auto", out=None, workspace=None,
                  return_routing=False):
    return _fused(hidden_states, gating_output, w_gate_up, w_down, top_k, correction_bias,
                  scoring, renormalize, num_expert_group, topk_group, routed_scaling_factor,
                  None, None, path, out, workspace, return_routing)


NOALLOC_SCRATCH_BYTES = 128 << 20


def fused_moe_fwd_noalloc(hidden_states, gating_output, w_gate_up, w_down, top_k,
                          correction_bias=None, scoring="softmax", renormalize=True,
                          num_expert_group=1, topk_group=1, routed_scaling_factor=1.0,
                          path="auto", out=None, topk_ids_out=None, topk_weights_out=None):
    """fused_moe_fwd without a workspace: the library's own fixed scratch array is used (see
    include/moe.h).  out / topk_ids_out / topk_weights_out may be given (preallocated)."""
    T, H = hidden_states.shape
    E, F2, _ = w_gate_up.shape
    F = F2 // 2
    dev = hidden_states.device
    dt = _pass_dtype(hidden_states)
    _check(hidden_states, "hidden_states", dt, (T, H))
    _check(gating_output, "gating_output", torch.float32, (T, E), dev)
    _check(w_gate_up, "w_gate_up", dt, (E, 2 * F, H), dev)
    _check(w_down, "w_down", dt, (E, H, F), dev)
    if correction_bias is not None:
        _check(correction_bias, "correction_bias", torch.float32, (E,), dev)
    p = make_params(T, H, E, F, top_k, scoring, renormalize, num_expert_group, topk_group,
                    routed_scaling_factor, path, dt)
    if out is None:
        out = torch.empty((T, H), dtype=dt, device=dev)
    _check(out, "out", dt, (T, H), dev)
    if topk_ids_out is not None:
        _check(topk_ids_out, "topk_ids_out", torch.int32, (T, top_k), dev)
    if topk_weights_out is not None:
        _check(topk_weights_out, "topk_weights_out", torch.float32, (T, top_k), dev)
    with torch.cuda.device(dev):
        st = lib().fused_moe_fwd_noalloc(
            _ptr(hidden_states), _ptr(gating_output), _ptr(w_gate_up), _ptr(w_down),
            _ptr(correction_bias), ctypes.byref(p), _ptr(out), _ptr(topk_ids_out),
            _ptr(topk_weights_out), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_fwd_noalloc")
    return out


def fused_moe_shared_fwd(hidden_states, gating_output, w_gate_up, w_down, shared_w_gate_up,
                         shared_w_down, top_k, correction_bias=None, scoring="softmax",
                         renormalize=True, num_expert_group=1, topk_group=1,
                         routed_scaling_factor=1.0, path="auto", out=None, workspace=None,
                         return_routing=False):
    if shared_w_gate_up is None or shared_w_down is None:
        raise ValueError("fused_moe_shared_fwd needs shared_w_gate_up and shared_w_down")
    return _fused(hidden_states, gating_output, w_gate_up, w_down, top_k, correction_bias,
                  scoring, renormalize, num_expert_group, topk_group, routed_scaling_factor,
                  shared_w_gate_up, shared_w_down, path, out, workspace, return_routing)


def fused_moe_experts_fwd(hidden_states, w_gate_up, w_down, topk_ids, topk_weights, path="auto",
                          out=None, workspace=None):
    T, H = hidden_states.shape
    E, F2, _ = w_gate_up.shape
    F = F2 // 2
    k = topk_ids.shape[1]
    dev = hidden_states.device
    dt = _pass_dtype(hidden_states)
    _check(hidden_states, "hidden_states", dt, (T, H))
    _check(w_gate_up, "w_gate_up", dt, (E, 2 * F, H), dev)
    _check(w_down, "w_down", dt, (E, H, F), dev)
    _check(topk_ids, "topk_ids", torch.int32, (T, k), dev)
    _check(topk_weights, "topk_weights", torch.float32, (T, k), dev)
    p = make_params(T, H, E, F, k, path=path, dtype=dt)
    if out is None:
        out = torch.empty((T, H), dtype=dt, device=dev)
    _check(out, "out", dt, (T, H), dev)
    with torch.cuda.device(dev):
        ws, nbytes = _workspace(p, 0, dev, workspace)
        st = lib().fused_moe_experts_fwd(_ptr(hidden_states), _ptr(w_gate_up), _ptr(w_down),
                                         _ptr(topk_ids), _ptr(topk_weights), ctypes.byref(p),
                                         _ptr(out), _ptr(ws), nbytes, _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_experts_fwd")
    return out


def fused_moe_experts_stage(stage, params, hidden_states, w_gate_up, w_down, topk_ids,
                            topk_weights, out, workspace, shared_w_gate_up=None,
                            shared_w_down=None):
    """One stage of the expert part (see include/moe.h).  Low level: ``params`` is a
    MoEParams matching the tensors (built with make_params) and ``workspace`` a uint8 tensor of
    at least workspace_bytes(params, S) bytes; the caller keeps both across the stages of one
    pass.  Tensors are assumed checked by the caller."""
    S = 0 if shared_w_gate_up is None else shared_w_gate_up.shape[0] // 2
    dev = hidden_states.device
    with torch.cuda.device(dev):
        st = lib().fused_moe_experts_stage(
            int(stage), _ptr(hidden_states), _ptr(w_gate_up), _ptr(w_down), _ptr(topk_ids),
            _ptr(topk_weights), _ptr(shared_w_gate_up), _ptr(shared_w_down), S,
            ctypes.byref(params), _ptr(out), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_experts_stage(%s)" % STAGE_NAMES.get(stage, stage))


def masked_workspace_bytes(E, max_m, H, F):
    return int(lib().fused_moe_masked_workspace_bytes(int(E), int(max_m), int(H), int(F)))


def _masked_args(a, masked_m, w_gate_up, w_down, out, workspace):
    E, max_m, H = a.shape
    F = w_down.shape[2]
    dev = a.device
    _check(a, "a", torch.bfloat16, (E, max_m, H))
    _check(masked_m, "masked_m", torch.int32, (E,), dev)
    _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * F, H), dev)
    _check(w_down, "w_down", torch.bfloat16, (E, H, F), dev)
    if out is None:
        out = torch.zeros((E, max_m, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (E, max_m, H), dev)
    n = masked_workspace_bytes(E, max_m, H, F)
    if workspace is None:
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    return E, max_m, H, F, out, workspace


def fused_moe_masked_fwd(a, masked_m, w_gate_up, w_down, out=None, workspace=None):
    """Expert MLPs of one expert-parallel shard on the masked layout a [E, max_m, H]: rows
    i < masked_m[e] of expert e -> out [E, max_m, H].  Rows past masked_m are left as they are
    in ``out`` (zeros when out is allocated here)."""
    E, max_m, H, F, out, workspace = _masked_args(a, masked_m, w_gate_up, w_down, out, workspace)
    dev = a.device
    with torch.cuda.device(dev):
        st = lib().fused_moe_masked_fwd(_ptr(a), _ptr(masked_m), _ptr(w_gate_up), _ptr(w_down),
                                        E, max_m, H, F, _ptr(out), _ptr(workspace),
                                        workspace.numel(), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_masked_fwd")
    return out


def fused_moe_masked_stage(stage, a, masked_m, w_gate_up, w_down, out, workspace):
    """One stage (STAGE_ALIGN, STAGE_GATE_UP or STAGE_DOWN) of fused_moe_masked_fwd on the
    caller's workspace (at least masked_workspace_bytes bytes, kept across the stages)."""
    E, max_m, H = a.shape
    F = w_down.shape[2]
    dev = a.device
    with torch.cuda.device(dev):
        st = lib().fused_moe_masked_stage(int(stage), _ptr(a), _ptr(masked_m), _ptr(w_gate_up),
                                          _ptr(w_down), E, max_m, H, F, _ptr(out),
                                          _ptr(workspace), workspace.numel(), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_masked_stage(%s)" % STAGE_NAMES.get(stage, stage))


def moe_grouped_gemm_fp8(a, a_scale, b, b_scale, masked_m, out=None):
    """Block-scaled FP8 grouped GEMM of the masked layout: a [E,max_m,K] and b [E,N,K] e4m3
    (torch.float8_e4m3fn or uint8 codes), a_scale [E,max_m,K/128] and b_scale
    [E,ceil(N/128),K/128] f32, masked_m [E] int32 -> out [E,max_m,N] bf16 (rows past masked_m
    left as they are; zeros when out is allocated here)."""
    E, max_m, K = a.shape
    N = b.shape[1]
    dev = a.device
    codes = lambda t: t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t
    a8, b8 = codes(a), codes(b)
    _check(a8, "a", torch.uint8, (E, max_m, K))
    _check(b8, "b", torch.uint8, (E, N, K), dev)
    _check(a_scale, "a_scale", torch.float32, (E, max_m, (K + 127) // 128), dev)
    _check(b_scale, "b_scale", torch.float32, (E, (N + 127) // 128, (K + 127) // 128), dev)
    _check(masked_m, "masked_m", torch.int32, (E,), dev)
    if out is None:
        out = torch.zeros((E, max_m, N), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (E, max_m, N), dev)
    with torch.cuda.device(dev):
        st = lib().moe_grouped_gemm_fp8(_ptr(a8), _ptr(a_scale), _ptr(b8), _ptr(b_scale),
                                        _ptr(masked_m), E, max_m, N, K, _ptr(out),
                                        _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "moe_grouped_gemm_fp8")
    return out


def moe_grouped_gemm_fp8_contiguous(a, a_scale, b, b_scale, expert_offsets, out=None):
    """Block-scaled FP8 grouped GEMM of the contiguous layout: a [P,K] e4m3 (torch.float8_e4m3fn
    or uint8 codes) with a_scale [P,K/128] f32, b [E,N,K] e4m3 with b_scale [E,ceil(N/128),K/128]
    f32, expert_offsets [E+1] int32 (expert e owns rows [offsets[e], offsets[e+1])) -> out [P,N]
    bf16 (rows of no expert left as they are; zeros when out is allocated here)."""
    P, K = a.shape
    E, N = b.shape[0], b.shape[1]
    dev = a.device
    codes = lambda t: t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t
    a8, b8 = codes(a), codes(b)
    _check(a8, "a", torch.uint8, (P, K))
    _check(b8, "b", torch.uint8, (E, N, K), dev)
    _check(a_scale, "a_scale", torch.float32, (P, (K + 127) // 128), dev)
    _check(b_scale, "b_scale", torch.float32, (E, (N + 127) // 128, (K + 127) // 128), dev)
    _check(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    if out is None:
        out = torch.zeros((P, N), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (P, N), dev)
    with torch.cuda.device(dev):
        st = lib().moe_grouped_gemm_fp8_contiguous(_ptr(a8), _ptr(a_scale), _ptr(b8),
                                                   _ptr(b_scale), _ptr(expert_offsets), E, P, N,
                                                   K, _ptr(out), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "moe_grouped_gemm_fp8_contiguous")
    return out


def moe_quant_fp8(x, q=None, scale=None):
    """bf16 x [M,K] -> (q [M,K] uint8 e4m3 codes, scale [M,ceil(K/128)] f32): per 1 x 128 group
    scale = amax / 448 (1 for an all-zero group), codes nearest to x / scale, ties to even."""
    M, K = x.shape
    dev = x.device
    _check(x, "x", torch.bfloat16, (M, K))
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((M, (K + 127) // 128), dtype=torch.float32, device=dev)
    _check(q, "q", torch.uint8, (M, K), dev)
    _check(scale, "scale", torch.float32, (M, (K + 127) // 128), dev)
    with torch.cuda.device(dev):
        st = lib().moe_quant_fp8(_ptr(x), M, K, _ptr(q), _ptr(scale), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "moe_quant_fp8")
    return q, scale


def fused_moe_mxfp4_fwd(hidden_states, gating_output, w_gate_up_q, w_gate_up_scale, w_down_q,
                        w_down_scale, top_k, correction_bias=None, scoring="softmax",
                        renormalize=True, num_expert_group=1, topk_group=1,
                        routed_scaling_factor=1.0, path="auto", out=None, workspace=None,
                        return_routing=False):
    """The fused pass with MXFP4 expert weights (uint8 e2m1 code pairs [E,2F,H/2] / [E,H,F/2],
    uint8 E8M0 scales [E,2F,H/32] / [E,H,F/32]) and bf16 activations."""
    T, H = hidden_states.shape
    E, F2, _ = w_gate_up_q.shape
    F = F2 // 2
    dev = hidden_states.device
    _check(hidden_states, "hidden_states", torch.bfloat16, (T, H))
    _check(gating_output, "gating_output", torch.float32, (T, E), dev)
    _check(w_gate_up_q, "w_gate_up_q", torch.uint8, (E, 2 * F, H // 2), dev)
    _check(w_gate_up_scale, "w_gate_up_scale", torch.uint8, (E, 2 * F, H // 32), dev)
    _check(w_down_q, "w_down_q", torch.uint8, (E, H, F // 2), dev)
    _check(w_down_scale, "w_down_scale", torch.uint8, (E, H, F // 32), dev)
    if correction_bias is not None:
        _check(correction_bias, "correction_bias", torch.float32, (E,), dev)
    p = make_params(T, H, E, F, top_k, scoring, renormalize, num_expert_group, topk_group,
                    routed_scaling_factor, path)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, H), dev)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev) if return_routing else None
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev) if return_routing else None
    with torch.cuda.device(dev):
        n = int(lib().fused_moe_mxfp4_workspace_bytes(ctypes.byref(p)))
        if workspace is None:
            workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        elif workspace.dtype != torch.uint8 or workspace.numel() < n:
            raise ValueError("workspace must be a uint8 tensor with >= %d bytes" % n)
        st = lib().fused_moe_mxfp4_fwd(
            _ptr(hidden_states), _ptr(gating_output), _ptr(w_gate_up_q), _ptr(w_gate_up_scale),
            _ptr(w_down_q), _ptr(w_down_scale), _ptr(correction_bias), ctypes.byref(p),
            _ptr(out), _ptr(ids), _ptr(w), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_mxfp4_fwd")
    if return_routing:
        return out, ids, w
    return out


def fused_moe_mxfp4_stage(stage, params, hidden_states, mx, topk_ids, topk_weights, out,
                          workspace):
    """One stage of the MXFP4 expert part (see include/moe.h): ``mx`` holds w_gate_up_q,
    w_gate_up_scale, w_down_q, w_down_scale; ``params`` a MoEParams; the workspace at least
    fused_moe_mxfp4_workspace_bytes(params) bytes.  Tensors are assumed checked by the caller."""
    dev = hidden_states.device
    with torch.cuda.device(dev):
        st = lib().fused_moe_mxfp4_stage(
            int(stage), _ptr(hidden_states), _ptr(mx["w_gate_up_q"]),
            _ptr(mx["w_gate_up_scale"]), _ptr(mx["w_down_q"]), _ptr(mx["w_down_scale"]),
            _ptr(topk_ids), _ptr(topk_weights), ctypes.byref(params), _ptr(out),
            _ptr(workspace), workspace.numel(), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_mxfp4_stage(%s)" % STAGE_NAMES.get(stage, stage))


def mxfp4_workspace_bytes(params):
    return int(lib().fused_moe_mxfp4_workspace_bytes(ctypes.byref(params)))


def fused_moe_fp8_fwd(hidden_states, gating_output, w_gate_up, w_gate_up_scale, w_down,
                      w_down_scale, top_k, correction_bias=None, scoring="softmax",
                      renormalize=True, num_expert_group=1, topk_group=1,
                      routed_scaling_factor=1.0, out=None, workspace=None,
                      return_routing=False, path="auto"):
    """The fused pass with FP8 expert weights: w_gate_up [E,2F,H] / w_down [E,H,F] e4m3
    (torch.float8_e4m3fn or uint8 codes) with f32 scales [E,2F/128,H/128] / [E,H/128,F/128];
    bf16 activations quantised per 1 x 128 group on the way in.  path: "direct" (T*k <= 64:
    no align and no quantiser launches), "sorted", or "auto"."""
    T, H = hidden_states.shape
    codes = lambda t: t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t
    wgu, wd = codes(w_gate_up), codes(w_down)
    E, F2, _ = wgu.shape
    F = F2 // 2
    dev = hidden_states.device
    _check(hidden_states, "hidden_states", torch.bfloat16, (T, H))
    _check(gating_output, "gating_output", torch.float32, (T, E), dev)
    _check(wgu, "w_gate_up", torch.uint8, (E, 2 * F, H), dev)
    _check(w_gate_up_scale, "w_gate_up_scale", torch.float32, (E, 2 * F // 128, H // 128), dev)
    _check(wd, "w_down", torch.uint8, (E, H, F), dev)
    _check(w_down_scale, "w_down_scale", torch.float32, (E, H // 128, F // 128), dev)
    if correction_bias is not None:
        _check(correction_bias, "correction_bias", torch.float32, (E,), dev)
    p = make_params(T, H, E, F, top_k, scoring, renormalize, num_expert_group, topk_group,
                    routed_scaling_factor, path)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, H), dev)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev) if return_routing else None
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev) if return_routing else None
    with torch.cuda.device(dev):
        n = int(lib().fused_moe_fp8_workspace_bytes(ctypes.byref(p)))
        if workspace is None:
            workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        elif workspace.dtype != torch.uint8 or workspace.numel() < n:
            raise ValueError("workspace must be a uint8 tensor with >= %d bytes" % n)
        st = lib().fused_moe_fp8_fwd(
            _ptr(hidden_states), _ptr(gating_output), _ptr(wgu), _ptr(w_gate_up_scale), _ptr(wd),
            _ptr(w_down_scale), _ptr(correction_bias), ctypes.byref(p), _ptr(out), _ptr(ids),
            _ptr(w), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_fp8_fwd")
    if return_routing:
        return out, ids, w
    return out


def fused_moe_fp8_stage(stage, params, hidden_states, fw, topk_ids, topk_weights, out,
                        workspace):
    """One stage of the FP8 pass's expert part (see include/moe.h): ``fw`` holds w_gate_up,
    w_gate_up_scale, w_down, w_down_scale (uint8 codes); ``params`` a MoEParams; the workspace
    at least fp8_workspace_bytes(params) bytes.  Tensors are assumed checked by the caller."""
    dev = hidden_states.device
    with torch.cuda.device(dev):
        st = lib().fused_moe_fp8_stage(
            int(stage), _ptr(hidden_states), _ptr(fw["w_gate_up"]), _ptr(fw["w_gate_up_scale"]),
            _ptr(fw["w_down"]), _ptr(fw["w_down_scale"]), _ptr(topk_ids), _ptr(topk_weights),
            ctypes.byref(params), _ptr(out), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "fused_moe_fp8_stage(%s)" % STAGE_NAMES.get(stage, stage))


def fp8_workspace_bytes(params):
    return int(lib().fused_moe_fp8_workspace_bytes(ctypes.byref(params)))


def moe_stream_read(buf, sink=None):
    """One streaming read of the bytes of the device tensor buf (the HBM read ceiling the
    expert GEMMs' weight streams are compared with).  Returns the int32 sink tensor (one word
    per CU) that the kernel writes."""
    dev = buf.device
    if sink is None:
        sink = torch.empty(int(lib().moe_stream_read_sink_words()), dtype=torch.int32,
                           device=dev)
    nbytes = buf.numel() * buf.element_size()
    with torch.cuda.device(dev):
        st = lib().moe_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(dev))
    if st != MOE_OK:
        raise MoEError(st, "moe_stream_read")
    return sink
