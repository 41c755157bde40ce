"""The C-ABI library loads without a GPU, exports every function include/moe.h declares, and
rejects invalid arguments on the host before touching the GPU (no compute call here)."""
import ctypes
import os
import re

import pytest

import mixture_experts_forward_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n not in skip})


def test_library_exports_every_declared_function():
    L = moe.lib()
    names = _declared_functions()
    assert "fused_moe_fwd" in names and "moe_route" in names and len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe.SIGNATURES), "binding and header disagree"


def test_abi_version_and_status_strings():
    assert moe.lib().moe_abi_version() == 3
    for s in (0, -1, -2, -3, -4, -5):
        assert moe.status_string(s) and moe.status_string(s) != "unknown status"
    assert moe.status_string(7) == "unknown status"


def _check(p, bias=0, S=0):
    return moe.lib().moe_check_params(ctypes.byref(p), bias, S)


def test_check_params_rules():
    ok = moe.make_params(32, 2048, 128, 768, 8)
    assert _check(ok) == 0
    assert moe.lib().moe_check_params(None, 0, 0) == -1
    assert _check(moe.make_params(-1, 2048, 128, 768, 8)) == -2
    assert _check(moe.make_params(0, 2048, 128, 768, 8)) == 0          # T = 0 is valid
    assert _check(moe.make_params(4, 0, 8, 64, 2)) == -2
    assert _check(moe.make_params(4, 128, 8, 64, 9)) == -2              # k > E
    assert _check(moe.make_params(4, 128, 64, 64, 33)) == -3            # k > 32
    assert _check(moe.make_params(4, 128, 2048, 64, 2)) == -3           # E > 1024
    assert _check(moe.make_params(4, 96, 8, 64, 2)) == -3               # H % 64
    assert _check(moe.make_params(4, 128, 8, 80, 2)) == -3              # F % 64
    bad_dtype = moe.make_params(4, 128, 8, 64, 2)
    bad_dtype.dtype = 2
    assert _check(bad_dtype) == -3                                      # unknown element type
    assert _check(moe.make_params(4, 128, 8, 64, 2, dtype=__import__("torch").float16)) == 0
    assert _check(moe.make_params(4, 128, 8, 64, 2), bias=1) == -3      # softmax + bias
    g = moe.make_params(4, 128, 8, 64, 2, "sigmoid", True, 3, 1)        # 8 % 3
    assert _check(g) == -3
    g = moe.make_params(4, 128, 8, 64, 2, "softmax", True, 2, 1)        # softmax + groups
    assert _check(g) == -3
    g = moe.make_params(4, 128, 8, 64, 5, "sigmoid", True, 4, 2)        # k > 2 groups * 2
    assert _check(g) == -3
    g = moe.make_params(4, 128, 8, 64, 4, "sigmoid", True, 4, 2)
    assert _check(g, bias=1) == 0
    assert _check(moe.make_params(65, 128, 8, 64, 8, path="direct")) == -3  # 520 routes > 512
    assert _check(moe.make_params(64, 128, 8, 64, 8, path="direct")) == 0
    assert _check(ok, S=-64) == -2
    assert _check(ok, S=100) == -3
    assert _check(ok, S=18432) == 0


def test_workspace_bytes():
    # decode batch (2 routed rows per expert): direct path, h and y in route order
    p = moe.make_params(32, 2048, 128, 768, 8)
    n = moe.workspace_bytes(p)
    P = 256
    assert n >= P * 768 * 2 + P * 2048 * 2
    assert n % 256 == 0
    assert moe.workspace_bytes(p, 18432) >= n + 32 * 18432 * 2 + 32 * 2048 * 2
    assert moe.workspace_bytes(moe.make_params(0, 2048, 128, 768, 8)) == 0
    # the same shape forced onto the sorted path also holds the sorted lists, padded to 16 rows
    s = moe.workspace_bytes(moe.make_params(32, 2048, 128, 768, 8, path="sorted"))
    slots = P + 128 * 15
    assert s >= slots * 768 * 2 + P * 2048 * 2 and s > n
    # prefill: 256-row tiles
    q = moe.workspace_bytes(moe.make_params(4096, 7168, 256, 2048, 8))
    assert q >= (32768 + 256 * 255) * 2048 * 2 + 32768 * 7168 * 2


def test_entry_points_reject_before_launch():
    """Invalid calls return their error code without any HIP call (runs without a GPU)."""
    L = moe.lib()
    p = moe.make_params(4, 128, 8, 64, 2)
    fake = ctypes.c_void_p(4096)
    assert L.fused_moe_fwd(None, fake, fake, fake, None, ctypes.byref(p), fake, None, None, fake,
                           1 << 30, None) == -1
    assert L.fused_moe_fwd(fake, fake, fake, fake, None, None, fake, None, None, fake, 1 << 30,
                           None) == -1
    bad = moe.make_params(4, 128, 8, 64, 9)
    assert L.fused_moe_fwd(fake, fake, fake, fake, None, ctypes.byref(bad), fake, None, None,
                           fake, 1 << 30, None) == -2
    assert L.fused_moe_fwd(fake, fake, fake, fake, fake, ctypes.byref(p), fake, None, None, fake,
                           1 << 30, None) == -3   # softmax with a bias
    assert L.fused_moe_fwd(fake, fake, fake, fake, None, ctypes.byref(p), fake, None, None, fake,
                           16, None) == -4        # workspace too small
    odd = ctypes.c_void_p(4096 + 2)
    assert L.fused_moe_fwd(odd, fake, fake, fake, None, ctypes.byref(p), fake, None, None, fake,
                           1 << 30, None) == -3   # misaligned bf16 pointer
    assert L.fused_moe_shared_fwd(fake, fake, fake, fake, None, None, None, 64, ctypes.byref(p),
                                  fake, None, None, fake, 1 << 30, None) == -1
    assert L.fused_moe_shared_fwd(fake, fake, fake, fake, None, fake, fake, 0, ctypes.byref(p),
                                  fake, None, None, fake, 1 << 30, None) == -2
    assert L.fused_moe_experts_fwd(fake, fake, fake, None, fake, ctypes.byref(p), fake, fake,
                                   1 << 30, None) == -1
    z = moe.make_params(0, 128, 8, 64, 2)
    assert L.fused_moe_fwd(fake, fake, fake, fake, None, ctypes.byref(z), fake, None, None, None,
                           0, None) == 0          # T = 0: nothing to do
    assert L.moe_route(fake, None, None, fake, fake, None) == -1
    assert L.moe_route(fake, fake, ctypes.byref(p), fake, fake, None) == -3
    assert L.moe_route(None, None, ctypes.byref(p), fake, fake, None) == -1
    assert L.moe_align_sort(fake, 4, 2, 0, 16, fake, fake, fake, fake, fake, None, 0,
                            None) == -2
    assert L.moe_align_sort(fake, 4, 2, 2048, 16, fake, fake, fake, fake, fake, None, 0,
                            None) == -3
    assert L.moe_align_sort(fake, 4, 2, 8, 0, fake, fake, fake, fake, fake, None, 0, None) == -3
    assert L.moe_align_sort(None, 4, 2, 8, 16, fake, fake, fake, fake, fake, None, 0,
                            None) == -1


def test_align_sort_workspace_checks():
    """The align workspace: 0 bytes up to 1024 routes, a chunks x E count table above; a short
    or missing workspace is rejected before anything is launched."""
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: checks come first
    q = L.moe_align_sort_workspace_bytes
    assert q(128, 8, 128, 16) == 0                      # 1024 routes: one workgroup
    assert q(129, 8, 128, 16) == 2 * 128 * 4            # 1032 routes: two chunks
    assert q(4096, 8, 256, 256) == 32 * 256 * 4         # DeepSeek-V3 prefill: 32 chunks
    assert q(4096, 8, 0, 16) == 0 and q(4, 2, 8, 0) == 0 and q(-1, 2, 8, 16) == 0
    need = q(4096, 8, 256, 256)
    args = (fake, 4096, 8, 256, 256, fake, fake, fake, fake, fake)
    assert L.moe_align_sort(*args, fake, need - 4, None) == -4        # too small
    assert L.moe_align_sort(*args, None, 0, None) == -4               # none given
    assert L.moe_align_sort(*args, None, need, None) == -1            # size without a buffer
    assert L.moe_align_sort(*args, ctypes.c_void_p((1 << 20) + 2), need, None) == -3


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.fused_moe_experts_fwd(x, torch.zeros(8, 128, 128, dtype=torch.bfloat16),
                                  torch.zeros(8, 128, 64, dtype=torch.bfloat16),
                                  torch.zeros(4, 2, dtype=torch.int32),
                                  torch.zeros(4, 2, dtype=torch.float32))


def test_masked_entry_points_reject_before_launch():
    L = moe.lib()
    ws_need = L.fused_moe_masked_workspace_bytes(32, 128, 7168, 2048)
    assert ws_need > 0
    assert L.fused_moe_masked_workspace_bytes(32, 0, 7168, 2048) == 0   # nothing to do
    assert L.fused_moe_masked_workspace_bytes(0, 128, 7168, 2048) == 0
    assert L.fused_moe_masked_workspace_bytes(4, 8, 96, 64) == 0        # H % 64
    # larger row blocks need more workspace (sorted layout and h grow with E * max_m)
    assert L.fused_moe_masked_workspace_bytes(32, 256, 7168, 2048) > ws_need
    fake = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: checks come first
    args = lambda E, m, H, F, ws, n: (fake, fake, fake, fake, E, m, H, F, fake, ws, n, None)
    assert L.fused_moe_masked_fwd(*args(0, 8, 128, 64, fake, 1 << 30)) == -2
    assert L.fused_moe_masked_fwd(*args(4, -1, 128, 64, fake, 1 << 30)) == -2
    assert L.fused_moe_masked_fwd(*args(4, 8, 96, 64, fake, 1 << 30)) == -3
    assert L.fused_moe_masked_fwd(*args(2048, 8, 128, 64, fake, 1 << 30)) == -3   # E > 1024
    assert L.fused_moe_masked_fwd(*args(4, 8, 128, 64, None, 1 << 30)) == -1
    n = L.fused_moe_masked_workspace_bytes(4, 8, 128, 64)
    assert L.fused_moe_masked_fwd(*args(4, 8, 128, 64, fake, n - 1)) == -4
    assert L.fused_moe_masked_fwd(*args(4, 0, 128, 64, None, 0)) == 0   # max_m = 0: no-op
    assert L.fused_moe_masked_fwd(fake, None, fake, fake, 4, 8, 128, 64, fake, fake, n,
                                  None) == -1                            # masked_m missing
    assert L.fused_moe_masked_stage(5, fake, fake, fake, fake, 4, 8, 128, 64, fake, fake, n,
                                    None) == -3                          # no combine stage
    # a stage checks only what it reads: the down stage needs no activations or masked_m
    assert L.fused_moe_masked_stage(3, None, None, None, fake, 4, 8, 128, 64, None, fake, n,
                                    None) == -1                          # but out is needed


def test_fp8_contiguous_and_quant_reject_before_launch():
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: checks come first
    odd = ctypes.c_void_p((1 << 20) + 4)
    g = lambda E, P, N, K, a=fake, off=fake: L.moe_grouped_gemm_fp8_contiguous(
        a, fake, fake, fake, off, E, P, N, K, fake, None)
    assert g(0, 16, 128, 128) == -2
    assert g(4, -1, 128, 128) == -2
    assert g(4, 16, 96, 128) == -3                 # N % 64
    assert g(4, 16, 128, 200) == -3                # K % 128
    assert g(2048, 16, 128, 128) == -3             # E > 1024
    assert g(4, 16, 128, 128, a=odd) == -3         # a not 16-byte aligned
    assert g(4, 16, 128, 128, off=None) == -1
    assert g(4, 0, 128, 128, a=None, off=None) == 0   # P = 0: nothing to do
    assert g(4, (1 << 30) - 64, 1 << 16, 128) == -3    # tile count past the launch bound
    q = lambda M, K, x=fake, qq=fake: L.moe_quant_fp8(x, M, K, qq, fake, None)
    assert q(-1, 128) == -2
    assert q(4, 0) == -2
    assert q(4, 100) == -3                         # K % 8
    assert q(4, 128, qq=ctypes.c_void_p((1 << 20) + 4)) == -3   # q not 8-byte aligned
    assert q(4, 128, x=None) == -1
    assert q(0, 128, x=None) == 0                  # M = 0: nothing to do


def test_mxfp4_entry_points_reject_before_launch():
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)
    ok = moe.make_params(32, 2048, 128, 768, 8)
    n = L.fused_moe_mxfp4_workspace_bytes(ctypes.byref(ok))
    assert n > 0
    call = lambda p, ws, nb, hidden=fake: L.fused_moe_mxfp4_fwd(
        hidden, fake, fake, fake, fake, fake, None, ctypes.byref(p), fake, None, None, ws, nb,
        None)
    assert call(moe.make_params(32, 2048, 128, 768, 8), fake, n - 1) == -4
    assert call(moe.make_params(32, 2048, 128, 768, 8), fake, n, hidden=None) == -1
    assert call(moe.make_params(32, 2112, 128, 768, 8), fake, 1 << 30) == -3     # H % 128
    assert call(moe.make_params(32, 2048, 128, 704, 8), fake, 1 << 30) == -3     # F % 128
    f16 = moe.make_params(32, 2048, 128, 768, 8, dtype=__import__("torch").float16)
    assert call(f16, fake, 1 << 30) == -3                                        # bf16 only
    assert L.fused_moe_mxfp4_workspace_bytes(ctypes.byref(f16)) == 0
    assert call(moe.make_params(0, 2048, 128, 768, 8), None, 0) == 0             # T = 0


def test_fp8_pass_path_rules():
    """The FP8 pass's direct form: chosen by AUTO for a few routes, refused past 64 routes or
    for K that is not a multiple of 256 or too long for one workgroup's LDS."""
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)
    ws = lambda p: L.fused_moe_fp8_workspace_bytes(ctypes.byref(p))
    call = lambda p: L.fused_moe_fp8_fwd(fake, fake, fake, fake, fake, fake, None,
                                         ctypes.byref(p), fake, None, None, fake, 1 << 40, None)
    # T = 1, k = 8 at Qwen3-30B-A3B dimensions: direct, ids / weights / h / y only
    d = ws(moe.make_params(1, 2048, 128, 768, 8))
    assert d == 2 * 256 + 8 * 768 * 2 + 8 * 2048 * 2
    assert ws(moe.make_params(1, 2048, 128, 768, 8, path="direct")) == d
    assert ws(moe.make_params(1, 2048, 128, 768, 8, path="sorted")) > d
    # AUTO keeps the sorted form past 64 routes or 8 routes per expert
    assert ws(moe.make_params(9, 2048, 128, 768, 8)) > 9 * 8 * (768 + 2048) * 2 + 512
    assert ws(moe.make_params(8, 256, 4, 256, 8)) == \
        ws(moe.make_params(8, 256, 4, 256, 8, path="sorted"))
    # DIRECT refused: 65 routes, K % 256 != 0 (F = 384), K past the LDS limit (H = 9728)
    assert call(moe.make_params(65, 2048, 128, 768, 1, path="direct")) == -3
    assert call(moe.make_params(2, 2048, 128, 384, 8, path="direct")) == -3
    assert call(moe.make_params(2, 9728, 128, 768, 8, path="direct")) == -3
    assert ws(moe.make_params(65, 2048, 128, 768, 1, path="direct")) == 0
    # the same shapes on AUTO fall to the sorted form
    assert ws(moe.make_params(2, 2048, 128, 384, 8)) == \
        ws(moe.make_params(2, 2048, 128, 384, 8, path="sorted"))


def test_stream_read_rejects_before_launch():
    """The streaming-read measurement validates its arguments before any HIP call."""
    L = moe.lib()
    fake = ctypes.c_void_p(4096)
    assert L.moe_stream_read(None, 0, None, None) == 0                   # nothing to read
    assert L.moe_stream_read(None, 1024, fake, None) == -1
    assert L.moe_stream_read(fake, 1024, None, None) == -1
    assert L.moe_stream_read(ctypes.c_void_p(4096 + 8), 1024, fake, None) == -3  # alignment
    assert L.moe_stream_read(fake, 1000, fake, None) == -3                # bytes % 16



def test_noalloc_checks_before_touching_the_gpu():
    """fused_moe_fwd_noalloc rejects a pass whose workspace exceeds its fixed array, and passes
    fused_moe_fwd's own argument errors through, before any HIP call."""
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)
    big = moe.make_params(4096, 7168, 256, 2048, 8, "sigmoid")
    assert moe.workspace_bytes(big) > moe.NOALLOC_SCRATCH_BYTES
    assert L.fused_moe_fwd_noalloc(fake, fake, fake, fake, fake, ctypes.byref(big), fake, None,
                                   None, None) == -4
    assert L.fused_moe_fwd_noalloc(fake, fake, fake, fake, None, None, fake, None, None,
                                   None) == -1
    bad = moe.make_params(4, 128, 8, 64, 9)
    assert L.fused_moe_fwd_noalloc(fake, fake, fake, fake, None, ctypes.byref(bad), fake, None,
                                   None, None) == -2
    z = moe.make_params(0, 128, 8, 64, 2)
    assert L.fused_moe_fwd_noalloc(None, None, None, None, None, ctypes.byref(z), None, None,
                                   None, None) == 0
