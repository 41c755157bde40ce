"""Host-side tools of bench.py: the one-GPU guard, the rocprofv3 kernel-trace summary (its
median column) and the kernel-source hash that marks a counter summary as stale."""
import os
import shutil
import subprocess
import sys
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

WIDE = "void moe_wide::k_wide_gemm<true, 0, 3, 0>(moe::GemmProblem, int, int)"
WS = "void moe_ws::k_ws_gemm<false, 3, 2, 1, 2, 3, 0, 1>(moe::GemmProblem)"


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_trace_summary_reports_the_median_of_the_dispatches(tmp_path, monkeypatch):
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    (d / "run_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n"
        '"%s",4,14000,3500,100,2000,6000,1\n' % WIDE)
    # four dispatches of 2, 3, 3 and 6 us: average 3.5, median 3.0
    rows = [(0, 2000), (10, 3010), (20, 3020), (30, 6030)]
    (d / "run_kernel_trace.csv").write_text(
        "Kernel_Name,Start_Timestamp,End_Timestamp\n" +
        "".join('"%s",%d,%d\n' % (WIDE, a, b) for a, b in rows))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path / "out"))
    args = types.SimpleNamespace(config="ds-v3-grouped-prefill",
                                 summarize_trace=str(tmp_path / "trace"), weights="16bit",
                                 pmc_commands=["rocprofv3 ..."])
    bench.summarize_trace(args)
    text = (tmp_path / "out" / "kernel_trace_ds-v3-grouped-prefill.md").read_text()
    assert "| `moe_wide::k_wide_gemm<true, 0, 3, 0>` | 4 | 3.50 | 3.00 | 2.00 | 6.00 |" in text


def test_kernel_source_hash_follows_the_kernel_family(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "mixture_experts_forward_amd", "csrc")
    csrc = tmp_path / "mixture_experts_forward_amd" / "csrc"
    shutil.copytree(src, csrc, ignore=shutil.ignore_patterns("*.o", "_build"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    wide0, ws0 = bench.kernel_source_hash(WIDE), bench.kernel_source_hash(WS)
    assert wide0 != ws0
    # an edit to the 256 x 256 kernel marks only its summaries stale
    with open(csrc / "moe_wide_kernel.h", "a") as f:
        f.write("\n")
    wide1, ws1 = bench.kernel_source_hash(WIDE), bench.kernel_source_hash(WS)
    assert wide1 != wide0 and ws1 == ws0
    # an edit to the shared device helpers marks every family stale
    with open(csrc / "moe_device.h", "a") as f:
        f.write("\n")
    assert bench.kernel_source_hash(WIDE) != wide1 and bench.kernel_source_hash(WS) != ws1


def test_gemm_roles_of_kernel_names():
    """Counter summaries are filed by the GEMM role read from the kernel name: the 16-bit
    families carry their row source as the second template argument (2: the shared expert's
    dense rows); the MXFP4 row-tiled and 256 x 256 kernels run on sorted rows only, so their
    second argument (a tile width) never marks them as the shared expert."""
    assert bench._role(WIDE) == "gate_up"
    assert bench._role(WS) == "down"
    assert bench._role("void moe_wide::k_wide_gemm<false, 2, 3, 0>(moe::GemmProblem, int, int)") \
        == "shared_down"
    assert bench._role("void moe_wide::k_wide_mx<true>(moe::GemmProblem, int, int)") == "gate_up"
    assert bench._role("void moe_mx::k_mx_tiled<false, 2, 3>(moe::GemmProblem, int, int)") \
        == "down"
    assert bench._role("void moe_mx::k_mx_gemm<true, 3, 1, 2, 3>(moe::GemmProblem)") == "gate_up"
    assert bench._role("void k_combine<0>(unsigned short const*)") is None
