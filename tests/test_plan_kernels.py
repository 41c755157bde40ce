"""The host plan and the instantiated GEMM kernels agree: every tile shape that make_plan picks
over a sweep of shapes, routing densities, paths and weight formats has a kernel instantiated
for its direction (a launcher that finds none returns an error at run time), and every
instantiated shape is picked by some plan (no kernel in the library is unreachable).

The planner is host-only C++ (no HIP call), so it is compiled here with g++ beside a small
driver; the instantiation lists are read from the launcher sources."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_forward_amd", "csrc")

KIND = {0: "ws", 1: "tiled", 3: "wide", 4: "mx", 5: "mx_tiled", 6: "mx_wide"}

DRIVER = r"""
#include <stdio.h>
#include <initializer_list>
#include "moe_plan.h"
static void put(const char *dir, const moe::TileChoice &t)
{
    printf("%s %d %d %d %d %d\n", dir, t.kind, t.nt, t.mt, t.ksplit, t.stages);
}
int main()
{
    const int Ts[] = {1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384};
    const int Es[] = {8, 32, 64, 128, 256};
    const int ks[] = {1, 2, 4, 6, 8};
    const int HF[][2] = {{2048, 768}, {4096, 1536}, {7168, 2048}, {320, 192}};
    const int paths[] = {MOE_PATH_AUTO, MOE_PATH_DIRECT, MOE_PATH_SORTED};
    for (int T : Ts)
        for (int E : Es)
            for (int k : ks)
                for (auto &hf : HF)
                    for (int ng : {1, 8})
                        for (int path : paths)
                            for (int wfmt = 0; wfmt < 2; ++wfmt) {
                                if (E % ng != 0 || k > E)
                                    continue;
                                moe_params_t p = {};
                                p.num_tokens = T;
                                p.hidden = hf[0];
                                p.num_experts = E;
                                p.inter = hf[1];
                                p.top_k = k;
                                p.scoring = ng > 1 ? MOE_SCORING_SIGMOID : MOE_SCORING_SOFTMAX;
                                p.renormalize = 1;
                                p.num_expert_group = ng;
                                p.topk_group = ng > 1 ? 4 : 1;
                                p.routed_scaling_factor = 1.0f;
                                p.path = path;
                                p.dtype = MOE_DTYPE_BF16;
                                if (moe::check_dims(&p) != MOE_OK ||
                                    moe::check_routing(&p, 0) != MOE_OK)
                                    continue;
                                for (int S : {0, 2048}) {
                                    moe::Plan pl;
                                    moe::make_plan(&p, S, &pl, wfmt);
                                    put("G", pl.gate_up);
                                    put("D", pl.down);
                                    if (S > 0) {
                                        put("G", pl.shared_gate_up);
                                        put("D", pl.shared_down);
                                    }
                                }
                            }
    return 0;
}
"""


def _split_directions(text, start_marker):
    """Case lines of one dispatch: (gate-up part, down part) of its `if constexpr (GATE_UP)`."""
    i = text.index(start_marker)
    body = text[text.index("if constexpr (GATE_UP) {", i):text.index("#undef", i)]
    up, down = body.split("} else {")
    return up, down


def _cases(part, macro):
    return [tuple(int(v) for v in m.split(","))
            for m in re.findall(r"^\s*%s\(([\d,\s]+)\)" % macro, part, re.M)]


def instantiated():
    """(direction, kind, key) of every instantiated routed-GEMM shape; key holds the tile
    fields that the kind's launcher matches on."""
    out = set()
    ws = open(os.path.join(CSRC, "moe_gemm_ws.hip")).read()
    for d, part in zip("GD", _split_directions(ws, "#define MOE_WS_CASE")):
        for nt, mt, ks, st in _cases(part, "MOE_WS_CASE"):
            out.add((d, "ws", (nt, mt, ks, st)))
    tiled = open(os.path.join(CSRC, "moe_gemm_tiled.hip")).read()
    for d, part in zip("GD", _split_directions(tiled, "#define MOE_TILED_CASE")):
        for bm, ntw, st in _cases(part, "MOE_TILED_CASE"):
            out.add((d, "tiled", (ntw, bm // 16, st)))
    mx = open(os.path.join(CSRC, "moe_gemm_mx.hip")).read()
    for d, part in zip("GD", _split_directions(mx, "#define MOE_MX_CASE")):
        for nt, ks, st in _cases(part, "MOE_MX_CASE"):
            out.add((d, "mx", (nt, ks, st)))
    for m in re.findall(r"^\s*MOE_MXT_CASE\((true|false),\s*(\d+),\s*(\d+)\)", mx, re.M):
        out.add(("G" if m[0] == "true" else "D", "mx_tiled", (int(m[1]), 4, int(m[2]))))
    # the 256 x 256 kernels take no tile fields; both directions are instantiated
    for d in "GD":
        out.add((d, "wide", ()))
        out.add((d, "mx_wide", ()))
    return out


def key(kind, nt, mt, ks, st):
    return {"ws": (nt, mt, ks, st), "tiled": (nt, mt, st), "mx": (nt, ks, st),
            "mx_tiled": (nt, mt, st), "wide": (), "mx_wide": ()}[kind]


@pytest.fixture(scope="module")
def planned(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    d = tmp_path_factory.mktemp("plan")
    (d / "driver.cpp").write_text(DRIVER)
    exe = d / "plan_sweep"
    subprocess.run([gxx, "-std=c++17", "-O1", "-I" + CSRC, str(d / "driver.cpp"),
                    os.path.join(CSRC, "moe_plan.cpp"), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], check=True, capture_output=True,
                           text=True).stdout.split("\n")
    out = set()
    for ln in lines:
        if not ln:
            continue
        d_, kind, nt, mt, ks, st = ln.split()
        k = KIND[int(kind)]
        out.add((d_, k, key(k, int(nt), int(mt), int(ks), int(st))))
    return out


def test_instantiation_lists_are_read():
    inst = instantiated()
    assert ("G", "ws", (1, 1, 4, 3)) in inst and ("D", "tiled", (4, 4, 2)) in inst
    assert len([x for x in inst if x[1] == "ws"]) >= 3


def test_every_planned_shape_is_instantiated(planned):
    missing = sorted(planned - instantiated())
    assert not missing, "plan picks shapes with no kernel: %s" % missing


def test_every_instantiated_shape_is_planned(planned):
    unreachable = sorted(instantiated() - planned)
    assert not unreachable, "kernels no plan picks: %s" % unreachable
