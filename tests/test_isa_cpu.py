"""Structural check of the compiled exchange kernels (CPU only: hipcc -S).

The exchange kernel runs a work-ticket loop in which thread 0 claims tickets
and finishes chunks between work-group barriers. If a thread-0 region spans
the loop's back edge, the compiler may turn it into a divergent loop exit:
lane 0 is parked outside the loop while the other lanes pass the barrier and
re-read a stale ticket forever. This test compiles the kernels for gfx950
and asserts that no exchange-kernel variant has a divergent loop exit
(`s_andn2_b64 exec, exec, ...`), and that every barrier-bearing loop of the
map builder keeps its divergent exits in barrier-free inner loops.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "domain_decomposition_halo_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def _isa(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "--cuda-device-only", "-S", src, "-o", str(out)],
                   check=True, capture_output=True)
    kernels, cur = {}, None
    for line in out.read_text().splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            kernels[cur] = []
            continue
        if cur is not None:
            kernels[cur].append(line)
            if "s_endpgm" in line:
                cur = None
    return kernels


def test_exchange_kernels_have_uniform_loops(tmp_path):
    kernels = _isa(os.path.join(CSRC, "ddh_exchange.hip"), tmp_path)
    ex = {k: v for k, v in kernels.items() if "exchange_kernel" in k}
    assert len(ex) == 3
    for name, lines in ex.items():
        assert sum("s_barrier" in ln for ln in lines) >= 4, name
        assert not any("s_andn2_b64 exec, exec" in ln for ln in lines), name


def _loops_with_barriers_and_divergent_exits(lines):
    """Loop headers (by label) whose own body (not an inner loop) holds both a
    barrier and a divergent exit."""
    depth_of = {}
    own = {}
    cur_loop = None
    for ln in lines:
        m = re.match(r"^\.(LBB\S+):.*(?:Loop Header: Depth=(\d+)|Parent Loop BB\S+ Depth=(\d+)|"
                     r"in Loop: Header=(BB\S+) Depth=(\d+))", ln)
        if m:
            if m.group(2):
                cur_loop = m.group(1)[1:] if m.group(1).startswith("L") else m.group(1)
                cur_loop = m.group(1).replace("LBB", "BB")
            elif m.group(4):
                cur_loop = m.group(4)
            own.setdefault(cur_loop, [0, 0])
            continue
        if re.match(r"^\.LBB\S+:", ln):
            cur_loop = None
            continue
        if cur_loop is None:
            continue
        if "s_barrier" in ln:
            own[cur_loop][0] += 1
        if "s_andn2_b64 exec, exec" in ln:
            own[cur_loop][1] += 1
    return [k for k, (b, d) in own.items() if b and d]


def test_builder_barriers_never_share_a_loop_with_divergent_exits(tmp_path):
    kernels = _isa(os.path.join(CSRC, "ddh_build.hip"), tmp_path)
    assert any("select_write_kernel" in k for k in kernels)
    for name, lines in kernels.items():
        assert _loops_with_barriers_and_divergent_exits(lines) == [], name
