"""The C ABI on a machine without a GPU: library, exports, host logic.

No device work runs here. Checks: libddh.so loads and exports every function
declared in include/ddh.h; the binding fails loudly when the library is
missing; parameter validation and the pulse schedule (host code of the
library) agree with the oracle's schedule; calls that need maps report
DDH_ESTATE; the product package never touches the oracle.
"""

import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import domain_decomposition_halo_amd as ddh
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddh.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddh_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 20
    lib = ctypes.CDLL(ddh.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(ddh.EXPORTS) == names
    out = subprocess.run(["nm", "-D", "--defined-only", ddh.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ddh_\w+)", out))
    assert set(names) <= exported


def test_binding_fails_loudly_without_library(tmp_path):
    pkg = tmp_path / "domain_decomposition_halo_amd"
    pkg.mkdir()
    src = open(os.path.join(ROOT, "domain_decomposition_halo_amd", "__init__.py")).read()
    (pkg / "__init__.py").write_text(src)
    res = subprocess.run([sys.executable, "-c", "import domain_decomposition_halo_amd"],
                         cwd=tmp_path, capture_output=True, text=True)
    assert res.returncode != 0 and "ImportError" in res.stderr and "build" in res.stderr


def test_product_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "domain_decomposition_halo_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "ddh_oracle" not in text, f
                assert "ddho_" not in text, f


def _schedule_via_abi(grid, box, rc):
    plan = ddh.Plan(grid, box, rc)
    try:
        return plan.layout()["pulses"]
    finally:
        plan.close()


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_schedule_matches_oracle_workloads(k):
    p = W.WORKLOADS[k].params()
    assert _schedule_via_abi(p["grid"], p["box"], p["rc"]) == oracle.schedule(p["grid"], p["box"],
                                                                             p["rc"])


def test_schedule_matches_oracle_random():
    rng = np.random.default_rng(0)
    for _ in range(300):
        grid = tuple(int(v) for v in rng.integers(1, 9, size=3))
        box = tuple(float(np.float32(v)) for v in rng.uniform(2.0, 30.0, size=3))
        rc = float(np.float32(rng.uniform(0.1, 6.0)))
        try:
            want = oracle.schedule(grid, box, rc)
        except oracle.OracleError as e:
            with pytest.raises(ddh.DDHError) as g:
                _schedule_via_abi(grid, box, rc)
            assert g.value.code == ddh.DDH_ERANGE and e.code == oracle.ERANGE
            continue
        assert _schedule_via_abi(grid, box, rc) == want


def test_parameter_errors():
    for grid, box, rc in [((0, 1, 1), (4, 4, 4), 1.0), ((2, 1, 1), (4, 4, 4), 0.0),
                          ((2, 1, 1), (4, 4, 4), -1.0), ((2, 1, 1), (0, 4, 4), 1.0),
                          ((2, 1, 1), (4, 4, 4), float("nan")), ((2, 1, 1), (4, 4, 4), float("inf"))]:
        with pytest.raises(ddh.DDHError) as e:
            ddh.Plan(grid, box, rc)
        assert e.value.code == ddh.DDH_EINVAL
    with pytest.raises(ddh.DDHError) as e:
        ddh.Plan((2, 1, 1), (4, 4, 4), 2.25)        # rc > L - w
    assert e.value.code == ddh.DDH_ERANGE
    with pytest.raises(ddh.DDHError) as e:
        ddh.Plan((40, 1, 1), (40, 4, 4), 17.5)      # 18 pulses > DDH_MAX_PULSES
    assert e.value.code == ddh.DDH_ERANGE


def test_calls_before_build_report_state():
    plan = ddh.Plan((2, 2, 2), (8.0, 8.0, 8.0), 1.0)
    b, nh, nt = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    assert ddh.ddh_domain_info(plan._h, 0, ctypes.byref(b), ctypes.byref(nh),
                               ctypes.byref(nt)) == ddh.DDH_ESTATE
    assert ddh.ddh_exchange_coords(plan._h, None, 0, None) == ddh.DDH_ESTATE
    assert ddh.ddh_exchange_forces(plan._h, None, 0, None) == ddh.DDH_ESTATE
    assert ddh.ddh_exchange_step(plan._h, None, None, 0, None) == ddh.DDH_ESTATE
    assert "ddh_build_maps" in ddh.last_error()
    assert ddh.ddh_query(plan._h, None) == ddh.DDH_EINVAL
    assert ddh.ddh_exchange_coords(None, None, 0, None) == ddh.DDH_EINVAL
    plan.close()


def test_mode_and_tune_validation():
    plan = ddh.Plan((2, 2, 2), (8.0, 8.0, 8.0), 1.0)
    plan.set_mode(ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH)
    plan.set_mode(ddh.DDH_MODE_FUSED)
    plan.set_mode(ddh.DDH_MODE_AUTO | ddh.DDH_MODE_GRAPH)
    plan.set_mode(ddh.DDH_MODE_STAGED)
    with pytest.raises(ddh.DDHError):
        plan.set_mode(ddh.DDH_MODE_STAGED | ddh.DDH_MODE_GRAPH)
    for bad in (4, 8, 32):
        with pytest.raises(ddh.DDHError):
            plan.set_mode(bad)
    plan.tune(ddh.DDH_TUNE_CHUNK, 100)
    plan.tune(ddh.DDH_TUNE_CHUNK, 0)
    for v in (1024, 512, 256, 0):
        plan.tune(ddh.DDH_TUNE_BLOCK, v)
    for v in (1, 2, 0):
        plan.tune(ddh.DDH_TUNE_EXIT_PUBLISH, v)
        plan.tune(ddh.DDH_TUNE_PAD_MAPS, v)
    for v in (1, 0):
        plan.tune(ddh.DDH_TUNE_HEADS_FIRST, v)
        plan.tune(ddh.DDH_TUNE_LDS_STAGE, v)
    plan.tune(ddh.DDH_TUNE_LDS_STAGE, 2)
    plan.tune(ddh.DDH_TUNE_STATIC_FIRST, 1)
    plan.tune(ddh.DDH_TUNE_STATIC_FIRST, 0)
    plan.tune(ddh.DDH_TUNE_FLAGS, 0)
    plan.tune(ddh.DDH_TUNE_FLAGS, 1)
    plan.tune(ddh.DDH_TUNE_NARROW_MAPS, 0)
    plan.tune(ddh.DDH_TUNE_NARROW_MAPS, 1)
    plan.tune(ddh.DDH_TUNE_WAVE_CHUNKS, 1)
    plan.tune(ddh.DDH_TUNE_WAVE_CHUNKS, 0)
    for v in (1, 2, 0):
        plan.tune(ddh.DDH_TUNE_HOME_SORT, v)
    for key, val in [(ddh.DDH_TUNE_CHUNK, 10), (ddh.DDH_TUNE_CHUNK, 70000),
                     (ddh.DDH_TUNE_GRID, -1), (ddh.DDH_TUNE_SPIN_LIMIT, 0), (99, 1),
                     (ddh.DDH_TUNE_BLOCK, 768), (ddh.DDH_TUNE_STATIC_FIRST, 2),
                     (ddh.DDH_TUNE_EXIT_PUBLISH, 3), (ddh.DDH_TUNE_PAD_MAPS, -1),
                     (ddh.DDH_TUNE_FLAGS, 2), (ddh.DDH_TUNE_NARROW_MAPS, -1),
                     (ddh.DDH_TUNE_WAVE_CHUNKS, 3), (ddh.DDH_TUNE_HOME_SORT, 3),
                     (ddh.DDH_TUNE_HOME_SORT, -1), (ddh.DDH_TUNE_LDS_STAGE, 3)]:
        with pytest.raises(ddh.DDHError) as e:
            plan.tune(key, val)
        assert e.value.code == ddh.DDH_EINVAL
    plan.close()


def test_build_without_device_fails_cleanly():
    plan = ddh.Plan((2, 2, 2), (8.0, 8.0, 8.0), 1.0)
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a device is present")
    except ImportError:
        pass
    code = ddh.ddh_build_maps(plan._h, ctypes.c_void_p(0), 0, None)
    assert code == ddh.DDH_EHIP
    plan.close()


def test_single_hip_runtime_in_process():
    # the binding must bind libddh.so to torch's HIP runtime, whatever the
    # import order of the caller
    code = ("import domain_decomposition_halo_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "libs = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "1"


def test_binding_constants_match_the_header():
    # every integer #define of the header that the binding mirrors has the
    # header's value
    hdr = open(os.path.join(ROOT, "include", "ddh.h")).read()
    defs = dict(re.findall(r"^#define\s+(DDH_[A-Z0-9_]+)\s+\(?(-?\d+)\)?", hdr, re.M))
    assert len(defs) >= 20
    mirrored = [k for k in defs if hasattr(ddh, k)]
    assert len(mirrored) >= 15, mirrored
    for k in mirrored:
        assert getattr(ddh, k) == int(defs[k]), k


def test_header_is_c99_and_links(tmp_path):
    """A C99 program that includes the header and takes the address of every
    declared call compiles with gcc and links against the library."""
    import shutil
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    hdr = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(ddh_[a-z_]+)\s*\(", hdr)))
    src = tmp_path / "uses_ddh.c"
    body = "\n".join(f"    (void)&{n};" for n in names)
    src.write_text('#include "ddh.h"\n#include <stdio.h>\n'
                   "int main(void)\n{\n" + body + "\n"
                   "    ddh_params prm = {{2, 2, 2}, {8.0f, 8.0f, 8.0f}, 1.0f, 0.5f, 0};\n"
                   "    (void)prm;\n    return 0;\n}\n")
    exe = tmp_path / "uses_ddh"
    libdir = os.path.dirname(ddh.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        "-L", libdir, "-lddh", "-Wl,--unresolved-symbols=ignore-in-shared-libs"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert len(names) >= 19


def test_bench_runs_on_one_gpu_only():
    # every domain is a virtual rank inside one GPU: more GPUs is an error
    # that names the reason, before any device is touched
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_bench_reports_counter_traffic_only_for_current_sources(tmp_path, monkeypatch):
    # the HBM traffic of a stored counter summary is reported only while the
    # kernel sources hash to the value stored with it
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "traffic_pulse_demo.md"
    path.write_text(f"- kernel_source_sha256: `{bench.kernel_hash()}`\n"
                    "- traffic_bytes_per_launch: 12345\n")
    assert bench.read_traffic("pulse", "demo") == 12345.0
    path.write_text("- kernel_source_sha256: `0000000000000000`\n"
                    "- traffic_bytes_per_launch: 12345\n")
    assert bench.read_traffic("pulse", "demo") is None
    assert bench.read_traffic("pulse", "absent") is None


def test_kernel_hash_ignores_comments_but_not_code():
    # the stored counters stay current across comment edits of the kernel
    # sources, and go stale on any change of the code itself
    import bench
    base = 'int f(int a) { return a + 1; } // one\nconst char* s = "x // y /* z */";\n'
    assert bench.code_text(base) == bench.code_text(
        "/* lead */ int f(int a) {\n  return a + 1;  // changed comment\n}\n"
        'const char* s = "x // y /* z */";')
    assert bench.code_text(base) != bench.code_text(base.replace("a + 1", "a + 2"))
    assert bench.code_text(base) != bench.code_text(base.replace("x // y", "x / y"))
    assert "/* z */" in bench.code_text(base)


def test_bench_timed_graphs_leave_at_least_five_replays():
    # exactly --steps steps are timed, in graphs of G steps, with at least
    # five replays whenever there are five steps, so p10 and p90 can differ
    import bench
    for steps, cap in [(20, 50), (200, 50), (1000, 50), (7, 50), (5, 50), (3, 50), (20, 1), (97, 50)]:
        G = bench.graph_size(steps, cap)
        assert steps % G == 0 and 1 <= G <= max(1, cap)
        if steps >= 5:
            assert steps // G >= 5, (steps, G)
    assert bench.graph_size(20, 50) == 4
    assert bench.graph_size(200, 50) == 40


def test_bench_host_cpu_fields():
    import bench
    cpu = bench.host_cpu()
    assert cpu["cpu_count"] >= 1 and 1 <= cpu["affinity"] <= cpu["cpu_count"]
    assert isinstance(cpu["model"], str) and cpu["model"]


def test_bench_marker_summary(tmp_path):
    # the host ranges of a rocprofv3 --marker-trace --stats run, largest
    # total first, durations in microseconds
    import bench
    d = tmp_path / "run" / "host"
    d.mkdir(parents=True)
    (d / "run_marker_api_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"build: pulses",2,1000000,500000.0,10.0,400000,600000,1.0\n'
        '"ddh_build_maps",2,3000000,1500000.0,30.0,1200000,1800000,1.0\n')
    text = bench.summarize_markers(str(tmp_path), "Map build", "cmd --x")
    lines = text.splitlines()
    assert lines[0] == "## Map build" and "cmd --x" in lines
    rows = [ln for ln in lines if ln.startswith("| `")]
    assert rows[0] == "| `ddh_build_maps` | 2 | 1500.0 | 1200.0 | 1800.0 |"
    assert rows[1] == "| `build: pulses` | 2 | 500.0 | 400.0 | 600.0 |"
