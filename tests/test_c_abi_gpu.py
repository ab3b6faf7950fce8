"""The C ABI used from C alone (no Python binding, no torch).

tests/c/c_abi_roundtrip.c builds the maps of a seeded uniform system through
include/ddh.h, runs the coordinate and force passes in every execution mode
(fused, per-pulse, automatic, host-orchestrated, and both graph-cached forms)
over two steps, and compares every slot bit for bit with the CPU oracle,
which only this test program links. The program is compiled with gcc here;
the library and the oracle are the in-tree builds.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "c_abi_roundtrip.c")
LIBDIR = os.path.join(ROOT, "domain_decomposition_halo_amd")
ORACLEDIR = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def compile_roundtrip(out_dir) -> str:
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    for lib in (os.path.join(LIBDIR, "libddh.so"), os.path.join(ORACLEDIR, "libddh_oracle.so")):
        if not os.path.exists(lib):
            pytest.fail(f"{lib} is missing: run __graft_entry__.build() first")
    exe = os.path.join(str(out_dir), "c_abi_roundtrip")
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"), SRC,
           "-o", exe, "-L", LIBDIR, "-lddh", "-L", ORACLEDIR, "-lddh_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}:{ORACLEDIR}:{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_compiles(tmp_path):
    compile_roundtrip(tmp_path)


@pytest.mark.gpu
@pytest.mark.parametrize("args", [
    [],                                          # 20000 atoms, 2x2x2, box 6 nm, rc 1 nm
    ["6000", "4", "2", "1", "4.0", "1.2"],       # two relay pulses in X
    ["0", "2", "2", "2", "6.0", "1.0"],          # no atoms at all
])
def test_c_program_matches_the_oracle(tmp_path, args):
    exe = compile_roundtrip(tmp_path)
    print(f"[c-abi] {os.path.basename(exe)} {' '.join(args)}", flush=True)
    r = subprocess.run([exe] + args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all modes bit-identical to the oracle" in r.stdout
