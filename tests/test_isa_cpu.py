"""Structural check of the compiled exchange kernels (CPU only: hipcc -S).

The exchange kernel runs a work-ticket loop in which thread 0 claims tickets
and finishes chunks between work-group barriers. If a thread-0 region spans
the loop's back edge, the compiler may turn it into a divergent loop exit:
lane 0 is parked outside the loop while the other lanes pass the barrier and
re-read a stale ticket forever. This test compiles the kernels for gfx950
and asserts that no loop holding a barrier also has a divergent exit
(`s_andn2_b64 exec, exec, ...`) of its own; divergent exits of barrier-free
inner loops are fine.
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
            # a kernel may end early (s_endpgm) before its main loop: the body
            # runs to the function's end label
            if line.startswith(".Lfunc_end"):
                cur = None
                continue
            kernels[cur].append(line)
    return kernels


def loops_with_barrier_and_divergent_exit(lines):
    """Loops whose own blocks (innermost-loop attribution) hold both an
    s_barrier and a divergent loop exit (s_andn2_b64 exec, exec, ...).

    LLVM annotates every block label: "=>This Loop Header: Depth=n" for an
    outermost header, "Parent Loop BBa Depth=n" followed by a line "=>  This
    Inner Loop Header: Depth=n+1" for an inner header, and "in Loop:
    Header=BBa Depth=n" for other blocks of loop BBa.
    """
    own = {}
    cur = None
    for k, ln in enumerate(lines):
        m = re.match(r"^\.(LBB\S+):(.*)$", ln)
        if m:
            label, rest = m.group(1).replace("LBB", "BB"), m.group(2)
            nxt = lines[k + 1] if k + 1 < len(lines) else ""
            if "This Loop Header" in rest or ("Parent Loop" in rest and "Inner Loop Header" in nxt):
                cur = label
            else:
                h = re.search(r"in Loop: Header=(BB\S+)", rest)
                cur = h.group(1) if h else None
            if cur is not None:
                own.setdefault(cur, [0, 0])
            continue
        if cur is None:
            continue
        if "s_barrier" in ln:
            own[cur][0] += 1
        if "s_andn2_b64 exec, exec" in ln:
            own[cur][1] += 1
    return sorted(k for k, (b, d) in own.items() if b and d)


def test_exchange_kernels_barrier_loops_are_uniform(tmp_path):
    kernels = _isa(os.path.join(CSRC, "ddh_exchange.hip"), tmp_path)
    ex = {k: v for k, v in kernels.items() if "exchange_kernel" in k}
    assert len(ex) >= 3
    for name, lines in ex.items():
        assert sum("s_barrier" in ln for ln in lines) >= 4, name
        assert loops_with_barrier_and_divergent_exit(lines) == [], name


def test_checker_flags_the_hazard():
    # a loop shaped like the miscompiled ticket loop: barrier at the head of
    # an inner loop whose exit removes lanes from exec
    lines = [
        ".LBB3_4:                                ; =>This Loop Header: Depth=1",
        "\ts_and_saveexec_b64 s[2:3], s[50:51]",
        ".LBB3_11:                               ;   in Loop: Header=BB3_12 Depth=2",
        "\ts_andn2_b64 exec, exec, s[60:61]",
        "\ts_cbranch_execz .LBB3_79",
        ".LBB3_12:                               ;   Parent Loop BB3_4 Depth=1",
        "                                        ; =>  This Inner Loop Header: Depth=2",
        "\ts_barrier",
        "\tds_read_b32 v2, v21",
        ".LBB3_79:                               ;   in Loop: Header=BB3_4 Depth=1",
    ]
    assert loops_with_barrier_and_divergent_exit(lines) == ["BB3_12"]


def test_builder_barriers_never_share_a_loop_with_divergent_exits(tmp_path):
    kernels = _isa(os.path.join(CSRC, "ddh_build.hip"), tmp_path)
    assert any("select_write_kernel" in k for k in kernels)
    for name, lines in kernels.items():
        assert loops_with_barrier_and_divergent_exit(lines) == [], name


def release_barriers_without_store_wait(lines, window=8):
    """Indexes of buffer_wbl2 (agent-scope release) whose preceding s_barrier
    is not preceded, within `window` lines, by s_waitcnt vmcnt(0): the other
    waves' stores would then not be covered by the one wave's release."""
    bad = []
    for i, ln in enumerate(lines):
        if "buffer_wbl2" not in ln:
            continue
        j = max((k for k in range(i) if "s_barrier" in lines[k]), default=None)
        if j is None:
            continue
        if not any("s_waitcnt vmcnt(0)" in lines[k] for k in range(max(0, j - window), j)):
            bad.append(i)
    return bad


def test_exchange_kernel_releases_cover_every_wave(tmp_path):
    kernels = _isa(os.path.join(CSRC, "ddh_exchange.hip"), tmp_path)
    ex = {k: v for k, v in kernels.items() if "exchange_kernel" in k}
    assert len(ex) >= 3
    for name, lines in ex.items():
        assert sum("buffer_wbl2" in ln for ln in lines) >= 2, name
        assert release_barriers_without_store_wait(lines) == [], name


def test_release_checker_flags_a_bare_barrier():
    lines = ["\tglobal_store_dwordx3 v[8:9], v[4:6], off nt", "\ts_or_b64 exec, exec, s[16:17]",
             "\ts_barrier", "\tbuffer_wbl2 sc1", "\ts_waitcnt vmcnt(0)", "\tglobal_atomic_add v[4:5], v3, off"]
    assert release_barriers_without_store_wait(lines) == [3]
    fixed = lines[:2] + ["\ts_waitcnt vmcnt(0)"] + lines[2:]
    assert release_barriers_without_store_wait(fixed) == []


def test_wave_kernel_takes_no_barrier_and_releases(tmp_path):
    # wavefront workers are independent: a work-group barrier in their ticket
    # loop would tie a waiting wavefront to its neighbours; each one releases
    # its own records with an agent-scope fence (buffer_wbl2)
    kernels = _isa(os.path.join(CSRC, "ddh_exchange.hip"), tmp_path)
    wk = {k: v for k, v in kernels.items() if "wave_kernel" in k}
    assert len(wk) >= 2
    for name, lines in wk.items():
        assert not any("s_barrier" in ln for ln in lines), name
        assert sum("buffer_wbl2" in ln for ln in lines) >= 2, name


def _scratch_users(src, tmp_path):
    """Kernels of `src` that touch private (scratch) memory: register arrays
    the compiler demoted to the stack, which turn every gathered record into
    extra memory traffic."""
    kernels = _isa(src, tmp_path)
    return sorted(k for k, lines in kernels.items() if any("scratch_" in ln for ln in lines))


def test_no_kernel_spills_to_scratch(tmp_path):
    for name in ("ddh_exchange.hip", "ddh_build.hip"):
        assert _scratch_users(os.path.join(CSRC, name), tmp_path) == [], name


def test_pulse_kernels_gather_without_branches(tmp_path):
    # a lane's gathers issue back to back: within a per-pulse kernel's first
    # round no s_waitcnt vmcnt separates the coordinate gathers of one lane
    kernels = _isa(os.path.join(CSRC, "ddh_exchange.hip"), tmp_path)
    pk = {k: v for k, v in kernels.items() if "pulse_kernel" in k}
    assert len(pk) >= 6
    for name, lines in pk.items():
        loads = [i for i, ln in enumerate(lines) if "global_load_dwordx3" in ln]
        assert loads, name
        # some pair of consecutive record loads with nothing but address
        # arithmetic between them (the unrolled gather of one round)
        assert any(all("s_waitcnt" not in lines[k] and "s_cbranch" not in lines[k]
                       for k in range(a, b))
                   for a, b in zip(loads, loads[1:])), name
