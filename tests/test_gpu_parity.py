"""GPU parity: the HIP library, through its C ABI, against the CPU oracle.

Bar (coordinates, maps, layout, ids: exact; forces: exact given the fixed
reverse pulse order): every comparison is bit for bit on the raw float32
words. Cases: the workloads at full size (maps, layout, coordinates, forces,
both passes in one call); every execution mode (fused persistent launch, one
launch per pulse, both replayed from the library's graphs, automatic, the
host-orchestrated baseline) over several consecutive steps; calls captured
in a caller's graph with the halo cleared before each replay; the fused
launch with wavefront workers; 16- and 32-bit map entries; ragged and
extreme chunk/grid/width settings (down to a single work-group, with and
without static first tickets); exact dyadic boxes with multi-pulse relay up
to the most pulses a grid allows; seeded random decompositions; rebuilds for
moving atoms; two plans on two streams; completion flags (counts, consumer
streams waiting on them, turned off); device memory released by destroyed
plans; the exchange beside a compute load on another stream; empty and
one-sided inputs, many domains with short or empty maps, error paths and the
bounded-wait timeout paths.
"""

import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import domain_decomposition_halo_amd as ddh  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

MODES = {
    "fused": ddh.DDH_MODE_FUSED,
    "pulse": ddh.DDH_MODE_PULSE,
    "fused_graph": ddh.DDH_MODE_FUSED | ddh.DDH_MODE_GRAPH,
    "pulse_graph": ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH,
    "auto": ddh.DDH_MODE_AUTO,
    "staged": ddh.DDH_MODE_STAGED,
}


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


class GpuPlan:
    """A device plan built from host positions, with host views of its output."""

    def __init__(self, x, grid, box, rc, cell=0.5, mode=0, chunk=0, wg=0, refined=1, block=0,
                 static_first=0, narrow=1, wave=0, home_sort=0, heads_first=0, lds_stage=0):
        self.plan = ddh.Plan(grid, box, rc, cell)
        self.plan.tune(ddh.DDH_TUNE_LDS_STAGE, lds_stage)
        self.plan.tune(ddh.DDH_TUNE_HOME_SORT, home_sort)
        self.plan.tune(ddh.DDH_TUNE_HEADS_FIRST, heads_first)
        self.plan.tune(ddh.DDH_TUNE_STATIC_FIRST, static_first)
        self.plan.tune(ddh.DDH_TUNE_NARROW_MAPS, narrow)
        self.plan.tune(ddh.DDH_TUNE_WAVE_CHUNKS, wave)
        self.plan.tune(ddh.DDH_TUNE_CHUNK, chunk)
        self.plan.tune(ddh.DDH_TUNE_GRID, wg)
        self.plan.tune(ddh.DDH_TUNE_BLOCK, block)
        self.plan.tune(ddh.DDH_TUNE_REFINED_WAITS, refined)
        self.plan.set_mode(mode)
        self.xg = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        self.lay = self.plan.build_maps(self.xg)
        self.n_slots = self.lay["n_slots"]
        self.D, self.P = self.lay["n_domains"], self.lay["n_pulses"]

    def tables(self):
        info = [self.plan.domain_info(D) for D in range(self.D)]
        base = np.array([i[0] for i in info], np.int64)
        nhome = np.array([i[1] for i in info], np.int32)
        ntotal = np.array([i[2] for i in info], np.int32)
        pul = np.array([[self.plan.pulse_info(S, p) for p in range(self.P)] for S in range(self.D)],
                       np.int32).reshape(self.D, self.P, 5)
        return base, nhome, ntotal, pul

    def maps(self):
        out = torch.empty(max(self.lay["n_halo"], 1), dtype=torch.int32, device="cuda")
        self.plan.copy_maps(out)
        return out.cpu().numpy()[:self.lay["n_halo"]]

    def ids(self):
        out = torch.empty(max(self.n_slots, 1), dtype=torch.int32, device="cuda")
        self.plan.local_ids(out)
        return out.cpu().numpy()[:self.n_slots]

    def new_coords(self):
        xl = torch.zeros((max(self.n_slots, 1), 3), dtype=torch.float32, device="cuda")
        self.plan.gather_home(self.xg, xl)
        return xl

    def close(self):
        self.plan.close()


def check_layout(g: GpuPlan, ref: oracle.OraclePlan):
    assert (g.D, g.P, g.n_slots, g.lay["n_halo"]) == (ref.n_domains, ref.n_pulses, ref.n_slots,
                                                       ref.halo_atoms)
    assert g.lay["pulses"] == ref.pulses
    base, nhome, ntotal, pul = g.tables()
    assert np.array_equal(base, ref.base)
    assert np.array_equal(nhome, ref.nhome)
    assert np.array_equal(ntotal, ref.ntotal)
    for k, arr in enumerate((ref.send, ref.split, ref.recv, ref.roff, ref.shift)):
        assert np.array_equal(pul[:, :, k], arr), ("send", "split", "recv", "roff", "shift")[k]
    want = np.concatenate([ref.maps[(S, p)] for S in range(ref.n_domains)
                           for p in range(ref.n_pulses)] or [np.zeros(0, np.int32)])
    assert np.array_equal(g.maps(), want)
    assert np.array_equal(g.ids(), ref.slot_ids)


def check_steps(g: GpuPlan, ref: oracle.OraclePlan, w_key, steps=3, fused_step=False):
    """Several consecutive steps; every one bit-identical to the oracle."""
    xl = g.new_coords()
    fl = torch.empty((max(g.n_slots, 1), 3), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(w_key)
    for s in range(steps):
        f0 = rng.normal(0, 10, size=(g.n_slots, 3)).astype(np.float32)
        fl[:g.n_slots].copy_(torch.from_numpy(f0))
        if fused_step:
            g.plan.exchange_step(xl, fl)
        else:
            g.plan.exchange_coords(xl)
            g.plan.exchange_forces(fl)
        assert g.plan.check() == ddh.DDH_OK
        assert np.array_equal(bits(xl.cpu().numpy()[:g.n_slots]), bits(ref.x_local)), f"coords step {s}"
        fr = f0.copy()
        ref.exchange_forces(fr)
        assert np.array_equal(bits(fl.cpu().numpy()[:g.n_slots]), bits(fr)), f"forces step {s}"


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_layout_maps_ids(k, workload_plan):
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, **w.params())
    check_layout(g, ref)
    g.close()


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_coords_forces(k, mode, workload_plan):
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, **w.params(), mode=MODES[mode])
    check_steps(g, ref, k)
    g.close()


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("k", [2, 4])
def test_workload_fused_step(k, mode, workload_plan):
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, **w.params(), mode=MODES[mode])
    check_steps(g, ref, 10 + k, fused_step=True)
    g.close()


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("mode", ["auto", "pulse", "fused", "wave"])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_captured_in_a_caller_graph(k, mode, split, workload_plan):
    """Calls captured in a torch CUDA graph and replayed several times, with
    eager work (new forces, a check) between replays: every replay matches
    the oracle bit for bit. "wave": the fused launch with wavefront workers."""
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, **w.params(), mode=MODES.get(mode, ddh.DDH_MODE_FUSED), wave=int(mode == "wave"))
    xl = g.new_coords()
    fl = torch.zeros((max(g.n_slots, 1), 3), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        if split:
            g.plan.exchange_coords(xl)
            g.plan.exchange_forces(fl)
        else:
            g.plan.exchange_step(xl, fl)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        if split:
            g.plan.exchange_coords(xl)
            g.plan.exchange_forces(fl)
        else:
            g.plan.exchange_step(xl, fl)
    rng = np.random.default_rng(300 + k)
    for r in range(4):
        xl.copy_(g.new_coords())
        f0 = rng.normal(0, 10, size=(g.n_slots, 3)).astype(np.float32)
        fl[:g.n_slots].copy_(torch.from_numpy(f0))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert g.plan.check() == ddh.DDH_OK
        assert np.array_equal(bits(xl.cpu().numpy()[:g.n_slots]), bits(ref.x_local)), f"replay {r}"
        fr = f0.copy()
        ref.exchange_forces(fr)
        assert np.array_equal(bits(fl.cpu().numpy()[:g.n_slots]), bits(fr)), f"replay {r}"
    del graph
    g.close()


def random_configs(n, seed):
    """Seeded random decompositions the schedule accepts: 1-6 domains per
    dimension, boxes of 2-9 nm per edge, cutoffs up to the largest the
    widths allow (so several pulses per dimension occur), 200-6000 uniform
    atoms."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        grid = tuple(int(g) for g in rng.integers(1, 7, size=3))
        box = tuple(float(np.float32(b)) for b in rng.uniform(2.0, 9.0, size=3))
        wmin = min(box[d] / grid[d] for d in range(3) if grid[d] > 1) if max(grid) > 1 else 1.0
        rc = float(np.float32(rng.uniform(0.2, 2.5) * wmin))
        try:
            P = len(oracle.schedule(grid, box, rc))
        except oracle.OracleError:
            continue
        if P > ddh.DDH_MAX_PULSES:
            continue
        out.append((grid, box, rc, int(rng.integers(200, 6000))))
    return out


@pytest.mark.parametrize("cfg", random_configs(24, 2024))
def test_random_decompositions(cfg):
    """Random grids, boxes, cutoffs (one to several pulses per dimension) and
    atom counts: layout, maps, ids, coordinates and forces bit-identical to
    the oracle in every mode (and with wavefront workers), over two steps."""
    grid, box, rc, n = cfg
    x = W.uniform_positions(n, box, seed=n)
    ref = oracle.OraclePlan(x, grid, box, rc)
    runs = [(m, 0, 0) for m in MODES.values()] + [(ddh.DDH_MODE_FUSED, 1, 0),
                                                  (ddh.DDH_MODE_FUSED, 0, 1)]
    for mode, wave, heads_first in runs:
        g = GpuPlan(x, grid, box, rc, mode=mode, wave=wave, heads_first=heads_first)
        check_layout(g, ref)
        check_steps(g, ref, n, steps=2)
        check_steps(g, ref, n + 1, steps=1, fused_step=True)
        g.close()


def lattice_configs(n, seed):
    """Seeded random decompositions on a coarse lattice: 1-5 domains per
    dimension, boxes of 2-8 nm per edge in steps of 1/8 nm, cutoffs up to
    twice the narrowest domain in steps of 1/16 nm, cell sizes from 0.2 to
    1.5 nm (any float), 300-5000 atoms on a 1/32 nm lattice, so atoms sit
    exactly on domain boundaries, cell edges and slab thresholds."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        grid = tuple(int(g) for g in rng.integers(1, 6, size=3))
        box = tuple(float(b) / 8.0 for b in rng.integers(16, 65, size=3))
        wmin = min(box[d] / grid[d] for d in range(3))
        rc = float(rng.integers(2, max(3, int(32 * wmin)))) / 16.0
        cell = float(np.float32(rng.uniform(0.2, 1.5)))
        try:
            P = len(oracle.schedule(grid, box, rc))
        except oracle.OracleError:
            continue
        if P > ddh.DDH_MAX_PULSES:
            continue
        out.append((grid, box, rc, cell, int(rng.integers(300, 5000)), int(rng.integers(1, 3))))
    return out


@pytest.mark.parametrize("cfg", lattice_configs(16, 77))
def test_lattice_decompositions(cfg):
    """Random grids, dyadic boxes and cutoffs, random cell sizes and a 1/32 nm
    lattice (ties everywhere the build compares): layout, maps, ids,
    coordinates and forces bit-identical to the oracle with either home sort,
    per-pulse and fused."""
    grid, box, rc, cell, n, home_sort = cfg
    x = W.lattice_positions(n, box, seed=n + 5, frac_bits=5)
    ref = oracle.OraclePlan(x, grid, box, rc, cell=cell)
    for mode in (ddh.DDH_MODE_PULSE, ddh.DDH_MODE_FUSED):
        g = GpuPlan(x, grid, box, rc, cell=cell, mode=mode, home_sort=home_sort)
        check_layout(g, ref)
        check_steps(g, ref, n + 9, steps=1)
        g.close()


@pytest.mark.parametrize("mode,wave", [("fused", 0), ("fused", 1), ("pulse", 0)])
def test_exchange_beside_a_compute_load(mode, wave, workload_plan):
    """The exchange on one stream while a chain of matrix products (the local
    non-bonded work's stand-in) holds compute units on another, both at
    default priority: the fused launch's claimed tickets must still drain,
    and every result stays bit-identical to the oracle."""
    w, x, ref = workload_plan(2)
    g = GpuPlan(x, **w.params(), mode=MODES[mode], wave=wave)
    xl = g.new_coords()
    fl = torch.empty((g.n_slots, 3), dtype=torch.float32, device="cuda")
    a = torch.randn(2048, 2048, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(2048, 2048, device="cuda", dtype=torch.bfloat16)
    side = torch.cuda.Stream()
    rng = np.random.default_rng(500)
    for r in range(5):
        f0 = rng.normal(0, 10, size=(g.n_slots, 3)).astype(np.float32)
        fl.copy_(torch.from_numpy(f0))
        xl.copy_(g.new_coords())
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            c = a
            for _ in range(4):
                c = torch.mm(c, b)
        for _ in range(3):                      # several steps overlap the load
            g.plan.exchange_step(xl, fl)
            if _ < 2:
                fl.copy_(torch.from_numpy(f0))
        torch.cuda.synchronize()
        assert g.plan.check() == ddh.DDH_OK
        assert np.array_equal(bits(xl.cpu().numpy()), bits(ref.x_local)), r
        fr = f0.copy()
        ref.exchange_forces(fr)
        assert np.array_equal(bits(fl.cpu().numpy()), bits(fr)), r
    g.close()


def test_rebuild_after_atoms_move():
    """One plan rebuilt for moving atoms (as at every neighbour-search step,
    sizes changing between builds): every build and exchange bit-identical
    to a fresh oracle plan of the same positions, in both main modes."""
    w = W.WORKLOADS[2]
    p = w.params()
    L = np.float32(p["box"][0])
    x = W.positions(w)
    rng = np.random.default_rng(41)
    for mode in (ddh.DDH_MODE_PULSE, ddh.DDH_MODE_FUSED):
        plan = ddh.Plan(**p)
        plan.set_mode(mode)
        xs = x.copy()
        for it in range(4):
            if it:
                step = rng.normal(0.0, 0.05 * it, size=xs.shape).astype(np.float32)
                xs = np.mod(xs + step, L).astype(np.float32)
                xs[xs >= L] = 0.0
            ref = oracle.OraclePlan(xs, **p)
            xg = torch.from_numpy(np.ascontiguousarray(xs)).cuda()
            lay = plan.build_maps(xg)
            assert (lay["n_slots"], lay["n_halo"]) == (ref.n_slots, ref.halo_atoms)
            xl = torch.zeros((lay["n_slots"], 3), dtype=torch.float32, device="cuda")
            plan.gather_home(xg, xl)
            plan.exchange_coords(xl)
            f0 = rng.normal(0, 10, size=(ref.n_slots, 3)).astype(np.float32)
            fl = torch.from_numpy(f0).cuda()
            plan.exchange_forces(fl)
            assert plan.check() == ddh.DDH_OK
            assert np.array_equal(bits(xl.cpu().numpy()), bits(ref.x_local)), it
            fr = f0.copy()
            ref.exchange_forces(fr)
            assert np.array_equal(bits(fl.cpu().numpy()), bits(fr)), it
        plan.close()


def test_rebuilds_that_grow_and_shrink():
    """One plan rebuilt for 2000, 40000, 500 and 40000 atoms: the build's
    device memory grows, is reused while large enough, and every build and
    exchange matches a fresh oracle plan in both main modes."""
    grid, box, rc = (2, 2, 2), (8.0, 8.0, 8.0), 1.25
    plan = ddh.Plan(grid, box, rc)
    for n in (2000, 40000, 500, 40000):
        x = W.uniform_positions(n, box, seed=700 + n)
        ref = oracle.OraclePlan(x, grid, box, rc)
        g = GpuPlan.__new__(GpuPlan)
        g.plan = plan
        g.xg = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        g.lay = plan.build_maps(g.xg)
        g.n_slots = g.lay["n_slots"]
        g.D, g.P = g.lay["n_domains"], g.lay["n_pulses"]
        check_layout(g, ref)
        for mode in (ddh.DDH_MODE_FUSED, ddh.DDH_MODE_PULSE):
            plan.set_mode(mode)
            check_steps(g, ref, n + mode, steps=1)
    plan.close()


def test_two_plans_on_two_streams(workload_plan):
    """Two plans (different decompositions) exchanging at the same time on
    two streams, fused and per-pulse: each keeps its own tickets, counters
    and flags, and both match the oracle."""
    cases = [workload_plan(2), workload_plan(4)]
    for modes in ((ddh.DDH_MODE_FUSED, ddh.DDH_MODE_FUSED), (ddh.DDH_MODE_PULSE, ddh.DDH_MODE_FUSED)):
        gs, xs, fs, f0s = [], [], [], []
        for (w, x, ref), mode in zip(cases, modes):
            g = GpuPlan(x, **w.params(), mode=mode)
            gs.append(g)
            xs.append(g.new_coords())
            f0 = np.random.default_rng(g.n_slots).normal(0, 10, size=(g.n_slots, 3)).astype(np.float32)
            f0s.append(f0)
            fs.append(torch.from_numpy(f0).cuda())
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        torch.cuda.synchronize()
        for _ in range(3):
            for g, xl, fl, st in zip(gs, xs, fs, streams):
                with torch.cuda.stream(st):
                    g.plan.exchange_coords(xl)
        for g, xl, fl, st in zip(gs, xs, fs, streams):
            with torch.cuda.stream(st):
                g.plan.exchange_forces(fl)
        torch.cuda.synchronize()
        for g, xl, fl, f0, (w, x, ref) in zip(gs, xs, fs, f0s, cases):
            assert g.plan.check() == ddh.DDH_OK
            assert np.array_equal(bits(xl.cpu().numpy()[:g.n_slots]), bits(ref.x_local))
            fr = f0.copy()
            ref.exchange_forces(fr)
            assert np.array_equal(bits(fl.cpu().numpy()[:g.n_slots]), bits(fr))
            g.close()


def test_plans_release_their_device_memory(workload_plan):
    """Build, exchange and destroy a plan many times (and rebuild one plan
    repeatedly): the free device memory returns to where it was."""
    w, x, ref = workload_plan(3)
    xg = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    torch.cuda.synchronize()

    def cycle():
        plan = ddh.Plan(**w.params())
        lay = plan.build_maps(xg)
        plan.build_maps(xg)
        xl = torch.zeros((lay["n_slots"], 3), dtype=torch.float32, device="cuda")
        plan.gather_home(xg, xl)
        for mode in (ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH, ddh.DDH_MODE_STAGED):
            plan.set_mode(mode)
            plan.exchange_coords(xl)
        assert plan.check() == ddh.DDH_OK
        plan.close()
        del xl
        torch.cuda.synchronize()

    cycle()
    torch.cuda.empty_cache()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(8):
        cycle()
    torch.cuda.empty_cache()
    free1 = torch.cuda.mem_get_info()[0]
    assert free0 - free1 < 16 << 20, (free0, free1)


@pytest.mark.parametrize("k", [2, 4])
def test_without_completion_flags(k, workload_plan):
    """With DDH_TUNE_FLAGS = 0 every mode still matches the oracle, the flag
    calls report DDH_ESTATE, and turning the flags back on resumes them."""
    w, x, ref = workload_plan(k)
    for mode in MODES.values():
        g = GpuPlan(x, **w.params(), mode=mode)
        g.plan.tune(ddh.DDH_TUNE_FLAGS, 0)
        check_steps(g, ref, 50 + k, steps=2)
        check_steps(g, ref, 60 + k, steps=1, fused_step=True)
        with pytest.raises(ddh.DDHError) as e:
            g.plan.flags_address()
        assert e.value.code == ddh.DDH_ESTATE
        with pytest.raises(ddh.DDHError) as e:
            g.plan.wait_flag(ddh.DDH_PASS_COORDS, 0, 1)
        assert e.value.code == ddh.DDH_ESTATE
        g.plan.tune(ddh.DDH_TUNE_FLAGS, 1)
        buf = torch.zeros(2 * ddh.DDH_MAX_PULSES, dtype=torch.int32, device="cuda")
        g.plan.copy_flags(buf)
        assert int(buf.cpu().numpy()[0]) == 0  # no pass counted while off
        check_steps(g, ref, 70 + k, steps=1)
        g.plan.copy_flags(buf)
        v = buf.cpu().numpy().view(np.uint32)
        assert (v[:g.P] == 1).all() and (v[ddh.DDH_MAX_PULSES:ddh.DDH_MAX_PULSES + g.P] == 1).all()
        g.close()


@pytest.mark.parametrize("exit_pub", [0, 1, 2])
def test_completion_flags_count_passes(exit_pub, workload_plan):
    """Every mode publishes every pulse's completion flag with the number of
    passes completed so far; words past the plan's pulses stay zero. Per-pulse
    calls publish the last launch's flags from that launch's last block
    (exit_pub 1) or from a one-wave launch after it (2)."""
    w, x, ref = workload_plan(4)
    g = GpuPlan(x, **w.params())
    g.plan.tune(ddh.DDH_TUNE_EXIT_PUBLISH, exit_pub)
    P = g.P
    xl = g.new_coords()
    fl = torch.zeros((max(g.n_slots, 1), 3), dtype=torch.float32, device="cuda")
    buf = torch.zeros(2 * ddh.DDH_MAX_PULSES, dtype=torch.int32, device="cuda")
    assert g.plan.flags_address() != 0

    def check(nx, nf):
        g.plan.copy_flags(buf)
        v = buf.cpu().numpy().view(np.uint32)
        m = ddh.DDH_MAX_PULSES
        assert (v[:P] == nx).all() and (v[P:m] == 0).all(), (nx, v[:m])
        assert (v[m:m + P] == nf).all() and (v[m + P:] == 0).all(), (nf, v[m:])

    check(0, 0)
    nx = nf = 0
    for mode in (ddh.DDH_MODE_PULSE, ddh.DDH_MODE_FUSED, ddh.DDH_MODE_STAGED, ddh.DDH_MODE_AUTO,
                 ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH, ddh.DDH_MODE_FUSED | ddh.DDH_MODE_GRAPH):
        g.plan.set_mode(mode)
        g.plan.exchange_coords(xl)
        nx += 1
        check(nx, nf)
        g.plan.exchange_forces(fl)
        nf += 1
        check(nx, nf)
        g.plan.exchange_step(xl, fl)
        nx += 1
        nf += 1
        check(nx, nf)
    assert g.plan.check() == ddh.DDH_OK
    # the coordinates are still the oracle's after all these passes
    assert np.array_equal(bits(xl.cpu().numpy()[:g.n_slots]), bits(ref.x_local))
    g.close()


@pytest.mark.parametrize("mode,exit_pub", [("pulse", 2), ("pulse", 1), ("fused", 0)])
@pytest.mark.parametrize("k", [2, 3])
def test_wait_flag_orders_a_consumer_stream(k, mode, exit_pub, workload_plan):
    """A consumer stream that waits on a pulse's flag reads that pulse's
    delivered records: the exchange on one stream, then on a second stream
    a flag wait followed by a gather of every receiver's region of the pulse,
    for each pulse and two passes (per-pulse calls: the last pulse's flag from
    its launch's last block, or from a one-wave launch after it)."""
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, **w.params(), mode=MODES[mode])
    g.plan.tune(ddh.DDH_TUNE_EXIT_PUBLISH, exit_pub)
    base, nhome, ntotal, pul = g.tables()
    xl = g.new_coords()
    prod = torch.cuda.Stream()
    cons = torch.cuda.Stream()
    for p in range(g.P):
        idx = np.concatenate([base[pul[S, p, 2]] + pul[S, p, 3] + np.arange(pul[S, p, 0])
                              for S in range(g.D)]).astype(np.int64)
        idx_d = torch.from_numpy(idx).cuda()
        for epoch in (2 * p + 1, 2 * p + 2):
            torch.cuda.synchronize()
            xl.copy_(g.new_coords())  # halo slots cleared
            torch.cuda.synchronize()
            with torch.cuda.stream(prod):
                g.plan.exchange_coords(xl)
            with torch.cuda.stream(cons):
                g.plan.wait_flag(ddh.DDH_PASS_COORDS, p, epoch)
                got = xl.index_select(0, idx_d)
            torch.cuda.synchronize()
            assert g.plan.check() == ddh.DDH_OK
            assert np.array_equal(bits(got.cpu().numpy()), bits(ref.x_local[idx])), (p, epoch)
    g.close()


@pytest.mark.parametrize("exit_pub,pad", [(1, 1), (1, 2), (2, 2)])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_pulse_publish_and_map_forms(k, exit_pub, pad, workload_plan):
    """Per-pulse launches whose last launch publishes the flags itself
    (DDH_TUNE_EXIT_PUBLISH 1) or leaves them to a one-wave launch (2), and
    whose blocks read the chunk-aligned map copy (DDH_TUNE_PAD_MAPS 1) or the
    maps after the descriptor (2): several steps, eager and from the library's
    graphs, then calls captured in a caller's graph and replayed with the
    halo cleared before each replay."""
    w, x, ref = workload_plan(k)
    for mode in (ddh.DDH_MODE_PULSE, ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH):
        g = GpuPlan(x, **w.params(), mode=mode)
        g.plan.tune(ddh.DDH_TUNE_EXIT_PUBLISH, exit_pub)
        g.plan.tune(ddh.DDH_TUNE_PAD_MAPS, pad)
        check_steps(g, ref, 200 + k, steps=2)
        check_steps(g, ref, 210 + k, steps=1, fused_step=True)
        g.close()
    g = GpuPlan(x, **w.params(), mode=ddh.DDH_MODE_PULSE)
    g.plan.tune(ddh.DDH_TUNE_EXIT_PUBLISH, exit_pub)
    g.plan.tune(ddh.DDH_TUNE_PAD_MAPS, pad)
    xl = g.new_coords()
    home = g.new_coords()
    f0 = np.random.default_rng(220 + k).normal(0, 10, size=(g.n_slots, 3)).astype(np.float32)
    fl = torch.from_numpy(f0).cuda()
    fr = f0.copy()
    ref.exchange_forces(fr)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.plan.exchange_step(xl, fl)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.plan.exchange_step(xl, fl)
    for r in range(3):
        xl.copy_(home)
        fl.copy_(torch.from_numpy(f0))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(xl.cpu().numpy()[:g.n_slots]), bits(ref.x_local)), r
        assert np.array_equal(bits(fl.cpu().numpy()[:g.n_slots]), bits(fr)), r
    assert g.plan.check() == ddh.DDH_OK
    del graph
    g.close()


@pytest.mark.parametrize("chunk,wg", [(0, 0), (64, 0), (1000, 3), (0, 1)])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_heads_first_tickets(k, chunk, wg, workload_plan):
    """The fused launch with heads-first tickets (DDH_TUNE_HEADS_FIRST): every
    map's independent head in chunks of its own, all heads before any tail.
    Ragged and many-chunk tables, grids down to one work-group, the
    conservative waits, and calls captured in a caller's graph replayed with
    the halo cleared (a missing wait or release cannot hide behind stale
    values)."""
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, **w.params(), mode=ddh.DDH_MODE_FUSED, chunk=chunk, wg=wg, heads_first=1)
    check_steps(g, ref, 500 + k, steps=2)
    check_steps(g, ref, 510 + k, steps=1, fused_step=True)
    g.plan.tune(ddh.DDH_TUNE_REFINED_WAITS, 0)
    g.plan.build_maps(g.xg)
    check_steps(g, ref, 520 + k, steps=1, fused_step=True)
    g.plan.tune(ddh.DDH_TUNE_REFINED_WAITS, 1)
    g.plan.build_maps(g.xg)
    home = g.new_coords()
    xl = g.new_coords()
    f0 = np.random.default_rng(530 + k).normal(0, 10, size=(g.n_slots, 3)).astype(np.float32)
    fl = torch.from_numpy(f0).cuda()
    fr = f0.copy()
    ref.exchange_forces(fr)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.plan.exchange_step(xl, fl)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.plan.exchange_step(xl, fl)
    for r in range(3):
        xl.copy_(home)
        fl.copy_(torch.from_numpy(f0))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(xl.cpu().numpy()[:g.n_slots]), bits(ref.x_local)), r
        assert np.array_equal(bits(fl.cpu().numpy()[:g.n_slots]), bits(fr)), r
    assert g.plan.check() == ddh.DDH_OK
    del graph
    g.close()


def test_wait_flag_errors_and_timeout(workload_plan):
    w, x, ref = workload_plan(1)
    g = GpuPlan(x, **w.params())
    for kind, pulse in ((2, 0), (ddh.DDH_PASS_COORDS, g.P), (ddh.DDH_PASS_FORCES, -1)):
        with pytest.raises(ddh.DDHError) as e:
            g.plan.wait_flag(kind, pulse, 1)
        assert e.value.code == ddh.DDH_EINVAL
    # a pass that never comes: the wait gives up after the spin limit
    g.plan.tune(ddh.DDH_TUNE_SPIN_LIMIT, 2000)
    g.plan.wait_flag(ddh.DDH_PASS_FORCES, 0, 5)
    assert g.plan.check() == ddh.DDH_ETIMEOUT
    assert g.plan.check() == ddh.DDH_OK
    xl = g.new_coords()
    g.plan.exchange_coords(xl)
    g.plan.wait_flag(ddh.DDH_PASS_COORDS, 0, 1)
    assert g.plan.check() == ddh.DDH_OK
    assert np.array_equal(bits(xl.cpu().numpy()[:g.n_slots]), bits(ref.x_local))
    g.close()


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_staged_mode_refuses_capture(workload_plan):
    w, x, ref = workload_plan(1)
    g = GpuPlan(x, **w.params(), mode=ddh.DDH_MODE_STAGED)
    xl = g.new_coords()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(ddh.DDHError) as e:
        with torch.cuda.graph(graph):
            g.plan.exchange_coords(xl)
    assert e.value.code == ddh.DDH_EINVAL
    del graph
    torch.cuda.synchronize()
    # the plan still works eagerly afterwards
    g.plan.exchange_coords(xl)
    assert g.plan.check() == ddh.DDH_OK
    assert np.array_equal(bits(xl.cpu().numpy()[:g.n_slots]), bits(ref.x_local))
    g.close()


@pytest.mark.parametrize("chunk,wg,refined,block", [
    (64, 0, 1, 0), (320, 0, 1, 0), (8192, 0, 1, 0), (64, 1, 1, 0), (192, 3, 0, 0),
    (256, 1, 0, 0), (1024, 5, 1, 0), (2048, 0, 1, 1024), (4096, 0, 0, 1024), (1024, 0, 1, 256),
    (3000, 7, 1, 1024), (8192, 1, 1, 1024), (640, 300, 1, 256)])
@pytest.mark.parametrize("k", [2, 4])
def test_chunk_and_grid_variants(k, chunk, wg, refined, block, workload_plan):
    # a single work-group must drain every ticket in order without waiting forever
    w, x, ref = workload_plan(k)
    for mode, sf in ((ddh.DDH_MODE_FUSED, 0), (ddh.DDH_MODE_FUSED, 1), (ddh.DDH_MODE_PULSE, 0)):
        g = GpuPlan(x, **w.params(), mode=mode, chunk=chunk, wg=wg, refined=refined, block=block,
                    static_first=sf)
        check_steps(g, ref, 20 + k, steps=2)
        check_steps(g, ref, 30 + k, steps=1, fused_step=True)
        g.close()


@pytest.mark.parametrize("mode", ["fused", "pulse", "pulse_graph", "staged"])
@pytest.mark.parametrize("k", [2, 4])
def test_32bit_maps(k, mode, workload_plan):
    """DDH_TUNE_NARROW_MAPS = 0: the kernels read the 32-bit maps, the path
    of every plan with a domain above 65536 slots."""
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, **w.params(), mode=MODES[mode], narrow=0)
    check_steps(g, ref, 40 + k, steps=2)
    check_steps(g, ref, 50 + k, steps=1, fused_step=True)
    g.close()


@pytest.mark.parametrize("k", [2, 4])
def test_map_width_switched_after_build(k, workload_plan):
    """A build with the 16-bit maps on makes only the 16-bit chunk-aligned
    map copy; switching to the 32-bit maps afterwards makes the per-pulse
    launches read the 32-bit maps after each descriptor (whatever
    DDH_TUNE_PAD_MAPS says), and switching back uses the copy again."""
    w, x, ref = workload_plan(k)
    for mode in (ddh.DDH_MODE_PULSE, ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH):
        g = GpuPlan(x, **w.params(), mode=mode)
        for narrow, pad in ((0, 1), (0, 0), (1, 1), (0, 2)):
            g.plan.tune(ddh.DDH_TUNE_NARROW_MAPS, narrow)
            g.plan.tune(ddh.DDH_TUNE_PAD_MAPS, pad)
            check_steps(g, ref, 700 + 10 * narrow + pad, steps=1)
            check_steps(g, ref, 720 + 10 * narrow + pad, steps=1, fused_step=True)
        g.close()


@pytest.mark.parametrize("n,wide", [(100_000, False), (140_000, True)])
def test_map_width_threshold(n, wide):
    """Two domains of about 50k and 70k home atoms: the first stays within
    65536 slots per domain, so the 16-bit maps hold indices above 32767; the
    second exceeds it, so every kernel reads the 32-bit maps."""
    grid, box, rc = (2, 1, 1), (8.0, 4.0, 4.0), 1.0
    x = W.uniform_positions(n, box, seed=n)
    ref = oracle.OraclePlan(x, grid, box, rc)
    assert (int(ref.ntotal.max()) > 65536) == wide
    assert int(ref.ntotal.max()) > 32768
    for mode in (ddh.DDH_MODE_FUSED, ddh.DDH_MODE_PULSE):
        g = GpuPlan(x, grid, box, rc, mode=mode)
        check_layout(g, ref)
        check_steps(g, ref, n, steps=2)
        check_steps(g, ref, n + 1, steps=1, fused_step=True)
        g.close()


@pytest.mark.parametrize("chunk,wg", [(0, 0), (64, 0), (1000, 0), (0, 1), (192, 3), (4096, 0)])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_wave_chunks(k, chunk, wg, workload_plan):
    """Fused launch with wavefront workers (DDH_TUNE_WAVE_CHUNKS): contiguous
    map slices, a wavefront waits only when its slice holds dependent
    entries and releases its own records. Down to one work-group of four
    wavefronts; ragged and multi-round slices."""
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, **w.params(), mode=ddh.DDH_MODE_FUSED, chunk=chunk, wg=wg, wave=1)
    check_steps(g, ref, 60 + k, steps=2)
    check_steps(g, ref, 70 + k, steps=1, fused_step=True)
    # the setting belongs to the chunk table: it changes at the next build
    g.plan.tune(ddh.DDH_TUNE_WAVE_CHUNKS, 0)
    check_steps(g, ref, 80 + k, steps=1, fused_step=True)
    g.plan.build_maps(g.xg)
    check_steps(g, ref, 90 + k, steps=1)
    g.close()


DYADIC = [
    ((1, 1, 1), (4.0, 4.0, 4.0), 0.75, 500),
    ((2, 1, 1), (8.0, 4.0, 4.0), 1.25, 2000),
    ((2, 2, 2), (8.0, 8.0, 8.0), 1.25, 4000),
    ((3, 2, 2), (12.0, 8.0, 8.0), 2.5, 4000),
    ((4, 2, 1), (8.0, 6.0, 4.0), 1.5, 3000),
    ((8, 2, 2), (8.0, 8.0, 8.0), 2.5, 4000),
    ((4, 1, 1), (8.0, 4.0, 4.0), 2.0, 1500),
    ((2, 2, 2), (8.0, 8.0, 8.0), 4.0, 1500),
    ((4, 4, 2), (4.0, 4.0, 4.0), 1.0, 3000),
    ((1, 8, 1), (4.0, 16.0, 4.0), 4.5, 3000),
    ((16, 1, 1), (16.0, 4.0, 4.0), 15.0, 2000),   # rc = L - w: 15 pulses, the most 16 domains allow
    ((8, 8, 1), (8.0, 8.0, 4.0), 7.0, 3000),      # 7 + 7 = 14 pulses over two dimensions
]


@pytest.mark.parametrize("grid,box,rc,n", DYADIC)
def test_dyadic_boxes(grid, box, rc, n):
    x = W.lattice_positions(n, box, seed=40 + n)
    x[:5] = 0.0                                   # atoms exactly on the origin
    ref = oracle.OraclePlan(x, grid, box, rc)
    for mode in MODES.values():
        g = GpuPlan(x, grid, box, rc, mode=mode, chunk=64)
        check_layout(g, ref)
        check_steps(g, ref, n, steps=2)
        check_steps(g, ref, n + 1, steps=1, fused_step=True)
        g.close()
    for chunk in (0, 64):                         # wavefront workers
        g = GpuPlan(x, grid, box, rc, mode=ddh.DDH_MODE_FUSED, chunk=chunk, wave=1)
        check_steps(g, ref, n + 2, steps=2)
        check_steps(g, ref, n + 3, steps=1, fused_step=True)
        g.close()


def test_empty_and_one_sided_inputs():
    box = (8.0, 8.0, 8.0)
    # no atoms
    ref = oracle.OraclePlan(np.zeros((0, 3), np.float32), (2, 2, 2), box, 1.0)
    g = GpuPlan(np.zeros((0, 3), np.float32), (2, 2, 2), box, 1.0)
    assert g.n_slots == 0 and g.lay["n_halo"] == 0 and g.P == 3
    xl = torch.zeros((1, 3), dtype=torch.float32, device="cuda")
    g.plan.exchange_coords(xl)
    g.plan.exchange_forces(xl)
    assert g.plan.check() == ddh.DDH_OK
    g.close()
    # all atoms in one domain: seven domains own nothing but still receive
    x = W.lattice_positions(700, (4.0, 4.0, 4.0), seed=3)
    ref = oracle.OraclePlan(x, (2, 2, 2), box, 1.25)
    g = GpuPlan(x, (2, 2, 2), box, 1.25)
    check_layout(g, ref)
    check_steps(g, ref, 5)
    g.close()
    # cell <= 0: one cell per domain (home atoms by class, then global id)
    x = W.lattice_positions(900, box, seed=4)
    ref = oracle.OraclePlan(x, (2, 2, 2), box, 1.25, cell=0.0)
    g = GpuPlan(x, (2, 2, 2), box, 1.25, cell=0.0)
    check_layout(g, ref)
    g.close()


@pytest.mark.parametrize("mode", ["pulse", "pulse_graph", "fused", "auto"])
@pytest.mark.parametrize("grid,n", [((16, 4, 4), 3000), ((8, 8, 8), 1500), ((16, 4, 4), 40000)])
def test_many_small_maps(grid, n, mode):
    """At least one domain per compute unit and short maps, many of them
    empty (chunks of empty maps, chunks holding a whole map)."""
    box = (15.66, 15.66, 15.66)
    x = W.uniform_positions(n, box, seed=n + grid[0])
    ref = oracle.OraclePlan(x, grid, box, 1.2)
    g = GpuPlan(x, grid, box, 1.2, mode=MODES[mode])
    check_layout(g, ref)
    check_steps(g, ref, n, steps=2)
    check_steps(g, ref, n + 1, steps=1, fused_step=True)
    g.close()


@pytest.mark.parametrize("home_sort", [0, 1, 2])
def test_home_sort_forms(home_sort, workload_plan):
    """Both orderings of the home atoms (the counting sort with device
    atomics, the partition sort with LDS counters) give the oracle's layout,
    maps and results: on the workloads, exact boxes with multi-pulse relay,
    random decompositions, many small domains, domains too large for the
    partition's LDS copy (40,000 atoms each), an empty input and a position
    outside the box."""
    for k in (1, 2, 3, 4):
        w, x, ref = workload_plan(k)
        g = GpuPlan(x, **w.params(), mode=ddh.DDH_MODE_PULSE, home_sort=home_sort)
        check_layout(g, ref)
        check_steps(g, ref, k, steps=1)
        g.close()
    cases = [(grid, box, rc, W.lattice_positions(n, box, seed=40 + n)) for grid, box, rc, n in DYADIC]
    cases += [(grid, box, rc, W.uniform_positions(n, box, seed=n))
              for grid, box, rc, n in random_configs(6, 77)]
    cases.append(((16, 4, 4), (15.66, 15.66, 15.66), 1.2,
                  W.uniform_positions(3000, (15.66, 15.66, 15.66), seed=3016)))
    cases.append(((2, 1, 1), (7.0, 7.0, 7.0), 1.0,
                  W.uniform_positions(80_000, (7.0, 7.0, 7.0), seed=8011)))
    for grid, box, rc, x in cases:
        ref = oracle.OraclePlan(x, grid, box, rc)
        g = GpuPlan(x, grid, box, rc, mode=ddh.DDH_MODE_AUTO, home_sort=home_sort)
        check_layout(g, ref)
        check_steps(g, ref, len(x), steps=1)
        g.close()
    g = GpuPlan(np.zeros((0, 3), np.float32), (2, 2, 2), (8.0, 8.0, 8.0), 1.0, home_sort=home_sort)
    assert g.n_slots == 0 and g.lay["n_halo"] == 0
    g.close()
    # more sort cells per domain than the partition's tables hold (13 x 25 x
    # 25 = 8125 at 2 x 1 x 1, box 12.5, cell 0.5) or more domains (2304): the
    # forced partition refuses, the automatic choice and the counting sort
    # build
    for grid, box in (((2, 1, 1), (12.5, 12.5, 12.5)), ((16, 16, 9), (40.0, 40.0, 22.5))):
        x = W.uniform_positions(4000, box, seed=77)
        if home_sort == 2:
            plan = ddh.Plan(grid, box, 1.0)
            plan.tune(ddh.DDH_TUNE_HOME_SORT, 2)
            with pytest.raises(ddh.DDHError) as e:
                plan.build_maps(torch.from_numpy(x).cuda())
            assert e.value.code == ddh.DDH_EINVAL
            plan.close()
        else:
            ref = oracle.OraclePlan(x, grid, box, 1.0)
            g = GpuPlan(x, grid, box, 1.0, mode=ddh.DDH_MODE_AUTO, home_sort=home_sort)
            check_layout(g, ref)
            g.close()
    plan = ddh.Plan((2, 2, 2), (8.0, 8.0, 8.0), 1.0)
    plan.tune(ddh.DDH_TUNE_HOME_SORT, home_sort)
    x = W.lattice_positions(200, (8.0, 8.0, 8.0), seed=1)
    x[7, 2] = 8.0
    with pytest.raises(ddh.DDHError) as e:
        plan.build_maps(torch.from_numpy(x).cuda())
    assert e.value.code == ddh.DDH_EINVAL
    plan.close()


@pytest.mark.parametrize("home_sort", [1, 2])
def test_selection_by_cells_and_by_slots(home_sort):
    """The home slots of a dimension's first pulse are selected by cells while
    the cells hold at most 64 home atoms on average (whole cells taken without
    a test, partly selected ones tested atom by atom, the partition sort
    gathering only the cells a selection reads), else by slot tiles with every
    home position gathered: both give the oracle's layout, maps and results.
    2 x 1 x 1 domains of 2 x 4 x 4 cells of 0.5 nm hold 60 atoms per cell on
    average (by cells, cells past 32 atoms taken in several batches) and 94
    (by slots); a cell size of 0 puts one cell in each domain (by slots)."""
    box = (2.0, 2.0, 2.0)
    for n, cell in ((3840, 0.5), (6000, 0.5), (2000, 0.0)):
        x = W.uniform_positions(n, box, seed=500 + n)
        ref = oracle.OraclePlan(x, (2, 1, 1), box, 0.5, cell=cell)
        for mode in (ddh.DDH_MODE_PULSE, ddh.DDH_MODE_FUSED):
            g = GpuPlan(x, (2, 1, 1), box, 0.5, cell=cell, mode=mode, home_sort=home_sort)
            check_layout(g, ref)
            check_steps(g, ref, 600 + n, steps=1)
            g.close()


@pytest.mark.parametrize("k,first", [(3, ddh.DDH_MODE_AUTO), (3, ddh.DDH_MODE_PULSE),
                                     (2, ddh.DDH_MODE_AUTO | ddh.DDH_MODE_GRAPH)])
def test_fused_table_made_at_mode_switch(k, first, workload_plan):
    """A build under a mode that never runs the fused launch (AUTO over more
    than 200k halo atoms, PULSE, AUTO with GRAPH) leaves its table out;
    switching to FUSED makes it then. Results stay the oracle's: eager and
    graph-replayed fused steps after the switch, a rebuild under FUSED, and
    a switch back and forth."""
    w, x, ref = workload_plan(k)
    g = GpuPlan(x, mode=first, **w.params())
    check_layout(g, ref)
    check_steps(g, ref, k + 70, steps=1)
    g.plan.set_mode(ddh.DDH_MODE_FUSED)
    check_steps(g, ref, k + 71, steps=1, fused_step=True)
    g.plan.set_mode(ddh.DDH_MODE_PULSE)
    g.plan.set_mode(ddh.DDH_MODE_FUSED | ddh.DDH_MODE_GRAPH)
    check_steps(g, ref, k + 72, steps=2)
    g.lay = g.plan.build_maps(g.xg)
    g.plan.set_mode(ddh.DDH_MODE_FUSED)
    check_steps(g, ref, k + 73, steps=1, fused_step=True)
    g.plan.set_mode(first)
    g.lay = g.plan.build_maps(g.xg)
    g.plan.set_mode(ddh.DDH_MODE_FUSED)
    check_steps(g, ref, k + 74, steps=1)
    g.close()


@pytest.mark.parametrize("refined", [0, 1])
def test_fused_table_keeps_the_build_settings(refined, workload_plan):
    """The fused table made at a later mode switch uses the refined-waits
    setting of its build, even when the setting changed in between: the
    conservative masks, or the refined ones, never none."""
    w, x, ref = workload_plan(3)
    g = GpuPlan(x, mode=ddh.DDH_MODE_PULSE, refined=refined, **w.params())
    g.plan.tune(ddh.DDH_TUNE_REFINED_WAITS, 1 - refined)
    g.plan.set_mode(ddh.DDH_MODE_FUSED)
    check_steps(g, ref, 90 + refined, steps=2, fused_step=True)
    check_steps(g, ref, 92 + refined, steps=1)
    g.close()


CELL_CASES = [((2, 2, 2), (4.0, 4.0, 4.0), 1.0, 4000, 11),
              ((3, 2, 1), (6.0, 3.0, 2.5), 0.75, 5000, 12),
              ((4, 1, 2), (5.0, 2.0, 4.0), 1.5, 3000, 13)]


@pytest.mark.parametrize("cell", [0.3, 0.37, 0.375, 0.7, 1.1, 3.0])
def test_cell_sizes(cell):
    """Cell sizes whose reciprocal is inexact in fp32 (0.3, 0.37, 0.7, 1.1),
    dyadic (0.375), and wider than every domain (3.0, one cell per domain),
    with positions on a 1/16 nm lattice, so that many atoms lie exactly on
    cell edges and on the slab thresholds (rc 1.0, 0.75, 1.5; two pulses
    along x in the last case). The cell coordinate is floor(fl(fl(x - lo) *
    fl(1/c))), clamped; the home selection's whole-cell decisions rest on it
    being monotone in fl(x - lo). Both home sorts and both launch forms give
    the oracle's layout, maps and results."""
    for grid, box, rc, n, seed in CELL_CASES:
        x = W.lattice_positions(n, box, seed=seed, frac_bits=4)
        ref = oracle.OraclePlan(x, grid, box, rc, cell=cell)
        for home_sort, mode in ((1, ddh.DDH_MODE_PULSE), (2, ddh.DDH_MODE_PULSE),
                                (2, ddh.DDH_MODE_FUSED)):
            g = GpuPlan(x, grid, box, rc, cell=cell, mode=mode, home_sort=home_sort)
            check_layout(g, ref)
            check_steps(g, ref, n + seed, steps=1)
            g.close()


def test_error_paths():
    box = (8.0, 8.0, 8.0)
    plan = ddh.Plan((2, 2, 2), box, 1.0)
    for bad in (8.0, -0.5, float("nan")):
        x = W.lattice_positions(200, box, seed=1)
        x[7, 2] = bad
        with pytest.raises(ddh.DDHError) as e:
            plan.build_maps(torch.from_numpy(x).cuda())
        assert e.value.code == ddh.DDH_EINVAL
    x = W.lattice_positions(2000, box, seed=2)
    lay = plan.build_maps(torch.from_numpy(x).cuda())
    small = torch.zeros((lay["n_slots"] - 1, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ddh.DDHError) as e:
        plan.exchange_coords(small)
    assert e.value.code == ddh.DDH_ECAPACITY
    full = torch.zeros((lay["n_slots"], 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ddh.DDHError) as e:
        plan.exchange_step(full, full)
    assert e.value.code == ddh.DDH_EINVAL
    # more atoms than a home sort value's 29 id bits hold: refused before
    # any position is read
    rc = ddh._lib.ddh_build_maps(plan._h, ctypes.c_void_p(full.data_ptr()), (1 << 29) + 1, None)
    assert rc == ddh.DDH_EINVAL
    plan.close()


def test_timeout_path_is_reported_and_recovers(workload_plan):
    w, x, ref = workload_plan(2)
    for mode, wave in ((ddh.DDH_MODE_FUSED, 0), (ddh.DDH_MODE_FUSED, 1), (ddh.DDH_MODE_PULSE, 0)):
        g = GpuPlan(x, **w.params(), mode=mode, wave=wave)
        g.plan.tune(ddh.DDH_TUNE_SPIN_LIMIT, 64)
        g.plan.tune(ddh.DDH_TUNE_FORCE_TIMEOUT, 1)
        xl = g.new_coords()
        fl = torch.zeros_like(xl)
        # only the fused launch waits on the device; pulse mode is ordered
        # by the stream and has nothing that can time out
        want = ddh.DDH_ETIMEOUT if mode == ddh.DDH_MODE_FUSED else ddh.DDH_OK
        g.plan.exchange_coords(xl)
        assert g.plan.check() == want
        g.plan.exchange_step(xl, fl)
        assert g.plan.check() == want
        g.plan.tune(ddh.DDH_TUNE_FORCE_TIMEOUT, 0)
        g.plan.tune(ddh.DDH_TUNE_SPIN_LIMIT, 1 << 20)
        check_steps(g, ref, 77, steps=2)
        g.close()


def test_repeated_force_passes_are_deterministic(workload_plan):
    w, x, ref = workload_plan(3)
    g = GpuPlan(x, **w.params())
    f0 = W.forces(w, g.n_slots)
    fr = f0.copy()
    ref.exchange_forces(fr)
    fl = torch.empty((g.n_slots, 3), dtype=torch.float32, device="cuda")
    src = torch.from_numpy(f0).cuda()
    for _ in range(20):
        fl.copy_(src)
        g.plan.exchange_forces(fl)
        assert np.array_equal(bits(fl.cpu().numpy()), bits(fr))
    assert g.plan.check() == ddh.DDH_OK
    g.close()


@pytest.mark.parametrize("stage", [1, 2])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_lds_staged_stores(k, stage, workload_plan):
    """Coordinate stores staged through LDS (DDH_TUNE_LDS_STAGE 1: records
    gathered into registers, 2: gathered by LDS loads) give the oracle's
    coordinates and forces: per-pulse launches and the fused launch (work-
    group chunks and wavefront workers), eager and from the library's graphs, with 16- and 32-bit maps, with chunks of
    several rounds (DDH_TUNE_CHUNK 4096 and 8192), in the host-orchestrated
    baseline, and into
    coordinate arrays that start 4, 8 or 12 bytes past a 16-byte boundary
    (every alignment of a run), with nothing written outside them."""
    w, x, ref = workload_plan(k)
    forms = ((ddh.DDH_MODE_PULSE, 1, 0), (ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH, 1, 0),
             (ddh.DDH_MODE_PULSE, 0, 0), (ddh.DDH_MODE_PULSE, 1, 4096),
             (ddh.DDH_MODE_STAGED, 1, 0), (ddh.DDH_MODE_FUSED, 1, 0),
             (ddh.DDH_MODE_FUSED | ddh.DDH_MODE_GRAPH, 0, 0), (ddh.DDH_MODE_FUSED, 1, 8192))
    for mode, narrow, chunk in forms:
        g = GpuPlan(x, **w.params(), mode=mode, narrow=narrow, chunk=chunk, lds_stage=stage)
        check_steps(g, ref, 300 + k, steps=2)
        check_steps(g, ref, 310 + k, steps=1, fused_step=True)
        g.close()
    # the fused launch's wavefront workers, slices of 256 and 1024 entries
    for chunk in (256, 1024):
        g = GpuPlan(x, **w.params(), mode=ddh.DDH_MODE_FUSED, wave=1, chunk=chunk, lds_stage=stage)
        check_steps(g, ref, 320 + k, steps=2)
        check_steps(g, ref, 330 + k, steps=1, fused_step=True)
        g.close()
    g = GpuPlan(x, **w.params(), mode=ddh.DDH_MODE_PULSE, lds_stage=stage)
    n = g.n_slots
    for off in (1, 2, 3):
        buf = torch.full((3 * n + 8,), -7.0, dtype=torch.float32, device="cuda")
        xl = buf[off:off + 3 * n].view(n, 3)
        xl.zero_()
        g.plan.gather_home(g.xg, xl)
        g.plan.exchange_coords(xl)
        assert g.plan.check() == ddh.DDH_OK
        assert np.array_equal(bits(xl.cpu().numpy()), bits(ref.x_local)), off
        rest = torch.cat([buf[:off], buf[off + 3 * n:]]).cpu().numpy()
        assert np.all(rest == -7.0), off
    g.close()


def test_workload5_full_size():
    """12M atoms, 8x8x8 domains, at full size: the fused launch (work-group
    chunks and wavefront workers), the library's graph of per-pulse launches
    (stores from registers, staged through LDS from registers and by LDS
    loads), the host-orchestrated
    baseline, and the bench's own launch (the automatic mode captured in a
    caller's graph and replayed twice)."""
    w = W.WORKLOADS[5]
    x = W.positions(w)
    ref = oracle.OraclePlan(x, **w.params())
    f0 = W.forces(w, ref.n_slots)
    fr = f0.copy()
    ref.exchange_forces(fr)
    for mode, wave, stg in ((ddh.DDH_MODE_FUSED, 0, 0), (ddh.DDH_MODE_FUSED, 1, 0),
                            (ddh.DDH_MODE_FUSED, 0, 2),
                            (ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH, 0, 0),
                            (ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH, 0, 1),
                            (ddh.DDH_MODE_PULSE | ddh.DDH_MODE_GRAPH, 0, 2),
                            (ddh.DDH_MODE_STAGED, 0, 0), (ddh.DDH_MODE_AUTO, 0, 0)):
        g = GpuPlan(x, **w.params(), mode=mode, wave=wave, lds_stage=stg)
        if mode == ddh.DDH_MODE_FUSED and not wave:
            check_layout(g, ref)
        xl = g.new_coords()
        fl = torch.from_numpy(f0).cuda()
        if mode != ddh.DDH_MODE_AUTO:
            g.plan.exchange_step(xl, fl)
            replays = 1
        else:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                g.plan.exchange_step(xl, fl)      # warm-up outside the capture
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                g.plan.exchange_step(xl, fl)
            replays = 2
        for r in range(replays):
            if mode == ddh.DDH_MODE_AUTO:
                xl.copy_(g.new_coords())
                fl.copy_(torch.from_numpy(f0))
                torch.cuda.synchronize()
                graph.replay()
            assert g.plan.check() == ddh.DDH_OK
            assert np.array_equal(bits(xl.cpu().numpy()), bits(ref.x_local)), (mode, wave, stg, r)
            assert np.array_equal(bits(fl.cpu().numpy()), bits(fr)), (mode, wave, stg, r)
        if mode == ddh.DDH_MODE_AUTO:
            del graph
        g.close()
