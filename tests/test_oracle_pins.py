"""Pins of the CPU oracle on small exact (dyadic) boxes.

Every check here compares the oracle with something other than itself: the
brute-force halo definition, closed forms, the structural facts the guide
states (tests/golden/guide_schedule.json), force conservation, integer-force
exactness and the reverse-pulse summation tree (tests/bruteforce.py).
"""

import json
import math
import os

import numpy as np
import pytest

import bruteforce as bf
import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "guide_schedule.json")

# (grid, box, rc, n_atoms): all boundaries, cutoffs and lattice positions are
# dyadic, so every fp32 operation of the exchange is exact.
DYADIC = [
    ((1, 1, 1), (4.0, 4.0, 4.0), 0.75, 500),      # nothing to exchange
    ((2, 1, 1), (8.0, 4.0, 4.0), 1.25, 2000),     # one dimension
    ((2, 2, 2), (8.0, 8.0, 8.0), 1.25, 4000),     # 3D, one pulse each
    ((3, 2, 2), (12.0, 8.0, 8.0), 2.5, 4000),     # odd domain count
    ((4, 2, 1), (8.0, 6.0, 4.0), 1.5, 3000),      # anisotropic
    ((8, 2, 2), (8.0, 8.0, 8.0), 2.5, 4000),      # X width 1 < rc: 3 pulses
    ((4, 1, 1), (8.0, 4.0, 4.0), 2.0, 1500),      # rc == width: one pulse
    ((2, 2, 2), (8.0, 8.0, 8.0), 4.0, 1500),      # rc == L - w: largest allowed
    ((4, 4, 2), (4.0, 4.0, 4.0), 1.0, 3000),      # rc == w in X/Y, 1 pulse
    ((16, 1, 1), (16.0, 4.0, 4.0), 15.0, 2000),   # rc == L - w: 15 pulses, the most 16 allow
    ((8, 8, 1), (8.0, 8.0, 4.0), 7.0, 3000),      # 7 + 7 = 14 pulses over two dimensions
]


def _bounds(grid, box):
    return [bf.exact_bounds(box[d], grid[d]) for d in range(3)]


def _pulses_per_dim(plan):
    m = [0, 0, 0]
    for d, _ in plan.pulses:
        m[d] += 1
    return m


def _with_boundary_atoms(x, grid, box, rc, rng):
    """Put some atoms exactly on domain boundaries and on slab thresholds."""
    x = x.copy()
    n = x.shape[0]
    picks = rng.choice(n, size=min(n, 60), replace=False)
    for t, a in enumerate(picks):
        d = t % 3
        i = int(rng.integers(0, grid[d]))
        lo = box[d] * i / grid[d]
        cand = [lo, lo + rc, (lo + rc) % box[d], 0.0]
        v = cand[t % len(cand)]
        if 0.0 <= v < box[d]:
            x[a, d] = np.float32(v)
    return x


@pytest.mark.parametrize("grid,box,rc,n", DYADIC)
def test_bruteforce_halo_exact(grid, box, rc, n):
    rng = np.random.default_rng(7)
    x = W.lattice_positions(n, box, seed=11 + n)
    x = _with_boundary_atoms(x, grid, box, rc, rng)
    plan = oracle.OraclePlan(x, grid, box, rc)
    bounds = _bounds(grid, box)
    for d in range(3):
        assert np.array_equal(plan.bounds[d].astype(np.float64), bounds[d])
    bf.check_halo_against(plan, x, grid, box, rc, bounds)
    # home slots: exactly the atoms inside each domain
    home = bf.domain_id(bf.home_index(x, bounds), grid)
    for D in range(plan.n_domains):
        b, nh = int(plan.base[D]), int(plan.nhome[D])
        assert np.array_equal(np.sort(plan.slot_ids[b:b + nh]), np.nonzero(home == D)[0])
        assert np.array_equal(plan.x_local[b:b + nh], x[plan.slot_ids[b:b + nh]])


@pytest.mark.parametrize("grid,box,rc,n", DYADIC)
def test_home_order_is_cell_class_then_id(grid, box, rc, n):
    """Home order from its definition, in exact arithmetic (dyadic box, lattice
    positions): sort cell (rows cy + ncy cz in turn, x upward in even rows and
    downward in odd ones), then the class of the first pulses that send the
    atom (the cells' selected atoms together, first or last by the parity of
    the x index counted from the cell that holds the cut, flipped in odd
    rows), then global id."""
    x = W.lattice_positions(n, box, seed=3 + n)
    plan = oracle.OraclePlan(x, grid, box, rc, cell=0.5)
    bounds = _bounds(grid, box)
    px = math.floor(rc / 0.5)
    for D in range(plan.n_domains):
        c = (D % grid[0], (D // grid[0]) % grid[1], D // (grid[0] * grid[1]))
        b, nh = int(plan.base[D]), int(plan.nhome[D])
        ids = plan.slot_ids[b:b + nh]
        xs = x[ids].astype(np.float64)
        ci, nc = [], []
        sent = np.zeros(nh, dtype=np.int64)
        for d in range(3):
            lo, hi = bounds[d][c[d]], bounds[d][c[d] + 1]
            ncd = max(1, math.ceil((hi - lo) / 0.5))
            ci.append(np.minimum(np.floor((xs[:, d] - lo) / 0.5), ncd - 1).astype(np.int64))
            nc.append(ncd)
            sent |= (xs[:, d] - lo < rc).astype(np.int64) << d
        row = ci[1] + nc[1] * ci[2]
        odd = row % 2 == 1
        key = np.where(odd, nc[0] - 1 - ci[0], ci[0]) + nc[0] * row
        first = ((ci[0] - px) % 2 == 0) != odd
        cls = np.where(first, 7 - sent, sent)
        order = np.lexsort((ids, cls, key))
        assert np.array_equal(order, np.arange(nh))


def test_cut_cells_keep_each_pulse_contiguous():
    """In every cell that one slab cuts, the atoms that dimension's first pulse
    sends form one run, at the cell's start when the cell's x index has the
    parity of the cut's cell (the other parity in odd rows, which run
    downward in x) and at its end otherwise, so a cell below the cut along x
    runs straight into the sent part of the next. And the X pulse's home
    atoms of an odd row end where those of the next row begin."""
    grid, box, rc = (2, 2, 2), (8.0, 8.0, 8.0), 1.25
    x = W.lattice_positions(30000, box, seed=41)
    plan = oracle.OraclePlan(x, grid, box, rc, cell=0.5)
    cut_cells = joined = 0
    for D in range(plan.n_domains):
        c = (D % 2, (D // 2) % 2, D // 4)
        lo = [4.0 * c[d] for d in range(3)]
        b, nh = int(plan.base[D]), int(plan.nhome[D])
        xs = x[plan.slot_ids[b:b + nh]].astype(np.float64)
        cell = np.floor((xs - np.array(lo)) / 0.5).astype(np.int64)
        key = cell[:, 0] + 8 * (cell[:, 1] + 8 * cell[:, 2])
        starts = np.flatnonzero(np.r_[True, key[1:] != key[:-1]])
        ends = np.r_[starts[1:], nh]
        for s, e in zip(starts, ends):
            cx = cell[s, 0]
            sent = [xs[s:e, d] - lo[d] < rc for d in range(3)]
            cut = [d for d in range(3) if sent[d].any() and not sent[d].all()]
            if len(cut) != 1:
                continue  # where two slabs cut a cell only the higher dimension's run is whole
            cut_cells += 1
            hit = np.flatnonzero(sent[cut[0]])
            assert hit[-1] - hit[0] + 1 == len(hit), "a pulse's atoms split inside a cell"
            odd = (cell[s, 1] + 8 * cell[s, 2]) % 2 == 1
            if ((cx - 2) % 2 == 0) != odd:
                assert hit[0] == 0
            else:
                assert hit[-1] == e - s - 1
        # serpentine: odd row r ends with its x-sent cells and row r + 1
        # starts with them, so both rows' X pulse atoms form one run (rows
        # that the y or z slab also cuts excepted: there a cell cut twice
        # keeps only its z or y run whole)
        row = cell[:, 1] + 8 * cell[:, 2]
        xsent = xs[:, 0] - lo[0] < rc
        for r in range(1, 63, 2):
            if 2 in (r % 8, r // 8, (r + 1) % 8, (r + 1) // 8):
                continue
            a, b = np.flatnonzero(row == r), np.flatnonzero(row == r + 1)
            assert b[0] == a[-1] + 1
            hit = np.flatnonzero(xsent[a[0]:b[-1] + 1])
            assert hit[-1] - hit[0] + 1 == len(hit), "rows r and r + 1 split the X pulse's run"
            joined += 1
    assert cut_cells > 100 and joined > 100


@pytest.mark.parametrize("grid,box,rc,n", DYADIC)
def test_map_invariants(grid, box, rc, n):
    x = W.lattice_positions(n, box, seed=5 + n)
    plan = oracle.OraclePlan(x, grid, box, rc)
    P = plan.n_pulses
    for S in range(plan.n_domains):
        for p in range(P):
            m = plan.maps[(S, p)]
            assert len(m) == plan.send[S, p]
            assert np.all(np.diff(m) > 0), "map entries must be unique and increasing"
            assert np.count_nonzero(m < plan.nhome[S]) == plan.split[S, p]
            if len(m):
                assert m.min() >= 0 and m.max() < plan.ntotal[S]
    # regions are contiguous, in pulse order, right after the home slots
    for R in range(plan.n_domains):
        regions = []
        for p in range(P):
            S = int(np.nonzero(plan.recv[:, p] == R)[0][0])
            regions.append((int(plan.roff[S, p]), int(plan.send[S, p])))
        off = int(plan.nhome[R])
        for start, size in regions:
            assert start == off
            off += size
        assert off == plan.ntotal[R]


def test_pulse_counts_closed_form():
    # np = ceil(rc / w) pulses per decomposed dimension, none for n_d = 1
    cases = [((8, 2, 2), (8.0, 8.0, 8.0), 2.5, [3, 1, 1]),
             ((4, 1, 1), (8.0, 4.0, 4.0), 2.0, [1, 0, 0]),
             ((16, 4, 4), (16.0, 16.0, 16.0), 3.0, [3, 1, 1]),
             ((1, 1, 1), (4.0, 4.0, 4.0), 1.0, [0, 0, 0]),
             ((1, 8, 1), (4.0, 16.0, 4.0), 4.5, [0, 3, 0])]
    for grid, box, rc, expect in cases:
        sched = oracle.schedule(grid, box, rc)
        per = [0, 0, 0]
        for d, _ in sched:
            per[d] += 1
        assert per == expect
        for d in range(3):
            if grid[d] > 1:
                assert per[d] == math.ceil(rc / (box[d] / grid[d]))
        # order: Z first, then Y, then X, k increasing inside a dimension
        dims = [d for d, _ in sched]
        assert dims == sorted(dims, reverse=True)
        assert all(k == i - dims.index(d) for i, (d, k) in enumerate(sched))


def test_errors():
    x = W.lattice_positions(100, (4.0, 4.0, 4.0), seed=1)
    # halo would wrap onto itself: rc > L - w
    with pytest.raises(oracle.OracleError) as e:
        oracle.OraclePlan(x, (2, 1, 1), (4.0, 4.0, 4.0), 2.25)
    assert e.value.code == oracle.ERANGE
    for bad in (np.float32(4.0), np.float32(-0.25), np.float32(np.nan)):
        y = x.copy()
        y[17, 1] = bad
        with pytest.raises(oracle.OracleError) as e:
            oracle.OraclePlan(y, (2, 2, 1), (4.0, 4.0, 4.0), 1.0)
        assert e.value.code == oracle.EINVAL
    for grid, rc in (((0, 1, 1), 1.0), ((2, 1, 1), 0.0), ((2, 1, 1), -1.0)):
        with pytest.raises(oracle.OracleError) as e:
            oracle.OraclePlan(x, grid, (4.0, 4.0, 4.0), rc)
        assert e.value.code == oracle.EINVAL


def test_empty_and_sparse_inputs():
    # no atoms at all
    plan = oracle.OraclePlan(np.zeros((0, 3), np.float32), (2, 2, 2), (8.0, 8.0, 8.0), 1.0)
    assert plan.n_slots == 0 and plan.halo_atoms == 0 and plan.n_pulses == 3
    # atoms in one domain only: the others have no home atoms but still receive
    x = W.lattice_positions(300, (4.0, 4.0, 4.0), seed=9)
    plan = oracle.OraclePlan(x, (2, 2, 2), (8.0, 8.0, 8.0), 1.25)
    assert plan.nhome[0] == 300 and np.all(plan.nhome[1:] == 0)
    bf.check_halo_against(plan, x, (2, 2, 2), (8.0, 8.0, 8.0), 1.25, _bounds((2, 2, 2), (8.0,) * 3))


def test_largest_cutoff_every_domain_sees_every_atom():
    # rc == L - w: every domain's extended region covers the whole box
    x = W.lattice_positions(1500, (8.0, 8.0, 8.0), seed=21)
    plan = oracle.OraclePlan(x, (2, 2, 2), (8.0, 8.0, 8.0), 4.0)
    assert np.all(plan.ntotal == 1500)


def test_golden_schedule():
    with open(GOLDEN) as fh:
        gold = json.load(fh)
    cases = {c["id"]: c for c in gold["cases"]}

    c = cases["phase_order_coordinates"]
    assert [d for d, _ in oracle.schedule(c["grid"], (8.0, 8.0, 8.0), 1.0)] == c["pulse_dims"]

    c = cases["phase_order_forces"]
    assert [d for d, _ in oracle.schedule(c["grid"], (8.0, 8.0, 8.0), 1.0)][::-1] == c["force_pulse_dims"]

    c = cases["one_pulse_per_dim_waits"]
    sched = oracle.schedule(c["grid"], (8.0, 8.0, 8.0), 1.0)
    assert len(sched) == c["pulses"]
    assert 2 * c["waits_per_pulse"] * len(sched) == c["waits_per_step"]

    c = cases["two_pulse_2d"]
    assert len(oracle.schedule(c["grid"], (8.0, 8.0, 8.0), 1.0)) == c["pulses"]

    c = cases["multi_pulse_relay"]
    sched = oracle.schedule(c["grid"], c["box"], c["rc"])
    assert [d for d, _ in sched] == c["pulse_dims"]

    # dependencies: the forwarded entries of pulse p reference exactly the
    # regions received in the earlier pulses named by the guide
    c = cases["global_pulse_dependencies"]
    x = W.lattice_positions(6000, (8.0, 8.0, 8.0), seed=4)
    plan = oracle.OraclePlan(x, c["grid"], (8.0, 8.0, 8.0), 1.5)
    names = c["names"]
    for p, name in enumerate(names):
        refs = set()
        for S in range(plan.n_domains):
            tail = plan.maps[(S, p)][plan.split[S, p]:]
            for q in range(p):
                Q = int(np.nonzero(plan.recv[:, q] == S)[0][0])
                lo = plan.roff[Q, q]
                hi = lo + plan.send[Q, q]
                if np.any((tail >= lo) & (tail < hi)):
                    refs.add(names[q])
        assert sorted(refs) == sorted(c["depends_on"][name])


def test_relay_pulse_forwards_only():
    # in the second X pulse a domain forwards only what it received in the first
    box = (8.0, 8.0, 8.0)
    x = W.lattice_positions(4000, box, seed=8)
    plan = oracle.OraclePlan(x, (8, 2, 2), box, 2.5)
    dims = [d for d, _ in plan.pulses]
    assert dims == [2, 1, 0, 0, 0]
    for p in (3, 4):
        assert np.all(plan.split[:, p] == 0)
        for S in range(plan.n_domains):
            Q = int(np.nonzero(plan.recv[:, p - 1] == S)[0][0])
            lo = plan.roff[Q, p - 1]
            m = plan.maps[(S, p)]
            assert np.all((m >= lo) & (m < lo + plan.send[Q, p - 1]))


@pytest.mark.parametrize("grid,box,rc,n", DYADIC)
def test_forces_exact_and_tree(grid, box, rc, n):
    x = W.lattice_positions(n, box, seed=13 + n)
    plan = oracle.OraclePlan(x, grid, box, rc)
    home_rows = np.concatenate([np.arange(plan.base[D], plan.base[D] + plan.nhome[D])
                                for D in range(plan.n_domains)])
    # integers: every copy reaches its home slot exactly once
    fi = W.integer_forces(plan.n_slots, seed=n)
    f = fi.copy()
    plan.exchange_forces(f)
    expect = bf.integer_force_expectation(plan, fi)
    assert np.array_equal(f[home_rows].astype(np.float64), expect[home_rows])
    # conservation in fp64
    fn = np.random.default_rng(n).normal(0, 10, size=(plan.n_slots, 3)).astype(np.float32)
    f = fn.copy()
    plan.exchange_forces(f)
    tot_before = fn.astype(np.float64).sum(0)
    tot_after = f[home_rows].astype(np.float64).sum(0)
    scale = np.abs(fn).astype(np.float64).sum(0) + 1e-30
    assert np.all(np.abs(tot_after - tot_before) <= 1e-6 * scale)
    # non-integer forces: the fixed reverse-pulse summation tree, bit for bit
    tree = bf.force_tree(plan, grid, fn, _pulses_per_dim(plan))
    assert np.array_equal(f[home_rows], tree[home_rows])


@pytest.mark.parametrize("grid,box,rc,n", DYADIC)
def test_coordinate_pass_reproduces_build(grid, box, rc, n):
    x = W.lattice_positions(n, box, seed=17 + n)
    plan = oracle.OraclePlan(x, grid, box, rc)
    xl = plan.home_coords(x)
    plan.exchange_coords(xl)
    assert np.array_equal(xl, plan.x_local)
    plan.exchange_coords(xl)       # a second pass changes nothing
    assert np.array_equal(xl, plan.x_local)
