"""Planted mistakes: the checks that pin the oracle must catch each one.

Each test takes a correct oracle result on an exact (dyadic) box, plants one
plausible mistake in it on the CPU (a dropped pulse, a duplicated map entry, a
missing periodic shift, `<=` in the slab test, pulses sent to the wrong
neighbour, no relay of received records, a lost force term, a wrong add
order) and asserts that the corresponding independent check fails.
"""

import copy

import numpy as np
import pytest

import bruteforce as bf
import oracle
import workloads as W

GRID, BOX, RC = (2, 2, 2), (8.0, 8.0, 8.0), 1.25


@pytest.fixture(scope="module")
def base():
    x = W.lattice_positions(4000, BOX, seed=31)
    plan = oracle.OraclePlan(x, GRID, BOX, RC)
    bounds = [bf.exact_bounds(BOX[d], GRID[d]) for d in range(3)]
    return x, plan, bounds


class _View:
    """A mutable copy of the arrays a check reads."""

    def __init__(self, plan):
        for k in ("base", "nhome", "ntotal", "slot_ids", "x_local", "n_slots"):
            setattr(self, k, copy.deepcopy(getattr(plan, k)))


def test_dropped_pulse_is_caught(base):
    x, plan, bounds = base
    v = _View(plan)
    # domain 0 never receives its last region: truncate its slots
    S = int(np.nonzero(plan.recv[:, 2] == 0)[0][0])
    v.ntotal[0] -= plan.send[S, 2]
    with pytest.raises(AssertionError):
        bf.check_halo_against(v, x, GRID, BOX, RC, bounds)


def test_duplicate_entry_is_caught(base):
    x, plan, bounds = base
    v = _View(plan)
    b, nh = int(v.base[3]), int(v.nhome[3])
    v.slot_ids[b + nh + 1] = v.slot_ids[b + nh]
    v.x_local[b + nh + 1] = v.x_local[b + nh]
    with pytest.raises(AssertionError):
        bf.check_halo_against(v, x, GRID, BOX, RC, bounds)


def test_missing_shift_is_caught(base):
    x, plan, bounds = base
    v = _View(plan)
    # undo the periodic image of one wrapped halo record
    for R in range(plan.n_domains):
        b, nh, nt = int(v.base[R]), int(v.nhome[R]), int(v.ntotal[R])
        for d in range(3):
            lo = bounds[d][[R % 2, (R // 2) % 2, R // 4][d]]
            wrapped = np.nonzero(v.x_local[b + nh:b + nt, d] >= BOX[d])[0]
            if len(wrapped):
                v.x_local[b + nh + wrapped[0], d] -= np.float32(BOX[d])
                with pytest.raises(AssertionError):
                    bf.check_halo_against(v, x, GRID, BOX, RC, bounds)
                return
    pytest.fail("no wrapped record found")


def test_wrong_slab_edge_is_caught():
    # an oracle that used <= instead of < would send atoms sitting exactly at rc;
    # model it by building with a slightly larger cutoff and checking at RC
    x = W.lattice_positions(4000, BOX, seed=32)
    lo_edges = np.arange(0.0, 8.0, 4.0)
    x[:40, 0] = np.float32(lo_edges[1] + RC)   # exactly on the X threshold
    bounds = [bf.exact_bounds(BOX[d], GRID[d]) for d in range(3)]
    loose = oracle.OraclePlan(x, GRID, BOX, np.nextafter(np.float32(RC), np.float32(10)))
    with pytest.raises(AssertionError):
        bf.check_halo_against(loose, x, GRID, BOX, RC, bounds)


def _home_rows(plan):
    return np.concatenate([np.arange(plan.base[D], plan.base[D] + plan.nhome[D])
                           for D in range(plan.n_domains)])


def test_lost_force_term_is_caught(base):
    x, plan, bounds = base
    fi = W.integer_forces(plan.n_slots, seed=5)
    f = fi.copy()
    plan.exchange_forces(f)
    expect = bf.integer_force_expectation(plan, fi)
    rows = _home_rows(plan)
    assert np.array_equal(f[rows].astype(np.float64), expect[rows])
    # a pass that skipped one pulse: drop the contributions of pulse 0
    g = fi.copy()
    for S in range(plan.n_domains):
        for p in range(plan.n_pulses - 1, 0, -1):
            R = plan.recv[S, p]
            src = plan.base[R] + plan.roff[S, p]
            m = plan.maps[(S, p)]
            g[plan.base[S] + m] += g[src:src + len(m)]
    assert not np.array_equal(g[rows].astype(np.float64), expect[rows])


def test_wrong_add_order_is_caught(base):
    x, plan, bounds = base
    fn = np.random.default_rng(3).normal(0, 10, size=(plan.n_slots, 3)).astype(np.float32)
    rows = _home_rows(plan)
    tree = bf.force_tree(plan, GRID, fn, [1, 1, 1])
    # forward pulse order instead of reverse: relay copies are added before
    # they have collected their own contributions, so values differ
    g = fn.copy()
    for p in range(plan.n_pulses):
        for S in range(plan.n_domains):
            R = plan.recv[S, p]
            src = plan.base[R] + plan.roff[S, p]
            m = plan.maps[(S, p)]
            g[plan.base[S] + m] = g[plan.base[S] + m] + g[src:src + len(m)]
    assert not np.array_equal(g[rows], tree[rows])
    # reverse order reproduces the tree
    h = fn.copy()
    plan.exchange_forces(h)
    assert np.array_equal(h[rows], tree[rows])


def _relaid_view(plan, per_domain):
    """A view whose domain R holds its home slots and then the halo records
    per_domain(R) returns (ids, coordinates), packed domain after domain."""
    v = _View(plan)
    ids, xs, bases, ntot = [], [], [], []
    pos = 0
    for R in range(plan.n_domains):
        b, nh = int(plan.base[R]), int(plan.nhome[R])
        hid, hx = per_domain(R)
        ids += [plan.slot_ids[b:b + nh], hid]
        xs += [plan.x_local[b:b + nh], hx]
        bases.append(pos)
        ntot.append(nh + len(hid))
        pos += nh + len(hid)
    v.slot_ids = np.concatenate(ids).astype(np.int32)
    v.x_local = np.concatenate(xs).astype(np.float32)
    v.base = np.asarray(bases, np.int64)
    v.ntotal = np.asarray(ntot, np.int32)
    v.n_slots = pos
    return v


def _mirror_domain(D, grid):
    c = [D % grid[0], (D // grid[0]) % grid[1], D // (grid[0] * grid[1])]
    c = [grid[d] - 1 - c[d] for d in range(3)]
    return c[0] + grid[0] * (c[1] + grid[1] * c[2])


def test_wrong_send_side_is_caught(base):
    # an oracle that sent every pulse to the +d neighbour (not -d) would
    # leave each domain the slab below its lower faces: exactly what the
    # correct oracle gives for the mirror image of the system, read back
    x, plan, bounds = base
    L = np.asarray(BOX, dtype=np.float32)
    xm = np.mod(L - x, L).astype(np.float32)  # exact on the 2^-12 nm lattice
    mp = oracle.OraclePlan(xm, GRID, BOX, RC)

    def halo(R):
        M = _mirror_domain(R, GRID)
        mb, mnh, mnt = int(mp.base[M]), int(mp.nhome[M]), int(mp.ntotal[M])
        return mp.slot_ids[mb + mnh:mb + mnt], L - mp.x_local[mb + mnh:mb + mnt]

    v = _relaid_view(plan, halo)
    with pytest.raises(AssertionError):
        bf.check_halo_against(v, x, GRID, BOX, RC, bounds)


def test_no_relay_is_caught(base):
    # an oracle whose pulses sent home atoms only (no forwarding of records
    # received in earlier pulses) leaves out every edge and corner copy
    x, plan, bounds = base
    keep = np.ones(plan.n_slots, dtype=bool)
    relayed = 0
    for S in range(plan.n_domains):
        for p in range(plan.n_pulses):
            R = int(plan.recv[S, p])
            o = int(plan.base[R] + plan.roff[S, p])
            keep[o + int(plan.split[S, p]):o + int(plan.send[S, p])] = False
            relayed += int(plan.send[S, p] - plan.split[S, p])
    assert relayed > 0

    def halo(R):
        b, nh, nt = int(plan.base[R]), int(plan.nhome[R]), int(plan.ntotal[R])
        k = keep[b + nh:b + nt]
        return plan.slot_ids[b + nh:b + nt][k], plan.x_local[b + nh:b + nt][k]

    v = _relaid_view(plan, halo)
    with pytest.raises(AssertionError):
        bf.check_halo_against(v, x, GRID, BOX, RC, bounds)
    # the unmutated view passes the same check
    full = _relaid_view(plan, lambda R: (
        plan.slot_ids[int(plan.base[R] + plan.nhome[R]):int(plan.base[R] + plan.ntotal[R])],
        plan.x_local[int(plan.base[R] + plan.nhome[R]):int(plan.base[R] + plan.ntotal[R])]))
    bf.check_halo_against(full, x, GRID, BOX, RC, bounds)
