"""Planted mistakes: the checks that pin the oracle must catch each one.

Each test takes a correct oracle result on an exact (dyadic) box, plants one
plausible mistake in it on the CPU (a dropped pulse, a duplicated or wrong map
entry, a missing periodic shift, a lost or doubled force term, a wrong add
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
