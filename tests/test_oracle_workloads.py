"""Pins of the CPU oracle on the five synthetic workloads (non-dyadic inputs).

The brute-force halo is exact in real arithmetic; the exchange works in fp32,
so atoms within a few ulps of a threshold are set aside (a tie band) and
counted. Forces are pinned by conservation, integer exactness and the
reverse-pulse summation tree, all independent of the oracle's code.
"""

import numpy as np
import pytest

import bruteforce as bf
import oracle
import workloads as W

EXPECTED_PULSES = {1: [0], 2: [2, 1, 0], 3: [2, 1, 0], 4: [2, 1, 0, 0], 5: [2, 1, 0]}


def _pulses_per_dim(plan):
    m = [0, 0, 0]
    for d, _ in plan.pulses:
        m[d] += 1
    return m


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_schedule(k):
    w = W.WORKLOADS[k]
    p = w.params()
    assert [d for d, _ in oracle.schedule(p["grid"], p["box"], p["rc"])] == EXPECTED_PULSES[k]


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_halo_vs_bruteforce(k, workload_plan):
    w, x, plan = workload_plan(k)
    p = w.params()
    band = 4.0 * float(np.spacing(np.float32(max(p["box"]))))
    n_band = bf.check_halo_against(plan, x, p["grid"], p["box"], p["rc"], plan.bounds, band=band)
    assert n_band <= 1e-4 * plan.halo_atoms + 5


def test_workload1_closed_form(workload_plan):
    # 2 x 1 x 1: each domain receives the atoms within rc above its upper edge,
    # rho * rc * L^2 = (3000 / 27) * 0.9 * 9 = 900 expected per domain
    w, x, plan = workload_plan(1)
    L = w.box32[0]
    for S in range(2):
        R = int(plan.recv[S, 0])
        hi = float(plan.bounds[0][R + 1])
        s = np.mod(x[:, 0].astype(np.float64) - hi, L)
        assert plan.send[S, 0] == np.count_nonzero(s < np.float32(w.rc))
    rho = w.n_atoms / L ** 3
    expect = rho * w.rc * L * L
    assert abs(plan.send.mean() - expect) < 5 * np.sqrt(expect)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_workload_slab_sizes_close_to_density(k, workload_plan):
    # expected send sizes: density x slab volume; Poisson scatter around it
    w, x, plan = workload_plan(k)
    L = w.box32[0]
    rho = w.n_atoms / L ** 3
    wd = [L / n for n in w.grid]
    rc = w.rc
    # Z0 sends the home slab within rc (or the whole domain if narrower)
    z0 = rho * wd[0] * wd[1] * min(rc, wd[2])
    assert abs(plan.send[:, 0].mean() - z0) < 0.02 * z0 + 3 * np.sqrt(z0 / plan.n_domains)
    assert plan.halo_atoms > 0


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_forces(k, workload_plan):
    w, x, plan = workload_plan(k)
    home_rows = np.concatenate([np.arange(plan.base[D], plan.base[D] + plan.nhome[D])
                                for D in range(plan.n_domains)])
    fi = W.integer_forces(plan.n_slots, seed=100 + k)
    f = fi.copy()
    plan.exchange_forces(f)
    expect = bf.integer_force_expectation(plan, fi)
    assert np.array_equal(f[home_rows].astype(np.float64), expect[home_rows])

    fn = W.forces(w, plan.n_slots)
    f = fn.copy()
    plan.exchange_forces(f)
    tot_before = fn.astype(np.float64).sum(0)
    tot_after = f[home_rows].astype(np.float64).sum(0)
    scale = np.abs(fn).astype(np.float64).sum(0)
    assert np.all(np.abs(tot_after - tot_before) <= 1e-6 * scale)
    tree = bf.force_tree(plan, w.grid, fn, _pulses_per_dim(plan))
    assert np.array_equal(f[home_rows], tree[home_rows])


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_copies_bounded(k, workload_plan):
    # one pulse per dimension: at most 7 halo copies per atom; 384k atoms on
    # 16x4x4 domains (two X pulses) allow (2+1)*(1+1)*(1+1) - 1 = 11
    w, x, plan = workload_plan(k)
    counts = np.bincount(plan.slot_ids, minlength=w.n_atoms)
    bound = 1
    for m in _pulses_per_dim(plan):
        bound *= m + 1
    assert counts.min() >= 1 and counts.max() <= bound
    assert counts.sum() == plan.n_slots


@pytest.mark.slow
def test_workload5_schedule_and_counts():
    w = W.WORKLOADS[5]
    x = W.positions(w)
    plan = oracle.OraclePlan(x, **w.params())
    assert plan.n_pulses == 3
    counts = np.bincount(plan.slot_ids, minlength=w.n_atoms)
    assert counts.max() <= 8
    # density x slab volume: about 8.46M halo atoms per pass
    assert abs(plan.halo_atoms - 8_463_804) < 0.01 * 8_463_804


def _random_configs(n, seed):
    """Seeded random decompositions the schedule accepts (1-6 domains per
    dimension, 2-9 nm edges, cutoffs up to the largest the widths allow)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        grid = tuple(int(g) for g in rng.integers(1, 7, size=3))
        box = tuple(float(np.float32(b)) for b in rng.uniform(2.0, 9.0, size=3))
        wmin = min(box[d] / grid[d] for d in range(3) if grid[d] > 1) if max(grid) > 1 else 1.0
        rc = float(np.float32(rng.uniform(0.2, 2.5) * wmin))
        try:
            oracle.schedule(grid, box, rc)
        except oracle.OracleError:
            continue
        out.append((grid, box, rc, int(rng.integers(200, 3000))))
    return out


@pytest.mark.parametrize("cfg", _random_configs(10, 77))
def test_random_decompositions_vs_bruteforce(cfg):
    """Random boxes and cutoffs (several pulses per dimension included): the
    received sets against brute force (tie band as above), and forces
    against the order-free integer expectation."""
    grid, box, rc, n = cfg
    x = W.uniform_positions(n, box, seed=n + 1)
    plan = oracle.OraclePlan(x, grid, box, rc)
    band = 4.0 * float(np.spacing(np.float32(max(box))))
    n_band = bf.check_halo_against(plan, x, grid, box, rc, plan.bounds, band=band)
    assert n_band <= 1e-3 * plan.halo_atoms + 5
    home_rows = np.concatenate([np.arange(plan.base[D], plan.base[D] + plan.nhome[D])
                                for D in range(plan.n_domains)])
    fi = W.integer_forces(plan.n_slots, seed=n)
    f = fi.copy()
    plan.exchange_forces(f)
    expect = bf.integer_force_expectation(plan, fi)
    assert np.array_equal(f[home_rows].astype(np.float64), expect[home_rows])
