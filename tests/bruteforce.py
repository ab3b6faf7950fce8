"""Independent checks for the staged halo exchange (test helper).

Nothing here reuses the oracle's code. Each check states a property that the
staged exchange of the NVIDIA guide "A Practical Guide to GPU-Initiated
Communication for Molecular Dynamics at Scale" must have, computed directly:

* `halo_sets`: the definition of the halo. With data relayed pulse by pulse
  through neighbours (section "Accelerating GROMACS using Device-initiated
  Remote Memory Access") and each domain receiving from its +d side, domain R
  must end up holding every atom that is not its own and lies, in every
  decomposed dimension, within [lo_d(R), hi_d(R) + rc) modulo L_d, each exactly
  once, with coordinate x_d + L_d wherever x_d < lo_d(R) (periodic image).
* `force_tree`: the value the reverse pass must produce. Forces travel back
  along the relay chain (section "Force halo exchange: Reversing the
  dependency chain"), last pulse first, accumulating in place. For a home atom
  whose copies sit s_d domain steps away in dimension d, the pass reduces each
  dimension's chain right-nested, v_0 + (v_1 + (... + v_m)), X first (the
  last pulses), then Y, then Z, giving a fixed fp32 summation tree.
"""

from __future__ import annotations

import numpy as np


def exact_bounds(L: float, n: int) -> np.ndarray:
    """Boundaries L*i/n in float64, asserting they are exact float32 values."""
    b = np.array([L * i / n for i in range(n + 1)], dtype=np.float64)
    assert np.all(b.astype(np.float32).astype(np.float64) == b), "box/grid not dyadic"
    return b


def home_index(x: np.ndarray, bounds) -> np.ndarray:
    """[N, 3] domain index per dimension: the i with b[i] <= x < b[i+1]."""
    out = np.zeros(x.shape, dtype=np.int64)
    for d in range(3):
        b = np.asarray(bounds[d], dtype=np.float64)
        xd = x[:, d].astype(np.float64)
        out[:, d] = np.searchsorted(b, xd, side="right") - 1
    return out


def domain_id(ci: np.ndarray, grid) -> np.ndarray:
    return ci[..., 0] + grid[0] * (ci[..., 1] + grid[1] * ci[..., 2])


def halo_sets(x: np.ndarray, grid, box, rc: float, bounds, band: float = 0.0):
    """Brute-force halo of every domain.

    Returns {R: (gids sorted, coords [n, 3] float64 in gid order, n_band)}.
    With band > 0, atoms whose exact distance lies within `band` of a
    threshold are left out and counted instead (non-dyadic inputs).
    """
    x64 = x.astype(np.float64)
    hi_ = home_index(x, bounds)
    home = domain_id(hi_, grid)
    out = {}
    n_dom = grid[0] * grid[1] * grid[2]
    for R in range(n_dom):
        c = (R % grid[0], (R // grid[0]) % grid[1], R // (grid[0] * grid[1]))
        keep = home != R
        amb = np.zeros(x.shape[0], dtype=bool)
        coords = x64.copy()
        for d in range(3):
            if grid[d] == 1:
                continue
            lo = float(bounds[d][c[d]])
            hi = float(bounds[d][c[d] + 1])
            L = float(box[d])
            s = np.mod(x64[:, d] - lo, L)
            thr = (hi - lo) + rc
            keep &= s < thr
            if band > 0:
                amb |= np.abs(s - thr) < band
                amb |= np.abs(x64[:, d] - lo) < band
                amb |= np.abs(x64[:, d] - hi) < band
            coords[:, d] = np.where(x64[:, d] < lo, x64[:, d] + L, x64[:, d])
        n_band = int(np.count_nonzero(amb & keep)) if band > 0 else 0
        sel = keep & ~amb
        gids = np.nonzero(sel)[0]
        out[R] = (gids, coords[gids], n_band, amb)
    return out


def check_halo_against(plan, x, grid, box, rc, bounds, band=0.0):
    """Compare a plan's halo slots with the brute force. Returns #band atoms.

    `plan` needs base, nhome, ntotal, slot_ids and x_local (numpy).
    Raises AssertionError on any mismatch.
    """
    ref = halo_sets(x, grid, box, rc, bounds, band)
    total_band = 0
    for R, (gids, coords, n_band, amb) in ref.items():
        b, nh, nt = int(plan.base[R]), int(plan.nhome[R]), int(plan.ntotal[R])
        ids = plan.slot_ids[b + nh:b + nt].astype(np.int64)
        xs = plan.x_local[b + nh:b + nt].astype(np.float64)
        assert len(np.unique(ids)) == len(ids), f"domain {R}: an atom arrives twice"
        # drop the ambiguous atoms from the plan's side as well
        mask = ~amb[ids]
        ids_c, xs_c = ids[mask], xs[mask]
        order = np.argsort(ids_c)
        ids_c, xs_c = ids_c[order], xs_c[order]
        assert ids_c.shape == gids.shape and np.array_equal(ids_c, gids), (
            f"domain {R}: halo set differs ({len(ids_c)} vs {len(gids)} atoms)")
        if band == 0.0:
            assert np.array_equal(xs_c, coords), f"domain {R}: halo coordinates differ"
        else:
            # away from the thresholds only the periodic image can differ
            assert np.allclose(xs_c, coords, rtol=0, atol=4 * band), f"domain {R}: image differs"
        total_band += n_band
    return total_band


def copy_offsets(plan, grid):
    """For each slot: owner domain, and the domain steps s_d back to its home."""
    owner = np.zeros(plan.n_slots, dtype=np.int64)
    for D in range(len(plan.base)):
        owner[plan.base[D]:plan.base[D] + plan.ntotal[D]] = D
    home_slot = np.full(int(plan.slot_ids.max()) + 1 if plan.n_slots else 0, -1, dtype=np.int64)
    for D in range(len(plan.base)):
        b, nh = int(plan.base[D]), int(plan.nhome[D])
        home_slot[plan.slot_ids[b:b + nh]] = np.arange(b, b + nh)
    gid = plan.slot_ids.astype(np.int64)
    hs = home_slot[gid]
    hd = owner[hs]
    g = np.asarray(grid)

    def coords(D):
        return np.stack([D % g[0], (D // g[0]) % g[1], D // (g[0] * g[1])], axis=-1)

    steps = np.mod(coords(hd) - coords(owner), g)
    return owner, hs, steps


def force_tree(plan, grid, f_before: np.ndarray, pulses_per_dim) -> np.ndarray:
    """Expected home-slot forces after the reverse pass, by the summation tree.

    Returns float32 [n_slots, 3] holding the expected value at every home slot
    (halo rows are left as NaN).
    """
    owner, hs, steps = copy_offsets(plan, grid)
    m = [int(pulses_per_dim[d]) for d in range(3)]
    n_home_total = int(np.sum(plan.nhome))
    # dense table v[home index, sx, sy, sz, 3], zero where no copy exists
    home_rows = np.concatenate([np.arange(plan.base[D], plan.base[D] + plan.nhome[D])
                                for D in range(len(plan.base))]) if n_home_total else np.zeros(0, np.int64)
    row_of = np.full(plan.n_slots, -1, dtype=np.int64)
    row_of[home_rows] = np.arange(len(home_rows))
    v = np.zeros((len(home_rows), m[0] + 1, m[1] + 1, m[2] + 1, 3), dtype=np.float32)
    r = row_of[hs]
    assert np.all(steps[:, 0] <= m[0]) and np.all(steps[:, 1] <= m[1]) and np.all(steps[:, 2] <= m[2])
    v[r, steps[:, 0], steps[:, 1], steps[:, 2]] = f_before
    # a right-nested chain per dimension, X innermost
    def chain(arr, axis):
        n = arr.shape[axis]
        acc = np.take(arr, n - 1, axis=axis)
        for i in range(n - 2, -1, -1):
            acc = (np.take(arr, i, axis=axis) + acc).astype(np.float32)
        return acc
    t = chain(v, 1)       # over sx -> [rows, sy, sz, 3]
    t = chain(t, 1)       # over sy -> [rows, sz, 3]
    t = chain(t, 1)       # over sz -> [rows, 3]
    out = np.full((plan.n_slots, 3), np.nan, dtype=np.float32)
    out[home_rows] = t
    return out


def integer_force_expectation(plan, f_before: np.ndarray) -> np.ndarray:
    """Home-slot forces after the reverse pass for integer-valued inputs.

    Every copy's force must reach its atom's home slot exactly once; with
    small integers every partial sum is exact, so the order does not matter.
    """
    # vectorised: sum every slot's force into the home slot of its atom
    owner_home = np.full(int(plan.slot_ids.max()) + 1 if plan.n_slots else 0, -1, dtype=np.int64)
    for D in range(len(plan.base)):
        b, nh = int(plan.base[D]), int(plan.nhome[D])
        owner_home[plan.slot_ids[b:b + nh]] = np.arange(b, b + nh)
    target = owner_home[plan.slot_ids.astype(np.int64)]
    acc = np.zeros((plan.n_slots, 3), dtype=np.float64)
    np.add.at(acc, target, f_before.astype(np.float64))
    return acc
