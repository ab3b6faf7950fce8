"""Seeded synthetic inputs for the staged halo exchange.

This module is shared by the CPU oracle's tests, the GPU tests and the bench.
It holds the workload table and the random generators only: no part of the
exchange itself (no domain assignment, no slab selection, no shifts, no adds)
lives here, so neither implementation borrows arithmetic from the other.

The five workloads stand in for the water-ethanol systems (45k to 23M atoms)
that the guide ("A Practical Guide to GPU-Initiated Communication for
Molecular Dynamics at Scale", section "A leap in scaling performance")
benchmarks on; those systems are not available, so each workload keeps a
water-like density of about 100 atoms/nm^3 and draws uniform positions.

Recipe (fixed, so every run and every side sees the same bytes):
  * workload k (1-based) draws positions from numpy default_rng(1000 + k):
    uniform(0, L) in float64 with L the float32 box edge, rounded to float32;
    a coordinate that rounds up to L is wrapped to 0 so all lie in [0, L).
  * per-slot forces are drawn after the layout is known, from
    default_rng(2000 + k): normal(0, 10) as float32, one xyz triple per local
    slot in slot order ("~N(0,100)" read as variance 100).
  * integer forces for the exactness checks: integers in [-1000, 1000].
  * lattice positions for the exact (dyadic) checks: multiples of 2^-12 nm.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    key: int            # 1-based index used for the seeds
    name: str
    n_atoms: int
    box: tuple          # box edges (nm), x, y, z
    grid: tuple         # virtual domains per dimension, x, y, z
    rc: float           # cutoff (nm)
    cell: float = 0.5   # edge of the sort cells for home atoms (nm)

    @property
    def box32(self):
        return tuple(float(np.float32(v)) for v in self.box)

    def params(self):
        """Plain dict form accepted by both the oracle wrapper and the binding."""
        return dict(grid=tuple(self.grid), box=self.box32,
                    rc=float(np.float32(self.rc)), cell=float(np.float32(self.cell)))


WORKLOADS = {
    1: Workload(1, "3k_2x1x1", 3_000, (3.0, 3.0, 3.0), (2, 1, 1), 0.9),
    2: Workload(2, "96k_2x2x2", 96_000, (9.86, 9.86, 9.86), (2, 2, 2), 1.0),
    3: Workload(3, "1M_4x4x4", 1_000_000, (21.5, 21.5, 21.5), (4, 4, 4), 1.2),
    4: Workload(4, "384k_16x4x4", 384_000, (15.66, 15.66, 15.66), (16, 4, 4), 1.2),
    5: Workload(5, "12M_8x8x8", 12_000_000, (49.3, 49.3, 49.3), (8, 8, 8), 1.2),
}


def positions(w: Workload) -> np.ndarray:
    """float32 [N, 3] positions of workload `w`, all inside [0, L)."""
    rng = np.random.default_rng(1000 + w.key)
    L = np.asarray(w.box32, dtype=np.float64)
    x = rng.uniform(0.0, 1.0, size=(w.n_atoms, 3)) * L
    x32 = x.astype(np.float32)
    L32 = L.astype(np.float32)
    x32 = np.where(x32 >= L32, np.float32(0.0), x32)
    return np.ascontiguousarray(x32, dtype=np.float32)


def forces(w: Workload, n_slots: int) -> np.ndarray:
    """float32 [n_slots, 3] per-slot forces, normal with sigma 10."""
    rng = np.random.default_rng(2000 + w.key)
    return np.ascontiguousarray(rng.normal(0.0, 10.0, size=(n_slots, 3)).astype(np.float32))


def integer_forces(n_slots: int, seed: int) -> np.ndarray:
    """float32 [n_slots, 3] small integers: every partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    return np.ascontiguousarray(rng.integers(-1000, 1001, size=(n_slots, 3)).astype(np.float32))


def lattice_positions(n_atoms: int, box, seed: int, frac_bits: int = 12) -> np.ndarray:
    """float32 [N, 3] positions on a 2^-frac_bits nm lattice inside [0, L).

    With dyadic box edges and cutoffs every subtraction, comparison and
    periodic shift of such coordinates is exact in fp32, so a float64
    brute force agrees with the staged exchange with no tie band.
    """
    rng = np.random.default_rng(seed)
    scale = float(1 << frac_bits)
    cols = []
    for L in box:
        n = int(round(L * scale))
        cols.append(rng.integers(0, n, size=n_atoms).astype(np.float64) / scale)
    return np.ascontiguousarray(np.stack(cols, axis=1).astype(np.float32))


def uniform_positions(n_atoms: int, box, seed: int) -> np.ndarray:
    """float32 [N, 3] uniform positions in [0, L) for ad-hoc sizes (tests)."""
    rng = np.random.default_rng(seed)
    L = np.asarray([float(np.float32(v)) for v in box], dtype=np.float64)
    x32 = (rng.uniform(0.0, 1.0, size=(n_atoms, 3)) * L).astype(np.float32)
    x32 = np.where(x32 >= L.astype(np.float32), np.float32(0.0), x32)
    return np.ascontiguousarray(x32, dtype=np.float32)
