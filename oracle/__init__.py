"""CPU oracle of the staged halo exchange (ctypes wrapper over ddh_oracle.c).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this package. The HIP library and its Python
binding never import it, and the two share no code: the only module both sides
use is the seeded input generator (`workloads`), which holds none of the
exchange's arithmetic.

The oracle follows the staged exchange of the NVIDIA guide "A Practical Guide
to GPU-Initiated Communication for Molecular Dynamics at Scale" (sections
"Accelerating GROMACS using Device-initiated Remote Memory Access" and "From
MPI baseline to optimized GPU-native halo exchange"): coordinates pulse by
pulse Z -> Y -> X with relay, forces in reverse order with scatter-add. Every
reading taken where the guide is silent is listed at the top of the C source.

Every function is pinned by tests that do not reuse the oracle's code:
brute-force halo sets and coordinates on dyadic boxes, closed forms for pulse
counts and slab sizes, force conservation, integer-force exactness, and the
reverse-pulse summation tree for non-integer forces.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ddh_oracle.c")
_LIB = os.path.join(_HERE, "libddh_oracle.so")

OK, EINVAL, ERANGE, ENOMEM = 0, -1, -2, -3
_ERRORS = {EINVAL: "EINVAL", ERANGE: "ERANGE", ENOMEM: "ENOMEM"}


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle error {_ERRORS.get(code, code)}")
        self.code = code


def build() -> str:
    """Compile the oracle with gcc (plain C99, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.ddho_build.argtypes = [P, I, P, P, F, F, ctypes.POINTER(ctypes.c_void_p)]
    lib.ddho_build.restype = I
    lib.ddho_schedule.argtypes = [P, P, F, P, P]
    lib.ddho_schedule.restype = I
    lib.ddho_free.argtypes = [P]
    lib.ddho_free.restype = None
    for name in ("ddho_ndomains", "ddho_npulses"):
        getattr(lib, name).argtypes = [P]
        getattr(lib, name).restype = I
    lib.ddho_nslots.argtypes = [P]
    lib.ddho_nslots.restype = I64
    lib.ddho_pulse_table.argtypes = [P, P, P]
    lib.ddho_bounds.argtypes = [P, I, P]
    lib.ddho_domain_table.argtypes = [P, P, P, P]
    lib.ddho_item_table.argtypes = [P, P, P, P, P, P]
    lib.ddho_maps.argtypes = [P, P]
    lib.ddho_slot_ids.argtypes = [P, P]
    lib.ddho_coords.argtypes = [P, P]
    lib.ddho_exchange_coords.argtypes = [P, P, I]
    lib.ddho_exchange_forces.argtypes = [P, P, I]
    for name in ("ddho_pulse_table", "ddho_bounds", "ddho_domain_table", "ddho_item_table",
                 "ddho_maps", "ddho_slot_ids", "ddho_coords", "ddho_exchange_coords",
                 "ddho_exchange_forces"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def schedule(grid, box, rc):
    """Pulse schedule [(dim, k), ...] for a grid/box/cutoff (dim 0 = X)."""
    lib = _load()
    nd = np.asarray(grid, dtype=np.int32)
    bx = np.asarray(box, dtype=np.float32)
    pdim = np.zeros(64, dtype=np.int32)
    pk = np.zeros(64, dtype=np.int32)
    P = lib.ddho_schedule(_ptr(nd), _ptr(bx), ctypes.c_float(rc), _ptr(pdim), _ptr(pk))
    if P < 0:
        raise OracleError(P)
    return [(int(pdim[p]), int(pk[p])) for p in range(P)]


class OraclePlan:
    """The oracle's exchange plan for one set of positions.

    Attributes (numpy, host):
      pulses      [(dim, k)] global pulse order, dim 0 = X, 1 = Y, 2 = Z
      bounds      three float32 arrays of domain boundaries
      base, nhome, ntotal   per domain (domain D = ix + nx*(iy + ny*iz))
      send, split, recv, roff, shift   [D, P] per (sender, pulse)
      maps        dict (S, p) -> int32 sender-local slot indices
      slot_ids    int32 [n_slots] global atom id per slot
      x_local     float32 [n_slots, 3] coordinates after the first pass
    """

    def __init__(self, x_global, grid, box, rc, cell=0.5):
        lib = _load()
        xg = np.ascontiguousarray(x_global, dtype=np.float32)
        assert xg.ndim == 2 and xg.shape[1] == 3
        self.grid = tuple(int(v) for v in grid)
        self.box = tuple(float(np.float32(v)) for v in box)
        self.rc = float(np.float32(rc))
        self.cell = float(np.float32(cell))
        nd = np.asarray(self.grid, dtype=np.int32)
        bx = np.asarray(self.box, dtype=np.float32)
        h = ctypes.c_void_p()
        t0 = time.perf_counter()
        rcode = lib.ddho_build(_ptr(xg), xg.shape[0], _ptr(nd), _ptr(bx), ctypes.c_float(self.rc),
                               ctypes.c_float(self.cell), ctypes.byref(h))
        self.build_seconds = time.perf_counter() - t0
        if rcode != OK:
            raise OracleError(rcode)
        self._h = h
        self._lib = lib
        D = lib.ddho_ndomains(h)
        P = lib.ddho_npulses(h)
        self.n_domains, self.n_pulses = D, P
        self.n_slots = int(lib.ddho_nslots(h))
        pdim = np.zeros(max(P, 1), dtype=np.int32)
        pk = np.zeros(max(P, 1), dtype=np.int32)
        lib.ddho_pulse_table(h, _ptr(pdim), _ptr(pk))
        self.pulses = [(int(pdim[p]), int(pk[p])) for p in range(P)]
        self.bounds = []
        for d in range(3):
            b = np.zeros(self.grid[d] + 1, dtype=np.float32)
            lib.ddho_bounds(h, d, _ptr(b))
            self.bounds.append(b)
        self.base = np.zeros(D, dtype=np.int64)
        self.nhome = np.zeros(D, dtype=np.int32)
        self.ntotal = np.zeros(D, dtype=np.int32)
        lib.ddho_domain_table(h, _ptr(self.base), _ptr(self.nhome), _ptr(self.ntotal))
        tabs = [np.zeros(max(D * P, 1), dtype=np.int32) for _ in range(5)]
        lib.ddho_item_table(h, *[_ptr(t) for t in tabs])
        self.send, self.split, self.recv, self.roff, self.shift = [
            t[:D * P].reshape(D, P) for t in tabs]
        flat = np.zeros(max(int(self.send.sum()), 1), dtype=np.int32)
        lib.ddho_maps(h, _ptr(flat))
        self.maps = {}
        pos = 0
        for S in range(D):
            for p in range(P):
                n = int(self.send[S, p])
                self.maps[(S, p)] = flat[pos:pos + n].copy()
                pos += n
        self.slot_ids = np.zeros(max(self.n_slots, 1), dtype=np.int32)[:self.n_slots]
        lib.ddho_slot_ids(h, _ptr(self.slot_ids))
        self.x_local = np.zeros((self.n_slots, 3), dtype=np.float32)
        lib.ddho_coords(h, _ptr(self.x_local))

    @property
    def halo_atoms(self) -> int:
        """Halo atoms moved per pass: the sum of every (domain, pulse) send size."""
        return int(self.send.sum())

    def domain_of_slot(self) -> np.ndarray:
        owner = np.zeros(self.n_slots, dtype=np.int32)
        for D in range(self.n_domains):
            owner[self.base[D]:self.base[D] + self.ntotal[D]] = D
        return owner

    def exchange_coords(self, x_local: np.ndarray, nthreads: int = 1) -> np.ndarray:
        """In-place coordinate pass on a flat [n_slots, 3] float32 array."""
        assert x_local.dtype == np.float32 and x_local.flags.c_contiguous
        assert x_local.shape == (self.n_slots, 3)
        self._lib.ddho_exchange_coords(self._h, _ptr(x_local), int(nthreads))
        return x_local

    def exchange_forces(self, f_local: np.ndarray, nthreads: int = 1) -> np.ndarray:
        """In-place force pass on a flat [n_slots, 3] float32 array."""
        assert f_local.dtype == np.float32 and f_local.flags.c_contiguous
        assert f_local.shape == (self.n_slots, 3)
        self._lib.ddho_exchange_forces(self._h, _ptr(f_local), int(nthreads))
        return f_local

    def home_coords(self, x_global: np.ndarray) -> np.ndarray:
        """Flat array with home slots filled from x_global and halo slots zero."""
        out = np.zeros((self.n_slots, 3), dtype=np.float32)
        for D in range(self.n_domains):
            b, n = int(self.base[D]), int(self.nhome[D])
            out[b:b + n] = x_global[self.slot_ids[b:b + n]]
        return out

    def close(self):
        if getattr(self, "_h", None):
            self._lib.ddho_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
