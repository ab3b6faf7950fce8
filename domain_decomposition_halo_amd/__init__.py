"""Staged halo exchange of a domain-decomposed MD step on one MI355X.

Thin ctypes binding over the HIP library `libddh.so` (C ABI in
include/ddh.h). Every function here only marshals arguments: all work of the
map build and of both exchange passes runs in the library's gfx950 kernels.
PyTorch is used for device buffers and streams only.

The library must be built first (`python -m domain_decomposition_halo_amd._build`
or `__graft_entry__.build()`); importing this package without it raises.

Raw entry points carry the C names (ddh_plan_create, ddh_build_maps, ...);
`Plan` wraps them for torch tensors.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libddh.so")

DDH_OK = 0
DDH_EINVAL, DDH_ERANGE, DDH_ECAPACITY, DDH_EHIP, DDH_ETIMEOUT, DDH_ENOTIMPL, DDH_ESTATE = (
    -1, -2, -3, -4, -5, -6, -7)
ERROR_NAMES = {DDH_EINVAL: "DDH_EINVAL", DDH_ERANGE: "DDH_ERANGE", DDH_ECAPACITY: "DDH_ECAPACITY",
               DDH_EHIP: "DDH_EHIP", DDH_ETIMEOUT: "DDH_ETIMEOUT", DDH_ENOTIMPL: "DDH_ENOTIMPL",
               DDH_ESTATE: "DDH_ESTATE"}
DDH_MAX_PULSES = 16
DDH_PASS_COORDS, DDH_PASS_FORCES = 0, 1
DDH_MODE_FUSED, DDH_MODE_PULSE, DDH_MODE_AUTO, DDH_MODE_STAGED, DDH_MODE_GRAPH = 0, 1, 2, 3, 16
DDH_AUTO_FUSED_MAX = 200000
DDH_TUNE_CHUNK, DDH_TUNE_GRID, DDH_TUNE_SPIN_LIMIT, DDH_TUNE_FORCE_TIMEOUT, DDH_TUNE_REFINED_WAITS = (
    1, 2, 3, 4, 5)
DDH_TUNE_TRACE = 6
DDH_TUNE_BLOCK = 7
DDH_TUNE_STATIC_FIRST = 8
DDH_TUNE_FLAGS = 9
DDH_TUNE_NARROW_MAPS = 10
DDH_TUNE_WAVE_CHUNKS = 11
DDH_TUNE_HOME_SORT = 12
DDH_TUNE_EXIT_PUBLISH = 13
DDH_TUNE_PAD_MAPS = 14
DDH_TUNE_HEADS_FIRST = 15
DDH_TUNE_LDS_STAGE = 16
TRACE_RECORDS = 64
TRACE_EVENTS = {1: "start", 2: "claim", 3: "head", 4: "waited", 5: "chunk", 6: "publish", 7: "exit"}

# every symbol declared in include/ddh.h
EXPORTS = ("ddh_plan_create", "ddh_plan_destroy", "ddh_last_error", "ddh_build_maps", "ddh_query",
           "ddh_domain_info", "ddh_pulse_info", "ddh_copy_maps", "ddh_local_ids",
           "ddh_flags", "ddh_copy_flags", "ddh_wait_flag",
           "ddh_gather_home", "ddh_exchange_coords", "ddh_exchange_forces",
           "ddh_exchange_step", "ddh_exchange_staged_static", "ddh_set_mode", "ddh_check",
           "ddh_tune")
DDH_STATIC_STAGE_BYTES = 64 << 20


class ddh_params(ctypes.Structure):
    _fields_ = [("ndom", ctypes.c_int32 * 3), ("box", ctypes.c_float * 3), ("rc", ctypes.c_float),
                ("cell", ctypes.c_float), ("flags", ctypes.c_int32)]


class ddh_layout(ctypes.Structure):
    _fields_ = [("n_domains", ctypes.c_int32), ("n_pulses", ctypes.c_int32),
                ("n_slots", ctypes.c_int64), ("n_halo", ctypes.c_int64),
                ("n_atoms", ctypes.c_int32),
                ("pulse_dim", ctypes.c_int32 * DDH_MAX_PULSES),
                ("pulse_k", ctypes.c_int32 * DDH_MAX_PULSES)]


class DDHError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {ERROR_NAMES.get(code, code)}")
        self.code = code


def _load():
    # torch brings its own HIP runtime (SONAME libamdhip64.so.7). Loading it
    # first makes libddh.so bind to that same runtime, so device pointers and
    # streams from torch are valid in the library; loading libddh.so first
    # would pull a second runtime into the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          "(python -m domain_decomposition_halo_amd._build)")
    lib = ctypes.CDLL(LIB_PATH)
    V, I32, I64, P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "ddh_plan_create": ([ctypes.POINTER(ddh_params), ctypes.POINTER(V)], ctypes.c_int),
        "ddh_plan_destroy": ([V], None),
        "ddh_last_error": ([], ctypes.c_char_p),
        "ddh_build_maps": ([V, P, I32, V], ctypes.c_int),
        "ddh_query": ([V, ctypes.POINTER(ddh_layout)], ctypes.c_int),
        "ddh_domain_info": ([V, I32, ctypes.POINTER(I64), ctypes.POINTER(I32),
                             ctypes.POINTER(I32)], ctypes.c_int),
        "ddh_pulse_info": ([V, I32, I32] + [ctypes.POINTER(I32)] * 5, ctypes.c_int),
        "ddh_copy_maps": ([V, P, I64, V], ctypes.c_int),
        "ddh_local_ids": ([V, P, I64, V], ctypes.c_int),
        "ddh_flags": ([V, ctypes.POINTER(ctypes.c_void_p)], ctypes.c_int),
        "ddh_copy_flags": ([V, P, V], ctypes.c_int),
        "ddh_wait_flag": ([V, I32, I32, ctypes.c_uint32, V], ctypes.c_int),
        "ddh_gather_home": ([V, P, P, I64, V], ctypes.c_int),
        "ddh_exchange_coords": ([V, P, I64, V], ctypes.c_int),
        "ddh_exchange_forces": ([V, P, I64, V], ctypes.c_int),
        "ddh_exchange_step": ([V, P, P, I64, V], ctypes.c_int),
        "ddh_exchange_staged_static": ([V, P, P, I64, V], ctypes.c_int),
        "ddh_set_mode": ([V, I32], ctypes.c_int),
        "ddh_check": ([V, V], ctypes.c_int),
        "ddh_tune": ([V, I32, I64], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()
for _name in EXPORTS:
    globals()[_name] = getattr(_lib, _name)


def last_error() -> str:
    return (_lib.ddh_last_error() or b"").decode()


def _check(code: int, what: str):
    if code != DDH_OK:
        raise DDHError(code, f"{what} ({last_error()})")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev_ptr(t, dtype_name: str, what: str):
    """Device pointer of a contiguous CUDA tensor, with its slot capacity."""
    import torch
    want = {"float32": torch.float32, "int32": torch.int32}[dtype_name]
    if not (t.is_cuda and t.dtype == want and t.is_contiguous()):
        raise DDHError(DDH_EINVAL, f"{what}: need a contiguous {dtype_name} CUDA tensor")
    return ctypes.c_void_p(t.data_ptr())


class Plan:
    """One decomposition: maps on the device, exchange calls on torch tensors."""

    def __init__(self, grid, box, rc, cell=0.5):
        prm = ddh_params()
        for d in range(3):
            prm.ndom[d] = int(grid[d])
            prm.box[d] = float(box[d])
        prm.rc = float(rc)
        prm.cell = float(cell)
        prm.flags = 0
        h = ctypes.c_void_p()
        _check(_lib.ddh_plan_create(ctypes.byref(prm), ctypes.byref(h)), "ddh_plan_create")
        self._h = h
        self.grid = tuple(int(v) for v in grid)

    # -- build and layout
    def build_maps(self, x_global, stream=None):
        if x_global.dim() != 2 or x_global.shape[1] != 3:
            raise DDHError(DDH_EINVAL, "build_maps: x_global must be an (n, 3) tensor")
        _check(_lib.ddh_build_maps(self._h, _dev_ptr(x_global, "float32", "x_global"),
                                   int(x_global.shape[0]), _stream(stream)), "ddh_build_maps")
        return self.layout()

    def layout(self) -> dict:
        lay = ddh_layout()
        _check(_lib.ddh_query(self._h, ctypes.byref(lay)), "ddh_query")
        P = lay.n_pulses
        return dict(n_domains=lay.n_domains, n_pulses=P, n_slots=lay.n_slots,
                    n_halo=lay.n_halo, n_atoms=lay.n_atoms,
                    pulses=[(lay.pulse_dim[p], lay.pulse_k[p]) for p in range(P)])

    def domain_info(self, dom: int):
        b, nh, nt = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.ddh_domain_info(self._h, dom, ctypes.byref(b), ctypes.byref(nh),
                                    ctypes.byref(nt)), "ddh_domain_info")
        return b.value, nh.value, nt.value

    def pulse_info(self, dom: int, pulse: int):
        v = [ctypes.c_int32() for _ in range(5)]
        _check(_lib.ddh_pulse_info(self._h, dom, pulse, *[ctypes.byref(x) for x in v]),
               "ddh_pulse_info")
        return tuple(x.value for x in v)  # send, split, recv_dom, recv_offset, shift

    def copy_maps(self, out, stream=None):
        _check(_lib.ddh_copy_maps(self._h, _dev_ptr(out, "int32", "maps"), out.numel(),
                                  _stream(stream)), "ddh_copy_maps")
        return out

    def flags_address(self) -> int:
        """Device address of the per-pulse completion flags (uint32[2 * 16])."""
        ptr = ctypes.c_void_p()
        _check(_lib.ddh_flags(self._h, ctypes.byref(ptr)), "ddh_flags")
        return ptr.value or 0

    def copy_flags(self, out, stream=None):
        """Snapshot of the flags into a device int32 tensor of >= 32 words (the
        words are uint32 counts; read them modulo 2**32)."""
        if out.numel() < 2 * DDH_MAX_PULSES:
            raise ValueError("copy_flags: the tensor needs 2 * DDH_MAX_PULSES words")
        _check(_lib.ddh_copy_flags(self._h, _dev_ptr(out, "int32", "flags"), _stream(stream)),
               "ddh_copy_flags")

    def wait_flag(self, pass_kind: int, pulse: int, epoch: int, stream=None):
        """Enqueue on stream a device wait for pulse `pulse` of a pass to reach `epoch`."""
        _check(_lib.ddh_wait_flag(self._h, pass_kind, pulse, epoch & 0xFFFFFFFF, _stream(stream)),
               "ddh_wait_flag")

    def local_ids(self, out, stream=None):
        _check(_lib.ddh_local_ids(self._h, _dev_ptr(out, "int32", "ids"), out.numel(),
                                  _stream(stream)), "ddh_local_ids")
        return out

    # -- exchanges
    def gather_home(self, x_global, x_local, stream=None):
        if x_global.dim() != 2 or x_global.shape[1] != 3 or \
                x_global.shape[0] < self.layout()["n_atoms"]:
            raise DDHError(DDH_EINVAL, "gather_home: x_global must hold every atom of the plan")
        _check(_lib.ddh_gather_home(self._h, _dev_ptr(x_global, "float32", "x_global"),
                                    _dev_ptr(x_local, "float32", "x_local"),
                                    x_local.numel() // 3, _stream(stream)), "ddh_gather_home")

    def exchange_coords(self, x_local, stream=None):
        _check(_lib.ddh_exchange_coords(self._h, _dev_ptr(x_local, "float32", "x_local"),
                                        x_local.numel() // 3, _stream(stream)),
               "ddh_exchange_coords")

    def exchange_forces(self, f_local, stream=None):
        _check(_lib.ddh_exchange_forces(self._h, _dev_ptr(f_local, "float32", "f_local"),
                                        f_local.numel() // 3, _stream(stream)),
               "ddh_exchange_forces")

    def exchange_step(self, x_local, f_local, stream=None):
        cap = min(x_local.numel(), f_local.numel()) // 3
        _check(_lib.ddh_exchange_step(self._h, _dev_ptr(x_local, "float32", "x_local"),
                                      _dev_ptr(f_local, "float32", "f_local"), cap,
                                      _stream(stream)), "ddh_exchange_step")

    def exchange_staged_static(self, x_local=None, f_local=None, stream=None):
        """The host-orchestrated exchange with its staging in the library's
        static device buffer (no allocation); either array may be None."""
        caps = [t.numel() // 3 for t in (x_local, f_local) if t is not None]
        xp = _dev_ptr(x_local, "float32", "x_local") if x_local is not None else None
        fp = _dev_ptr(f_local, "float32", "f_local") if f_local is not None else None
        _check(_lib.ddh_exchange_staged_static(self._h, xp, fp, min(caps) if caps else 0,
                                               _stream(stream)), "ddh_exchange_staged_static")

    # -- control
    def set_mode(self, mode: int):
        _check(_lib.ddh_set_mode(self._h, int(mode)), "ddh_set_mode")

    def tune(self, key: int, value: int):
        _check(_lib.ddh_tune(self._h, int(key), int(value)), "ddh_tune")

    def check(self, stream=None) -> int:
        """Wait for the stream; return DDH_OK or the device error code."""
        code = _lib.ddh_check(self._h, _stream(stream))
        if code not in (DDH_OK, DDH_ETIMEOUT):
            _check(code, "ddh_check")
        return code

    def close(self):
        if getattr(self, "_h", None):
            _lib.ddh_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
