"""Python binding of libgc: all-pairs angular-separation histograms on an MI355X.

The computation is the one of "CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080",
section "The problem": DD, DR and RR histograms of the angle between the radius
vectors of every ordered pair of galaxies, and the Landy-Szalay estimator
omega = (DD - 2 DR + RR) / RR.

Every function here marshals torch tensors (device memory, current HIP stream) into
the C ABI declared in include/gc.h; all arithmetic runs in the library's HIP kernels.
There is no CPU fallback: without the built library every call raises.

Typical use::

    import torch, two_point_angular_amd as gc
    pd = gc.prepare(ra_d, dec_d)            # fp32 arcmin tensors on cuda
    pr = gc.prepare(ra_r, dec_r)
    dd, dr, rr = gc.histogram_dd_dr_rr(pd, len(ra_d), pr, len(ra_r), 720, 0.25)
    w = gc.omega(dd, dr, rr, len(ra_d), len(ra_r))

Histograms are returned as int64 tensors holding the library's uint64 counts (all
counts here are below 2^63).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = ["GCError", "Tuning", "library_path", "load", "prepared_bytes", "workspace_bytes",
           "prepare", "histogram_dd_dr_rr", "histogram_totals", "omega", "eval_angle_core",
           "ceiling_valu", "ceiling_lds_atomic",
           "MAX_BINS", "MAX_GALAXIES", "ALIGNMENT"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "lib", "libgc.so")

MAX_BINS = 8192
MAX_GALAXIES = 2147483647
ALIGNMENT = 256

GC_OK = 0
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported size", 3: "workspace too small",
           4: "device error", 5: "file input/output error"}


class GCError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{where}: {_STATUS.get(status, 'unknown')} (status {status})"
        if status == 4:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


class _Tuning(ctypes.Structure):
    _fields_ = [("dot_precision", ctypes.c_int32), ("i_per_lane", ctypes.c_int32),
                ("blocks_per_cu", ctypes.c_int32), ("shared_histogram", ctypes.c_int32),
                ("span_kernel", ctypes.c_int32), ("fast_core", ctypes.c_int32),
                ("flush_interval", ctypes.c_int64), ("hist_columns", ctypes.c_int32),
                ("waves_per_group", ctypes.c_int32), ("l1_share", ctypes.c_int32),
                ("reserved_", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("core", "dot_precision", "i_per_lane", "hist_columns", "waves_per_group",
                                              "l1_share", "shared_histogram", "blocks_per_cu", "workgroups",
                                              "lds_bytes")] + \
               [("flush_interval", ctypes.c_int64), ("always_recheck", ctypes.c_int32), ("lut_m", ctypes.c_int32)]


@dataclass
class Tuning:
    """Launch-plan overrides (0 = library's choice); results do not depend on them."""

    dot_precision: int = 0
    i_per_lane: int = 0
    blocks_per_cu: int = 0
    flush_interval: int = 0
    shared_histogram: int = 0
    span_kernel: int = 0
    fast_core: int = 0
    hist_columns: int = 0
    waves_per_group: int = 0
    l1_share: int = 0

    def _c(self) -> _Tuning:
        return _Tuning(self.dot_precision, self.i_per_lane, self.blocks_per_cu, self.shared_histogram,
                       self.span_kernel, self.fast_core, self.flush_interval, self.hist_columns,
                       self.waves_per_group, self.l1_share, 0)


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libgc.so (built by two_point_angular_amd.build); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libgc.so not built ({_LIB_PATH}); run python -m two_point_angular_amd.build")
    # torch first: it ships its own HIP runtime, and libgc must bind to that one.  Loaded the
    # other way round, the process holds two runtimes and libgc's calls fail with
    # hipErrorNoDevice.
    _torch()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "gc_prepared_bytes": (sz, [i64]),
        "gc_prepare": (i32, [vp, vp, i64, vp, vp]),
        "gc_workspace_bytes": (sz, [i32]),
        "gc_histogram_dd_dr_rr": (i32, [vp, i64, vp, i64, i32, ctypes.c_double, vp, vp, vp, vp, sz, vp]),
        "gc_histogram_dd_dr_rr_tuned": (i32, [vp, i64, vp, i64, i32, ctypes.c_double, vp, vp, vp, vp, sz,
                                              ctypes.POINTER(_Tuning), vp]),
        "gc_histogram_part": (i32, [vp, i64, vp, i64, i32, ctypes.c_double, i64, i64, vp, vp, vp, vp, sz,
                                    ctypes.POINTER(_Tuning), vp]),
        "gc_histogram_dd_dr_rr_noalloc": (i32, [vp, i64, vp, i64, i32, ctypes.c_double, vp, vp, vp, vp]),
        "gc_histogram_totals": (i32, [vp, vp, vp, i32, vp, vp]),
        "gc_omega": (i32, [vp, vp, vp, i32, i64, i64, vp, vp]),
        "gc_eval_angle_core": (i32, [vp, vp, i64, i32, ctypes.c_double, i32, vp, vp, vp, vp, vp, sz, vp]),
        "gc_eval_dot_mfma": (i32, [vp, vp, vp, vp, vp, vp, i64, vp, vp]),
        "gc_ladder_workspace_bytes": (sz, [i64, i64]),
        "gc_ladder_histogram": (i32, [i32, i32, i32, i32, vp, vp, i64, vp, vp, i64, i32, ctypes.c_double, vp, vp,
                                      vp, vp, sz, vp]),
        "gc_catalog_count": (i32, [ctypes.c_char_p, ctypes.POINTER(i64)]),
        "gc_catalog_read": (i32, [ctypes.c_char_p, vp, vp, i64, ctypes.POINTER(i64)]),
        "gc_omega_write": (i32, [ctypes.c_char_p, vp, vp, vp, vp, i32, ctypes.c_double]),
        "gc_ceiling_sink_bytes": (sz, []),
        "gc_ceiling_valu": (i32, [i32, i64, vp, sz, ctypes.POINTER(ctypes.c_uint64), vp]),
        "gc_ceiling_lds_atomic": (i32, [i32, i32, i64, vp, sz, ctypes.POINTER(ctypes.c_uint64), vp]),
        "gc_launch_plan": (i32, [i64, i64, i32, ctypes.c_double, ctypes.POINTER(_Tuning), ctypes.POINTER(_Plan)]),
        "gc_ceiling_l1": (i32, [i32, i32, i64, vp, sz, ctypes.POINTER(ctypes.c_uint64), vp]),
        "gc_ceiling_lds": (i32, [i32, i32, i32, i32, i32, i64, vp, sz, ctypes.POINTER(ctypes.c_uint64), vp]),
        "gc_status_string": (ctypes.c_char_p, [i32]),
        "gc_last_device_error": (ctypes.c_int, []),
        "gc_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != GC_OK:
        raise GCError(status, where, load().gc_last_device_error() if status == 4 else 0)


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _buf(t, name, dtype, min_numel=0, device=None, optional=False, shape=None):
    """Check one tensor argument before its address goes to the library, which cannot see sizes:
    dtype and contiguity (TypeError), then element count or shape (ValueError).  Returns the
    tensor; None passes only when optional.  Where the tensors live is checked for all of a
    call's arguments at once, after these (_on_gpu), so these checks run on any machine."""
    torch = _torch()
    if t is None:
        if optional:
            return None
        raise TypeError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be a {dtype} tensor, got {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")
    return t


def _on_gpu(**tensors):
    """Every given tensor (None skipped) is a GPU tensor (TypeError), all on one device
    (ValueError)."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")


def _need(t, dtype, name, device=None):
    _buf(t, name, dtype)
    _on_gpu(**{name: t})
    return t


def prepared_bytes(n: int) -> int:
    return int(load().gc_prepared_bytes(int(n)))


def workspace_bytes(nbins: int) -> int:
    return int(load().gc_workspace_bytes(int(nbins)))


def _count(v, name, limit):
    v = int(v)
    if v < 0 or v > limit:
        raise ValueError(f"{name} = {v} outside [0, {limit}]")
    return v


def _bins(nbins):
    nbins = int(nbins)
    if nbins < 1 or nbins > MAX_BINS:
        raise ValueError(f"nbins = {nbins} outside [1, {MAX_BINS}]")
    return nbins


def prepare(ra_arcmin, dec_arcmin, out=None, stream=None):
    """Prepared (unit-vector) form of one catalog, as an opaque uint8 device tensor."""
    torch = _torch()
    _buf(ra_arcmin, "ra_arcmin", torch.float32)
    n = _count(ra_arcmin.numel(), "n", MAX_GALAXIES)
    _buf(dec_arcmin, "dec_arcmin", torch.float32)
    if dec_arcmin.numel() != n:
        raise ValueError("ra and dec must have the same length")
    nbytes = prepared_bytes(n)
    _buf(out, "out", torch.uint8, nbytes, optional=True)
    _on_gpu(ra_arcmin=ra_arcmin, dec_arcmin=dec_arcmin, out=out)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=ra_arcmin.device)
    _check(load().gc_prepare(_ptr(ra_arcmin), _ptr(dec_arcmin), n, _ptr(out), _stream(stream)), "gc_prepare")
    return out


def _job_args(prep_d, n_d, prep_r, n_r, nbins, out, workspace, out_required):
    """Checked arguments of a histogram call: the prepared catalogs hold prepared_bytes(n) bytes
    (either may be absent when its n is 0), out is a (3, nbins) int64 tensor, the workspace holds
    workspace_bytes(nbins) bytes, all on one device."""
    torch = _torch()
    n_d = _count(n_d, "n_d", MAX_GALAXIES)
    n_r = _count(n_r, "n_r", MAX_GALAXIES)
    nbins = _bins(nbins)
    _buf(prep_d, "prep_d", torch.uint8, prepared_bytes(n_d), optional=n_d == 0)
    _buf(prep_r, "prep_r", torch.uint8, prepared_bytes(n_r), optional=n_r == 0)
    _buf(out, "out", torch.int64, shape=(3, nbins), optional=not out_required)
    _buf(workspace, "workspace", torch.uint8, workspace_bytes(nbins), optional=True)
    _on_gpu(prep_d=prep_d, prep_r=prep_r, out=out, workspace=workspace)
    ref = next((t for t in (prep_d, prep_r, out, workspace) if t is not None), None)
    if ref is None:
        raise TypeError("no device tensor given (prepared catalogs, out or workspace)")
    if out is None:
        out = torch.empty((3, nbins), dtype=torch.int64, device=ref.device)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(nbins), dtype=torch.uint8, device=ref.device)
    return n_d, n_r, nbins, out, workspace


def histogram_dd_dr_rr(prep_d, n_d: int, prep_r, n_r: int, nbins: int, bin_width_deg: float,
                       out=None, workspace=None, tuning: Tuning | None = None, stream=None):
    """(DD, DR, RR) int64 device tensors of nbins counts each (rows of `out`)."""
    n_d, n_r, nbins, out, workspace = _job_args(prep_d, n_d, prep_r, n_r, nbins, out, workspace, False)
    dd, dr, rr = out[0], out[1], out[2]
    args = [_ptr(prep_d), n_d, _ptr(prep_r), n_r, nbins, float(bin_width_deg),
            _ptr(dd), _ptr(dr), _ptr(rr), _ptr(workspace), workspace.numel()]
    lib = load()
    if tuning is None:
        st = lib.gc_histogram_dd_dr_rr(*args, _stream(stream))
    else:
        tc = tuning._c()
        st = lib.gc_histogram_dd_dr_rr_tuned(*args, ctypes.byref(tc), _stream(stream))
    _check(st, "gc_histogram_dd_dr_rr")
    return dd, dr, rr


def histogram_dd_dr_rr_noalloc(prep_d, n_d: int, prep_r, n_r: int, nbins: int, bin_width_deg: float, out,
                               stream=None):
    """histogram_dd_dr_rr with the library's own per-GPU scratch (gc_histogram_dd_dr_rr_noalloc):
    nothing is allocated, so `out` ((3, nbins) int64 device tensor) is required.  Calls that
    overlap on one GPU share that scratch and race."""
    torch = _torch()
    n_d = _count(n_d, "n_d", MAX_GALAXIES)
    n_r = _count(n_r, "n_r", MAX_GALAXIES)
    nbins = _bins(nbins)
    _buf(prep_d, "prep_d", torch.uint8, prepared_bytes(n_d), optional=n_d == 0)
    _buf(prep_r, "prep_r", torch.uint8, prepared_bytes(n_r), optional=n_r == 0)
    _buf(out, "out", torch.int64, shape=(3, nbins))
    _on_gpu(prep_d=prep_d, prep_r=prep_r, out=out)
    dd, dr, rr = out[0], out[1], out[2]
    _check(load().gc_histogram_dd_dr_rr_noalloc(_ptr(prep_d), n_d, _ptr(prep_r), n_r, nbins, float(bin_width_deg),
                                                _ptr(dd), _ptr(dr), _ptr(rr), _stream(stream)),
           "gc_histogram_dd_dr_rr_noalloc")
    return dd, dr, rr


MAX_PARTS = 1 << 40


def histogram_part(prep_d, n_d: int, prep_r, n_r: int, nbins: int, bin_width_deg: float, part: int, parts: int,
                   out, workspace=None, tuning: Tuning | None = None, stream=None):
    """ADD part `part` of `parts` of the (DD, DR, RR) job into `out` ((3, nbins) int64 device
    tensor); the parts of one job sum exactly to histogram_dd_dr_rr's result."""
    n_d, n_r, nbins, out, workspace = _job_args(prep_d, n_d, prep_r, n_r, nbins, out, workspace, True)
    tc = tuning._c() if tuning is not None else None
    _check(load().gc_histogram_part(_ptr(prep_d), n_d, _ptr(prep_r), n_r, nbins,
                                    float(bin_width_deg), int(part), int(parts), _ptr(out[0]), _ptr(out[1]),
                                    _ptr(out[2]), _ptr(workspace), workspace.numel(),
                                    ctypes.byref(tc) if tc is not None else None, _stream(stream)),
           "gc_histogram_part")
    return out


def _families(dd, dr, rr):
    torch = _torch()
    _buf(dd, "dd", torch.int64)
    nbins = _bins(dd.numel())
    _buf(dr, "dr", torch.int64, shape=tuple(dd.shape))
    _buf(rr, "rr", torch.int64, shape=tuple(dd.shape))
    return nbins


def histogram_totals(dd, dr, rr, out=None, stream=None):
    torch = _torch()
    nbins = _families(dd, dr, rr)
    _buf(out, "out", torch.int64, 3, optional=True)
    _on_gpu(dd=dd, dr=dr, rr=rr, out=out)
    if out is None:
        out = torch.empty(3, dtype=torch.int64, device=dd.device)
    _check(load().gc_histogram_totals(_ptr(dd), _ptr(dr), _ptr(rr), nbins, _ptr(out), _stream(stream)),
           "gc_histogram_totals")
    return out


def omega(dd, dr, rr, n_d: int, n_r: int, out=None, stream=None):
    torch = _torch()
    nbins = _families(dd, dr, rr)
    n_d, n_r = _count(n_d, "n_d", MAX_GALAXIES), _count(n_r, "n_r", MAX_GALAXIES)
    _buf(out, "out", torch.float64, nbins, optional=True)
    _on_gpu(dd=dd, dr=dr, rr=rr, out=out)
    if out is None:
        out = torch.empty(nbins, dtype=torch.float64, device=dd.device)
    _check(load().gc_omega(_ptr(dd), _ptr(dr), _ptr(rr), nbins, n_d, n_r, _ptr(out), _stream(stream)), "gc_omega")
    return out


def eval_angle_core(x, nbins: int, bin_width_deg: float, with_exact: bool = True, with_t: bool = False,
                    stream=None):
    """The pair kernel's angle-to-bin core on cosines x (fp32 -> fp32-dot core, fp64 ->
    fp64-dot core).  Returns (bin, trip, exact_bin, t) device tensors (None where not asked)."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dtype not in (torch.float32, torch.float64):
        raise TypeError("x must be a float32 or float64 tensor")
    _buf(x, "x", x.dtype)
    nbins = _bins(nbins)
    _on_gpu(x=x)
    n = x.numel()
    dot = 64 if x.dtype == torch.float64 else 32
    bins = torch.empty(n, dtype=torch.int32, device=x.device)
    trip = torch.empty(n, dtype=torch.uint8, device=x.device)
    exact = torch.empty(n, dtype=torch.int32, device=x.device) if with_exact else None
    t = torch.empty(n, dtype=torch.float32, device=x.device) if with_t else None
    x32 = x if dot == 32 else None
    x64 = x if dot == 64 else None
    ws = torch.empty(workspace_bytes(nbins), dtype=torch.uint8, device=x.device)
    _check(load().gc_eval_angle_core(_ptr(x32), _ptr(x64), n, nbins, float(bin_width_deg), dot,
                                     _ptr(bins), _ptr(trip), _ptr(exact), _ptr(t), _ptr(ws),
                                     ws.numel(), _stream(stream)),
           "gc_eval_angle_core")
    return bins, trip, exact, t


def eval_dot_mfma(a, b, stream=None):
    """The bin-table core's matrix-core dot products: a and b are (3, 16 ntiles) fp32 device
    tensors (x, y, z rows); returns (ntiles, 16, 16) with [t, i, j] = a_(16t+i) . b_(16t+j)."""
    torch = _torch()
    if not isinstance(a, torch.Tensor) or a.dim() != 2 or a.shape[0] != 3 or a.shape[1] % 16:
        raise ValueError("a must have shape (3, 16 ntiles)")
    ntiles = a.shape[1] // 16
    a = _buf(a.contiguous(), "a", torch.float32)
    b = _buf(b.contiguous() if isinstance(b, torch.Tensor) else b, "b", torch.float32, shape=tuple(a.shape))
    _on_gpu(a=a, b=b)
    out = torch.empty((ntiles, 16, 16), dtype=torch.float32, device=a.device)
    _check(load().gc_eval_dot_mfma(_ptr(a[0]), _ptr(a[1]), _ptr(a[2]), _ptr(b[0]), _ptr(b[1]), _ptr(b[2]), ntiles,
                                   _ptr(out), _stream(stream)), "gc_eval_dot_mfma")
    return out


CLI_PATH = os.path.join(_PKG, "bin", "galaxy_gc")


def catalog_count(path: str) -> int:
    """Galaxy count of a catalog text file (its first token)."""
    n = ctypes.c_int64(0)
    _check(load().gc_catalog_count(os.fsencode(path), ctypes.byref(n)), "gc_catalog_count")
    return n.value


def read_catalog(path: str):
    """(alpha, delta) fp32 host arrays in arcminutes from a catalog text file."""
    import numpy as np
    n = catalog_count(path)
    ra = np.empty(n, dtype=np.float32)
    dec = np.empty(n, dtype=np.float32)
    got = ctypes.c_int64(0)
    _check(load().gc_catalog_read(os.fsencode(path), ra.ctypes.data_as(ctypes.c_void_p),
                                  dec.ctypes.data_as(ctypes.c_void_p), n, ctypes.byref(got)), "gc_catalog_read")
    return ra, dec


def write_omega(path: str, dd, dr, rr, omega_values, bin_width_deg: float) -> None:
    """Write the result file (the page's omega.out layout) from host arrays."""
    import numpy as np
    arrs = [np.ascontiguousarray(np.asarray(x), dtype=np.uint64) for x in (dd, dr, rr)]
    om = np.ascontiguousarray(np.asarray(omega_values), dtype=np.float64)
    nb = om.size
    if any(a.size != nb for a in arrs):
        raise ValueError("dd, dr, rr and omega must have the same length")
    vp = ctypes.c_void_p
    _check(load().gc_omega_write(os.fsencode(path), *[a.ctypes.data_as(vp) for a in arrs], om.ctypes.data_as(vp),
                                 nb, float(bin_width_deg)), "gc_omega_write")


LADDER_RUNGS = 6
LADDER_ACOS = {"rung": -1, "libm": 0, "handbook": 1, "fit6": 2}


def ladder_workspace_bytes(n_d: int, n_r: int) -> int:
    return int(load().gc_ladder_workspace_bytes(int(n_d), int(n_r)))


def ladder_histogram(rung: int, ra_d, dec_d, ra_r, dec_r, nbins: int, bin_width_deg: float, acos: str = "rung",
                     tile: int = 0, bin_stride: int = 0, out=None, workspace=None, stream=None):
    """(DD, DR, RR) of one rung of the page's ablation ladder (fp32 arithmetic, no guard; see
    include/gc_ladder.h) from fp32 arcmin device tensors."""
    torch = _torch()
    for t, nm in ((ra_d, "ra_d"), (dec_d, "dec_d"), (ra_r, "ra_r"), (dec_r, "dec_r")):
        _buf(t, nm, torch.float32)
    n_d, n_r = ra_d.numel(), ra_r.numel()
    if dec_d.numel() != n_d or dec_r.numel() != n_r:
        raise ValueError("ra and dec must have the same length")
    nbins = _bins(nbins)
    _buf(out, "out", torch.int64, shape=(3, nbins), optional=True)
    _buf(workspace, "workspace", torch.uint8, ladder_workspace_bytes(n_d, n_r), optional=True)
    _on_gpu(ra_d=ra_d, dec_d=dec_d, ra_r=ra_r, dec_r=dec_r, out=out, workspace=workspace)
    dev = ra_d.device
    if out is None:
        out = torch.empty((3, nbins), dtype=torch.int64, device=dev)
    if workspace is None:
        workspace = torch.empty(max(ladder_workspace_bytes(n_d, n_r), 1), dtype=torch.uint8, device=dev)
    _check(load().gc_ladder_histogram(int(rung), LADDER_ACOS[acos], int(tile), int(bin_stride), _ptr(ra_d),
                                      _ptr(dec_d), n_d, _ptr(ra_r), _ptr(dec_r), n_r, int(nbins),
                                      float(bin_width_deg), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                                      _ptr(workspace), workspace.numel(), _stream(stream)),
           "gc_ladder_histogram")
    return out[0], out[1], out[2]


def _timed(launch, stream=None):
    torch = _torch()
    st = torch.cuda.current_stream() if stream is None else stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    n = launch(_stream(st))
    e1.record(st)
    e1.synchronize()
    return n, e0.elapsed_time(e1) / 1e3


def ceiling_valu(kind: int, iters: int = 4096, repeats: int = 3):
    """Measured VALU rate (lane operations per second) of independent FMA chains (kind 0:
    fp32 FMA, 1: fp32 square root, 2: fp64 FMA); best of `repeats` timed launches."""
    torch = _torch()
    sink = torch.empty(load().gc_ceiling_sink_bytes(), dtype=torch.uint8, device="cuda")
    ops = ctypes.c_uint64(0)
    best = None
    for _ in range(repeats + 1):
        def launch(s):
            _check(load().gc_ceiling_valu(int(kind), int(iters), _ptr(sink), sink.numel(), ctypes.byref(ops), s),
                   "gc_ceiling_valu")
            return ops.value
        n, dt = _timed(launch)
        best = dt if best is None else min(best, dt)
    return ops.value / best


def ceiling_lds_atomic(nbins: int, same_bin: bool = False, iters: int = 2048, repeats: int = 3):
    """Measured LDS atomic increments per second into per-wave histograms of nbins bins."""
    torch = _torch()
    sink = torch.empty(load().gc_ceiling_sink_bytes(), dtype=torch.uint8, device="cuda")
    n_at = ctypes.c_uint64(0)
    best = None
    for _ in range(repeats + 1):
        def launch(s):
            _check(load().gc_ceiling_lds_atomic(int(nbins), int(bool(same_bin)), int(iters), _ptr(sink), sink.numel(),
                                                ctypes.byref(n_at), s), "gc_ceiling_lds_atomic")
            return n_at.value
        n, dt = _timed(launch)
        best = dt if best is None else min(best, dt)
    return n_at.value / best


LDS_PROBES = {"add": 0, "add_rtn": 1, "add64": 2, "add64_rtn": 3, "read32": 4, "read64": 5,
              "read64_then_add": 6, "add_sparse": 7}


def ceiling_lds(kind: str, words: int, threads: int = 256, sparse: int = 1, cols: int = 0, iters: int = 512,
                repeats: int = 3):
    """Measured rate of one kind of random-address LDS operation (64-lane instructions per
    second) into a table of `words` words shared by each workgroup (gc_ceiling_lds); cols > 0:
    a table of that many columns, one per lane group (lane mod cols)."""
    torch = _torch()
    sink = torch.empty(load().gc_ceiling_sink_bytes(), dtype=torch.uint8, device="cuda")
    n = ctypes.c_uint64(0)
    best = None
    for _ in range(repeats + 1):
        def launch(s):
            _check(load().gc_ceiling_lds(LDS_PROBES[kind], int(words), int(threads), int(sparse), int(cols), int(iters),
                                         _ptr(sink), sink.numel(), ctypes.byref(n), s), "gc_ceiling_lds")
            return n.value
        _, dt = _timed(launch)
        best = dt if best is None else min(best, dt)
    return n.value / best


def ceiling_l1(words: int, threads: int = 256, iters: int = 256, repeats: int = 3):
    """Measured rate of random 8-byte loads (64-lane instructions per second) from a table of
    `words` words in global memory (gc_ceiling_l1)."""
    torch = _torch()
    tab_bytes = (words * 4 + 255) // 256 * 256
    sink = torch.zeros(tab_bytes + load().gc_ceiling_sink_bytes(), dtype=torch.uint8, device="cuda")
    n = ctypes.c_uint64(0)
    best = None
    for _ in range(repeats + 1):
        def launch(s):
            _check(load().gc_ceiling_l1(int(words), int(threads), int(iters), _ptr(sink), sink.numel(),
                                        ctypes.byref(n), s), "gc_ceiling_l1")
            return n.value
        _, dt = _timed(launch)
        best = dt if best is None else min(best, dt)
    return n.value / best


def launch_plan(n_d: int, n_r: int, nbins: int, bin_width_deg: float, tuning: Tuning | None = None) -> dict:
    """The launch plan of a histogram call with these sizes, bins and overrides (gc_launch_plan):
    core, dot precision, galaxies per lane, histogram columns, waves per workgroup, L1 share,
    occupancy, grid and LDS per workgroup.  Enqueues nothing."""
    p = _Plan()
    tc = tuning._c() if tuning is not None else None
    _check(load().gc_launch_plan(int(n_d), int(n_r), int(nbins), float(bin_width_deg),
                                 ctypes.byref(tc) if tc is not None else None, ctypes.byref(p)), "gc_launch_plan")
    return {n: getattr(p, n) for n, _ in _Plan._fields_ if n != "reserved_"}
