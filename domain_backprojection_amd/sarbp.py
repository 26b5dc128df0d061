"""ctypes binding of the sarbp C ABI (include/sarbp.h).

Argument marshalling only: tensors become device pointers and the current
torch stream becomes the hipStream_t.  Every step of the computation runs in
the HIP library ``libsarbp.so`` built in this directory; importing this module
raises if that library is missing -- there is no fallback.

The functions keep the C names: :func:`sarbp_plan_create`,
:func:`sarbp_backproject`, :func:`sarbp_backproject_dem`, :func:`sarbp_range_compress`,
:func:`sarbp_interpolate_track`, :func:`sarbp_stream_create`,
:func:`sarbp_backproject_host`, :func:`sarbp_stream_destroy`, :func:`sarbp_destroy`,
:func:`sarbp_backproject_split_noalloc`,
:func:`sarbp_check_indices`, :func:`sarbp_status_string`, :func:`sarbp_version`.  :class:`Plan` and
:class:`HostStream` wrap the handles' lifetimes.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsarbp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m domain_backprojection_amd.build` "
        "(hipcc, gfx950). There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

SARBP_OK = 0
SARBP_EINVAL = -1
SARBP_ENOMEM = -2
SARBP_EDEVICE = -3
SARBP_EUNSUPPORTED = -4
SARBP_ESCRATCH = -5
SARBP_STATIC_SCRATCH_BYTES = 8 << 20

SARBP_NEAREST = 0
SARBP_LINEAR = 1
SARBP_SINC8 = 2
INTERP = {"nearest": SARBP_NEAREST, "linear": SARBP_LINEAR, "sinc8": SARBP_SINC8}
SARBP_ACC_FP32, SARBP_ACC_KAHAN, SARBP_ACC_CHUNK64 = 0, 1, 2
ACCUM = {"fp32": SARBP_ACC_FP32, "kahan": SARBP_ACC_KAHAN, "chunk64": SARBP_ACC_CHUNK64}


class sarbp_params(ctypes.Structure):
    """Mirror of ``sarbp_params`` (same field order and C alignment)."""

    _fields_ = [
        ("n_pulses", ctypes.c_int32),
        ("n_range", ctypes.c_int32),
        ("r0", ctypes.c_double),
        ("dr", ctypes.c_double),
        ("nx", ctypes.c_int32),
        ("ny", ctypes.c_int32),
        ("x0", ctypes.c_double),
        ("y0", ctypes.c_double),
        ("z0", ctypes.c_double),
        ("dx", ctypes.c_double),
        ("dy", ctypes.c_double),
        ("wavelength", ctypes.c_double),
        ("interp", ctypes.c_int32),
        ("n_fast", ctypes.c_int32),
        ("fs", ctypes.c_double),
        ("chirp_T", ctypes.c_double),
        ("chirp_B", ctypes.c_double),
        ("window", ctypes.c_int32),
        ("taylor_nbar", ctypes.c_int32),
        ("taylor_sll", ctypes.c_double),
        ("accum", ctypes.c_int32),
        ("dem_relief", ctypes.c_double),
        ("nz", ctypes.c_int32),
        ("dz", ctypes.c_double),
    ]


class sarbp_index_report(ctypes.Structure):
    """Mirror of ``sarbp_index_report``."""

    _fields_ = [
        ("decisions", ctypes.c_int64),
        ("window_violations", ctypes.c_int64),
        ("staging_violations", ctypes.c_int64),
        ("nearest_rechecks", ctypes.c_int64),
        ("nearest_recheck_clamped", ctypes.c_int64),
        ("nearest_escapes", ctypes.c_int64),
        ("nan_tiles", ctypes.c_int64),
        ("max_position_error", ctypes.c_double),
        ("max_error_to_band", ctypes.c_double),
        ("min_position", ctypes.c_double),
        ("max_position_margin", ctypes.c_double),
        ("window_mean", ctypes.c_double),
        ("chunks", ctypes.c_int64),
        ("chunks_in_record", ctypes.c_int64),
        ("window", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("pixels_per_lane", ctypes.c_int32),
        ("fp64_ranges", ctypes.c_int32),
        ("mode_chunks", ctypes.c_int32 * 3),
        ("tie_band_max", ctypes.c_float),
        ("tie_queue_words", ctypes.c_int64),
        ("tie_queue_drains", ctypes.c_int64),
        ("tie_queue_tile_max", ctypes.c_int32),
        ("tie_queue_capacity", ctypes.c_int32),
        ("tie_queue_tables", ctypes.c_int64),
        ("tie_queue_table_misses", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {f: (list(getattr(self, f)) if f == "mode_chunks" else getattr(self, f)) for f, _ in self._fields_}


_vp = ctypes.c_void_p
_lib.sarbp_plan_create.argtypes = [ctypes.POINTER(sarbp_params), ctypes.POINTER(_vp)]
_lib.sarbp_plan_create.restype = ctypes.c_int
_lib.sarbp_backproject.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp]
_lib.sarbp_backproject.restype = ctypes.c_int
_lib.sarbp_range_compress.argtypes = [_vp, _vp, _vp, ctypes.c_int32, _vp]
_lib.sarbp_range_compress.restype = ctypes.c_int
_lib.sarbp_destroy.argtypes = [_vp]
_lib.sarbp_destroy.restype = None
_lib.sarbp_status_string.argtypes = [ctypes.c_int]
_lib.sarbp_status_string.restype = ctypes.c_char_p
_lib.sarbp_version.argtypes = []
_lib.sarbp_version.restype = ctypes.c_int
_lib.sarbp_stream_create.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_vp)]
_lib.sarbp_stream_create.restype = ctypes.c_int
_lib.sarbp_backproject_host.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp]
_lib.sarbp_backproject_host.restype = ctypes.c_int
_lib.sarbp_stream_destroy.argtypes = [_vp]
_lib.sarbp_stream_destroy.restype = None
_lib.sarbp_interpolate_track.argtypes = [_vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp]
_lib.sarbp_interpolate_track.restype = ctypes.c_int
_lib.sarbp_backproject_dem.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp]
_lib.sarbp_backproject_dem.restype = ctypes.c_int
_lib.sarbp_split_workspace_bytes.argtypes = [_vp, ctypes.c_int32]
_lib.sarbp_split_workspace_bytes.restype = ctypes.c_size_t
_lib.sarbp_backproject_split.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_size_t,
                                         _vp]
_lib.sarbp_backproject_split.restype = ctypes.c_int
_lib.sarbp_backproject_split_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp]
_lib.sarbp_backproject_split_noalloc.restype = ctypes.c_int
_lib.sarbp_check_indices.argtypes = [ctypes.POINTER(sarbp_params), ctypes.c_int32, _vp, ctypes.c_int32, _vp,
                                     ctypes.POINTER(sarbp_index_report)]
_lib.sarbp_check_indices.restype = ctypes.c_int

EXPORTS = ("sarbp_plan_create", "sarbp_backproject", "sarbp_range_compress", "sarbp_destroy",
           "sarbp_status_string", "sarbp_version", "sarbp_stream_create", "sarbp_backproject_host",
           "sarbp_stream_destroy", "sarbp_interpolate_track", "sarbp_backproject_dem",
           "sarbp_split_workspace_bytes", "sarbp_backproject_split", "sarbp_backproject_split_noalloc",
           "sarbp_check_indices")


class SarbpError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {sarbp_status_string(status)} ({status})")
        self.status = status


def sarbp_status_string(status: int) -> str:
    return _lib.sarbp_status_string(int(status)).decode()


def sarbp_version() -> int:
    return int(_lib.sarbp_version())


def make_params(n_pulses, n_range, r0, dr, nx, ny, x0, y0, z0, dx, dy, wavelength, interp="linear",
                n_fast=0, fs=0.0, chirp_T=0.0, chirp_B=0.0, window=0, taylor_nbar=0, taylor_sll=0.0, accum="fp32", dem_relief=0.0, nz=0,
                dz=0.0) -> sarbp_params:
    return sarbp_params(int(n_pulses), int(n_range), float(r0), float(dr), int(nx), int(ny), float(x0),
                        float(y0), float(z0), float(dx), float(dy), float(wavelength),
                        INTERP[interp] if isinstance(interp, str) else int(interp), int(n_fast), float(fs),
                        float(chirp_T), float(chirp_B), int(window), int(taylor_nbar), float(taylor_sll),
                        ACCUM[accum] if isinstance(accum, str) else int(accum), float(dem_relief), int(nz),
                        float(dz))


def sarbp_plan_create(params: sarbp_params) -> int:
    """Create a plan on the current device; returns the opaque handle (an int)."""
    h = _vp()
    st = _lib.sarbp_plan_create(ctypes.byref(params), ctypes.byref(h))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_plan_create")
    return h.value


def sarbp_destroy(handle) -> None:
    _lib.sarbp_destroy(handle)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev_ptr(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def sarbp_backproject(handle, positions: torch.Tensor, echo: torch.Tensor, image: torch.Tensor,
                      n: int | None = None, accumulate: int = 0, stream=None) -> None:
    """positions float64 (n, 3), echo complex64 (n, n_range), image complex64 (ny, nx), all on the device."""
    if n is None:
        n = positions.shape[0]
    if positions.dim() != 2 or positions.shape[1] != 3 or positions.shape[0] < n or echo.shape[0] < n:
        raise ValueError("positions must be (>= n, 3) and echo (>= n, n_range)")
    st = _lib.sarbp_backproject(handle, _dev_ptr(positions, torch.float64, "positions"),
                                _dev_ptr(echo, torch.complex64, "echo"), _dev_ptr(image, torch.complex64, "image"),
                                int(n), int(accumulate), _stream(stream))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_backproject")


def sarbp_backproject_dem(handle, positions: torch.Tensor, echo: torch.Tensor, dem: torch.Tensor,
                          image: torch.Tensor, n: int | None = None, accumulate: int = 0, stream=None) -> None:
    """As :func:`sarbp_backproject`, with pixel heights dem float32 (ny, nx) on the device."""
    if n is None:
        n = positions.shape[0]
    if positions.dim() != 2 or positions.shape[1] != 3 or positions.shape[0] < n or echo.shape[0] < n:
        raise ValueError("positions must be (>= n, 3) and echo (>= n, n_range)")
    if tuple(dem.shape) != tuple(image.shape):
        raise ValueError("dem must have the image's shape (ny, nx)")
    st = _lib.sarbp_backproject_dem(handle, _dev_ptr(positions, torch.float64, "positions"),
                                    _dev_ptr(echo, torch.complex64, "echo"), _dev_ptr(dem, torch.float32, "dem"),
                                    _dev_ptr(image, torch.complex64, "image"), int(n), int(accumulate),
                                    _stream(stream))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_backproject_dem")


def sarbp_split_workspace_bytes(handle, n: int) -> int:
    """Bytes of workspace :func:`sarbp_backproject_split` needs for n pulses (0: the call runs unsplit)."""
    return int(_lib.sarbp_split_workspace_bytes(handle, int(n)))


def sarbp_backproject_split(handle, positions: torch.Tensor, echo: torch.Tensor, image: torch.Tensor,
                            workspace: torch.Tensor | None, n: int | None = None, accumulate: int = 0,
                            stream=None, dem: torch.Tensor | None = None) -> None:
    """As :func:`sarbp_backproject` (or with dem, :func:`sarbp_backproject_dem`), with the pulses split
    over several workgroups per pixel tile; workspace is a device tensor of at least
    :func:`sarbp_split_workspace_bytes` bytes (None when that is 0)."""
    if n is None:
        n = positions.shape[0]
    if positions.dim() != 2 or positions.shape[1] != 3 or positions.shape[0] < n or echo.shape[0] < n:
        raise ValueError("positions must be (>= n, 3) and echo (>= n, n_range)")
    dem_p = None
    if dem is not None:
        if tuple(dem.shape) != tuple(image.shape):
            raise ValueError("dem must have the image's shape (ny, nx)")
        dem_p = _dev_ptr(dem, torch.float32, "dem")
    ws_p, ws_bytes = None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
            raise TypeError("workspace must be a contiguous device tensor")
        ws_p, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = _lib.sarbp_backproject_split(handle, _dev_ptr(positions, torch.float64, "positions"),
                                      _dev_ptr(echo, torch.complex64, "echo"), dem_p,
                                      _dev_ptr(image, torch.complex64, "image"), int(n), int(accumulate), ws_p,
                                      ws_bytes, _stream(stream))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_backproject_split")


def sarbp_backproject_split_noalloc(handle, positions: torch.Tensor, echo: torch.Tensor, image: torch.Tensor,
                                    n: int | None = None, accumulate: int = 0, stream=None,
                                    dem: torch.Tensor | None = None) -> None:
    """As :func:`sarbp_backproject_split` with the partial images in the library's static
    device array (no workspace, no allocation; calls on one GPU must not overlap)."""
    if n is None:
        n = positions.shape[0]
    if positions.dim() != 2 or positions.shape[1] != 3 or positions.shape[0] < n or echo.shape[0] < n:
        raise ValueError("positions must be (>= n, 3) and echo (>= n, n_range)")
    dem_p = None
    if dem is not None:
        if tuple(dem.shape) != tuple(image.shape):
            raise ValueError("dem must have the image's shape (ny, nx)")
        dem_p = _dev_ptr(dem, torch.float32, "dem")
    st = _lib.sarbp_backproject_split_noalloc(handle, _dev_ptr(positions, torch.float64, "positions"),
                                              _dev_ptr(echo, torch.complex64, "echo"), dem_p,
                                              _dev_ptr(image, torch.complex64, "image"), int(n), int(accumulate),
                                              _stream(stream))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_backproject_split_noalloc")


def sarbp_check_indices(params: sarbp_params, positions, dem=None, n_cu: int = 0) -> dict:
    """Host emulation of the backprojection kernels' index arithmetic for the plan
    `params` over host float64 positions (n, 3) (and float32 heights (ny, nx) for the
    terrain kernels); returns the report's fields as a dict.  No device is used."""
    import numpy as np

    pos = np.ascontiguousarray(positions, dtype=np.float64)
    if pos.ndim != 2 or pos.shape[1] != 3:
        raise ValueError("positions must be (n, 3)")
    dem_p = None
    if dem is not None:
        dem = np.ascontiguousarray(dem, dtype=np.float32)
        if dem.shape != (params.ny, params.nx):
            raise ValueError("dem must be (ny, nx)")
        dem_p = dem.ctypes.data
    rep = sarbp_index_report()
    st = _lib.sarbp_check_indices(ctypes.byref(params), int(n_cu), pos.ctypes.data, int(pos.shape[0]), dem_p,
                                  ctypes.byref(rep))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_check_indices")
    return rep.as_dict()


def sarbp_range_compress(handle, raw: torch.Tensor, out: torch.Tensor, n: int | None = None, stream=None) -> None:
    """raw and out complex64 (n, n_fast) on the device, rows of the plan's n_fast samples
    (the caller's Plan checks n_fast itself; here the two must agree row for row)."""
    if raw.dim() != 2 or out.dim() != 2:
        raise ValueError("raw and out must be 2-D (pulses, samples)")
    if raw.shape[1] != out.shape[1]:
        raise ValueError(f"raw rows hold {raw.shape[1]} samples but out rows {out.shape[1]}")
    if n is None:
        n = raw.shape[0]
    if n < 0 or raw.shape[0] < n or out.shape[0] < n:
        raise ValueError("raw and out must hold n pulses")
    st = _lib.sarbp_range_compress(handle, _dev_ptr(raw, torch.complex64, "raw"),
                                   _dev_ptr(out, torch.complex64, "out"), int(n), _stream(stream))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_range_compress")


def _host_ptr(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.is_cuda:
        raise TypeError(f"{name} must be a host tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def sarbp_stream_create(plan_handle, chunk: int, compress: int = 0) -> int:
    h = _vp()
    st = _lib.sarbp_stream_create(plan_handle, int(chunk), int(compress), ctypes.byref(h))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_stream_create")
    return h.value


def sarbp_backproject_host(stream_handle, positions: torch.Tensor, data: torch.Tensor, image: torch.Tensor,
                           n: int | None = None, accumulate: int = 0, stream=None) -> None:
    """positions float64 (n, 3) and data complex64 (n, row) in host memory (page-locked for
    overlap), image complex64 (ny, nx) on the device."""
    if n is None:
        n = positions.shape[0]
    if positions.dim() != 2 or positions.shape[1] != 3 or positions.shape[0] < n or data.shape[0] < n:
        raise ValueError("positions must be (>= n, 3) and data (>= n, row)")
    st = _lib.sarbp_backproject_host(stream_handle, _host_ptr(positions, torch.float64, "positions"),
                                     _host_ptr(data, torch.complex64, "data"),
                                     _dev_ptr(image, torch.complex64, "image"), int(n), int(accumulate),
                                     _stream(stream))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_backproject_host")


def sarbp_stream_destroy(stream_handle) -> None:
    _lib.sarbp_stream_destroy(stream_handle)


def sarbp_interpolate_track(nav_t: torch.Tensor, nav_xyz: torch.Tensor, t: torch.Tensor,
                            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Positions float64 (n, 3) at pulse times t (n,) from navigation samples nav_t (M,)
    and nav_xyz (M, 3), all float64 on the device."""
    if nav_t.dim() != 1 or nav_xyz.shape != (nav_t.shape[0], 3) or t.dim() != 1:
        raise ValueError("nav_t must be (M,), nav_xyz (M, 3) and t (n,)")
    if out is None:
        out = torch.empty((t.shape[0], 3), dtype=torch.float64, device=t.device)
    if tuple(out.shape) != (t.shape[0], 3):
        raise ValueError("out must be (n, 3)")
    st = _lib.sarbp_interpolate_track(_dev_ptr(nav_t, torch.float64, "nav_t"),
                                      _dev_ptr(nav_xyz, torch.float64, "nav_xyz"), int(nav_t.shape[0]),
                                      _dev_ptr(t, torch.float64, "t"), _dev_ptr(out, torch.float64, "out"),
                                      int(t.shape[0]), _stream(stream))
    if st != SARBP_OK:
        raise SarbpError(st, "sarbp_interpolate_track")
    return out


class Plan:
    """Owns one plan handle; checks tensor shapes against the plan's sizes."""

    def __init__(self, **kw):
        self.params = make_params(**kw)
        self.handle = sarbp_plan_create(self.params)

    @classmethod
    def for_scene(cls, scene, n_fast=None, **over):
        kw = dict(scene.params())
        kw.update(over)
        if n_fast:
            kw.update(n_fast=n_fast, fs=scene.fs, chirp_T=scene.chirp_T, chirp_B=scene.chirp_B, window=scene.window)
        return cls(**kw)

    def close(self):
        if getattr(self, "handle", None):
            sarbp_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def image_shape(self) -> tuple:
        """(ny, nx), or (nz, ny, nx) for a volume."""
        p = self.params
        return (p.nz, p.ny, p.nx) if p.nz > 1 else (p.ny, p.nx)

    def new_image(self, device="cuda") -> torch.Tensor:
        return torch.zeros(self.image_shape, dtype=torch.complex64, device=device)

    def split_workspace_bytes(self, n: int) -> int:
        return sarbp_split_workspace_bytes(self.handle, n)

    def backproject(self, positions, echo, image=None, n=None, accumulate=0, stream=None, dem=None,
                    split=False, workspace=None) -> torch.Tensor:
        """split=True calls sarbp_backproject_split, with `workspace` or, when it is None, a
        workspace allocated here by torch (device memory is torch's; the kernels are the library's)."""
        if image is None:
            image = torch.empty(self.image_shape, dtype=torch.complex64, device=echo.device)
        if tuple(image.shape) != self.image_shape:
            raise ValueError("image shape does not match the plan")
        if echo.dim() != 2 or echo.shape[1] != self.params.n_range:
            raise ValueError("echo must be (n, n_range)")
        if split:
            npulses = positions.shape[0] if n is None else n
            if workspace is None:
                need = self.split_workspace_bytes(npulses)
                workspace = torch.empty(need, dtype=torch.uint8, device=echo.device) if need else None
            sarbp_backproject_split(self.handle, positions, echo, image, workspace, n=n, accumulate=accumulate,
                                    stream=stream, dem=dem)
        elif dem is None:
            sarbp_backproject(self.handle, positions, echo, image, n=n, accumulate=accumulate, stream=stream)
        else:
            sarbp_backproject_dem(self.handle, positions, echo, dem, image, n=n, accumulate=accumulate,
                                  stream=stream)
        return image

    def range_compress(self, raw, out=None, n=None, stream=None) -> torch.Tensor:
        if raw.dim() != 2 or raw.shape[1] != self.params.n_fast:
            raise ValueError("raw must be (n, n_fast)")
        if out is None:
            out = torch.empty_like(raw)
        if out.dim() != 2 or out.shape[1] != self.params.n_fast:
            raise ValueError("out must be (n, n_fast)")
        sarbp_range_compress(self.handle, raw, out, n=n, stream=stream)
        return out


class HostStream:
    """Owns one host-to-device pulse pipeline of a plan (``sarbp_stream_create``)."""

    def __init__(self, plan: Plan, chunk: int, compress: bool = False):
        self.plan = plan
        self.row = plan.params.n_range
        self.handle = sarbp_stream_create(plan.handle, chunk, 1 if compress else 0)

    def close(self):
        if getattr(self, "handle", None):
            sarbp_stream_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def backproject(self, positions, data, image=None, n=None, accumulate=0, stream=None) -> torch.Tensor:
        if image is None:
            image = torch.empty(self.plan.image_shape, dtype=torch.complex64, device="cuda")
        if tuple(image.shape) != self.plan.image_shape:
            raise ValueError("image shape does not match the plan")
        if data.dim() != 2 or data.shape[1] != self.row:
            raise ValueError("data must be (n, n_range)")
        sarbp_backproject_host(self.handle, positions, data, image, n=n, accumulate=accumulate, stream=stream)
        return image
