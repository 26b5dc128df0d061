"""CPU checks of the C-ABI library: it loads, exports every function include/sarbp.h
declares, its parameter struct matches the ctypes mirror, and host-side argument
validation returns the documented codes without touching a GPU."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sarbp.h")


@pytest.fixture(scope="module")
def sb():
    from domain_backprojection_amd import sarbp

    return sarbp


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sarbp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function(sb):
    names = declared_functions()
    assert set(names) == set(sb.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", sb.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sarbp_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(sb._lib, n)


def test_params_struct_layout_matches_c(sb):
    fields = [f for f, _ in sb.sarbp_params._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "sarbp.h"', "int main(void){",
            'printf("%zu\\n", sizeof(sarbp_params));']
    prog += [f'printf("%zu\\n", offsetof(sarbp_params, {f}));' for f in fields]
    prog += ["return 0;}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "p.c"), os.path.join(d, "p")
        open(src, "w").write("\n".join(prog))
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(sb.sarbp_params)
    for f, off in zip(fields, vals[1:]):
        assert getattr(sb.sarbp_params, f).offset == off, f


def test_status_strings(sb):
    for code, word in ((0, "success"), (-1, "invalid"), (-2, "memory"), (-3, "HIP"), (-4, "unsupported")):
        assert word in sb.sarbp_status_string(code)
    assert sb.sarbp_status_string(12345) == "unknown status"
    assert sb.sarbp_version() >= 100


def _good(sb, **over):
    kw = dict(n_pulses=16, n_range=64, r0=1000.0, dr=0.5, nx=8, ny=8, x0=0, y0=0, z0=0, dx=0.2, dy=0.2,
              wavelength=0.03, interp="linear")
    kw.update(over)
    return sb.make_params(**kw)


@pytest.mark.parametrize("bad", [
    dict(n_pulses=0), dict(n_range=1), dict(nx=0), dict(ny=-3), dict(dr=0.0), dict(dr=float("nan")),
    dict(dx=-1.0), dict(dy=float("inf")), dict(wavelength=0.0), dict(interp=7), dict(r0=float("nan")),
    dict(interp=2, n_range=7), dict(x0=float("inf")),
    dict(n_fast=100, fs=1e6, chirp_T=1e-5, chirp_B=1e5), dict(n_fast=32, fs=1e6, chirp_T=1e-5, chirp_B=1e5),
    dict(n_fast=1024, fs=0.0, chirp_T=1e-5, chirp_B=1e5), dict(n_fast=64, fs=1e8, chirp_T=1e-5, chirp_B=1e5),
    dict(n_fast=1024, fs=1e6, chirp_T=1e-5, chirp_B=1e5, window=3),
    dict(n_fast=1024, fs=1e6, chirp_T=1e-5, chirp_B=1e5, window=-1),
    dict(n_fast=1024, fs=1e6, chirp_T=1e-5, chirp_B=1e5, window=2, taylor_nbar=1),
    dict(n_fast=1024, fs=1e6, chirp_T=1e-5, chirp_B=1e5, window=2, taylor_nbar=65),
    dict(n_fast=1024, fs=1e6, chirp_T=1e-5, chirp_B=1e5, window=2, taylor_sll=10.0),
    dict(n_fast=1024, fs=1e6, chirp_T=1e-5, chirp_B=1e5, window=2, taylor_sll=float("nan")),
    dict(accum=3), dict(accum=-1),
    dict(dem_relief=-1.0), dict(dem_relief=float("nan")), dict(dem_relief=1e5),
    dict(nz=-1), dict(nz=70000), dict(nz=4, dz=0.0), dict(nz=4, dz=-0.5), dict(nz=4, dz=0.5, dem_relief=2.0),
])
def test_plan_create_rejects_invalid_parameters(sb, bad):
    h = ctypes.c_void_p(123)
    st = sb._lib.sarbp_plan_create(ctypes.byref(_good(sb, **bad)), ctypes.byref(h))
    assert st == sb.SARBP_EINVAL
    assert h.value is None


@pytest.mark.parametrize("dr, wavelength, unsupported", [(4.0, 0.03125, True), (7.97, 0.0625, True),
                                                      (3.98, 0.03125, False), (0.41637, 0.0086, False)])
def test_plan_create_bounds_cycles_per_bin(sb, dr, wavelength, unsupported):
    """2 dr / lambda carrier cycles per range bin must stay below 255 (the hardware sine
    and cosine take at most 256 cycles): 256 and 255.04 are refused before any device
    call; 254.7 and a Ka-band 96.8 pass validation (and fail, if at all, only at the
    device step, with no GPU here)."""
    h = ctypes.c_void_p()
    st = sb._lib.sarbp_plan_create(ctypes.byref(_good(sb, dr=dr, wavelength=wavelength, n_range=4096)),
                                   ctypes.byref(h))
    if unsupported:
        assert st == sb.SARBP_EUNSUPPORTED and h.value is None
    else:
        assert st not in (sb.SARBP_EINVAL, sb.SARBP_EUNSUPPORTED)
        if st == sb.SARBP_OK:
            sb._lib.sarbp_destroy(h)


@pytest.mark.parametrize("ok", [dict(window=2), dict(window=2, taylor_nbar=6, taylor_sll=45.0),
                                dict(window=1, taylor_nbar=1), dict(window=0)])
def test_plan_params_validate_window_fields(sb, ok):
    """Validation of the window fields without touching a device: a valid set passes
    validation and fails, if at all, only at the device step (no GPU here)."""
    h = ctypes.c_void_p()
    st = sb._lib.sarbp_plan_create(ctypes.byref(_good(sb, n_fast=1024, fs=1e6, chirp_T=1e-5, chirp_B=1e5, **ok)),
                                   ctypes.byref(h))
    assert st != sb.SARBP_EINVAL
    if st == sb.SARBP_OK:
        sb._lib.sarbp_destroy(h)


def test_null_arguments(sb):
    h = ctypes.c_void_p()
    assert sb._lib.sarbp_plan_create(None, ctypes.byref(h)) == sb.SARBP_EINVAL
    assert sb._lib.sarbp_plan_create(ctypes.byref(_good(sb)), None) == sb.SARBP_EINVAL
    assert sb._lib.sarbp_backproject(None, 8, 8, 8, 1, 0, None) == sb.SARBP_EINVAL
    assert sb._lib.sarbp_range_compress(None, 8, 16, 1, None) == sb.SARBP_EINVAL
    sb._lib.sarbp_destroy(None)  # no-op
    assert sb._lib.sarbp_stream_create(None, 8, 0, ctypes.byref(h)) == sb.SARBP_EINVAL
    assert sb._lib.sarbp_stream_create(None, 8, 0, None) == sb.SARBP_EINVAL
    assert sb._lib.sarbp_backproject_host(None, 8, 8, 8, 1, 0, None) == sb.SARBP_EINVAL
    sb._lib.sarbp_stream_destroy(None)  # no-op
    assert sb._lib.sarbp_backproject_dem(None, 8, 8, 8, 8, 1, 0, None) == sb.SARBP_EINVAL
    assert sb._lib.sarbp_interpolate_track(None, 8, 10, 8, 8, 4, None) == sb.SARBP_EINVAL
    assert sb._lib.sarbp_interpolate_track(8, 8, 3, 8, 8, 4, None) == sb.SARBP_EINVAL  # fewer than 4 samples
    assert sb._lib.sarbp_interpolate_track(8, 8, 10, 8, 8, 0, None) == sb.SARBP_EINVAL
    assert sb._lib.sarbp_split_workspace_bytes(None, 16) == 0
    assert sb._lib.sarbp_backproject_split(None, 8, 8, None, 8, 1, 0, None, 0, None) == sb.SARBP_EINVAL
    # output overlapping the sample positions
    assert sb._lib.sarbp_interpolate_track(4096, 8192, 10, 65536, 8192, 4, None) == sb.SARBP_EINVAL


def test_range_compress_shapes_checked_before_launch(sb):
    """A compressed row is n_fast samples: raw and out rows that disagree with each other
    (or, through a Plan, with the plan's n_fast) are refused on the host, before any
    device call, so the kernel never reads or writes past a narrower buffer."""
    import torch

    raw = torch.zeros(4, 64, dtype=torch.complex64)
    narrow = torch.zeros(4, 32, dtype=torch.complex64)
    with pytest.raises(ValueError):
        sb.sarbp_range_compress(None, raw, narrow)
    with pytest.raises(ValueError):
        sb.sarbp_range_compress(None, narrow, raw)
    with pytest.raises(ValueError):
        sb.sarbp_range_compress(None, raw, torch.zeros(256, dtype=torch.complex64))
    with pytest.raises(ValueError):
        sb.sarbp_range_compress(None, raw, torch.zeros(2, 64, dtype=torch.complex64))  # fewer pulses than raw
    # a Plan with n_fast = 64, its handle never created (no device here)
    plan = sb.Plan.__new__(sb.Plan)
    plan.params = _good(sb, n_fast=64, fs=1e6, chirp_T=1e-5, chirp_B=1e5)
    plan.handle = None
    with pytest.raises(ValueError):
        plan.range_compress(raw, out=narrow)
    with pytest.raises(ValueError):
        plan.range_compress(narrow)
    with pytest.raises(ValueError):
        plan.range_compress(raw, out=torch.zeros(4, 64, 1, dtype=torch.complex64))
