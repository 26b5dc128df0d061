"""Nearest-bin index probe on the GPU: one pulse per call with the real echo s[k] = k + 1, so
|I(p)| - 1 is the bin the kernel chose for pixel p (0 where that bin lies outside the record),
compared with the oracle's floor(u + 1/2) in double precision."""
import sys

import numpy as np

import oracle


def nearest_index_mismatches(sb, scene, pulses, dem=None, layers=None, **plan_kw):
    """Count pixels x pulses where the GPU's nearest bin differs from the oracle's.

    scene: a synth.Scene (its geometry; its echo is replaced by the ramp).
    dem:   float32 (ny, nx) heights (the terrain kernels), or None.
    layers: (nz, dz) for a volume, or None."""
    import torch

    nr = scene.nr
    ramp = torch.arange(1, nr + 1, dtype=torch.float32).to(torch.complex64).cuda()[None, :].contiguous()
    ii, jj = np.meshgrid(np.arange(scene.nx), np.arange(scene.ny), indexing="xy")
    ij = np.stack([ii.ravel(), jj.ravel()], 1)
    kw = dict(plan_kw)
    kw.update(interp="nearest", n_pulses=1)
    dem_d = None
    if dem is not None:
        kw["dem_relief"] = plan_kw.get("dem_relief", 0.0) or max(float(dem.max() - dem.min()), 1e-3)
        dem_d = torch.from_numpy(np.ascontiguousarray(dem, dtype=np.float32)).cuda()
    nz, dz = (layers if layers is not None else (1, 0.0))
    if layers is not None:
        kw.update(nz=nz, dz=dz)
    mismatches = 0
    with sb.Plan.for_scene(scene, **kw) as plan:
        img = plan.new_image()
        for n in pulses:
            pos = torch.from_numpy(np.ascontiguousarray(scene.positions[n:n + 1])).cuda()
            plan.backproject(pos, ramp, image=img, dem=dem_d)
            mag = img.abs().cpu().numpy().astype(np.float64).reshape(nz, -1)
            assert np.max(np.abs(mag - np.rint(mag))) < 0.02, "probe magnitude is not an integer"
            for layer in range(nz):
                k = oracle.nearest_index(scene.positions[n], scene.r0, scene.dr, scene.x0, scene.y0,
                                         scene.z0 + layer * dz, scene.dx, scene.dy, ij, dem=dem)
                want = np.where((k >= 0) & (k < nr), k + 1, 0)
                mismatches += int(np.count_nonzero(np.rint(mag[layer]) != want))
    return mismatches


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
