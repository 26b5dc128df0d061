"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle under the acceptance bar.

Acceptance bar (floating point, from the workload statement):
  * rel-L2 = ||I_gpu - I_oracle|| / ||I_oracle|| <= 2e-3 over the compared pixels
  * every target's strongest pixel in a +-ceil(rho_az/dx) x +-ceil(rho_rg/dy) window
    around its true pixel is the same pixel in both images (nearest: up to the
    definition's own plateaus, see PEAK_TIE; every such tie is reported)
  * | 20 log10(|I_gpu| / |I_oracle|) | <= 0.05 dB at the oracle's peak pixel
Integer decisions (nearest bin) must match exactly.
"""
import math

import numpy as np

REL_L2 = 2e-3
PEAK_DB = 0.05
# With nearest interpolation the definition itself has plateaus: neighbouring pixels that
# select the same range bin for every pulse differ only through the phase term (on the tiny
# scene three pixels of one target differ by 2e-6).  There, and only there, the GPU's peak
# may sit on another pixel of the oracle's plateau: the oracle's gap between that pixel and
# its maximum must be at most PEAK_TIE (relative) and at most the GPU's own measured error in
# that window (the largest |I_gpu - I_oracle| there, relative to the peak), so the two
# candidates are indistinguishable at the precision the run shows.  Every such tie is
# recorded in TIES and printed.  Linear and sinc8 are continuous in the range and must put
# every peak on the oracle's pixel.
PEAK_TIE = 1e-4
TIES = []


def rel_l2(got, want):
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


def target_windows(scene):
    """(K, list of (i, j) arrays) pixel windows around each target, clipped to the grid."""
    import synth

    rho_az, rho_rg = synth.resolution(scene)
    hx = max(1, math.ceil(rho_az / scene.dx))
    hy = max(1, math.ceil(rho_rg / scene.dy))
    wins = []
    for (i, j) in scene.targets:
        ii, jj = np.meshgrid(np.arange(i - hx, i + hx + 1), np.arange(j - hy, j + hy + 1), indexing="xy")
        ok = (ii >= 0) & (ii < scene.nx) & (jj >= 0) & (jj < scene.ny)
        wins.append(np.stack([ii[ok], jj[ok]], 1))
    return wins


def check_peaks(got_at, want_at, wins, interp, label=""):
    """got_at / want_at: callables mapping an (P, 2) pixel array to complex values.  Returns
    the worst peak magnitude difference in dB over the windows."""
    worst = 0.0
    for w in wins:
        g = got_at(w)
        o = want_at(w)
        ao = np.abs(o)
        kg, ko = int(np.argmax(np.abs(g))), int(np.argmax(ao))
        if kg != ko:
            gap = (ao[ko] - ao[kg]) / ao[ko]
            err = float(np.max(np.abs(g - o)) / ao[ko])
            tie = interp == "nearest" and gap <= PEAK_TIE and gap <= err
            rec = {"label": label, "gpu": w[kg].tolist(), "oracle": w[ko].tolist(), "gap": float(gap),
                   "window_error": err, "accepted": bool(tie)}
            TIES.append(rec)
            print(f"[peak tie] {label} gpu {w[kg].tolist()} oracle {w[ko].tolist()}: oracle gap {gap:.3g}, "
                  f"GPU error in the window {err:.3g} -> {'accepted' if tie else 'rejected'}", flush=True)
            assert tie, (f"peak moved: gpu {w[kg]} oracle {w[ko]} (oracle there {ao[kg]:.6g} vs {ao[ko]:.6g}, "
                         f"gap {gap:.3g}, window error {err:.3g}, {interp})")
        db = 20 * math.log10(abs(g[ko]) / ao[ko])
        assert abs(db) <= PEAK_DB, f"peak magnitude differs by {db:.4f} dB at {w[ko]}"
        worst = max(worst, abs(db))
    return worst


def sample_pixels(scene, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    i = rng.integers(0, scene.nx, count)
    j = rng.integers(0, scene.ny, count)
    edge = np.array([[0, 0], [scene.nx - 1, 0], [0, scene.ny - 1], [scene.nx - 1, scene.ny - 1]])
    return np.concatenate([np.stack([i, j], 1), edge])
