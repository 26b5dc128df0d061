"""CPU checks of the integer index schemes the kernels rely on, written out again here
from their stated rules (no GPU; the kernels' own arithmetic is covered by the GPU
parity tests):

* backprojection staging divides a step index u by the chunk window's step count wu
  as trunc(u * fl32(1 / wu)) in fp32, corrected by one either way; u stays below the
  LDS entries of a chunk (at most 150 KiB / 8 B = 19200), where the quotient must be
  exact;
* the range-compression FFT stores pass outputs in a padded LDS layout: a pass with
  Ns < 32 (other than a transform's last) stores entry i at i + Ns floor(i / (Ns R)).
  Every pass must write distinct slots inside 9N/8 entries, the next pass must read
  back exactly what was written, and each 32-lane half of a wave must store to 32
  distinct 8-byte slots modulo 32 (one bank row).  The inverse transform runs the
  forward's radices in reverse order, and its first pass is fused with the forward's
  last: butterfly j of both must cover the same points j + r N/R.
"""
import numpy as np
import pytest


def test_window_step_division_is_exact():
    u = np.arange(19200, dtype=np.int64)
    uf = u.astype(np.float32)
    for wu in range(3, 19201):
        rwu = np.float32(1.0) / np.float32(wu)  # correctly rounded fp32 reciprocal
        p = (uf * rwu).astype(np.int64)  # fp32 product, truncated
        r = u - p * wu
        p = np.where(r < 0, p - 1, np.where(r >= wu, p + 1, p))
        assert np.array_equal(p, u // wu), wu


def _radix(L, p, inv=False):
    n8 = {1: 3, 2: 2, 3: 1, 0: 0}[L % 4]
    P = _passes(L)
    q = P - 1 - p if inv else p
    return 8 if q < n8 else 16


def _passes(L):
    n8 = {1: 3, 2: 2, 3: 1, 0: 0}[L % 4]
    return n8 + (L - 3 * n8) // 4


@pytest.mark.parametrize("L", range(6, 15))
def test_rc_padded_layout(L):
    N = 1 << L
    P = _passes(L)
    assert np.prod([_radix(L, p) for p in range(P)]) == N
    cap = N // 8 * 9
    written = None
    for transform in range(2):
        ns, pad_prev = 1, 0
        for p in range(P):
            R = _radix(L, p, inv=transform == 1)
            nb = N // R
            last = p == P - 1
            pad_w = ns if (not last and ns < 32) else 0
            j = np.arange(nb)
            if p > 0 or transform == 1:
                pad_r = pad_prev if p > 0 else 0
                for r in range(R):
                    idx = j + r * nb
                    phys = idx + (pad_r * (j // ns) if pad_r else 0) + pad_r * (r * nb // ns)
                    assert phys.max() < cap
                    assert np.array_equal(written[phys], idx), (L, transform, p, r)
            k = j & (ns - 1)
            base = (j // ns) * ns * R + k + (pad_w * (j // ns) if pad_w else 0)
            out = np.full(cap, -1)
            for r in range(R):
                phys = base + r * ns
                logical = (j // ns) * ns * R + k + r * ns
                assert phys.max() < cap and np.all(out[phys] == -1), (L, transform, p, r)
                out[phys] = logical
                if not last or transform == 0:
                    for h in range(0, nb, 32):
                        assert len(np.unique(phys[h:h + 32] % 32)) == min(32, nb - h), (L, transform, p, r)
            written = out
            pad_prev = pad_w
            ns *= R
        if transform == 0:
            # the fused pass reads the forward transform's output in natural order
            assert np.array_equal(written[:N], np.arange(N))
            # ... where the forward's last butterfly j and the inverse's first cover the same points
            Rf, Ri = _radix(L, P - 1), _radix(L, 0, inv=True)
            assert Rf == Ri
            nb = N // Rf
            fwd_out = [sorted((np.arange(nb)[:, None] + np.arange(Rf)[None, :] * nb)[j]) for j in range(nb)]
            inv_in = [sorted(j + np.arange(Ri) * (N // Ri)) for j in range(N // Ri)]
            assert all(np.array_equal(a, b) for a, b in zip(fwd_out, inv_in))
