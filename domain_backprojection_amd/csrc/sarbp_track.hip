// Antenna positions interpolated from navigation samples (sarbp_interpolate_track,
// see include/sarbp.h): cubic Lagrange interpolation through the 4 samples around
// each pulse time, in double precision, one lane per pulse.
#include <math.h>

#include "sarbp_internal.h"

namespace {

__global__ __launch_bounds__(256) void track_kernel(const double* __restrict__ nav_t,
                                                    const double* __restrict__ nav_p, int m_nav,
                                                    const double* __restrict__ t_in, double* __restrict__ out,
                                                    int n) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= n) return;
    const double t = t_in[k];
    double px = NAN, py = NAN, pz = NAN;
    if (isfinite(t) && t >= nav_t[0] && t <= nav_t[m_nav - 1]) {
        // largest i with nav_t[i] <= t, within [0, m_nav - 2]
        int lo = 0, hi = m_nav - 1;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (nav_t[mid] <= t) lo = mid;
            else hi = mid;
        }
        int j0 = lo - 1;
        j0 = j0 < 0 ? 0 : (j0 > m_nav - 4 ? m_nav - 4 : j0);
        double ts[4];
        bool ok = true;
#pragma unroll
        for (int q = 0; q < 4; ++q) ts[q] = nav_t[j0 + q];
#pragma unroll
        for (int q = 0; q < 3; ++q) ok = ok && ts[q] < ts[q + 1];
        if (ok) {
            px = py = pz = 0.0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                double w = 1.0;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (r != q) w *= (t - ts[r]) / (ts[q] - ts[r]);
                const double* p = nav_p + 3 * (size_t)(j0 + q);
                px += w * p[0];
                py += w * p[1];
                pz += w * p[2];
            }
        }
    }
    out[3 * (size_t)k] = px;
    out[3 * (size_t)k + 1] = py;
    out[3 * (size_t)k + 2] = pz;
}

bool aligned8(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

} // namespace

extern "C" int sarbp_interpolate_track(const double* nav_t_d, const double* nav_xyz_d, int32_t n_nav,
                                       const double* t_d, double* positions_d, int32_t n, void* stream) {
    if (!aligned8(nav_t_d) || !aligned8(nav_xyz_d) || !aligned8(t_d) || !aligned8(positions_d) || n_nav < 4 ||
        n < 1)
        return SARBP_EINVAL;
    const uintptr_t o = reinterpret_cast<uintptr_t>(positions_d), ob = (uintptr_t)n * 3 * sizeof(double);
    const uintptr_t a = reinterpret_cast<uintptr_t>(nav_xyz_d), ab = (uintptr_t)n_nav * 3 * sizeof(double);
    const uintptr_t b = reinterpret_cast<uintptr_t>(nav_t_d), bb = (uintptr_t)n_nav * sizeof(double);
    const uintptr_t c = reinterpret_cast<uintptr_t>(t_d), cb = (uintptr_t)n * sizeof(double);
    if ((o < a + ab && a < o + ob) || (o < b + bb && b < o + ob) || (o < c + cb && c < o + ob))
        return SARBP_EINVAL; // the output overlaps an input
    hipLaunchKernelGGL(track_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), nav_t_d,
                       nav_xyz_d, (int)n_nav, t_d, positions_d, (int)n);
    return hipGetLastError() == hipSuccess ? SARBP_OK : SARBP_EDEVICE;
}
