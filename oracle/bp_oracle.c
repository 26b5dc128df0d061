/*
 * CPU ORACLE for time-domain SAR backprojection -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this library.  The product path (the HIP library and its binding)
 * never calls it, links it or shares code with it.
 *
 * It is the plain definition of the method, in IEEE double precision, built
 * with -O2 -ffp-contract=off (no fused multiply-add, no fast-math), written
 * from the page "基于GPU的SAR后向投影成像优化与CUDA加速实践" (GPU-based SAR
 * backprojection imaging and CUDA acceleration):
 *
 *   section 1.1: every pixel sums, over all pulses, the echo sample found at the
 *                pixel's range for that pulse, after phase compensation;
 *   section 2.2: per pulse, (1) pixel coordinates, (2) antenna-to-pixel
 *                distance, (3) range index and interpolation into the
 *                range-compressed echo, (4) multiply by the phase term and
 *                accumulate; interpolation is nearest, linear or sinc;
 *   section 3.3: the range axis is r_k = r0 + k*dr, the pixel plane is a grid
 *                x_i = x0 + i*dx, y_j = y0 + j*dy, the image is indexed
 *                [j*nx + i], the phase term is 4*pi*R/lambda with the carrier
 *                wavelength (section 4.2).
 *
 * For pixel p_ij = (x0 + i dx, y0 + j dy, z0) and pulse n (antenna a_n):
 *   R = sqrt(dx*dx + dy*dy + dz*dz),  (dx, dy, dz) = p - a_n, summed left to right
 *   u = (R - r0) / dr
 *   nearest: v = s_n[floor(u + 1/2)]
 *   linear : k = floor(u), f = u - k, v = (1 - f) s_n[k] + f s_n[k + 1]
 *   sinc8  : k = floor(u), f = u - k, v = sum_{m=-3..4} s_n[k + m] h(f - m),
 *            h(t) = sinc(t) (0.54 + 0.46 cos(pi t / 4)) for |t| < 4, else 0
 *   s_n[k] = 0 for k outside [0, nr - 1]
 *   I_ij  += v * exp(+j 4 pi R / lambda)      (complex128, pulses in order)
 *
 * The sinc8 kernel shape is a reading (the page names sinc interpolation but
 * does not define it): eight taps, Hamming-windowed, not normalised.
 *
 * Terrain (section 3.3 notes that terrain height may have to be taken into
 * account): the *_dem variants place pixel (i, j) at height z0 + dem[j*nx + i]
 * instead of the plane z = z0; dem is float32, each value taken exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_PI 3.14159265358979323846

enum { ORC_NEAREST = 0, ORC_LINEAR = 1, ORC_SINC8 = 2 };

typedef struct {
    int na, nr;
    const double* pos;  /* [na][3] */
    const double* echo; /* [na][nr] complex128, interleaved re/im */
    double r0, dr, lam;
    int interp;
} orc_problem;

/* Echo sample with zero extension outside the record. */
static void sample_at(const double* row, int nr, int64_t k, double* re, double* im) {
    if (k < 0 || k >= nr) {
        *re = 0.0;
        *im = 0.0;
    } else {
        *re = row[2 * k];
        *im = row[2 * k + 1];
    }
}

/* The 8-tap Hamming-windowed sinc weight h(t). */
double oracle_sinc8_weight(double t) {
    if (!(fabs(t) < 4.0)) return 0.0;
    double sinc = (t == 0.0) ? 1.0 : sin(ORC_PI * t) / (ORC_PI * t);
    return sinc * (0.54 + 0.46 * cos(ORC_PI * t / 4.0));
}

/* Interpolated echo of one pulse at fractional bin position u. */
static void interpolate(const double* row, int nr, double u, int interp, double* vr, double* vi) {
    double ar, ai, br, bi;
    if (interp == ORC_NEAREST) {
        sample_at(row, nr, (int64_t)floor(u + 0.5), vr, vi);
    } else if (interp == ORC_LINEAR) {
        double kf = floor(u);
        double f = u - kf;
        int64_t k = (int64_t)kf;
        sample_at(row, nr, k, &ar, &ai);
        sample_at(row, nr, k + 1, &br, &bi);
        *vr = (1.0 - f) * ar + f * br;
        *vi = (1.0 - f) * ai + f * bi;
    } else {
        double kf = floor(u);
        double f = u - kf;
        int64_t k = (int64_t)kf;
        double sr = 0.0, si = 0.0;
        for (int m = -3; m <= 4; ++m) {
            double w = oracle_sinc8_weight(f - (double)m);
            sample_at(row, nr, k + m, &ar, &ai);
            sr += w * ar;
            si += w * ai;
        }
        *vr = sr;
        *vi = si;
    }
}

/* The coherent sum over all pulses for one pixel at (x, y, z). */
static void pixel_sum(const orc_problem* P, double x, double y, double z, double* outr, double* outi) {
    double accr = 0.0, acci = 0.0;
    for (int n = 0; n < P->na; ++n) {
        double ddx = x - P->pos[3 * n];
        double ddy = y - P->pos[3 * n + 1];
        double ddz = z - P->pos[3 * n + 2];
        double R = sqrt(ddx * ddx + ddy * ddy + ddz * ddz);
        double u = (R - P->r0) / P->dr;
        double vr, vi;
        interpolate(P->echo + (size_t)2 * P->nr * n, P->nr, u, P->interp, &vr, &vi);
        double ph = 4.0 * ORC_PI * R / P->lam;
        double c = cos(ph), s = sin(ph);
        accr += vr * c - vi * s;
        acci += vr * s + vi * c;
    }
    *outr = accr;
    *outi = acci;
}

static int check(int na, int nr, double dr, double lam, int interp) {
    if (na < 0 || nr <= 0) return -1;
    if (!(dr > 0.0) || !(lam > 0.0)) return -1;
    if (interp < ORC_NEAREST || interp > ORC_SINC8) return -1;
    return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Full image, rows j in [j0, j1): image receives (j1 - j0) rows of nx complex128. */
int oracle_backproject_rows(int na, int nr, const double* pos, const double* echo, double r0,
                            double dr, int nx, int ny, double x0, double y0, double z0, double dx,
                            double dy, double lam, int interp, int j0, int j1, double* image,
                            int nthreads) {
    if (check(na, nr, dr, lam, interp) || nx <= 0 || ny <= 0 || j0 < 0 || j1 > ny || j1 < j0) return -1;
    set_threads(nthreads);
    orc_problem P = {na, nr, pos, echo, r0, dr, lam, interp};
#pragma omp parallel for schedule(static)
    for (int j = j0; j < j1; ++j) {
        double y = y0 + (double)j * dy;
        for (int i = 0; i < nx; ++i) {
            double x = x0 + (double)i * dx;
            double* o = image + (size_t)2 * ((size_t)(j - j0) * nx + i);
            pixel_sum(&P, x, y, z0, o, o + 1);
        }
    }
    return 0;
}

/* Selected pixels (i, j) of the grid: ij is [npix][2] int64; out is [npix] complex128. */
int oracle_backproject_pixels(int na, int nr, const double* pos, const double* echo, double r0,
                              double dr, double x0, double y0, double z0, double dx, double dy,
                              double lam, int interp, int npix, const int64_t* ij, double* out,
                              int nthreads) {
    if (check(na, nr, dr, lam, interp) || npix < 0) return -1;
    set_threads(nthreads);
    orc_problem P = {na, nr, pos, echo, r0, dr, lam, interp};
#pragma omp parallel for schedule(dynamic, 16)
    for (int p = 0; p < npix; ++p) {
        double x = x0 + (double)ij[2 * p] * dx;
        double y = y0 + (double)ij[2 * p + 1] * dy;
        pixel_sum(&P, x, y, z0, out + 2 * (size_t)p, out + 2 * (size_t)p + 1);
    }
    return 0;
}

/* Nearest-bin index floor(u + 1/2) chosen for pulse position a (3 doubles) at
 * selected pixels: the integer decision the nearest interpolator takes. */
int oracle_nearest_index(const double* a, double r0, double dr, double x0, double y0, double z0,
                         double dx, double dy, int npix, const int64_t* ij, int64_t* k_out) {
    if (!(dr > 0.0) || npix < 0) return -1;
    for (int p = 0; p < npix; ++p) {
        double x = x0 + (double)ij[2 * p] * dx;
        double y = y0 + (double)ij[2 * p + 1] * dy;
        double ddx = x - a[0], ddy = y - a[1], ddz = z0 - a[2];
        double R = sqrt(ddx * ddx + ddy * ddy + ddz * ddz);
        double u = (R - r0) / dr;
        k_out[p] = (int64_t)floor(u + 0.5);
    }
    return 0;
}

/* As oracle_nearest_index, with pixel (i, j) at height z0 + dem[j * nx + i]
 * (terrain: the pixel height of the definition above). */
int oracle_nearest_index_dem(const double* a, double r0, double dr, double x0, double y0, double z0,
                             double dx, double dy, int nx, int ny, const float* dem, int npix, const int64_t* ij,
                             int64_t* k_out) {
    if (!(dr > 0.0) || npix < 0 || !dem || nx <= 0 || ny <= 0) return -1;
    for (int p = 0; p < npix; ++p) {
        const int64_t i = ij[2 * p], j = ij[2 * p + 1];
        if (i < 0 || i >= nx || j < 0 || j >= ny) return -1;
        double x = x0 + (double)i * dx;
        double y = y0 + (double)j * dy;
        double z = z0 + (double)dem[j * nx + i];
        double ddx = x - a[0], ddy = y - a[1], ddz = z - a[2];
        double R = sqrt(ddx * ddx + ddy * ddy + ddz * ddz);
        double u = (R - r0) / dr;
        k_out[p] = (int64_t)floor(u + 0.5);
    }
    return 0;
}

/* As oracle_backproject_rows, with pixel (i, j) at height z0 + dem[j * nx + i]. */
int oracle_backproject_rows_dem(int na, int nr, const double* pos, const double* echo, double r0,
                                double dr, int nx, int ny, double x0, double y0, double z0, double dx,
                                double dy, const float* dem, double lam, int interp, int j0, int j1,
                                double* image, int nthreads) {
    if (check(na, nr, dr, lam, interp) || nx <= 0 || ny <= 0 || j0 < 0 || j1 > ny || j1 < j0 || !dem) return -1;
    set_threads(nthreads);
    orc_problem P = {na, nr, pos, echo, r0, dr, lam, interp};
#pragma omp parallel for schedule(static)
    for (int j = j0; j < j1; ++j) {
        double y = y0 + (double)j * dy;
        for (int i = 0; i < nx; ++i) {
            double x = x0 + (double)i * dx;
            double z = z0 + (double)dem[(size_t)j * nx + i];
            double* o = image + (size_t)2 * ((size_t)(j - j0) * nx + i);
            pixel_sum(&P, x, y, z, o, o + 1);
        }
    }
    return 0;
}

/* As oracle_backproject_pixels, with pixel (i, j) at height z0 + dem[j * nx + i]. */
int oracle_backproject_pixels_dem(int na, int nr, const double* pos, const double* echo, double r0,
                                  double dr, double x0, double y0, double z0, double dx, double dy, int nx,
                                  const float* dem, double lam, int interp, int npix, const int64_t* ij,
                                  double* out, int nthreads) {
    if (check(na, nr, dr, lam, interp) || npix < 0 || nx <= 0 || !dem) return -1;
    set_threads(nthreads);
    orc_problem P = {na, nr, pos, echo, r0, dr, lam, interp};
#pragma omp parallel for schedule(dynamic, 16)
    for (int p = 0; p < npix; ++p) {
        double x = x0 + (double)ij[2 * p] * dx;
        double y = y0 + (double)ij[2 * p + 1] * dy;
        double z = z0 + (double)dem[(size_t)ij[2 * p + 1] * nx + ij[2 * p]];
        pixel_sum(&P, x, y, z, out + 2 * (size_t)p, out + 2 * (size_t)p + 1);
    }
    return 0;
}
