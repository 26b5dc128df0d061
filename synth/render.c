/*
 * Seeded-scene echo renderer (test and benchmark input generator).
 *
 * This file produces the synthetic echoes that both the CPU oracle and the HIP
 * library consume.  It is a forward model (scene -> echo), not backprojection:
 * it holds none of the image-formation arithmetic and shares no code with
 * either consumer.
 *
 * Echo model (range-compressed, unit-amplitude point scatterers):
 *   s_n[k] += a * sinc(beta * (k - u)) * exp(-j 4 pi R / lambda),
 *   u = (R - r0) / dr,  R = |p - a_n|,  sinc(x) = sin(pi x) / (pi x),
 * with beta = B / fs (the range impulse response of a band-limited pulse
 * sampled at fs).  The point-target simulation approach follows the debugging
 * advice of the page "基于GPU的SAR后向投影成像优化与CUDA加速实践" (GPU-based
 * SAR backprojection imaging and CUDA acceleration), section 4.2.
 *
 * Raw LFM model (before range compression), section 3.1 of the same page:
 *   x_n[m] += a * exp(-j 4 pi R / lambda) * p(t_m - 2R/c),
 *   p(t) = exp(j pi K t^2) for -T/2 <= t < T/2, else 0,  t_m = t0 + m / fs.
 *
 * Every routine accumulates into a caller-owned complex128 buffer (interleaved
 * re, im), parallel over pulses with a fixed per-row order, so the result does
 * not depend on the thread count.  Built with -ffp-contract=off so that
 * vectorised and scalar code round identically.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SYN_PI 3.14159265358979323846

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* sin and cos of 2*pi*x (x in cycles): reduce to z in [-pi/4, pi/4] by quarter
 * turns, then Taylor series to z^15 (truncation < 3e-14).  Branch-free pure
 * arithmetic, so it vectorises and does not depend on the host's libm. */
static inline void sincos_cycles(double x, double* s, double* c) {
    double r = x - floor(x + 0.5);
    double y = 4.0 * r;
    double q = floor(y + 0.5);
    double z = (y - q) * (SYN_PI / 2.0);
    double z2 = z * z;
    double sz = z * (1.0 + z2 * (-1.0 / 6.0 + z2 * (1.0 / 120.0 + z2 * (-1.0 / 5040.0 +
                z2 * (1.0 / 362880.0 + z2 * (-1.0 / 39916800.0 + z2 * (1.0 / 6227020800.0 +
                z2 * (-1.0 / 1307674368000.0))))))));
    double cz = 1.0 + z2 * (-0.5 + z2 * (1.0 / 24.0 + z2 * (-1.0 / 720.0 + z2 * (1.0 / 40320.0 +
                z2 * (-1.0 / 3628800.0 + z2 * (1.0 / 479001600.0 + z2 * (-1.0 / 87178291200.0)))))));
    /* rotate by (q mod 4) quarter turns */
    double qm = q - 4.0 * floor(q * 0.25); /* 0, 1, 2, 3 */
    double odd = (qm == 1.0 || qm == 3.0) ? 1.0 : 0.0;
    double sgn = (qm >= 2.0) ? -1.0 : 1.0;
    *s = sgn * (odd * cz + (1.0 - odd) * sz);
    *c = sgn * (odd * (-sz) + (1.0 - odd) * cz);
}

static void tap_tables(int half, double beta, double* Sm, double* Cm) {
    for (int m = -half; m <= half; ++m) {
        Sm[m + half] = sin(SYN_PI * beta * m);
        Cm[m + half] = cos(SYN_PI * beta * m);
    }
}

/* Tap weights of one scatterer: the 2*half+1 bins k0-half .. k0+half around
 * k0 = round(u), each sinc(beta (k - u)) times the phase (cph, sph).
 * w receives (re, im) pairs; ws receives the rotated pairs (-im, re), so a
 * complex multiply-accumulate by sigma = (sr, si) is acc += sr*w + si*ws. */
static inline int tap_weights(double u, double beta, double cph, double sph, int half,
                              const double* Sm, const double* Cm, double* w, double* ws) {
    double k0 = floor(u + 0.5);
    double e = u - k0; /* in [-0.5, 0.5] */
    double se, ce;
    sincos_cycles(0.5 * beta * e, &se, &ce);
    for (int m = -half; m <= half; ++m) {
        double t = (double)m - e; /* = k - u */
        double s = Sm[m + half] * ce - Cm[m + half] * se; /* sin(pi beta t) */
        double den = SYN_PI * beta * t;
        double val = fabs(t) < 1e-12 ? 1.0 : s / den;
        int o = 2 * (m + half);
        w[o] = val * cph;
        w[o + 1] = val * sph;
        ws[o] = -val * sph;
        ws[o + 1] = val * cph;
    }
    return (int)k0;
}

/* Accumulate runs of consecutive scatterers that share the same tap window
 * (first bin) in registers, then add each run to the padded row.  K[p] is the
 * window's first bin in padded coordinates; W/WS hold 2*ntap doubles per p. */
static inline void accumulate_runs(int np, const int* K, const double* W, const double* WS,
                                   const double* sig, int ntap, double* prow, double* acc) {
    const int nw = 2 * ntap;
    int kcur = K[0];
    for (int t = 0; t < nw; ++t) acc[t] = 0.0;
    for (int p = 0; p < np; ++p) {
        if (K[p] != kcur) {
            double* r = prow + 2 * (size_t)kcur;
            for (int t = 0; t < nw; ++t) {
                r[t] += acc[t];
                acc[t] = 0.0;
            }
            kcur = K[p];
        }
        const double sr = sig[2 * p], si = sig[2 * p + 1];
        const double* w = W + (size_t)nw * p;
        const double* ws = WS + (size_t)nw * p;
#pragma omp simd
        for (int t = 0; t < nw; ++t) acc[t] += sr * w[t] + si * ws[t];
    }
    double* r = prow + 2 * (size_t)kcur;
    for (int t = 0; t < nw; ++t) r[t] += acc[t];
}

/* Padded accumulation rows cover bins [-pad, nr + pad) with pad = 2*half, so
 * every window that overlaps the record fits.  Returns the window's first bin
 * in padded coordinates, or -1 when the window misses the record entirely. */
static inline int padded_k(int k0, int half, int pad, int nr) {
    if (k0 + half < 0 || k0 - half > nr - 1) return -1;
    return k0 - half + pad;
}

/* A window that misses the record contributes nothing: zero its weights and
 * park it at padded bin 0. */
static inline int park_if_outside(int kp, int nw, double* w, double* ws) {
    if (kp >= 0) return kp;
    for (int t = 0; t < nw; ++t) w[t] = ws[t] = 0.0;
    return 0;
}

static void unpad_add(int na, int nr, int pad, const double* padded, double* echo) {
#pragma omp parallel for schedule(static)
    for (int n = 0; n < na; ++n) {
        const double* src = padded + (size_t)2 * (nr + 2 * pad) * n + 2 * pad;
        double* dst = echo + (size_t)2 * nr * n;
        for (int k = 0; k < 2 * nr; ++k) dst[k] += src[k];
    }
}

/*
 * Point scatterers at arbitrary positions, any trajectory (direct evaluation).
 * half >= 0 truncates each range profile to +-half bins around the peak;
 * half < 0 evaluates the full record.
 */
int synth_render_sinc(int na, int nr, const double* pos, double r0, double dr, double lam,
                      double beta, int npts, const double* pts, const double* amp, int half,
                      double* echo, int nthreads) {
    if (na <= 0 || nr <= 0 || npts < 0 || dr <= 0 || lam <= 0) return -1;
    if (npts == 0) return 0;
    set_threads(nthreads);
    if (half < 0) {
        /* full record: plain loops (used for the few targets of small scenes) */
#pragma omp parallel for schedule(static)
        for (int n = 0; n < na; ++n) {
            double* row = echo + (size_t)2 * nr * n;
            for (int p = 0; p < npts; ++p) {
                double dx = pts[3 * p] - pos[3 * n], dy = pts[3 * p + 1] - pos[3 * n + 1];
                double dz = pts[3 * p + 2] - pos[3 * n + 2];
                double R = sqrt(dx * dx + dy * dy + dz * dz);
                double u = (R - r0) / dr;
                double c, s;
                sincos_cycles(-2.0 * R / lam, &s, &c);
                double cph = amp[2 * p] * c - amp[2 * p + 1] * s;
                double sph = amp[2 * p] * s + amp[2 * p + 1] * c;
                for (int k = 0; k < nr; ++k) {
                    double t = (double)k - u;
                    double val = fabs(t) < 1e-12 ? 1.0 : sin(SYN_PI * beta * t) / (SYN_PI * beta * t);
                    row[2 * k] += val * cph;
                    row[2 * k + 1] += val * sph;
                }
            }
        }
        return 0;
    }
    const int ntap = 2 * half + 1, nw = 2 * ntap, pad = 2 * half;
    const int nrp = nr + 2 * pad;
    double* Sm = (double*)malloc(sizeof(double) * ntap);
    double* Cm = (double*)malloc(sizeof(double) * ntap);
    tap_tables(half, beta, Sm, Cm);
    double* padded = (double*)calloc((size_t)2 * nrp * na, sizeof(double));
    const int blk = 4096; /* scatterers per block */
#pragma omp parallel
    {
        int* K = (int*)malloc(sizeof(int) * blk);
        double* W = (double*)malloc(sizeof(double) * (size_t)nw * blk);
        double* WS = (double*)malloc(sizeof(double) * (size_t)nw * blk);
        double* SG = (double*)malloc(sizeof(double) * 2 * blk);
        double* acc = (double*)malloc(sizeof(double) * nw);
#pragma omp for schedule(static)
        for (int n = 0; n < na; ++n) {
            const double ax = pos[3 * n], ay = pos[3 * n + 1], az = pos[3 * n + 2];
            double* prow = padded + (size_t)2 * nrp * n;
            for (int p0 = 0; p0 < npts; p0 += blk) {
                int np = npts - p0 < blk ? npts - p0 : blk;
                for (int q = 0; q < np; ++q) {
                    int p = p0 + q;
                    double dx = pts[3 * p] - ax, dy = pts[3 * p + 1] - ay, dz = pts[3 * p + 2] - az;
                    double R = sqrt(dx * dx + dy * dy + dz * dz);
                    double u = (R - r0) / dr;
                    double c, s;
                    sincos_cycles(-2.0 * R / lam, &s, &c);
                    int k0 = tap_weights(u, beta, c, s, half, Sm, Cm, W + (size_t)nw * q,
                                         WS + (size_t)nw * q);
                    K[q] = park_if_outside(padded_k(k0, half, pad, nr), nw, W + (size_t)nw * q,
                                           WS + (size_t)nw * q);
                    SG[2 * q] = amp[2 * p];
                    SG[2 * q + 1] = amp[2 * p + 1];
                }
                accumulate_runs(np, K, W, WS, SG, ntap, prow, acc);
            }
        }
        free(K);
        free(W);
        free(WS);
        free(SG);
        free(acc);
    }
    unpad_add(na, nr, pad, padded, echo);
    free(padded);
    free(Sm);
    free(Cm);
    return 0;
}

/*
 * Distributed scatterers, one per grid cell (reflectivity sigma[j][i]), for a
 * straight track whose pulse spacing equals the grid's x spacing:
 *   a_n = (ax0 + n * dxg, ay, az),   cell (i, j) = (x0 + i dxg, y0 + j dy, z0).
 * Then x_i - ax_n depends only on q = i - n, so each cell row's tap weights
 * are tabulated once per q and reused for every pulse.  Same model as
 * synth_render_sinc with the same half (up to rounding of the coordinates).
 */
int synth_render_sinc_grid_straight(int na, int nr, double ax0, double ay, double az, double r0,
                                    double dr, double lam, double beta, int nx, int ny, double x0,
                                    double y0, double z0, double dxg, double dy, const double* sigma,
                                    int half, double* echo, int nthreads) {
    if (na <= 0 || nr <= 0 || nx <= 0 || ny <= 0 || half < 0 || dr <= 0 || lam <= 0) return -1;
    set_threads(nthreads);
    const int ntap = 2 * half + 1, nw = 2 * ntap, pad = 2 * half;
    const int nrp = nr + 2 * pad;
    double* Sm = (double*)malloc(sizeof(double) * ntap);
    double* Cm = (double*)malloc(sizeof(double) * ntap);
    tap_tables(half, beta, Sm, Cm);
    const int nq = na + nx - 1; /* q = i - n in [-(na-1), nx-1] */
    double* W = (double*)malloc(sizeof(double) * (size_t)nw * nq);
    double* WS = (double*)malloc(sizeof(double) * (size_t)nw * nq);
    int* K = (int*)malloc(sizeof(int) * (size_t)nq);
    double* padded = (double*)calloc((size_t)2 * nrp * na, sizeof(double));
    const double xoff = x0 - ax0; /* x_i - ax_n = xoff + q * dxg */
    for (int j = 0; j < ny; ++j) {
        const double ddy = (y0 + j * dy) - ay, ddz = z0 - az;
#pragma omp parallel for schedule(static)
        for (int iq = 0; iq < nq; ++iq) {
            int q = iq - (na - 1);
            double ddx = xoff + q * dxg;
            double R = sqrt(ddx * ddx + ddy * ddy + ddz * ddz);
            double u = (R - r0) / dr;
            double sp, cp;
            sincos_cycles(-2.0 * R / lam, &sp, &cp);
            int k0 = tap_weights(u, beta, cp, sp, half, Sm, Cm, W + (size_t)nw * iq, WS + (size_t)nw * iq);
            K[iq] = park_if_outside(padded_k(k0, half, pad, nr), nw, W + (size_t)nw * iq,
                                    WS + (size_t)nw * iq);
        }
        const double* srow = sigma + (size_t)2 * nx * j;
#pragma omp parallel
        {
            double* acc = (double*)malloc(sizeof(double) * nw);
#pragma omp for schedule(static)
            for (int n = 0; n < na; ++n) {
                const int iq0 = (na - 1) - n; /* iq of cell i = 0 */
                accumulate_runs(nx, K + iq0, W + (size_t)nw * iq0, WS + (size_t)nw * iq0, srow, ntap,
                                padded + (size_t)2 * nrp * n, acc);
            }
            free(acc);
        }
    }
    unpad_add(na, nr, pad, padded, echo);
    free(padded);
    free(W);
    free(WS);
    free(K);
    free(Sm);
    free(Cm);
    return 0;
}

/* Raw (uncompressed) LFM echoes of point scatterers, any trajectory. */
int synth_render_chirp(int na, int nfast, const double* pos, double t0, double fs, double lam,
                       double c, double chirp_T, double chirp_K, int npts, const double* pts,
                       const double* amp, double* raw, int nthreads) {
    if (na <= 0 || nfast <= 0 || fs <= 0 || chirp_T <= 0) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < na; ++n) {
        double ax = pos[3 * n], ay = pos[3 * n + 1], az = pos[3 * n + 2];
        double* row = raw + (size_t)2 * nfast * n;
        for (int p = 0; p < npts; ++p) {
            double dx = pts[3 * p] - ax, dy = pts[3 * p + 1] - ay, dz = pts[3 * p + 2] - az;
            double R = sqrt(dx * dx + dy * dy + dz * dz);
            double tau = 2.0 * R / c;
            double sp, cp;
            sincos_cycles(-2.0 * R / lam, &sp, &cp);
            double cph = amp[2 * p] * cp - amp[2 * p + 1] * sp;
            double sph = amp[2 * p] * sp + amp[2 * p + 1] * cp;
            /* samples m with -T/2 <= t0 + m/fs - tau < T/2 */
            long mlo = (long)ceil((tau - 0.5 * chirp_T - t0) * fs) - 1;
            long mhi = (long)floor((tau + 0.5 * chirp_T - t0) * fs) + 1;
            if (mlo < 0) mlo = 0;
            if (mhi > nfast - 1) mhi = nfast - 1;
            for (long m = mlo; m <= mhi; ++m) {
                double t = t0 + (double)m / fs - tau;
                if (t < -0.5 * chirp_T || t >= 0.5 * chirp_T) continue;
                double pr, pi_;
                sincos_cycles(0.5 * chirp_K * t * t, &pi_, &pr);
                row[2 * m] += cph * pr - sph * pi_;
                row[2 * m + 1] += cph * pi_ + sph * pr;
            }
        }
    }
    return 0;
}
