// Host side of the sarbp C ABI: argument validation, plan creation (the
// carrier-phase and matched-filter tables, the sinc8 polynomials, the progress
// hints), the device entry points' dispatch and status strings.  See
// include/sarbp.h.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <complex>
#include <new>
#include <vector>

#include "sarbp_geom.h"
#include "sarbp_internal.h"

int sarbp_rc_prepare_device();
int sarbp_bp_allow_lds(int interp, int accum, bool dem, int ppt, bool f64, size_t bytes);

namespace {

constexpr double kPi = 3.14159265358979323846;

bool finite_pos(double v) { return isfinite(v) && v > 0.0; }

bool aligned8(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// In-place iterative radix-2 FFT (forward, exp(-2 pi i n k / N)) in double
// precision, used once at plan creation for the matched filter's spectrum.
void fft_host(std::vector<std::complex<double>>& a) {
    const size_t n = a.size();
    for (size_t i = 1, j = 0; i < n; ++i) {
        size_t bit = n >> 1;
        for (; j & bit; bit >>= 1) j ^= bit;
        j ^= bit;
        if (i < j) std::swap(a[i], a[j]);
    }
    for (size_t len = 2; len <= n; len <<= 1) {
        for (size_t i = 0; i < n; i += len) {
            for (size_t k = 0; k < len / 2; ++k) {
                const double ang = -2.0 * kPi * (double)k / (double)len;
                const std::complex<double> w(cos(ang), sin(ang));
                const std::complex<double> u = a[i + k], v = a[i + k + len / 2] * w;
                a[i + k] = u + v;
                a[i + k + len / 2] = u - v;
            }
        }
    }
}

} // namespace

int sarbp_validate(const sarbp_params* p) {
    if (p == nullptr) return SARBP_EINVAL;
    if (p->n_pulses < 1 || p->nx < 1 || p->ny < 1) return SARBP_EINVAL;
    if (p->interp < SARBP_NEAREST || p->interp > SARBP_SINC8) return SARBP_EINVAL;
    if (p->accum < SARBP_ACC_FP32 || p->accum > SARBP_ACC_CHUNK64) return SARBP_EINVAL;
    if (!isfinite(p->dem_relief) || p->dem_relief < 0.0 || p->dem_relief > 1.0e4) return SARBP_EINVAL;
    if (p->nz < 0 || p->nz > 65535) return SARBP_EINVAL;
    if (p->nz > 1 && (!finite_pos(p->dz) || p->dem_relief > 0.0)) return SARBP_EINVAL; // volume xor terrain
    if (p->n_range < (p->interp == SARBP_SINC8 ? 8 : 2)) return SARBP_EINVAL;
    if (!isfinite(p->r0) || !finite_pos(p->dr) || !finite_pos(p->dx) || !finite_pos(p->dy)) return SARBP_EINVAL;
    if (!isfinite(p->x0) || !isfinite(p->y0) || !isfinite(p->z0) || !finite_pos(p->wavelength)) return SARBP_EINVAL;
    if ((int64_t)p->nx * p->ny > (int64_t)1 << 40) return SARBP_EINVAL;
    // The per-sample rotation takes v_sin/v_cos of kappa f revolutions, kappa = 2 dr /
    // lambda and f in [0, 1); those instructions accept at most 256 revolutions.
    if (!(2.0 * p->dr / p->wavelength < 255.0)) return SARBP_EUNSUPPORTED;
    if (p->n_fast != 0) {
        if (p->n_fast < 64 || p->n_fast > 16384 || (p->n_fast & (p->n_fast - 1)) != 0) return SARBP_EINVAL;
        if (!finite_pos(p->fs) || !finite_pos(p->chirp_T) || !finite_pos(p->chirp_B)) return SARBP_EINVAL;
        const double L = floor(p->chirp_T * p->fs + 0.5);
        if (L < 1.0 || L > (double)p->n_fast) return SARBP_EINVAL;
        if (p->window < 0 || p->window > 2) return SARBP_EINVAL;
        if (p->window == 2) {
            if (p->taylor_nbar != 0 && (p->taylor_nbar < 2 || p->taylor_nbar > 64)) return SARBP_EINVAL;
            if (p->taylor_sll != 0.0 && !(p->taylor_sll >= 13.0 && p->taylor_sll <= 150.0)) return SARBP_EINVAL;
        }
    }
    return SARBP_OK;
}

namespace {

template <typename T>
int upload(const std::vector<T>& host, T** dev) {
    *dev = nullptr;
    if (hipMalloc(reinterpret_cast<void**>(dev), host.size() * sizeof(T)) != hipSuccess) {
        *dev = nullptr;
        return SARBP_ENOMEM;
    }
    if (hipMemcpy(*dev, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return SARBP_EDEVICE;
    return SARBP_OK;
}

void release(sarbp_plan* plan) {
    if (plan == nullptr) return;
    int cur = -1;
    const bool switch_dev = hipGetDevice(&cur) == hipSuccess && cur != plan->device;
    if (switch_dev) (void)hipSetDevice(plan->device);
    if (plan->phase_tab) (void)hipFree(plan->phase_tab);
    if (plan->rc_filter) (void)hipFree(plan->rc_filter);
    if (plan->progress) (void)hipFree(plan->progress);
    if (switch_dev) (void)hipSetDevice(cur);
    delete plan;
}

// Carrier phase of each range bin: exp(+j 4 pi (r0 + k dr) / lambda) at [k + 4],
// k = -4 .. n_range + 3 (every bin whose interpolation taps can reach the
// record), reduced modulo one cycle in double precision.
std::vector<float2> phase_table(const sarbp_params& p) {
    // bins -4 .. n_range + 3, then two NaN entries (the window of a pulse with no finite geometry)
    std::vector<float2> t((size_t)p.n_range + 10, make_float2(NAN, NAN));
    for (int64_t k = -4; k <= (int64_t)p.n_range + 3; ++k) {
        const double cyc = 2.0 * (p.r0 + (double)k * p.dr) / p.wavelength;
        const double fr = cyc - floor(cyc);
        t[(size_t)(k + 4)] = make_float2((float)cos(2.0 * kPi * fr), (float)sin(2.0 * kPi * fr));
    }
    return t;
}

// Taylor taper at x in [-1/2, 1/2] with nbar nearly equal sidelobes at sll dB
// below the peak, scaled to 1 at x = 0 (the classical Taylor line-source
// weighting: A = acosh(10^(sll/20)) / pi, sigma^2 = nbar^2 / (A^2 + (nbar - 1/2)^2),
// w = 1 + 2 sum_m F_m cos(2 pi m x) with the F_m below).
struct TaylorTaper {
    double F[64];
    int nbar;
    double centre;
    TaylorTaper(int nbar_, double sll) : nbar(nbar_), centre(1.0) {
        const double A = acosh(pow(10.0, sll / 20.0)) / kPi;
        const double s2 = (double)nbar * nbar / (A * A + (nbar - 0.5) * (nbar - 0.5));
        for (int m = 1; m < nbar; ++m) {
            double num = 1.0, den = 1.0;
            for (int n = 1; n < nbar; ++n) {
                num *= 1.0 - (double)m * m / (s2 * (A * A + (n - 0.5) * (n - 0.5)));
                if (n != m) den *= 1.0 - (double)m * m / ((double)n * n);
            }
            F[m] = ((m & 1) ? 0.5 : -0.5) * num / den;
            centre += 2.0 * F[m];
        }
    }
    double operator()(double x) const {
        double w = 1.0;
        for (int m = 1; m < nbar; ++m) w += 2.0 * F[m] * cos(2.0 * kPi * m * x);
        return w / centre;
    }
};

// The 8-tap interpolation kernel of the page's sinc option: sinc(t) times a
// Hamming-type taper over its 8-sample support, h(t) = sinc(t) (0.54 + 0.46
// cos(pi t / 4)) for |t| < 4.
double sinc8_kernel(double t) {
    if (fabs(t) >= 4.0) return 0.0;
    const double s = t == 0.0 ? 1.0 : sin(kPi * t) / (kPi * t);
    return s * (0.54 + 0.46 * cos(kPi * t / 4.0));
}

// For taps mo = -3 .. 0 the weight h(f - mo), f in [0, 1), as a degree-7
// polynomial in g = f - 1/2: interpolation at the 8 Chebyshev nodes of
// [-1/2, 1/2] (largest deviation from h below 7e-7), solved in the monomial
// basis by Gaussian elimination in double precision.  Taps 1 - mo are the
// mirror images, h(f - (1 - mo)) = h(-g + 1/2 - mo), so they need no table.
// Layout: coefficient j of tap mo = t - 3 at [4 j + t].
void sinc8_polynomials(float* out) {
    for (int t = 0; t < 4; ++t) {
        const int mo = t - 3;
        double V[8][9];
        for (int i = 0; i < 8; ++i) {
            const double x = 0.5 * cos(kPi * (2 * i + 1) / 16.0);
            double xp = 1.0;
            for (int j = 0; j < 8; ++j, xp *= x) V[i][j] = xp;
            V[i][8] = sinc8_kernel(x + 0.5 - mo);
        }
        for (int c = 0; c < 8; ++c) {
            int piv = c;
            for (int r = c + 1; r < 8; ++r)
                if (fabs(V[r][c]) > fabs(V[piv][c])) piv = r;
            for (int j = 0; j < 9; ++j) std::swap(V[c][j], V[piv][j]);
            for (int r = 0; r < 8; ++r) {
                if (r == c) continue;
                const double q = V[r][c] / V[c][c];
                for (int j = c; j < 9; ++j) V[r][j] -= q * V[c][j];
            }
        }
        for (int j = 0; j < 8; ++j) out[4 * j + t] = (float)(V[j][8] / V[j][j]);
    }
}

} // namespace

int sarbp_plan_layout(const sarbp_params& p, int n_cu, BpLayout* L) {
    memset(L, 0, sizeof(*L));
    L->n_cu = n_cu < 1 ? 1 : n_cu;
    // Backprojection tiling and LDS window size.  Every pixel of a tile lies
    // within half_span of the tile centre, so (triangle inequality) its range
    // lies within R_t +- half_span and its bin within the window below.
    // Two pixels per lane (64 x 32 tiles) unless that leaves fewer than two tiles
    // per CU: then one (64 x 16), which doubles the workgroups (measured on a
    // 2048 x 128 grid: 4.22 -> 2.56 ms; on 1024 x 1024, one pixel per lane is 20 %
    // slower, so large grids keep two).  Terrain plans keep 64 x 32 tiles: the
    // relief bound and its NaN blocks are defined on them.
    const int64_t layers = p.nz > 1 ? p.nz : 1;
    L->tiles_x = (p.nx + BP_TX - 1) / BP_TX;
    const int64_t tiles2 = (int64_t)L->tiles_x * ((p.ny + 2 * BP_WAVES - 1) / (2 * BP_WAVES)) * layers;
    // The fp32 kernels carry a pixel's window position (0 .. W bins) to about 2^-24
    // of the window, and its phase to 2^-24 of the kappa W carrier cycles across
    // the window (kappa = 2 dr / lambda; W ~ 4 half_span / lambda for large tiles).
    // Past 4096 cycles (about 7.7e-4 rad per rounding) the plan uses the fp64-range
    // kernels instead (64 x 32 tiles).
    const double hs32 = 0.5 * sqrt((BP_TX * p.dx) * (BP_TX * p.dx) +
                                   (2.0 * BP_WAVES * p.dy) * (2.0 * BP_WAVES * p.dy) + p.dem_relief * p.dem_relief);
    const double win32 = ceil(2.0 * hs32 / p.dr) + 6.0; // the window of 64 x 32 tiles, margins included
    L->f64 = (2.0 * p.dr / p.wavelength) * win32 > 4096.0;
    // Nearest: the fp32 bin decision is rechecked in fp64 within a tie band that
    // grows with the window and the tile (tie_band_coefficients); where the band of
    // a 64 x 32 tile would pass BP_NEAREST_TIE_MAX, the fp64-range kernels serve
    // the plan.  (rho <= 1.06 half_span / dr while the series applies.)
    if (p.interp == SARBP_NEAREST && !L->f64) {
        float base[3], win_coef, rho_coef[3];
        tie_band_coefficients(false, base, &win_coef, rho_coef);
        const double band = (double)base[0] + (double)win_coef * win32 + (double)rho_coef[0] * 1.06 * hs32 / p.dr;
        if (band > BP_NEAREST_TIE_MAX) L->f64 = 1;
    }
    L->ppt = (tiles2 < 2 * (int64_t)L->n_cu && !(p.dem_relief > 0.0) && !L->f64) ? 1 : 2;
    const int ty = BP_WAVES * L->ppt;
    L->tiles_y = (p.ny + ty - 1) / ty;
    if ((int64_t)L->tiles_x * L->tiles_y * layers > INT32_MAX) return SARBP_EINVAL;
    // (with terrain, the tile centre is at the tile's mid-height: |dz| <= dem_relief / 2)
    L->half_span = 0.5 * sqrt((BP_TX * p.dx) * (BP_TX * p.dx) + ((double)ty * p.dy) * ((double)ty * p.dy) +
                              p.dem_relief * p.dem_relief);
    const double span_bins = ceil(2.0 * L->half_span / p.dr);
    // The window holds the bins floor(u) can take (the sinc8 taps are folded into
    // each bin's polynomial), with a spare bin each side.
    const int taps_hi = 1;
    L->margin_lo = 2;
    if (span_bins > 1.0e6) return SARBP_EUNSUPPORTED;
    L->win = (int)span_bins + L->margin_lo + 2 + taps_hi;
    // linear and nearest windows are staged two bins per lane step: make W even
    if (p.interp != SARBP_SINC8) L->win += L->win & 1;
    const int eb = p.interp == SARBP_NEAREST ? 8 : (p.interp == SARBP_LINEAR ? 16 : 64);
    if (p.interp == SARBP_SINC8) sinc8_polynomials(L->sinc_poly);
    // LDS of a workgroup: `entries` window entries, which each chunk fills with its
    // pulses' exact windows; two sets of per-pulse records of `rec` bytes for up to
    // `chunk` pulses (the pulse loop reads one while the next chunk's set-up writes
    // the other: constants, window start, bp_ext_doubles fp64 words); the chunk's
    // issue-priority word, its double-buffered mode, tie-band, window and edge words
    // (40 bytes) and the tile's pixel box and reference point (9 doubles); and for
    // nearest with fp32 ranges the workgroup's queue of tie-recheck words (16 bytes
    // each, a 2-byte owner each, the count, and 16 bytes of alignment): at least
    // BP_TIE_QUEUE words, and whatever LDS a full chunk's windows leave over.
    const int rec = ((p.dem_relief > 0.0 || L->f64) ? 3 : 2) * 16 + 4 + 8 * bp_ext_doubles(p.interp, L->f64 != 0);
    int tq = (p.interp == SARBP_NEAREST && !L->f64 && BP_NEAREST_DEFER) ? BP_TIE_QUEUE : 0;
    const auto fixed_bytes = [](int q) { return 40 + 72 + (q > 0 ? 16 + q * 18 + 4 : 0); };
    const int fixed = fixed_bytes(tq);
    const int cap = p.interp == SARBP_NEAREST ? BP_MAX_CHUNK_NEAREST : BP_MAX_CHUNK;
    // Pulses per chunk when every window is the plan's longest.  Coarse grids (long
    // windows) that would stage fewer than 8 use up to 150 KiB of LDS: one
    // workgroup per CU instead of two.
    int avail = BP_LDS_BUDGET - fixed;
    if (avail / (L->win * eb + 2 * rec) < 8) avail = 150 * 1024 - fixed;
    const int pmin = avail / (L->win * eb + 2 * rec);
    if (pmin < 1) return SARBP_EUNSUPPORTED;
    // Records for chunks of windows half that long (one pulse sees a tile's range
    // extent, typically about half the diagonal that bounds it), between pmin and
    // the cap; the window entries take the rest, at least one longest window.
    int chunk = avail / (L->win * eb / 2 + 2 * rec);
    chunk = std::min(cap, std::max(pmin, chunk));
    int entries = ((avail - 2 * chunk * rec) / eb) & ~1; // (even: 16-byte records follow)
    if (entries < L->win) {
        chunk = std::max(1, std::min(chunk, (avail - L->win * eb) / (2 * rec)));
        entries = ((avail - 2 * chunk * rec) / eb) & ~1;
    }
    if (entries < L->win) return SARBP_EUNSUPPORTED;
    // Nearest's chunk is capped by its mark bits, so LDS beyond a full chunk of the
    // longest windows goes to the tie queue: fewer queue drains between chunks.
    if (tq > 0 && chunk == cap && avail == BP_LDS_BUDGET - fixed) {
        const int need = (cap * L->win + 1) & ~1;
        const int more = std::min((entries - need) * eb / (18 * 64) * 64, 16384 - tq);
        if (more > 0) {
            tq += more;
            entries = ((BP_LDS_BUDGET - fixed_bytes(tq) - 2 * chunk * rec) / eb) & ~1;
        }
    }
    L->chunk = chunk;
    L->entries = entries;
    L->tie_queue = tq;
    L->lds_bytes = (size_t)entries * eb + 2 * (size_t)chunk * rec + fixed_bytes(tq);
    return SARBP_OK;
}

void sarbp_bp_args(const sarbp_params& p, const BpLayout& L, BpArgs* A) {
    *A = BpArgs();
    A->n_range = p.n_range;
    A->nx = p.nx;
    A->ny = p.ny;
    A->tiles_x = L.tiles_x;
    A->ntiles = L.tiles_x * L.tiles_y;
    A->group_blocks = A->ntiles * (p.nz > 1 ? p.nz : 1);
    A->nblocks = A->group_blocks;
    A->dz = p.nz > 1 ? p.dz : 0.0;
    A->win = L.win;
    A->fast_stage = (uint64_t)L.chunk * (uint64_t)p.n_range * 8u + 64u < (1ull << 32) ? 1 : 0;
    A->margin_lo = L.margin_lo;
    A->chunk = L.chunk;
    A->entries = L.entries;
    A->tie_queue = L.tie_queue;
    A->slots = L.n_cu;
    A->r0 = p.r0;
    A->dr = p.dr;
    A->inv_dr = 1.0 / p.dr;
    A->x0 = p.x0;
    A->y0 = p.y0;
    A->z0 = p.z0;
    A->dx = p.dx;
    A->dy = p.dy;
    A->half_span = L.half_span;
    A->dem_relief = p.dem_relief;
    for (int i = 0; i < 32; ++i) A->sinc_poly[i] = L.sinc_poly[i];
    A->half_span_bins = L.half_span / p.dr;
    A->kappa = (float)(2.0 * p.dr / p.wavelength);
    tie_band_coefficients(L.f64 != 0, A->tie_base, &A->tie_win, A->tie_rho);
    A->round_half = p.interp == SARBP_NEAREST ? 1 : 0;
}

extern "C" int sarbp_plan_create(const sarbp_params* params, sarbp_plan** out) {
    if (out == nullptr) return SARBP_EINVAL;
    *out = nullptr;
    int st = sarbp_validate(params);
    if (st != SARBP_OK) return st;
    sarbp_plan* plan = new (std::nothrow) sarbp_plan();
    if (plan == nullptr) return SARBP_ENOMEM;
    memset(plan, 0, sizeof(*plan));
    plan->p = *params;
    const sarbp_params& p = plan->p;
    int n_cu = 0;
    if (hipGetDevice(&plan->device) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, plan->device) != hipSuccess) {
        delete plan;
        return SARBP_EDEVICE;
    }
    plan->L.n_cu = n_cu;

    st = sarbp_plan_layout(p, n_cu, &plan->L);
    if (st != SARBP_OK) {
        release(plan);
        return st;
    }
    if (plan->L.lds_bytes > 64 * 1024) {
        st = sarbp_bp_allow_lds(p.interp, p.accum, false, plan->L.ppt, plan->L.f64, plan->L.lds_bytes);
        if (st == SARBP_OK && p.dem_relief > 0.0)
            st = sarbp_bp_allow_lds(p.interp, p.accum, true, plan->L.ppt, plan->L.f64, plan->L.lds_bytes);
        if (st != SARBP_OK) {
            release(plan);
            return st;
        }
    }

    // The device address of the library's static pulse-group scratch on this device
    // (sarbp_backproject_split_noalloc); taken here, once per device.
    st = sarbp_scratch_address(plan->device, &plan->scratch);
    if (st != SARBP_OK) {
        release(plan);
        return st;
    }

    st = upload(phase_table(p), &plan->phase_tab);
    if (st == SARBP_OK) st = upload(std::vector<int>((size_t)2 * plan->L.n_cu, 0), &plan->progress);
    if (st != SARBP_OK) {
        release(plan);
        return st;
    }

    if (p.n_fast != 0) {
        const int N = p.n_fast;
        int lg = 0;
        while ((1 << lg) < N) ++lg;
        plan->rc_log2 = lg;
        // reference chirp: ref[m mod N] = exp(j pi K t^2), t = m / fs, m = -L/2 .. L - L/2 - 1
        const int L = (int)floor(p.chirp_T * p.fs + 0.5);
        const double K = p.chirp_B / p.chirp_T;
        std::vector<std::complex<double>> ref((size_t)N, 0.0);
        for (int m = -(L / 2); m < L - L / 2; ++m) {
            const double t = (double)m / p.fs;
            const double ph = kPi * K * t * t;
            ref[(size_t)((m % N + N) % N)] = std::complex<double>(cos(ph), sin(ph));
        }
        fft_host(ref);
        std::vector<float2> filt((size_t)N);
        const TaylorTaper taylor(p.taylor_nbar ? p.taylor_nbar : 4, p.taylor_sll != 0.0 ? p.taylor_sll : 35.0);
        for (int m = 0; m < N; ++m) {
            const double f = (m < N / 2 ? (double)m : (double)(m - N)) * p.fs / (double)N; // fftfreq
            const bool in_band = fabs(f) <= 0.5 * p.chirp_B;
            double w = 1.0;
            if (p.window == 1) w = in_band ? 0.54 + 0.46 * cos(2.0 * kPi * f / p.chirp_B) : 0.0;
            if (p.window == 2) w = in_band ? taylor(f / p.chirp_B) : 0.0;
            const std::complex<double> h = std::conj(ref[(size_t)m]) * (w / (double)N);
            filt[(size_t)m] = make_float2((float)h.real(), (float)h.imag());
        }
        st = upload(filt, &plan->rc_filter);
        if (st == SARBP_OK) st = sarbp_rc_prepare_device();
        if (st != SARBP_OK) {
            release(plan);
            return st;
        }
    }
    *out = plan;
    return SARBP_OK;
}

int sarbp_check_device(const sarbp_plan* plan) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SARBP_EDEVICE;
    return cur == plan->device ? SARBP_OK : SARBP_EINVAL;
}

namespace {
int check_device(const sarbp_plan* plan) { return sarbp_check_device(plan); }
} // namespace

extern "C" int sarbp_backproject(const sarbp_plan* plan, const double* positions_d, const void* echo_d, void* image_d,
                                 int32_t n, int32_t accumulate, void* stream) {
    if (plan == nullptr || !aligned8(positions_d) || !aligned8(echo_d) || !aligned8(image_d)) return SARBP_EINVAL;
    if (n < 1 || n > plan->p.n_pulses || (accumulate != 0 && accumulate != 1)) return SARBP_EINVAL;
    const int st = check_device(plan);
    if (st != SARBP_OK) return st;
    return sarbp_launch_bp(plan, positions_d, static_cast<const float2*>(echo_d), nullptr,
                           static_cast<float2*>(image_d), n, accumulate, static_cast<hipStream_t>(stream));
}

extern "C" int sarbp_backproject_dem(const sarbp_plan* plan, const double* positions_d, const void* echo_d,
                                     const float* dem_d, void* image_d, int32_t n, int32_t accumulate,
                                     void* stream) {
    if (plan == nullptr || !(plan->p.dem_relief > 0.0) || dem_d == nullptr ||
        (reinterpret_cast<uintptr_t>(dem_d) & 3u) != 0 || !aligned8(positions_d) || !aligned8(echo_d) ||
        !aligned8(image_d))
        return SARBP_EINVAL;
    if (n < 1 || n > plan->p.n_pulses || (accumulate != 0 && accumulate != 1)) return SARBP_EINVAL;
    const int st = check_device(plan);
    if (st != SARBP_OK) return st;
    return sarbp_launch_bp(plan, positions_d, static_cast<const float2*>(echo_d), dem_d,
                           static_cast<float2*>(image_d), n, accumulate, static_cast<hipStream_t>(stream));
}

extern "C" size_t sarbp_split_workspace_bytes(const sarbp_plan* plan, int32_t n) {
    if (plan == nullptr || n < 1 || n > plan->p.n_pulses) return 0;
    const int s = sarbp_split_count(plan, n);
    if (s < 2) return 0;
    const size_t layers = plan->p.nz > 1 ? (size_t)plan->p.nz : 1;
    return (size_t)s * layers * (size_t)plan->p.ny * (size_t)plan->p.nx * sizeof(float2);
}

int sarbp_split_check(const sarbp_plan* plan, const double* positions_d, const void* echo_d, const float* dem_d,
                      const void* image_d, int32_t n, int32_t accumulate) {
    if (plan == nullptr || !aligned8(positions_d) || !aligned8(echo_d) || !aligned8(image_d)) return SARBP_EINVAL;
    if (n < 1 || n > plan->p.n_pulses || (accumulate != 0 && accumulate != 1)) return SARBP_EINVAL;
    if (dem_d != nullptr && (!(plan->p.dem_relief > 0.0) || (reinterpret_cast<uintptr_t>(dem_d) & 3u) != 0))
        return SARBP_EINVAL;
    return SARBP_OK;
}

extern "C" int sarbp_backproject_split(const sarbp_plan* plan, const double* positions_d, const void* echo_d,
                                       const float* dem_d, void* image_d, int32_t n, int32_t accumulate,
                                       void* workspace_d, size_t workspace_bytes, void* stream) {
    int st = sarbp_split_check(plan, positions_d, echo_d, dem_d, image_d, n, accumulate);
    if (st != SARBP_OK) return st;
    const size_t need = sarbp_split_workspace_bytes(plan, n);
    if (need > 0) {
        if (!aligned8(workspace_d) || workspace_bytes < need) return SARBP_EINVAL;
        const size_t layers = plan->p.nz > 1 ? (size_t)plan->p.nz : 1;
        const uintptr_t ib = (uintptr_t)(layers * (size_t)plan->p.ny * (size_t)plan->p.nx * sizeof(float2));
        const uintptr_t i = reinterpret_cast<uintptr_t>(image_d), w = reinterpret_cast<uintptr_t>(workspace_d);
        if (i < w + need && w < i + ib) return SARBP_EINVAL; // the workspace overlaps the image
    }
    st = check_device(plan);
    if (st != SARBP_OK) return st;
    return sarbp_launch_bp(plan, positions_d, static_cast<const float2*>(echo_d), dem_d,
                           static_cast<float2*>(image_d), n, accumulate, static_cast<hipStream_t>(stream),
                           need > 0 ? static_cast<float2*>(workspace_d) : nullptr,
                           need > 0 ? sarbp_split_count(plan, n) : 1);
}

extern "C" int sarbp_range_compress(const sarbp_plan* plan, const void* raw_d, void* out_d, int32_t n, void* stream) {
    if (plan == nullptr || plan->p.n_fast == 0 || !aligned8(raw_d) || !aligned8(out_d) || n < 1) return SARBP_EINVAL;
    const uintptr_t bytes = (uintptr_t)n * (uintptr_t)plan->p.n_fast * sizeof(float2);
    const uintptr_t a = reinterpret_cast<uintptr_t>(raw_d), b = reinterpret_cast<uintptr_t>(out_d);
    if (a < b + bytes && b < a + bytes) return SARBP_EINVAL; // overlapping buffers
    const int st = check_device(plan);
    if (st != SARBP_OK) return st;
    return sarbp_launch_rc(plan, static_cast<const float2*>(raw_d), static_cast<float2*>(out_d), n,
                           static_cast<hipStream_t>(stream));
}

extern "C" void sarbp_destroy(sarbp_plan* plan) { release(plan); }

extern "C" const char* sarbp_status_string(int status) {
    switch (status) {
        case SARBP_OK: return "success";
        case SARBP_EINVAL: return "invalid argument";
        case SARBP_ENOMEM: return "out of memory";
        case SARBP_EDEVICE: return "HIP runtime or kernel launch failure";
        case SARBP_EUNSUPPORTED: return "unsupported configuration";
        case SARBP_ESCRATCH: return "the call needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

extern "C" int sarbp_version(void) { return 200; }
