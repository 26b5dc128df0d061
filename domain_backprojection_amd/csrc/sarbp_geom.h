// Index and window-position arithmetic of the backprojection kernels, shared by
// the device code (sarbp_bp.hip) and the host-side emulation of it
// (sarbp_check_indices in sarbp_check.hip), so that the emulation runs the very
// operations the kernels run.
//
// Method: the page "基于GPU的SAR后向投影成像优化与CUDA加速实践" (GPU-based SAR
// backprojection), section 2.2: for each pixel and pulse the range R = |p - a_n|,
// the fractional bin u = (R - r0) / dr, the interpolated sample, and the phase
// term; section 2.2 also warns that fp32 ranges lose phase accuracy, and
// section 4.4 that an index outside the echo window fills the image with noise.
//
// The few operations whose gfx950 instruction has no bit-identical host twin go
// through a math policy: DevMath (the hardware instructions) or HostMath.  Only
// the fp32 square root and reciprocal of the exact-form window position differ
// (v_sqrt_f32 / v_rcp_f32 are within about one ulp, the host's are correctly
// rounded); every other operation is IEEE on both sides.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sarbp_internal.h"

#pragma clang fp contract(off)

struct DevMath {
    __device__ static float sqrt_hw(float x) { return __builtin_amdgcn_sqrtf(x); }
    __device__ static float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
    __device__ static float fract(float x) { return __builtin_amdgcn_fractf(x); }
    __device__ static uint32_t to_u32(float x) { return (uint32_t)x; } // v_cvt_u32_f32: truncates, saturates
    __device__ static double dadd(double a, double b) { return __dadd_rn(a, b); }
    __device__ static double dsub(double a, double b) { return __dsub_rn(a, b); }
    __device__ static double dmul(double a, double b) { return __dmul_rn(a, b); }
    __device__ static double ddiv(double a, double b) { return __ddiv_rn(a, b); }
    __device__ static double dsqrt(double a) { return __dsqrt_rn(a); }
};

struct HostMath {
    static float sqrt_hw(float x) { return sqrtf(x); }
    static float rcp_hw(float x) { return 1.0f / x; }
    // v_fract_f32: x - floor(x), kept below 1
    static float fract(float x) { return fminf(x - floorf(x), 0x1.fffffep-1f); }
    static uint32_t to_u32(float x) {
        if (!(x > 0.0f)) return 0u; // negative and NaN saturate to 0
        if (x >= 4294967296.0f) return 0xffffffffu;
        return (uint32_t)x;
    }
    static double dadd(double a, double b) { return a + b; }
    static double dsub(double a, double b) { return a - b; }
    static double dmul(double a, double b) { return a * b; }
    static double ddiv(double a, double b) { return a / b; }
    static double dsqrt(double a) { return sqrt(a); }
};

template <int INTERP>
__host__ __device__ constexpr int entry_bytes() {
    return INTERP == SARBP_NEAREST ? 8 : (INTERP == SARBP_LINEAR ? 16 : 64);
}

// The pixel tile of workgroup gb (within its pulse group): voxel layer, first
// column and row, last in-grid column and row, and the reference point c (the
// centre of the tile's in-grid pixels, on the layer's plane).  Tiles are
// remapped so that each XCD (workgroups go round-robin over 8 XCDs) owns a
// contiguous band of tiles, whose echo windows then overlap in its L2.
struct TileFrame {
    int layer, i0, j0, i_last, j_last;
    double cxp, cyp; // reference point in pixel units
    double cx, cy, zl;
};

template <int PPT>
__host__ __device__ __forceinline__ TileFrame tile_frame(const BpArgs& A, int gb) {
    TileFrame t;
    t.layer = gb / A.ntiles;
    int tile = gb - t.layer * A.ntiles;
    const int nt8 = (A.ntiles / 8) * 8;
    if (tile < nt8) tile = (tile & 7) * (nt8 / 8) + (tile >> 3);
    const int tx = tile % A.tiles_x, ty = tile / A.tiles_x;
    t.i0 = tx * BP_TX;
    t.j0 = ty * (BP_WAVES * PPT);
    t.i_last = min(t.i0 + BP_TX, A.nx) - 1;
    t.j_last = min(t.j0 + BP_WAVES * PPT, A.ny) - 1;
    t.cxp = 0.5 * (double)(t.i0 + t.i_last);
    t.cyp = 0.5 * (double)(t.j0 + t.j_last);
    t.cx = A.x0 + t.cxp * A.dx;
    t.cy = A.y0 + t.cyp * A.dy;
    t.zl = A.z0 + (double)t.layer * A.dz;
    return t;
}

// The box spanned by a tile's in-grid pixel centres: x in [xa, xb], y in [ya, yb]
// and heights z in [za, zb] (one plane: za = zb; terrain: the tile's height range).
struct TileBox {
    double xa, xb, ya, yb, za, zb;
};

__host__ __device__ __forceinline__ TileBox tile_box(const BpArgs& A, const TileFrame& t, double za, double zb) {
    TileBox b;
    b.xa = t.cx + ((double)t.i0 - t.cxp) * A.dx;
    b.xb = t.cx + ((double)t.i_last - t.cxp) * A.dx;
    b.ya = t.cy + ((double)t.j0 - t.cyp) * A.dy;
    b.yb = t.cy + ((double)t.j_last - t.cyp) * A.dy;
    b.za = za;
    b.zb = zb;
    return b;
}

// A uniform input of the per-pulse set-up, made opaque to the optimiser at each
// call: quantities derived from it (2 h, h^2, the margins as doubles) are then
// formed by the set-up lanes where they are used, instead of being computed once
// before the chunk loop and held in registers across the pulse loop, which has
// none to spare (they went to scratch).  No effect on the host build.
template <class T>
__host__ __device__ __forceinline__ T per_call(T x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+s"(x));
#endif
    return x;
}

// The echo window of one pulse for one tile: the bins floor(u) the tile's pixels
// can take, u = (R - r0) / dr, from the nearest and the farthest point of the
// tile's box to the antenna (the nearest: each coordinate clamped into the box;
// the farthest: the far corner), with margin_lo spare bins below and three above
// (room for the fp32 window position's error and for nearest's + 1/2).  Sets the
// first bin, or INT32_MIN for a pulse without finite geometry, and returns the
// length W_p = floor(u_max) - floor(u_min) + margin_lo + 3, which the triangle
// inequality keeps within the plan's window (the tile's diagonal in bins plus the
// same margins).
__host__ __device__ inline int pulse_window(const BpArgs& A, double ax, double ay, double az, const TileBox& b,
                                            int* klo) {
    const double nx = fmin(fmax(ax, b.xa), b.xb) - ax, ny = fmin(fmax(ay, b.ya), b.yb) - ay,
                 nz = fmin(fmax(az, b.za), b.zb) - az;
    const double fx = fmax(fabs(b.xa - ax), fabs(b.xb - ax)), fy = fmax(fabs(b.ya - ay), fabs(b.yb - ay)),
                 fz = fmax(fabs(b.za - az), fabs(b.zb - az));
    const double umin = (sqrt(nx * nx + ny * ny + nz * nz) - A.r0) * A.inv_dr;
    const double umax = (sqrt(fx * fx + fy * fy + fz * fz) - A.r0) * A.inv_dr;
    const int mlo = per_call(A.margin_lo), win = per_call(A.win);
    const double kmin = floor(umin) - (double)mlo;
    const double w = floor(umax) - floor(umin) + (double)(mlo + 3);
    if (!(fabs(kmin) < 1.0e9 && w >= 0.0 && w < 2.0e9)) {
        *klo = INT32_MIN;
        return mlo + 3;
    }
    *klo = (int)kmin;
    return w < (double)win ? (int)w : win;
}

// Whether a pulse's staged window, with what its staging reads beyond it, lies in
// the echo record (the fast staging path then needs no clamps): sinc8 reads the taps
// klo - 3 .. klo + W + 3, linear klo .. klo + W (its last step reads one past the
// window), nearest klo .. klo + W - 1; W is taken at the plan's longest window.
template <int INTERP>
__host__ __device__ __forceinline__ bool window_in_record(const BpArgs& A, int klo) {
    if (INTERP == SARBP_SINC8) return klo != INT32_MIN && klo >= 3 && klo <= A.n_range - 5 - A.win;
    return klo != INT32_MIN && klo >= 0 && klo <= A.n_range - 1 - A.win;
}

// The pulses of a chunk: as many of its cand set-up candidates as the LDS window
// entries hold at the chunk's window length; half as many (at least one) for the
// first chunk of staggered workgroups.
__host__ __device__ __forceinline__ int chunk_length(int cand, int entries, int win_c, bool half) {
    int np = entries / win_c;
    if (np > cand) np = cand;
    if (half) np = np > 1 ? np >> 1 : 1;
    return np;
}

// The window length of a chunk: the longest of its pulses' windows, even where
// staging takes two bins per step, and within the plan's window.
__host__ __device__ __forceinline__ int chunk_window(int wmax, int bins_per_step, int win) {
    int w = wmax < 6 ? 6 : wmax;
    if (bins_per_step == 2) w += w & 1;
    return w < win ? w : win;
}

// Per-pulse constants of the current tile, two float4 per pulse:
//   c0 = (2 ux, 2 uy, ft, a)   c1 = (b, c, 1/R_t^2, a2)
// with u = c - a_n, ft = u_c - k_lo (fractional bin of the tile centre within
// the window), a = 1/(2 R_t dr), b = -1/(8 R_t^3 dr), c = 1/(16 R_t^5 dr).
// In q = num / R_t^2, (R - R_t) / R_t = q/2 - q^2/8 + q^3/16 - 5 q^4/128 + ...
// The two-term form replaces the cubic by its Chebyshev-economised linear fit
// over |q| <= q_m, (3/4) q_m^2 q, so its linear coefficient is
// a2 = a (1 + 3 q_m^2 / 32) and its error at most R_t (q_m^3/64 + 5 q_m^4/128).
// Returns the accuracy mode this pulse needs (0: 2 terms, 1: 3 terms, 2: exact).
// Terrain (dem) kernels also store c2 = (2 uz, 0, 0, 0), the vertical term of 2 d.u.
// *rho_out receives the bound (|d|^2 + 2 |d| R_t) / (2 R_t dr), |d| <= half_span,
// on the range-difference terms in bins, from which the nearest tie band is sized.
__host__ __device__ inline int pulse_setup(const BpArgs& A, double ax, double ay, double az, double cx, double cy,
                                           double cz, float4* cst, double* uc_out, float* rho_out, bool dem) {
    const double ux = cx - ax, uy = cy - ay, uz = cz - az;
    const double R2 = ux * ux + uy * uy + uz * uz;
    const double Rt = sqrt(R2);
    const double uc = (Rt - A.r0) * A.inv_dr;
    const bool ok = isfinite(Rt) && Rt > 0.0 && isfinite(uc) && fabs(uc) < 1.0e9;
    if (!ok) {
        *uc_out = NAN; // parked by pulse_finish
        *rho_out = 0.f;
        return 0;
    }
    const double inv_r = 1.0 / Rt;
    const double idr = A.inv_dr;
    // q_m bounds |q| over the tile: |d| <= half_span and |u| = R_t.
    const double hs = per_call(A.half_span);
    const double q = (hs * hs + 2.0 * hs * Rt) * inv_r * inv_r;
    const double a = 0.5 * inv_r * idr;
    cst[0] = make_float4((float)(2.0 * ux), (float)(2.0 * uy), 0.f, (float)a); // .z: ft, set by pulse_finish
    cst[1] = make_float4((float)(-0.125 * inv_r * inv_r * inv_r * idr),
                         (float)(0.0625 * inv_r * inv_r * inv_r * inv_r * inv_r * idr), (float)(inv_r * inv_r),
                         (float)(a * (1.0 + (3.0 / 32.0) * q * q)));
    if (dem) cst[2] = make_float4((float)(2.0 * uz), 0.f, 0.f, 0.f);
    *uc_out = uc;
    *rho_out = (float)(0.5 * q * Rt * idr * 1.0000001);
    // Truncation error of each series for the worst pixel of the tile, in bins,
    // against 1e-6 bins (below the fp32 rounding of the window position).
    const double e2 = Rt * (q * q * q * (1.0 / 64.0) + q * q * q * q * (5.0 / 128.0)) * idr;
    const double e3 = Rt * q * q * q * q * (5.0 / 128.0) * idr;
    return (q > 0.25 || e3 > 1e-6) ? 2 : (e2 > 1e-6 ? 1 : 0);
}

// The tile centre's position within its pulse window, ft = u_c - k_lo (+ 1/2 for
// nearest, whose window positions carry u + 1/2), once both the set-up (u_c) and
// the window (k_lo) are known.  A pulse without finite geometry is parked: every
// pixel on window entry margin_lo, whose staged samples are NaN, so NaN propagates.
__host__ __device__ inline void pulse_finish(const BpArgs& A, double uc, int klo, float4* cst, bool dem, bool f64) {
    if (klo == INT32_MIN || !isfinite(uc)) {
        if (f64) {
            double2* cd = reinterpret_cast<double2*>(cst);
            cd[0] = make_double2(0.0, 0.0);
            cd[1] = make_double2((double)A.margin_lo + 0.25, 0.0);
            cd[2] = make_double2(0.0, 0.0);
        } else {
            cst[0] = make_float4(0.f, 0.f, (float)A.margin_lo + 0.25f, 0.f);
            cst[1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (dem) cst[2] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }
    const double ft = uc - (double)klo + (per_call(A.round_half) ? 0.5 : 0.0);
    if (f64)
        reinterpret_cast<double2*>(cst)[1].x = ft;
    else
        cst[0].z = (float)ft;
}

// Per-pulse constants of the fp64-range kernels (tiles whose range extent is too
// large for the fp32 difference): three double2 per pulse,
//   (2 ux, 2 uy), (ft, 1/R_t^2), (R_t/dr, 2 uz),
// and the window position ub = ft + (R_t/dr) (sqrt(1 + q) - 1), q = num / R_t^2,
// by its binomial series through q^4 (mode 0) or q^7 (mode 1), the shorter one
// whose first omitted term stays below 1e-7 bins over the tile, else exactly
// (mode 2).  (1e-7 bins is below the fp32 rounding of the fraction returned.)
__host__ __device__ inline int pulse_setup_f64(const BpArgs& A, double ax, double ay, double az, double cx, double cy,
                                               double cz, float4* cst, double* uc_out) {
    double2* cd = reinterpret_cast<double2*>(cst);
    const double ux = cx - ax, uy = cy - ay, uz = cz - az;
    const double Rt = sqrt(ux * ux + uy * uy + uz * uz);
    const double uc = (Rt - A.r0) * A.inv_dr;
    if (!(isfinite(Rt) && Rt > 0.0 && isfinite(uc) && fabs(uc) < 1.0e9)) {
        *uc_out = NAN; // parked by pulse_finish
        return 0;
    }
    const double inv_r = 1.0 / Rt;
    const double hs = per_call(A.half_span);
    const double q = (hs * hs + 2.0 * hs * Rt) * inv_r * inv_r;
    cd[0] = make_double2(2.0 * ux, 2.0 * uy);
    cd[1] = make_double2(0.0, inv_r * inv_r); // .x: ft, set by pulse_finish
    cd[2] = make_double2(Rt * A.inv_dr, 2.0 * uz); // 2 uz: the terrain kernels' vertical term
    *uc_out = uc;
    const double q2 = q * q, q4 = q2 * q2, rb = Rt * A.inv_dr; // R_t in bins
    if (q > 0.25 || rb * (429.0 / 32768.0) * q4 * q4 > 1e-7) return 2;
    return rb * (7.0 / 256.0) * q4 * q > 1e-7 ? 1 : 0;
}

// Window position of one pixel for pulse p in the fp64-range kernels: the bin
// k = floor(ub) and the fraction f = ub - k.
template <int MODE, bool DEM>
__host__ __device__ __forceinline__ void locate_f64(const float4* cst, int p, double dxd, double dyd, double ddd,
                                                    double dzd, float* f, uint32_t* k) {
    const double2* cd = reinterpret_cast<const double2*>(cst) + 3 * p;
    const double2 d0 = cd[0], d1 = cd[1], d2 = cd[2];
    const double num = fma(dxd, d0.x, fma(dyd, d0.y, DEM ? fma(dzd, d2.y, ddd) : ddd));
    const double q = num * d1.y;
    double s; // (sqrt(1 + q) - 1) / q
    if constexpr (MODE == 2) {
        s = 1.0 / (1.0 + sqrt(1.0 + q));
    } else {
        s = -5.0 / 128.0;
        if constexpr (MODE == 1) {
            s = fma(33.0 / 2048.0, q, -21.0 / 1024.0);
            s = fma(s, q, 7.0 / 256.0);
            s = fma(s, q, -5.0 / 128.0);
        }
        s = fma(s, q, 1.0 / 16.0);
        s = fma(s, q, -1.0 / 8.0);
        s = fma(s, q, 0.5);
    }
    const double ub = fma(d2.x * q, s, d1.x);
    const double kd = floor(ub);
    *k = (uint32_t)kd;
    *f = (float)(ub - kd);
}

// num = |d|^2 + 2 d.(c - a) of a pixel at offset d from the tile centre (fp32 kernels).
__host__ __device__ __forceinline__ float pixel_num(float dxl, float dy, float dd, float dz, const float4& c0,
                                                    const float4& c2, bool dem) {
    return fmaf(dxl, c0.x, fmaf(dy, c0.y, dem ? fmaf(dz, c2.x, dd) : dd));
}

// Bin position of a pixel within its pulse window: ub = ft + (R - R_t) / dr.
template <int MODE, class M>
__host__ __device__ __forceinline__ float bin_position(float num, const float4& c0, const float4& c1) {
    if constexpr (MODE == 0) {
        return fmaf(num, fmaf(num, c1.x, c1.w), c0.z);
    } else if constexpr (MODE == 1) {
        return fmaf(num, fmaf(num, fmaf(num, c1.y, c1.x), c0.w), c0.z);
    } else {
        // (R - R_t) / dr = (num / (R_t dr)) / (1 + s) = a num / (1/2 + s/2),  s = sqrt(1 + q)
        const float s = M::sqrt_hw(fmaxf(fmaf(num, c1.z, 1.0f), 0.0f));
        return fmaf(num * c0.w, M::rcp_hw(fmaf(0.5f, s, 0.5f)), c0.z);
    }
}

// Nearest interpolation: the fp32 bin decision floor(ub) is exact unless ub lies
// within the tie band of an integer.  The band is twice a bound on the fp32
// error of ub, in bins, built from u = 2^-24 per rounding:
//   * ft and ub themselves (|ft|, |ub| <= W):                     2 u W
//   * num = |d|^2 + 2 d.(c - a) from rounded offsets and constants and its
//     two (three with terrain) roundings, times a or a2, and the rounding of
//     the series' coefficient and product: at most 8 u rho (10 with terrain),
//     rho = (|d|^2 + 2 |d| R_t) / (2 R_t dr) the size of the range term in bins
//     (the chunk's largest, from pulse_setup);
//   * the exact form adds the fp32 square root and reciprocal (taken as within
//     2 ulp each) and the rounding of 1 + q: at most 26 u rho;
//   * the series' truncation, at most 1e-6 bins by the choice of mode (none in
//     the exact form).
// A little more is kept (10 / 30 for the rho terms, and 1e-9 bins for the fp64
// reference itself).  tie_band = base[MODE] + win_coef * W + rho_coef[MODE] * rho,
// W the chunk's window length.
#define SARBP_TIE_C_SERIES 10.0
#define SARBP_TIE_C_EXACT 30.0
#define SARBP_TIE_TRUNC 1e-6
// The fp64-range kernels keep ub in fp64 and return the fraction in fp32: their
// error is the series' 1e-7 bins plus the 2^-25 of that rounding.
#define SARBP_TIE_F64 1e-6

__host__ __device__ inline void tie_band_coefficients(bool f64, float base[3], float* win_coef, float rho_coef[3]) {
    const double u = 1.0 / 16777216.0;
    *win_coef = f64 ? 0.f : (float)(4.0 * u);
    for (int m = 0; m < 3; ++m) {
        if (f64) {
            base[m] = (float)SARBP_TIE_F64;
            rho_coef[m] = 0.f;
        } else {
            base[m] = (float)(2.0 * (m < 2 ? SARBP_TIE_TRUNC : 0.0) + 1e-9);
            rho_coef[m] = (float)(2.0 * u * (m < 2 ? SARBP_TIE_C_SERIES : SARBP_TIE_C_EXACT));
        }
    }
}

// Nearest interpolation measures the carrier phase from the middle of the chosen
// bin: a = kappa (g - 1/2) revolutions, g = fract(u + 1/2), taken with one rounding.
// The tie test is made on a as well: |a| > a_lim with a_lim = kappa tie_lim
// (1 - 2^-22) flags every decision with |g - 1/2| > tie_lim, because the two
// roundings of a_lim keep it below kappa tie_lim (1 - 2^-24) and the one of a
// keeps |a| at or above kappa |g - 1/2| (1 - 2^-24).  (A negative tie_lim flags all.)
__host__ __device__ inline float nearest_phase(float kappa, float g) { return fmaf(kappa, g, -0.5f * kappa); }
__host__ __device__ inline float nearest_tie_limit(float kappa, float tie_lim) {
    return kappa * tie_lim * (1.0f - 0x1p-22f);
}

// The definition's fractional bin of pixel (i, j) at height z for an antenna at
// (ax, ay, az), in its double-precision operation order (no contraction):
// u = (sqrt(dx^2 + dy^2 + dz^2) - r0) / dr.
template <class M>
__host__ __device__ __forceinline__ double definition_bin(double ax, double ay, double az, double x0, double y0,
                                                          double z, double dx, double dy, double r0, double dr, int i,
                                                          int j) {
    const double x = M::dadd(x0, M::dmul((double)i, dx));
    const double y = M::dadd(y0, M::dmul((double)j, dy));
    const double ddx = M::dsub(x, ax);
    const double ddy = M::dsub(y, ay);
    const double ddz = M::dsub(z, az);
    const double s2 = M::dadd(M::dadd(M::dmul(ddx, ddx), M::dmul(ddy, ddy)), M::dmul(ddz, ddz));
    const double R = M::dsqrt(s2);
    return M::ddiv(M::dsub(R, r0), dr);
}

// Exact nearest-bin decision for one pixel and pulse: floor(u + 1/2).
template <class M>
__host__ __device__ __forceinline__ int nearest_bin_fp64(double ax, double ay, double az, double x0, double y0,
                                                         double z, double dx, double dy, double r0, double dr, int i,
                                                         int j) {
    return (int)floor(M::dadd(definition_bin<M>(ax, ay, az, x0, y0, z, dx, dy, r0, dr, i, j), 0.5));
}

// Staging of one chunk: step u covers B consecutive bins of one pulse's window
// (B = 2 for linear and nearest, whose windows have even length W; 1 for sinc8).
// The pulse is p = u / (W / B), from an fp32 quotient trunc(u * (1 / (W / B)))
// corrected by one either way so that 0 <= u - p (W / B) < W / B exactly (u < 2^24);
// the step's first bin is k (absolute).  A pulse without finite geometry
// (klo = INT32_MIN) takes k = 0 and reads the carrier table's NaN entries.
template <int B>
__host__ __device__ __forceinline__ void stage_step_f32(const int* klo_s, int u, int wu, float rwu, int* p_out,
                                                        int* k_out, bool* bad_out) {
    int p = (int)((float)u * rwu);
    int r = u - p * wu;
    if (r < 0) {
        --p;
        r += wu;
    } else if (r >= wu) {
        ++p;
        r -= wu;
    }
    const int klo = klo_s[p];
    const bool bad = (klo == INT32_MIN);
    *p_out = p;
    *k_out = (bad ? 0 : klo) + B * r;
    *bad_out = bad;
}

// Index into the carrier table (bins -4 .. n_range + 3 at [k + 4], then two NaN
// entries) of the first of B bins starting at k.
template <int B>
__host__ __device__ __forceinline__ int carrier_index(int k, int nr, bool bad) {
    return bad ? nr + 8 : (k < -4 ? 0 : (k > nr + 4 - B ? nr + 8 - B : k + 4));
}
