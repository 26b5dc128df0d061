// Time-domain backprojection kernels for gfx950 (CDNA4, wave64).
//
// Computes, for every pixel p of the grid and every pulse n,
//   I(p) += interp(s_n, u) * exp(+j 4 pi R / lambda),  R = |p - a_n|,  u = (R - r0) / dr,
// the coherent sum of the page "基于GPU的SAR后向投影成像优化与CUDA加速实践"
// (GPU-based SAR backprojection): section 1.1 (per-pixel sum over pulses),
// section 2.2 (pixel coordinates -> range -> interpolated sample -> phase
// compensation and accumulation; nearest / linear / sinc interpolation;
// hardware square root and trigonometry), section 2.3 (stage the echo block a
// pixel tile touches in on-chip memory because every thread re-reads it).
//
// Design on gfx950 (not the page's one-thread-per-pixel CUDA kernel):
//
// * A workgroup of 16 wave64s owns a 64 (x) by 16 PPT (y) pixel tile (of one
//   voxel layer, for volumes); each lane keeps PPT pixels of one column (register
//   blocking) and accumulates them across all pulses, so the image is written
//   once.  PPT is 2, or 1 for grids too small to give each CU two tiles.
// * Pulses are processed in chunks.  For each pulse of a chunk one lane
//   computes, in fp64, the tile-centre range R_t and derived fp32 constants;
//   the pixels then need only the fp32 range *difference* to the tile centre,
//      num = |d|^2 + 2 d.(c - a),   d = p - c,
//      R - R_t = R_t (sqrt(1 + num / R_t^2) - 1)
//   evaluated by a series in q = num / R_t^2 (two terms, with the dropped cubic
//   Chebyshev-economised into the linear term, or three), picked per chunk from
//   a bound on the truncation error, or when q is not small by the exact form
//   num / (R_t (1 + sqrt(1 + q))).  This keeps the bin position to ~1e-6 bins,
//   which fp32 absolute ranges (~1e-3 m at 11 km) could not (section 2.2 warns
//   about fp32 range precision).  The fp32 window position itself carries ~2^-24
//   of the window, i.e. of the carrier cycles across it, so plans whose window
//   spans more than 4096 cycles (coarse pixels, or many cycles per range bin) run
//   the F64 variant: the same difference and series in fp64, with only the
//   fraction within the bin back in fp32.
// * The echo window a tile can touch (its range extent, bounded by the tile
//   diagonal) is staged per pulse in LDS, already multiplied by the bin-centre
//   carrier phase exp(+j 4 pi r_k / lambda).  For a pixel at u = k + f the
//   remaining phase is exp(j 2 pi kappa f) with kappa = 2 dr / lambda, so one
//   v_sin_f32 / v_cos_f32 pair (inputs in revolutions) on a bounded argument
//   replaces a large-argument reduction.
// * Staged per bin k: linear (A, D) = (s[k] E[k], (s[k+1] - s[k]) E[k]), a
//   sample is one ds_read_b128 and two FMAs; nearest s[k] E[k], its phase taken
//   from the bin's middle, exp(j 2 pi kappa (g - 1/2)) with g = fract(u + 1/2);
//   sinc8 the 8 coefficients of the degree-7 polynomial in f that is the
//   windowed-sinc interpolant at k + f, times E[k], so a sample is one complex
//   Horner evaluation.  The window position is positive by construction, so
//   v_cvt_u32_f32 (truncation) is its floor and v_fract_f32 its fraction.
// * Nearest interpolation rechecks lanes within the tie band of a rounding tie
//   in fp64, in the definition's operation order, so the chosen bin matches the
//   double-precision definition exactly.
// * Template parameters select the accumulator (fp32, Kahan-compensated, or
//   fp32 per chunk summed in fp64) and terrain (per-pixel heights: the tile is
//   centred at its mid-height and the range term gains 2 u_z dz).
// * The two workgroups that share a CU exchange pulse progress through a small
//   array and the one behind raises its wave priority, so neither ends up
//   running alone at half occupancy; larger grids lower the priority by quarter.
// * Workgroups are remapped so each XCD (8 per GPU, round-robin dispatch) owns
//   a contiguous band of tiles whose echo windows overlap in its L2.
#include <math.h>

#include "sarbp_geom.h"
#include "sarbp_internal.h"

#pragma clang fp contract(off)

namespace {



// Rotation of a complex sample by exp(j 2 pi x), x in revolutions (|x| < 256).
__device__ __forceinline__ void sincos_rev(float x, float* s, float* c) {
    *s = __builtin_amdgcn_sinf(x);
    *c = __builtin_amdgcn_cosf(x);
}

// Issue priority of this workgroup's waves for the next chunk.  Two workgroups
// share each CU and the wave arbiter favours the older one, so left alone the
// first finishes early and the second then runs by itself at half occupancy.
// When every tile is resident at once (at most two per CU; the partner of
// workgroup b is then b +- slots), each publishes its progress and whichever is
// behind takes the higher priority.  Larger grids use a fixed schedule instead:
// the priority drops by one with each quarter of the pulses done.  The values
// only steer scheduling; stale or racing reads cannot change a result.
__device__ int chunk_priority(const BpArgs& A, int n0, int total) {
    const int b = (int)blockIdx.x;
    if (A.nblocks <= 2 * A.slots) {
        __hip_atomic_store(A.progress + b, n0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int partner = b < A.slots ? b + A.slots : b - A.slots;
        if (partner >= A.nblocks) return 0;
        const int other = __hip_atomic_load(A.progress + partner, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return (n0 < other || (n0 == other && b >= A.slots)) ? 3 : 0;
    }
    return 3 - (int)((4 * (long long)n0) / total);
}

__device__ __forceinline__ void set_priority(int p) {
    if (p >= 3) __builtin_amdgcn_s_setprio(3);
    else if (p == 2) __builtin_amdgcn_s_setprio(2);
    else if (p == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// Complex product, as the staging forms its entries.
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(fmaf(a.x, b.x, -(a.y * b.y)), fmaf(a.x, b.y, a.y * b.x));
}

// acc += v * (cs + j sn).  ACC_FP32 and ACC_CHUNK64 use four FMAs on the fp32
// accumulator; ACC_KAHAN forms the product first and adds it with a compensation
// term (Kahan summation: the low part lost by each add is carried to the next).
template <int ACC>
__device__ __forceinline__ void mac(float& ar, float& ai, float& cr, float& ci, float vr, float vi, float cs,
                                    float sn) {
    if constexpr (ACC == SARBP_ACC_KAHAN) {
        const float tr = fmaf(vr, cs, -(vi * sn));
        const float ti = fmaf(vr, sn, vi * cs);
        const float yr = tr - cr, yi = ti - ci;
        const float sr = ar + yr, si = ai + yi;
        cr = (sr - ar) - yr;
        ci = (si - ai) - yi;
        ar = sr;
        ai = si;
    } else {
        ar = fmaf(vr, cs, ar);
        ar = fmaf(-vi, sn, ar);
        ai = fmaf(vr, sn, ai);
        ai = fmaf(vi, cs, ai);
    }
}

// Nearest interpolation over G consecutive pulses p0 .. p0+G-1: every bin
// decision of the group first, then one (rare) branch that retakes the decisions
// within the tie band of a rounding tie in fp64 (antenna positions from LDS), then
// the fetches and accumulations.  ub carries u + 1/2: its floor is the nearest bin
// and g - 1/2 = u - bin; the staged sample carries the bin's carrier, and
// exp(j 2 pi a), a = kappa (g - 1/2), completes the phase.  The tie test is made on a
// (nearest_phase / nearest_tie_limit), which the phase needs anyway.
template <int G, int MODE, int ACC, bool DEM, int PPT, bool F64, bool DEFER = false>
__device__ __forceinline__ bool nearest_group(const BpArgs& A, const char* smem, const float4* cst, const int* klo_s,
                                              const double* pos_s, int p0, int i_pix, int j_pix0, float dxl,
                                              const float* dyv, const float* ddv, float* accr, float* acci,
                                              float* cmpr, float* cmpi, const float* dzv, const float* hv, double zl,
                                              uint32_t wstride, const double* pxd, float a_lim, int win_c) {
    constexpr int CS = (DEM || F64) ? 3 : 2;
    float a[G][PPT];
    uint32_t kb[G][PPT];
    float amax = 0.f; // the group's largest |a| (NaN positions, of pulses with no geometry, drop out)
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const float4 c0 = cst[CS * (p0 + q)];
        const float4 c1 = cst[CS * (p0 + q) + 1];
        const float4 c2 = DEM ? cst[CS * (p0 + q) + 2] : c1;
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            float g;
            if constexpr (F64) {
                locate_f64<MODE, DEM>(cst, p0 + q, pxd[0], pxd[1 + m], pxd[1 + PPT + m], pxd[1 + 2 * PPT + m], &g,
                                      &kb[q][m]);
            } else {
                const float num = pixel_num(dxl, dyv[m], ddv[m], dzv[m], c0, c2, DEM);
                const float ub = bin_position<MODE, DevMath>(num, c0, c1);
                g = DevMath::fract(ub);
                kb[q][m] = DevMath::to_u32(ub);
            }
            a[q][m] = nearest_phase(A.kappa, g);
            amax = fmaxf(amax, fabsf(a[q][m]));
        }
    }
    const bool tie = amax > a_lim;
    if (!DEFER && tie) {
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const double* ps = pos_s + 3 * (p0 + q);
#pragma unroll
            for (int m = 0; m < PPT; ++m) {
                if (fabsf(a[q][m]) > a_lim) {
                    const double zp = DEM ? A.z0 + (double)hv[m] : zl; // the pixel's height
                    const int kabs = nearest_bin_fp64<DevMath>(ps[0], ps[1], ps[2], A.x0, A.y0, zp, A.dx, A.dy, A.r0,
                                                               A.dr, i_pix, j_pix0 + BP_WAVES * m);
                    int kr = kabs - klo_s[p0 + q];
                    kr = kr < 0 ? 0 : (kr > win_c - 1 ? win_c - 1 : kr);
                    // g moves by the bins the decision moved: a = kappa (g + kb - kr - 1/2)
                    a[q][m] = fmaf(A.kappa, (float)((int)kb[q][m] - kr), a[q][m]);
                    kb[q][m] = (uint32_t)kr;
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const uint32_t wbase = (uint32_t)(p0 + q) * wstride;
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            const float2 sv = *reinterpret_cast<const float2*>(smem + ((kb[q][m] << 3) + wbase));
            float sn, cs;
            sincos_rev(a[q][m], &sn, &cs);
            mac<ACC>(accr[m], acci[m], cmpr[m], cmpi[m], sv.x, sv.y, cs, sn);
        }
    }
    return tie;
}

// acc += d, through the compensated sum for ACC_KAHAN.
template <int ACC>
__device__ __forceinline__ void add_delta(float& ar, float& ai, float& cr, float& ci, float dr, float di) {
    if constexpr (ACC == SARBP_ACC_KAHAN) {
        const float yr = dr - cr, yi = di - ci;
        const float sr = ar + yr, si = ai + yi;
        cr = (sr - ar) - yr;
        ci = (si - ai) - yi;
        ar = sr;
        ai = si;
    } else {
        ar += dr;
        ai += di;
    }
}

// Deferred tie rechecks (fp32 ranges).  The chunk's loop takes every nearest
// decision in fp32 and only marks, per lane, the groups of pulses with a decision
// inside the tie band, so the loop needs no branch.  After the loop each lane with
// marks appends one word to the workgroup's queue in LDS: (the chunk's first
// pulse; the lane, the chunk's accuracy mode, its number of full groups and the
// wave; the marks; the chunk's tie limit).  A chunk adds at most one word per
// lane, so the queue holds A.tie_queue >= 2 BP_THREADS words and is resolved
// between chunks once it holds more than A.tie_queue - BP_THREADS, and at the end
// of the tile (drain_ties).  There every lane of the workgroup takes words of any
// wave: it repeats the marked pulses' set-up and the owner lane's decisions with
// the same code and the owner's offsets from the same function (so the same
// constants, a and k_f), finds the definition's bin k_d in fp64 for the decisions
// inside the band and, where k_d differs from k_f, forms the correction
// S(k_d) exp(j 2 pi a_d) - S(k_f) exp(j 2 pi a), a_d = a + kappa (k_f - k_d) and
// S(k) = s[k] E[k] formed as the staging forms it, which it leaves in the word's
// slot.  Then each owner adds its corrections in queue order (for one lane, the
// order of its chunks).
static_assert(BP_WAVES <= 16 && BP_MAX_CHUNK_NEAREST / BP_NEAREST_GROUP < 32, "a tie-queue word's wave and group-count fields");
struct TieQueue {
    int4* q;             // the workgroup's A.tie_queue words in LDS (a word's correction replaces it)
    unsigned short* own; // each word's owner: wave << 6 | lane
    int* count;          // words held (an LDS word)
    int pulse0;          // global index of the chunk's first pulse
};

__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// The staged nearest entry of absolute bin k: s[k] E[k], zero outside the record.
__device__ __forceinline__ float2 nearest_entry(const float2* row, const float2* phase, int k, int nr) {
    if ((uint32_t)k >= (uint32_t)nr) return make_float2(0.f, 0.f);
    return cmul(row[k], phase[k + 4]); // carrier of bin k
}

// The fp32 offsets from the tile's reference point of the pixels that lane ln of
// wave wv works with: x (dxl), y (dyv), |d|^2 (ddv) and, on terrain, the height h
// (hv) and its difference to the tile's mid-height hc (dzv).  Lanes past the
// grid's edge take the last column or row, so every lane's range stays within the
// staged window.  The pulse loop and the tie rechecks of its decisions (made by
// any lane of the workgroup) both take them from here.
template <int PPT, bool DEM>
__device__ __forceinline__ void lane_offsets(const BpArgs& A, const TileFrame& T, double hc, int ln, int wv,
                                             float* dxl, float* dyv, float* ddv, float* dzv, float* hv) {
    const int i_off = min(T.i0 + ln, T.i_last);
    const double ddx = ((double)i_off - T.cxp) * A.dx;
    *dxl = (float)ddx;
#pragma unroll
    for (int m = 0; m < PPT; ++m) {
        const int j_off = min(T.j0 + wv + BP_WAVES * m, T.j_last);
        const double ddy = ((double)j_off - T.cyp) * A.dy;
        dyv[m] = (float)ddy;
        if constexpr (DEM) {
            hv[m] = A.dem[(size_t)j_off * A.nx + i_off];
            const double ddz = (double)hv[m] - hc;
            dzv[m] = (float)ddz;
            ddv[m] = (float)(ddx * ddx + ddy * ddy + ddz * ddz);
        } else {
            hv[m] = dzv[m] = 0.f;
            ddv[m] = (float)(ddx * ddx + ddy * ddy);
        }
    }
}

// One pulse's constants and window start for the current tile, as the chunk's
// set-up forms them (the same code, so the same fp32 values).
template <bool DEM>
__device__ __forceinline__ void replay_setup(const BpArgs& A, int n, const double* box_s, float4* cl, int* klo) {
    const double ax = A.pos[3 * (size_t)n], ay = A.pos[3 * (size_t)n + 1], az = A.pos[3 * (size_t)n + 2];
    const TileBox box = {box_s[0], box_s[1], box_s[2], box_s[3], box_s[4], box_s[5]};
    double uc;
    float rho;
    pulse_setup(A, ax, ay, az, box_s[6], box_s[7], box_s[8], cl, &uc, &rho, DEM);
    pulse_window(A, ax, ay, az, box, klo);
    pulse_finish(A, uc, *klo, cl, DEM, false);
}

// Resolve the workgroup's queue of qn words into the owners' accumulators (every
// lane of the workgroup calls it, after a barrier that follows the last append).
// box_s: the tile's pixel box at [0 .. 5] and reference point at [6 .. 8]; T, hc:
// the tile frame and mid-height; zl: the layer's height; pb, pn: the first pulse
// and the pulse count of the workgroup's pulse group.
//
// Lanes of one row tend to mark the same pulses, so each marked pulse's set-up is
// made once: a bitmap of the marked pulses (relative to pb) and its prefix counts
// go to the echo-window LDS (free between chunks), then a table of the marked
// pulses' constants and window starts, in that LDS after them and in the queue's
// unused words.  When the table does not fit, each word repeats its pulses' set-up.
template <int G, int ACC, bool DEM, int PPT>
__device__ __forceinline__ void drain_ties(const BpArgs& A, const TieQueue& tq, int qn, const double* box_s,
                                           const TileFrame& T, double hc, double zl, char* smem, int pb, int pn,
                                           float* accr, float* acci, float* cmpr, float* cmpi) {
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int CS = DEM ? 3 : 2;      // float4 constants per pulse
    constexpr int TE = CS * 16 + 4;      // table bytes per pulse
    float4* dq = reinterpret_cast<float4*>(tq.q);
    const int nbw = (pn + 31) >> 5;      // bitmap words
    uint32_t* bm = reinterpret_cast<uint32_t*>(smem);
    int* pref = reinterpret_cast<int*>(bm + nbw); // [nbw + 1]: marked pulses before each bitmap word
    const int head = ((2 * nbw + 1) * 4 + 15) & ~15;
    const int region = A.entries * entry_bytes<SARBP_NEAREST>();
    bool table = head <= region;
    int cap1 = 0, cap2 = 0;
    if (table) {
        for (int w = tid; w < nbw; w += BP_THREADS) bm[w] = 0;
        __syncthreads();
        for (int e = tid; e < qn; e += BP_THREADS) {
            const int4 t = tq.q[e];
            const int nfull = (t.y >> 8) & 31, r0 = t.x - pb;
            uint32_t marks = (uint32_t)t.z;
            while (marks != 0) {
                const int g = __builtin_ctz(marks);
                marks &= marks - 1;
                const int r = r0 + (g < nfull ? g * G : nfull * G + (g - nfull)), gsz = g < nfull ? G : 1;
                const uint64_t bits = ((1ull << gsz) - 1) << (r & 31);
                atomicOr(&bm[r >> 5], (uint32_t)bits);
                if (bits >> 32) atomicOr(&bm[(r >> 5) + 1], (uint32_t)(bits >> 32));
            }
        }
        __syncthreads();
        if (wave == 0) {
            int run = 0;
            for (int b = 0; b < nbw; b += 64) {
                const int w = b + lane;
                const int c = w < nbw ? __popc(bm[w]) : 0;
                int x = c; // inclusive prefix over the wave
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int y = __shfl_up(x, off);
                    if (lane >= off) x += y;
                }
                if (w < nbw) pref[w] = run + x - c;
                run += __shfl(x, 63);
            }
            if (lane == 0) pref[nbw] = run;
        }
        __syncthreads();
        const int K = pref[nbw]; // the marked pulses (the same for every lane)
        cap1 = (region - head) / TE;
        cap2 = (A.tie_queue - qn) * 16 / TE;
        table = K <= cap1 + cap2;
        if (table) {
            // the k-th marked pulse: the last bitmap word with at most k marks before it, then its bit
            for (int k = tid; k < K; k += BP_THREADS) {
                int lo = 0, hi = nbw - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (pref[mid] <= k)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                uint32_t bits = bm[lo];
                for (int j = k - pref[lo]; j > 0; --j) bits &= bits - 1;
                float4 cl[3];
                int klo;
                replay_setup<DEM>(A, pb + 32 * lo + __builtin_ctz(bits), box_s, cl, &klo);
                const bool first = k < cap1;
                float4* tc = first ? reinterpret_cast<float4*>(smem + head) + k * CS
                                   : reinterpret_cast<float4*>(tq.q + qn) + (k - cap1) * CS;
                int* tk = first ? reinterpret_cast<int*>(reinterpret_cast<float4*>(smem + head) + cap1 * CS) + k
                                : reinterpret_cast<int*>(reinterpret_cast<float4*>(tq.q + qn) + cap2 * CS) + (k - cap1);
#pragma unroll
                for (int c = 0; c < CS; ++c) tc[c] = cl[c];
                *tk = klo;
            }
        }
        __syncthreads();
    }
    for (int e = tid; e < qn; e += BP_THREADS) {
        const int4 t = tq.q[e];
        const int ow = t.y & 63, mode = (t.y >> 6) & 3, nfull = (t.y >> 8) & 31, wo = (t.y >> 13) & 15;
        const int pulse0 = t.x;
        uint32_t marks = (uint32_t)t.z;
        const float a_lim = __int_as_float(t.w);
        float o_dx, o_dy[PPT], o_dd[PPT], o_dz[PPT], o_h[PPT], dr[PPT], di[PPT];
        lane_offsets<PPT, DEM>(A, T, hc, ow, wo, &o_dx, o_dy, o_dd, o_dz, o_h);
#pragma unroll
        for (int m = 0; m < PPT; ++m) dr[m] = di[m] = 0.f;
        while (marks != 0) {
            const int g = __builtin_ctz(marks);
            marks &= marks - 1;
            const int p0 = g < nfull ? g * G : nfull * G + (g - nfull), gsz = g < nfull ? G : 1;
            for (int q = 0; q < gsz; ++q) {
                const int n = pulse0 + p0 + q;
                float4 cl[3];
                int klo;
                if (table) {
                    const int r = n - pb;
                    const int k = pref[r >> 5] + __popc(bm[r >> 5] & ((1u << (r & 31)) - 1u));
                    const bool first = k < cap1;
                    const float4* tc = first ? reinterpret_cast<const float4*>(smem + head) + k * CS
                                             : reinterpret_cast<const float4*>(tq.q + qn) + (k - cap1) * CS;
                    const int* tk =
                        first ? reinterpret_cast<const int*>(reinterpret_cast<const float4*>(smem + head) + cap1 * CS) + k
                              : reinterpret_cast<const int*>(reinterpret_cast<const float4*>(tq.q + qn) + cap2 * CS) +
                                    (k - cap1);
#pragma unroll
                    for (int c = 0; c < CS; ++c) cl[c] = tc[c];
                    klo = *tk;
                } else {
                    replay_setup<DEM>(A, n, box_s, cl, &klo);
                }
                const float4 c0 = cl[0], c1 = cl[1], c2 = DEM ? cl[2] : cl[1];
#pragma unroll
                for (int m = 0; m < PPT; ++m) {
                    const float num = pixel_num(o_dx, o_dy[m], o_dd[m], o_dz[m], c0, c2, DEM);
                    const float ub = mode == 2 ? bin_position<2, DevMath>(num, c0, c1)
                                               : (mode == 1 ? bin_position<1, DevMath>(num, c0, c1)
                                                            : bin_position<0, DevMath>(num, c0, c1));
                    const float a = nearest_phase(A.kappa, DevMath::fract(ub));
                    if (!(fabsf(a) > a_lim)) continue;
                    const int kf = (int)DevMath::to_u32(ub) + klo;
                    const double ax = A.pos[3 * (size_t)n], ay = A.pos[3 * (size_t)n + 1],
                                 az = A.pos[3 * (size_t)n + 2];
                    const double zp = DEM ? A.z0 + (double)o_h[m] : zl; // the pixel's height
                    const int kd = nearest_bin_fp64<DevMath>(ax, ay, az, A.x0, A.y0, zp, A.dx, A.dy, A.r0, A.dr,
                                                             T.i0 + ow, T.j0 + wo + BP_WAVES * m);
                    if (kd == kf) continue;
                    const float2* row = A.echo + (size_t)n * (size_t)A.n_range;
                    const float2 vf = nearest_entry(row, A.phase, kf, A.n_range);
                    const float2 vd = nearest_entry(row, A.phase, kd, A.n_range);
                    float sf, cf, sd, cd;
                    sincos_rev(a, &sf, &cf);
                    sincos_rev(fmaf(A.kappa, (float)(kf - kd), a), &sd, &cd);
                    const float2 tf = cmul(vf, make_float2(cf, sf)), td = cmul(vd, make_float2(cd, sd));
                    dr[m] += td.x - tf.x;
                    di[m] += td.y - tf.y;
                }
            }
        }
        dq[e] = make_float4(dr[0], di[0], PPT > 1 ? dr[PPT - 1] : 0.f, PPT > 1 ? di[PPT - 1] : 0.f);
    }
    __syncthreads();
    // each owner adds its corrections, in queue order: 64 words at a time, the
    // wave's own words with a correction found by a ballot
    static_assert(PPT <= 2, "a correction word holds two pixels");
    for (int b = 0; b < qn; b += 64) {
        const int e = b + lane;
        bool hit = false;
        if (e < qn) {
            const float4 d = dq[e];
            hit = (tq.own[e] >> 6) == wave && (d.x != 0.f || d.y != 0.f || d.z != 0.f || d.w != 0.f);
        }
        uint64_t hits = __builtin_amdgcn_ballot_w64(hit);
        while (hits != 0) {
            const int k = (int)__builtin_ctzll(hits);
            hits &= hits - 1;
            if (lane == (tq.own[b + k] & 63)) {
                const float4 d = dq[b + k];
                if (d.x != 0.f || d.y != 0.f) add_delta<ACC>(accr[0], acci[0], cmpr[0], cmpi[0], d.x, d.y);
                if (PPT > 1 && (d.z != 0.f || d.w != 0.f))
                    add_delta<ACC>(accr[PPT - 1], acci[PPT - 1], cmpr[PPT - 1], cmpi[PPT - 1], d.z, d.w);
            }
        }
    }
}

template <int INTERP, int MODE, int ACC, bool DEM, int PPT, bool F64>
__device__ __forceinline__ void accumulate_chunk(const BpArgs& A, const char* smem, const float4* cst,
                                                 const int* klo_s, const double* pos_s, int np, int i_pix,
                                                 int j_pix0, float dxl, const float* dyv, const float* ddv,
                                                 float* accr, float* acci, float* cmpr, float* cmpi,
                                                 const float* dzv, const float* hv, double zl, const double* pxd,
                                                 float a_lim, int win_c, const TieQueue& tq) {
    const int eb = entry_bytes<INTERP>();
    const uint32_t wstride = (uint32_t)(win_c * eb);
    const float kappa = A.kappa;
    if constexpr (INTERP == SARBP_NEAREST) {
        int p = 0;
        constexpr int G = F64 ? 1 : BP_NEAREST_GROUP;
        if constexpr (!F64 && BP_NEAREST_DEFER) {
            static_assert(BP_MAX_CHUNK_NEAREST / BP_NEAREST_GROUP + BP_NEAREST_GROUP - 1 <= 32, "one mark bit per group");
            uint32_t marks = 0; // bit g: group g had a decision inside the tie band on this lane
            int gi = 0;
            for (; p + G <= np; p += G, ++gi) {
                const bool tie = nearest_group<G, MODE, ACC, DEM, PPT, F64, true>(
                    A, smem, cst, klo_s, pos_s, p, i_pix, j_pix0, dxl, dyv, ddv, accr, acci, cmpr, cmpi, dzv, hv, zl,
                    wstride, pxd, a_lim, win_c);
                marks |= (uint32_t)tie << gi;
            }
            const int nfull = gi;
            for (; p < np; ++p, ++gi) {
                const bool tie = nearest_group<1, MODE, ACC, DEM, PPT, F64, true>(
                    A, smem, cst, klo_s, pos_s, p, i_pix, j_pix0, dxl, dyv, ddv, accr, acci, cmpr, cmpi, dzv, hv, zl,
                    wstride, pxd, a_lim, win_c);
                marks |= (uint32_t)tie << gi;
            }
            // queue this lane's marks (one word per lane with any; the queue has room
            // for a word from every lane of the workgroup)
            const uint64_t mm = __builtin_amdgcn_ballot_w64(marks != 0);
            if (mm != 0) {
                const int lane = lane_id(), wave = (int)(threadIdx.x >> 6);
                int base = 0;
                if (lane == 0) base = atomicAdd(tq.count, __popcll(mm));
                base = __builtin_amdgcn_readfirstlane(base);
                if (marks != 0) {
                    const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mm >> 32),
                                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0u));
                    tq.q[slot] = make_int4(tq.pulse0, lane | (MODE << 6) | (nfull << 8) | (wave << 13), (int)marks,
                                           __float_as_int(a_lim));
                    tq.own[slot] = (unsigned short)((wave << 6) | lane);
                }
            }
            return;
        }
        for (; p + G <= np; p += G)
            nearest_group<G, MODE, ACC, DEM, PPT, F64>(A, smem, cst, klo_s, pos_s, p, i_pix, j_pix0, dxl, dyv, ddv,
                                                       accr, acci, cmpr, cmpi, dzv, hv, zl, wstride, pxd, a_lim, win_c);
        for (; p < np; ++p)
            nearest_group<1, MODE, ACC, DEM, PPT, F64>(A, smem, cst, klo_s, pos_s, p, i_pix, j_pix0, dxl, dyv, ddv,
                                                       accr, acci, cmpr, cmpi, dzv, hv, zl, wstride, pxd, a_lim, win_c);
        return;
    }
    constexpr int kUnroll = F64 ? BP_PUNROLL_F64 : (INTERP == SARBP_LINEAR ? BP_PUNROLL_LINEAR : BP_PUNROLL_SINC8);
#pragma unroll kUnroll
    for (int p = 0; p < np; ++p) {
        constexpr int CS = (DEM || F64) ? 3 : 2; // float4 constants per pulse
        const float4 c0 = cst[CS * p];
        const float4 c1 = cst[CS * p + 1];
        const float4 c2 = DEM ? cst[CS * p + 2] : c1;
        const uint32_t wbase = (uint32_t)p * wstride;
        if constexpr (INTERP == SARBP_LINEAR) {
#pragma unroll
            for (int m = 0; m < PPT; ++m) {
                float f;
                uint32_t kw;
                if constexpr (F64) {
                    locate_f64<MODE, DEM>(cst, p, pxd[0], pxd[1 + m], pxd[1 + PPT + m], pxd[1 + 2 * PPT + m], &f, &kw);
                } else {
                    const float num = pixel_num(dxl, dyv[m], ddv[m], dzv[m], c0, c2, DEM);
                    const float ub = bin_position<MODE, DevMath>(num, c0, c1);
                    f = DevMath::fract(ub);
                    kw = DevMath::to_u32(ub);
                }
                const uint32_t addr = (kw << 4) + wbase;
                const float4 ad = *reinterpret_cast<const float4*>(smem + addr);
                const float vr = fmaf(f, ad.z, ad.x);
                const float vi = fmaf(f, ad.w, ad.y);
                float sn, cs;
                sincos_rev(kappa * f, &sn, &cs);
                mac<ACC>(accr[m], acci[m], cmpr[m], cmpi[m], vr, vi, cs, sn);
            }
        } else {
            // 8-tap windowed sinc: entry k of the window holds the coefficients of the
            // degree-7 polynomial v(g) = sum_j C_j g^j, g = f - 1/2, that gives the
            // interpolated sample at k + f, already multiplied by the carrier of bin k
            // (built by stage_chunk).  Stored highest degree first, two per float4.
#pragma unroll
            for (int m = 0; m < PPT; ++m) {
                float f;
                uint32_t kw;
                if constexpr (F64) {
                    locate_f64<MODE, DEM>(cst, p, pxd[0], pxd[1 + m], pxd[1 + PPT + m], pxd[1 + 2 * PPT + m], &f, &kw);
                } else {
                    const float num = pixel_num(dxl, dyv[m], ddv[m], dzv[m], c0, c2, DEM);
                    const float ub = bin_position<MODE, DevMath>(num, c0, c1);
                    f = DevMath::fract(ub);
                    kw = DevMath::to_u32(ub);
                }
                const float g = f - 0.5f;
                const float4* e = reinterpret_cast<const float4*>(smem + ((kw << 6) + wbase));
                const float4 q0 = e[0], q1 = e[1], q2 = e[2], q3 = e[3];
                float vr = fmaf(q0.x, g, q0.z), vi = fmaf(q0.y, g, q0.w);
                vr = fmaf(vr, g, q1.x);
                vi = fmaf(vi, g, q1.y);
                vr = fmaf(vr, g, q1.z);
                vi = fmaf(vi, g, q1.w);
                vr = fmaf(vr, g, q2.x);
                vi = fmaf(vi, g, q2.y);
                vr = fmaf(vr, g, q2.z);
                vi = fmaf(vi, g, q2.w);
                vr = fmaf(vr, g, q3.x);
                vi = fmaf(vi, g, q3.y);
                vr = fmaf(vr, g, q3.z);
                vi = fmaf(vi, g, q3.w);
                float sn, cs;
                sincos_rev(kappa * f, &sn, &cs);
                mac<ACC>(accr[m], acci[m], cmpr[m], cmpi[m], vr, vi, cs, sn);
            }
        }
    }
}

// Stage the echo windows of one chunk into LDS.  Entry e = p W + kk of the
// chunk's np x W entries is bin kk of pulse p's window (the LDS order).  Lanes
// take B consecutive bins of one window per step (B = 2 for linear and nearest,
// whose windows have even W; 1 for sinc8), and the steps are spread evenly over
// all lanes of the workgroup, so short windows leave no lane idle; the pulse
// p = (e / B) / (W / B) is one multiply-high by the plan's ceil(2^32 B / W).
// Samples outside the record are zero: the loads read a clamped index and a
// select zeroes them.  The carrier table holds bins -4 .. n_range + 3 (every
// bin whose taps can reach the record; beyond them the samples are zero, so the
// clamped carrier is never seen) and then two NaN entries, which a pulse with
// no finite geometry reads instead, so its whole window is NaN.
__device__ __forceinline__ float2 sample_or_zero(const float2* row, int k, int nr) {
    const bool in = (uint32_t)k < (uint32_t)nr;
    const float2 v = row[in ? (uint32_t)k : 0u];
    return make_float2(in ? v.x : 0.f, in ? v.y : 0.f);
}

// One sinc8 window entry from its 8 taps k-3 .. k+4 and the carrier of bin k.
// Taps pair up as (k+t-3, k+4-t), t = 0..3: tap k+4-t's weight polynomial is tap
// k+t-3's with g -> -g, so coefficient j takes the pair's sum (j even) or
// difference (j odd) times sinc_poly[4 j + t].  Stored highest degree first.
__device__ __forceinline__ void sinc8_entry(const BpArgs& A, char* smem, int u, const float2* tap, float2 c0) {
    float2 ps[4], pd[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float2 sa = tap[t], sb = tap[7 - t];
        ps[t] = make_float2(sa.x + sb.x, sa.y + sb.y);
        pd[t] = make_float2(sa.x - sb.x, sa.y - sb.y);
    }
    float2 cj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float2* src = (j & 1) ? pd : ps;
        float r = 0.f, i = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            r = fmaf(A.sinc_poly[4 * j + t], src[t].x, r);
            i = fmaf(A.sinc_poly[4 * j + t], src[t].y, i);
        }
        cj[j] = cmul(make_float2(r, i), c0);
    }
    float4* dst = reinterpret_cast<float4*>(smem) + (size_t)u * 4;
    dst[0] = make_float4(cj[7].x, cj[7].y, cj[6].x, cj[6].y);
    dst[1] = make_float4(cj[5].x, cj[5].y, cj[4].x, cj[4].y);
    dst[2] = make_float4(cj[3].x, cj[3].y, cj[2].x, cj[2].y);
    dst[3] = make_float4(cj[1].x, cj[1].y, cj[0].x, cj[0].y);
}

// Staging when every window of the chunk, with its taps, lies inside the record
// (the set-up checks): no clamped indices or zero selects, and the samples
// addressed by 32-bit byte offsets from the chunk's first record (taken only while
// a chunk's records span less than 4 GiB).  Same entries as stage_chunk.
template <int INTERP>
__device__ void stage_inside(const BpArgs& A, char* smem, const int* klo_s, int np, int n0, int tid, int W) {
    constexpr int B = INTERP == SARBP_SINC8 ? 1 : 2;
    const int Wu = W / B, nr = A.n_range;
    const int nu = np * Wu;
    const float rwu = 1.0f / (float)Wu;
    const char* base = reinterpret_cast<const char*>(A.echo + (size_t)n0 * (size_t)nr);
    const char* ph = reinterpret_cast<const char*>(A.phase + 4); // carrier of bin 0
    for (int u = tid; u < nu; u += BP_THREADS) {
        int p, k;
        bool bad;
        stage_step_f32<B>(klo_s, u, Wu, rwu, &p, &k, &bad);
        const uint32_t off = ((uint32_t)p * (uint32_t)nr + (uint32_t)k) * 8u;
        const float2* e = reinterpret_cast<const float2*>(ph + (uint32_t)k * 8u);
        if constexpr (INTERP == SARBP_LINEAR) {
            const float2* q = reinterpret_cast<const float2*>(base + off);
            const float2 s0 = q[0], s1 = q[1], s2 = q[2], c0 = e[0], c1 = e[1];
            const float2 a0 = cmul(s0, c0), d0 = cmul(make_float2(s1.x - s0.x, s1.y - s0.y), c0);
            const float2 a1 = cmul(s1, c1), d1 = cmul(make_float2(s2.x - s1.x, s2.y - s1.y), c1);
            float4* dst = reinterpret_cast<float4*>(smem) + 2 * u;
            dst[0] = make_float4(a0.x, a0.y, d0.x, d0.y);
            dst[1] = make_float4(a1.x, a1.y, d1.x, d1.y);
        } else if constexpr (INTERP == SARBP_NEAREST) {
            const float2* q = reinterpret_cast<const float2*>(base + off);
            const float2 s0 = q[0], s1 = q[1], c0 = e[0], c1 = e[1];
            const float2 v0 = cmul(s0, c0), v1 = cmul(s1, c1);
            reinterpret_cast<float4*>(smem)[u] = make_float4(v0.x, v0.y, v1.x, v1.y);
        } else {
            const float2* q = reinterpret_cast<const float2*>(base + off - 24u); // taps k-3 .. k+4
            float2 tap[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) tap[t] = q[t];
            sinc8_entry(A, smem, u, tap, e[0]);
        }
    }
}

template <int INTERP>
__device__ void stage_chunk(const BpArgs& A, char* smem, const int* klo_s, int np, int n0, int tid, int W) {
    constexpr int B = INTERP == SARBP_SINC8 ? 1 : 2;
    const int Wu = W / B, nr = A.n_range;
    const int nu = np * Wu;
    // the pulse of a step: an fp32 quotient by the chunk's window, exactly corrected
    const float rwu = 1.0f / (float)Wu;
    for (int u = tid; u < nu; u += BP_THREADS) {
        int p, k;
        bool bad;
        stage_step_f32<B>(klo_s, u, Wu, rwu, &p, &k, &bad);
        const float2* row = A.echo + (size_t)(n0 + p) * (size_t)nr;
        const int ke = carrier_index<B>(k, nr, bad);
        const float2 c0 = A.phase[ke];
        if constexpr (INTERP == SARBP_LINEAR) {
            // every load of the step before any of its selects, so that their latencies overlap
            const bool in0 = (uint32_t)k < (uint32_t)nr, in1 = (uint32_t)(k + 1) < (uint32_t)nr,
                       in2 = (uint32_t)(k + 2) < (uint32_t)nr;
            const float2 r0 = row[in0 ? (uint32_t)k : 0u], r1 = row[in1 ? (uint32_t)(k + 1) : 0u],
                         r2 = row[in2 ? (uint32_t)(k + 2) : 0u];
            const float2 c1 = A.phase[ke + 1];
            __builtin_amdgcn_sched_barrier(0);
            const float2 s0 = make_float2(in0 ? r0.x : 0.f, in0 ? r0.y : 0.f),
                         s1 = make_float2(in1 ? r1.x : 0.f, in1 ? r1.y : 0.f),
                         s2 = make_float2(in2 ? r2.x : 0.f, in2 ? r2.y : 0.f);
            const float2 a0 = cmul(s0, c0), d0 = cmul(make_float2(s1.x - s0.x, s1.y - s0.y), c0);
            const float2 a1 = cmul(s1, c1), d1 = cmul(make_float2(s2.x - s1.x, s2.y - s1.y), c1);
            float4* dst = reinterpret_cast<float4*>(smem) + 2 * u;
            dst[0] = make_float4(a0.x, a0.y, d0.x, d0.y);
            dst[1] = make_float4(a1.x, a1.y, d1.x, d1.y);
        } else if constexpr (INTERP == SARBP_NEAREST) {
            const bool in0 = (uint32_t)k < (uint32_t)nr, in1 = (uint32_t)(k + 1) < (uint32_t)nr;
            const float2 r0 = row[in0 ? (uint32_t)k : 0u], r1 = row[in1 ? (uint32_t)(k + 1) : 0u];
            const float2 c1 = A.phase[ke + 1];
            __builtin_amdgcn_sched_barrier(0);
            const float2 s0 = make_float2(in0 ? r0.x : 0.f, in0 ? r0.y : 0.f),
                         s1 = make_float2(in1 ? r1.x : 0.f, in1 ? r1.y : 0.f);
            const float2 v0 = cmul(s0, c0), v1 = cmul(s1, c1);
            reinterpret_cast<float4*>(smem)[u] = make_float4(v0.x, v0.y, v1.x, v1.y);
        } else {
            float2 tap[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) tap[t] = sample_or_zero(row, k + t - 3, nr);
            sinc8_entry(A, smem, u, tap, c0);
        }
    }
}

// Set-up of the next chunk's candidate pulses n .. n + cand - 1 into one set of
// records and chunk words (the words must be zero).  Lanes 0 .. cand-1 take each
// pulse's constants in fp64 and its tile-centre bin u_c; lanes wl .. wl+cand-1 (wl
// a wave boundary past cand) take its exact window in parallel.  The chunk's length
// follows from the longest of these windows (chunk_length), so some candidates may
// be left for the chunk after; the chunk's accuracy mode, tie-band size and
// in-record flag are taken over all candidates, which only makes them cautious.
static_assert(BP_MAX_CHUNK <= 448 && BP_MAX_CHUNK_NEAREST <= BP_MAX_CHUNK,
              "set-up lanes 0 .. chunk - 1 and window lanes wl .. wl + chunk - 1 lie in one workgroup");
template <int INTERP, bool DEM, bool F64>
__device__ __forceinline__ void chunk_setup(const BpArgs& A, int tid, int n, int cand, int wl, float4* cst,
                                            int* klo_s, double* ext, int* mode_w, int* rho_w, int* wlen_w,
                                            int* edge_w, const double* box_s) {
    constexpr int CS = (DEM || F64) ? 3 : 2;
    if (tid < cand) {
        const size_t pa = 3 * (size_t)(n + tid);
        const double ax = A.pos[pa], ay = A.pos[pa + 1], az = A.pos[pa + 2];
        if constexpr (bp_ext_doubles(INTERP, F64) == 4) {
            double* ps = ext + A.chunk + 3 * tid; // the antenna positions follow the u_c words
            ps[0] = ax;
            ps[1] = ay;
            ps[2] = az;
        }
        const double gx = box_s[6], gy = box_s[7], gz = box_s[8];
        float rho = 0.f;
        double uc;
        const int need = F64 ? pulse_setup_f64(A, ax, ay, az, gx, gy, gz, cst + CS * tid, &uc)
                             : pulse_setup(A, ax, ay, az, gx, gy, gz, cst + CS * tid, &uc, &rho, DEM);
        ext[tid] = uc;
        if (need) atomicOr(mode_w, need);
        if constexpr (INTERP == SARBP_NEAREST && !F64) atomicMax(rho_w, __float_as_int(rho));
    } else if (tid >= wl && tid < wl + cand) {
        const int t = tid - wl;
        const size_t pa = 3 * (size_t)(n + t);
        const TileBox box = {box_s[0], box_s[1], box_s[2], box_s[3], box_s[4], box_s[5]};
        atomicMax(wlen_w, pulse_window(A, A.pos[pa], A.pos[pa + 1], A.pos[pa + 2], box, klo_s + t));
        if (!window_in_record<INTERP>(A, klo_s[t])) atomicOr(edge_w, 1);
    }
}

// At most 64 VGPRs, so two 1024-lane workgroups (8 waves per SIMD) fit on a CU:
// the loop needs that many waves to hide LDS and transcendental latency.
// F64: the fp64-range variant (pulse_setup_f64 / locate_f64) for plans whose echo
// window spans too many carrier cycles for the fp32 window position.
template <int INTERP, int ACC, bool DEM, int PPT, bool F64>
__global__ __launch_bounds__(BP_THREADS) __attribute__((amdgpu_waves_per_eu(8))) void bp_kernel(BpArgs A) {
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // XCD-aware tile order: workgroup b runs on XCD (b mod 8); give each XCD a
    // contiguous range of tiles (rows of tiles share echo bins in its L2).
    // Workgroup b handles tile (b mod ntiles) of voxel layer b / ntiles (one layer,
    // z = z0, for a 2-D image).
    // A split launch runs group_blocks workgroups per pulse group: group g takes
    // pulses g split_len .. and writes its partial image split_stride further on.
    const int group = (int)blockIdx.x / A.group_blocks;
    const int gb = (int)blockIdx.x - group * A.group_blocks;
    const int pb = group * A.split_len;             // this group's first pulse
    const int pn = min(A.split_len, A.n - pb);      // its pulses (a trailing group may have none)
    const TileFrame T = tile_frame<PPT>(A, gb);
    const int layer = T.layer, i0 = T.i0, j0 = T.j0;

    // Tile centre (fp64): the centre of the part of the tile inside the grid, which
    // brings the pixels of a ragged edge tile (or of a grid smaller than a tile)
    // closer to it than the full tile's half diagonal.  Lanes past the grid's edge
    // take the offsets of the last column or row, so every lane's range stays
    // within the staged window; their results are not stored.
    const int i_last = T.i_last, j_last = T.j_last;
    const double cxp = T.cxp, cyp = T.cyp;
    const double cx = T.cx, cy = T.cy;
    const double zl = T.zl; // this layer's height
    double cz = zl;
    const int i_off = min(i0 + lane, i_last); // the pixel column whose offsets this lane uses
    int j_off[PPT];
#pragma unroll
    for (int m = 0; m < PPT; ++m) j_off[m] = min(j0 + wave + BP_WAVES * m, j_last);
    const double ddx = ((double)i_off - cxp) * A.dx;
    float dxl;
    double pxd[1 + 3 * PPT]; // F64: ddx, then ddy, |d|^2 and (terrain) dz of each of the lane's pixels
    pxd[0] = ddx;
    float dyv[PPT], ddv[PPT], accr[PPT], acci[PPT];
    float cmpr[PPT], cmpi[PPT]; // Kahan compensation (ACC_KAHAN)
    double sumr[PPT], sumi[PPT]; // fp64 totals of the chunk partials (ACC_CHUNK64)
#pragma unroll
    for (int m = 0; m < PPT; ++m) {
        const double ddy = ((double)j_off[m] - cyp) * A.dy;
        pxd[1 + m] = ddy;
        pxd[1 + PPT + m] = ddx * ddx + ddy * ddy;
        pxd[1 + 2 * PPT + m] = 0.0;
        accr[m] = 0.f;
        acci[m] = 0.f;
        cmpr[m] = 0.f;
        cmpi[m] = 0.f;
        sumr[m] = 0.0;
        sumi[m] = 0.0;
    }

    // Terrain: pixel heights h (z = z0 + h); the tile centre sits at the tile's
    // mid-height, so |dz| <= half the tile's height range, which the plan's
    // window allows for up to dem_relief.  A tile beyond that bound is NaN.
    float dzv[PPT], hv[PPT];
    bool bad_tile = false;
    double za = zl, zb = zl; // the tile's height range (one plane, or the terrain's)
    double hc = 0.0;         // terrain: the tile's mid-height
    if constexpr (DEM) {
        float hmin = INFINITY, hmax = -INFINITY;
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            hv[m] = A.dem[(size_t)j_off[m] * A.nx + i_off]; // lanes past the edge repeat an edge pixel
            hmin = fminf(hmin, hv[m]);
            hmax = fmaxf(hmax, hv[m]);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            hmin = fminf(hmin, __shfl_xor(hmin, off));
            hmax = fmaxf(hmax, __shfl_xor(hmax, off));
        }
        float* red = reinterpret_cast<float*>(smem);
        if (lane == 0) {
            red[2 * wave] = hmin;
            red[2 * wave + 1] = hmax;
        }
        __syncthreads();
        hmin = red[0];
        hmax = red[1];
        for (int w = 1; w < BP_WAVES; ++w) {
            hmin = fminf(hmin, red[2 * w]);
            hmax = fmaxf(hmax, red[2 * w + 1]);
        }
        __syncthreads();
        bad_tile = !((double)hmax - (double)hmin <= A.dem_relief);
        hc = 0.5 * ((double)hmin + (double)hmax);
        cz = A.z0 + hc;
        za = A.z0 + (double)hmin;
        zb = A.z0 + (double)hmax;
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            const double ddy = ((double)j_off[m] - cyp) * A.dy;
            const double ddz = (double)hv[m] - hc;
            pxd[1 + PPT + m] = ddx * ddx + ddy * ddy + ddz * ddz;
            pxd[1 + 2 * PPT + m] = ddz;
        }
    }
    // the fp32 offsets of the pulse loop (the tie rechecks of its decisions take
    // them from the same function)
    lane_offsets<PPT, DEM>(A, T, hc, lane, wave, &dxl, dyv, ddv, dzv, hv);

    const int P = A.chunk; // pulses per chunk, at most (the record capacity)
    constexpr int CS = (DEM || F64) ? 3 : 2; // float4 constants per pulse
    constexpr int EXT = bp_ext_doubles(INTERP, F64);
    constexpr int B = INTERP == SARBP_SINC8 ? 1 : 2; // bins per staging step
    // LDS: A.entries window entries, which each chunk fills with its pulses' exact
    // windows (as many pulses as fit at its longest window: the tile's range extent
    // for this pulse, typically about half the tile diagonal the plan bounds it by);
    // then two sets of per-pulse records (constants, window start, the tile centre's
    // bin u_c and, for nearest with fp64 ranges, the antenna position its in-loop tie
    // rechecks read), so that the next chunk's set-up can write one set while the
    // loop reads the other; then the chunk words and the tile's pixel box.
    float4* cst0 = reinterpret_cast<float4*>(smem + (size_t)A.entries * entry_bytes<INTERP>());
    int* klo0 = reinterpret_cast<int*>(cst0 + 2 * CS * P);
    double* ext0 = reinterpret_cast<double*>(klo0 + 2 * P);
    int* prio_s = reinterpret_cast<int*>(ext0 + 2 * EXT * P);
    // The accuracy mode of a chunk is the OR of its pulses' modes, its window length
    // the longest of theirs, and its nearest tie band follows from the largest of
    // their range-term sizes rho.  The words are double-buffered with the records:
    // chunk c's set-up writes word set c & 1, which the staging phase of chunk c - 1
    // cleared after chunk c - 2 had finished reading it.  (rho >= 0, so its float
    // bits order as integers.)
    int* mode_s = prio_s + 1;
    int* rho_s = mode_s + 2;
    int* wlen_s = rho_s + 2;
    int* edge_s = wlen_s + 2; // nonzero: a window of the chunk reaches past the record (or has no geometry)
    // the tile's pixel box and reference point, read by the set-up lanes of each chunk
    double* box_s = reinterpret_cast<double*>(prio_s + 10);
    // nearest (fp32 ranges): the workgroup's queue of tie-recheck words, after the
    // box: the words, their owners and the count
    constexpr bool QUEUE = INTERP == SARBP_NEAREST && !F64 && BP_NEAREST_DEFER;
    TieQueue tq;
    tq.q = reinterpret_cast<int4*>(smem + ((reinterpret_cast<char*>(box_s + 9) - smem + 15) & ~(ptrdiff_t)15));
    tq.own = reinterpret_cast<unsigned short*>(tq.q + A.tie_queue);
    tq.count = reinterpret_cast<int*>(tq.own + A.tie_queue);
    tq.pulse0 = 0;
    if (tid == 0) {
        if constexpr (QUEUE) *tq.count = 0;
        mode_s[0] = mode_s[1] = rho_s[0] = rho_s[1] = wlen_s[0] = wlen_s[1] = edge_s[0] = edge_s[1] = 0;
        box_s[6] = cx;
        box_s[7] = cy;
        box_s[8] = cz;
        const TileBox b = tile_box(A, T, za, zb);
        box_s[0] = b.xa;
        box_s[1] = b.xb;
        box_s[2] = b.ya;
        box_s[3] = b.yb;
        box_s[4] = b.za;
        box_s[5] = b.zb;
    }
    __syncthreads();

    // The first chunk is half size on alternate workgroups: both placements of a
    // CU's two workgroups (b, b + slots) and (b, b + 8) get opposite parities.
    const int stagger = BP_STAGGER ? (((int)blockIdx.x / A.slots) ^ ((int)blockIdx.x >> 3)) & 1 : 0;
    const int pend = bad_tile ? 0 : pn; // the pulses this workgroup runs
    const int wl = (P + 63) & ~63;     // the first window lane of the set-up
    int cand = min(P, pend);
    if (cand > 0)
        chunk_setup<INTERP, DEM, F64>(A, tid, pb, cand, wl, cst0, klo0, ext0, mode_s, rho_s, wlen_s, edge_s, box_s);
    __syncthreads();
    // Each chunk: staging, barrier, the pulse loop, then the next chunk's set-up on
    // lanes 0 .. cand-1 and wl .. wl+cand-1, barrier.  The oldest waves of a
    // workgroup issue first and end the loop long before the youngest, so the set-up
    // runs while those finish instead of in a phase of its own.
    for (int n0 = 0, c = 0; n0 < pend; ++c) {
        const int s = c & 1;
        const float4* cst = cst0 + s * CS * P;
        const int* klo_s = klo0 + s * P;
        const double* ext = ext0 + s * EXT * P;
        const int win_c = chunk_window(__builtin_amdgcn_readfirstlane(wlen_s[s]), B, A.win);
        const int np = chunk_length(cand, A.entries, win_c, c == 0 && stagger);
        if (tid == 0) {
            *prio_s = chunk_priority(A, n0, pn);
            mode_s[s ^ 1] = 0;
            rho_s[s ^ 1] = 0;
            wlen_s[s ^ 1] = 0;
            edge_s[s ^ 1] = 0;
        }
        // each pulse's tile-centre position within its window (read by the pulse loop
        // after the next barrier), while all lanes stage the windows
        if (tid < np) pulse_finish(A, ext[tid], klo_s[tid], cst0 + s * CS * P + CS * tid, DEM, F64);
        if (A.fast_stage && __builtin_amdgcn_readfirstlane(edge_s[s]) == 0)
            stage_inside<INTERP>(A, smem, klo_s, np, pb + n0, tid, win_c);
        else
            stage_chunk<INTERP>(A, smem, klo_s, np, pb + n0, tid, win_c);
        __syncthreads();
        set_priority(*prio_s);
        const int mode = __builtin_amdgcn_readfirstlane(mode_s[s]); // the same word for every lane
        const int m1 = mode & 1, m2 = mode & 2;
        const int mi = m2 ? 2 : (m1 ? 1 : 0);
        // nearest: |fract(ub) - 1/2| beyond tie_lim means ub is within the tie band of an
        // integer; the test is made on the phase a = kappa (fract(ub) - 1/2) against a_lim
        float a_lim = 0.f;
        tq.pulse0 = pb + n0;
        if constexpr (INTERP == SARBP_NEAREST) {
            const float rho = __int_as_float(__builtin_amdgcn_readfirstlane(rho_s[s]));
            const float tie_lim = 0.5f - fmaf(A.tie_rho[mi], rho, fmaf(A.tie_win, (float)win_c, A.tie_base[mi]));
            a_lim = nearest_tie_limit(A.kappa, tie_lim);
        }
        if (m2)
            accumulate_chunk<INTERP, 2, ACC, DEM, PPT, F64>(A, smem, cst, klo_s, ext + P, np, i0 + lane, j0 + wave, dxl,
                                                            dyv, ddv, accr, acci, cmpr, cmpi, dzv, hv, zl, pxd, a_lim,
                                                            win_c, tq);
        else if (m1)
            accumulate_chunk<INTERP, 1, ACC, DEM, PPT, F64>(A, smem, cst, klo_s, ext + P, np, i0 + lane, j0 + wave, dxl,
                                                            dyv, ddv, accr, acci, cmpr, cmpi, dzv, hv, zl, pxd, a_lim,
                                                            win_c, tq);
        else
            accumulate_chunk<INTERP, 0, ACC, DEM, PPT, F64>(A, smem, cst, klo_s, ext + P, np, i0 + lane, j0 + wave, dxl,
                                                            dyv, ddv, accr, acci, cmpr, cmpi, dzv, hv, zl, pxd, a_lim,
                                                            win_c, tq);
        if constexpr (ACC == SARBP_ACC_CHUNK64) {
#pragma unroll
            for (int m = 0; m < PPT; ++m) {
                sumr[m] += (double)accr[m];
                sumi[m] += (double)acci[m];
                accr[m] = 0.f;
                acci[m] = 0.f;
            }
        }
        const int n1 = n0 + np;
        cand = min(P, pend - n1);
        if (cand > 0)
            chunk_setup<INTERP, DEM, F64>(A, tid, pb + n1, cand, wl, cst0 + (s ^ 1) * CS * P, klo0 + (s ^ 1) * P,
                                          ext0 + (s ^ 1) * EXT * P, mode_s + (s ^ 1), rho_s + (s ^ 1),
                                          wlen_s + (s ^ 1), edge_s + (s ^ 1), box_s);
        __syncthreads();
        n0 = n1;
        if constexpr (QUEUE) {
            // resolve the tie queue when it could not take another chunk's words
            const int qn = __builtin_amdgcn_readfirstlane(*tq.count);
            if (n0 < pend && qn > A.tie_queue - BP_THREADS) {
                drain_ties<BP_NEAREST_GROUP, ACC, DEM, PPT>(A, tq, qn, box_s, T, hc, zl, smem, pb, pn, accr, acci,
                                                            cmpr, cmpi);
                if (tid == 0) *tq.count = 0; // read again after the next chunk's first barrier
            }
        }
    }

    if constexpr (QUEUE) {
        const int qn = __builtin_amdgcn_readfirstlane(*tq.count);
        if (qn > 0) {
            drain_ties<BP_NEAREST_GROUP, ACC, DEM, PPT>(A, tq, qn, box_s, T, hc, zl, smem, pb, pn, accr, acci, cmpr,
                                                        cmpi);
            if constexpr (ACC == SARBP_ACC_CHUNK64) {
#pragma unroll
                for (int m = 0; m < PPT; ++m) {
                    sumr[m] += (double)accr[m];
                    sumi[m] += (double)acci[m];
                }
            }
        }
    }
    if (bad_tile) {
#pragma unroll
        for (int m = 0; m < PPT; ++m) accr[m] = acci[m] = sumr[m] = sumi[m] = NAN;
    }
    const int i = i0 + lane;
    if (i < A.nx) {
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            const int j = j0 + wave + BP_WAVES * m;
            if (j < A.ny) {
                float2* o = A.image + (size_t)group * A.split_stride + ((size_t)layer * A.ny + j) * A.nx + i;
                if constexpr (ACC == SARBP_ACC_CHUNK64) {
                    double r = sumr[m], im = sumi[m];
                    if (A.accumulate) {
                        const float2 old = *o;
                        r += (double)old.x;
                        im += (double)old.y;
                    }
                    *o = make_float2((float)r, (float)im);
                } else {
                    float r = accr[m], im = acci[m];
                    if constexpr (ACC == SARBP_ACC_KAHAN) {
                        r -= cmpr[m];
                        im -= cmpi[m];
                    }
                    if (A.accumulate) {
                        const float2 old = *o;
                        r = old.x + r;
                        im = old.y + im;
                    }
                    *o = make_float2(r, im);
                }
            }
        }
    }
}

template <int INTERP, int ACC, bool DEM, int PPT, bool F64>
int allow_lds_one(size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(bp_kernel<INTERP, ACC, DEM, PPT, F64>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess
               ? SARBP_OK
               : SARBP_EDEVICE;
}

template <int INTERP, bool DEM, int PPT, bool F64>
int allow_lds_acc(int accum, size_t bytes) {
    switch (accum) {
        case SARBP_ACC_KAHAN: return allow_lds_one<INTERP, SARBP_ACC_KAHAN, DEM, PPT, F64>(bytes);
        case SARBP_ACC_CHUNK64: return allow_lds_one<INTERP, SARBP_ACC_CHUNK64, DEM, PPT, F64>(bytes);
        default: return allow_lds_one<INTERP, SARBP_ACC_FP32, DEM, PPT, F64>(bytes);
    }
}

// Kernel variants: ppt 1 or 2 with fp32 ranges, and ppt 2 with fp64 ranges.
template <int INTERP, bool DEM>
int allow_lds(int accum, int ppt, bool f64, size_t bytes) {
    if (f64) return allow_lds_acc<INTERP, DEM, 2, true>(accum, bytes);
    return ppt == 1 ? allow_lds_acc<INTERP, DEM, 1, false>(accum, bytes)
                    : allow_lds_acc<INTERP, DEM, 2, false>(accum, bytes);
}

template <int INTERP, bool DEM, int PPT, bool F64>
void launch_acc(const BpArgs& A, int accum, size_t lds, hipStream_t stream) {
    const dim3 grid(A.nblocks), block(BP_THREADS);
    switch (accum) {
        case SARBP_ACC_KAHAN:
            hipLaunchKernelGGL((bp_kernel<INTERP, SARBP_ACC_KAHAN, DEM, PPT, F64>), grid, block, lds, stream, A);
            break;
        case SARBP_ACC_CHUNK64:
            hipLaunchKernelGGL((bp_kernel<INTERP, SARBP_ACC_CHUNK64, DEM, PPT, F64>), grid, block, lds, stream, A);
            break;
        default:
            hipLaunchKernelGGL((bp_kernel<INTERP, SARBP_ACC_FP32, DEM, PPT, F64>), grid, block, lds, stream, A);
            break;
    }
}

template <int INTERP, bool DEM>
void launch(const BpArgs& A, int accum, int ppt, bool f64, size_t lds, hipStream_t stream) {
    if (f64) return launch_acc<INTERP, DEM, 2, true>(A, accum, lds, stream);
    if (ppt == 1) launch_acc<INTERP, DEM, 1, false>(A, accum, lds, stream);
    else launch_acc<INTERP, DEM, 2, false>(A, accum, lds, stream);
}

// Sum of the pulse groups' partial images of a split backprojection, in group
// order and in fp64, added to the image (accumulate = 1) or written over it.
__global__ __launch_bounds__(256) void split_sum_kernel(const float2* __restrict__ part, int nsplit, size_t elems,
                                                        float2* __restrict__ image, int accumulate) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < elems; e += stride) {
        double r = 0.0, im = 0.0;
        for (int g = 0; g < nsplit; ++g) {
            const float2 v = part[(size_t)g * elems + e];
            r += (double)v.x;
            im += (double)v.y;
        }
        if (accumulate) {
            const float2 old = image[e];
            r += (double)old.x;
            im += (double)old.y;
        }
        image[e] = make_float2((float)r, (float)im);
    }
}

} // namespace

int sarbp_split_count(const sarbp_plan* plan, int n) {
    // Pulse groups so that the launch has about two workgroups per CU, at most 16,
    // each of at least 32 pulses; grids that already fill the GPU are not split.
    const int64_t layers = plan->p.nz > 1 ? plan->p.nz : 1;
    const int64_t blocks = (int64_t)plan->L.tiles_x * plan->L.tiles_y * layers;
    int64_t s = (2 * (int64_t)plan->L.n_cu) / blocks;
    if (s > 16) s = 16;
    if (s > n / 32) s = n / 32;
    return s < 2 ? 1 : (int)s;
}

int sarbp_bp_allow_lds(int interp, int accum, bool dem, int ppt, bool f64, size_t bytes) {
    switch (interp) {
        case SARBP_NEAREST:
            return dem ? allow_lds<SARBP_NEAREST, true>(accum, ppt, f64, bytes)
                       : allow_lds<SARBP_NEAREST, false>(accum, ppt, f64, bytes);
        case SARBP_LINEAR:
            return dem ? allow_lds<SARBP_LINEAR, true>(accum, ppt, f64, bytes)
                       : allow_lds<SARBP_LINEAR, false>(accum, ppt, f64, bytes);
        default:
            return dem ? allow_lds<SARBP_SINC8, true>(accum, ppt, f64, bytes)
                       : allow_lds<SARBP_SINC8, false>(accum, ppt, f64, bytes);
    }
}

int sarbp_launch_bp(const sarbp_plan* plan, const double* pos, const float2* echo, const float* dem,
                    float2* image, int n, int accumulate, hipStream_t stream, float2* workspace, int nsplit) {
    const sarbp_params& p = plan->p;
    const BpLayout& L = plan->L;
    BpArgs A;
    sarbp_bp_args(p, L, &A);
    A.pos = pos;
    A.echo = echo;
    A.image = image;
    A.phase = plan->phase_tab;
    A.progress = plan->progress;
    A.dem = dem;
    A.n = n;
    const size_t elems = (size_t)(p.nz > 1 ? p.nz : 1) * (size_t)p.ny * (size_t)p.nx;
    const bool split = nsplit > 1 && workspace != nullptr;
    if (!split) nsplit = 1;
    A.nblocks = A.group_blocks * nsplit;
    A.split_len = split ? (n + nsplit - 1) / nsplit : n;
    A.split_stride = split ? elems : 0;
    if (split) {
        A.image = workspace; // partial images, written over; summed into `image` below
        A.accumulate = 0;
    } else {
        A.accumulate = accumulate;
    }
    const bool d = dem != nullptr;
    switch (p.interp) {
        case SARBP_NEAREST:
            d ? launch<SARBP_NEAREST, true>(A, p.accum, L.ppt, L.f64, L.lds_bytes, stream)
              : launch<SARBP_NEAREST, false>(A, p.accum, L.ppt, L.f64, L.lds_bytes, stream);
            break;
        case SARBP_LINEAR:
            d ? launch<SARBP_LINEAR, true>(A, p.accum, L.ppt, L.f64, L.lds_bytes, stream)
              : launch<SARBP_LINEAR, false>(A, p.accum, L.ppt, L.f64, L.lds_bytes, stream);
            break;
        default:
            d ? launch<SARBP_SINC8, true>(A, p.accum, L.ppt, L.f64, L.lds_bytes, stream)
              : launch<SARBP_SINC8, false>(A, p.accum, L.ppt, L.f64, L.lds_bytes, stream);
            break;
    }
    if (hipGetLastError() != hipSuccess) return SARBP_EDEVICE;
    if (split) {
        const size_t blocks = (elems + 255) / 256;
        hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, stream,
                           static_cast<const float2*>(workspace), nsplit, elems, image, accumulate);
        if (hipGetLastError() != hipSuccess) return SARBP_EDEVICE;
    }
    return SARBP_OK;
}
