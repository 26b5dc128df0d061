// Host-side emulation of the backprojection kernels' index and window-position
// arithmetic (sarbp_check_indices, include/sarbp.h).  It runs, on the CPU, the
// same per-tile frame, per-pulse set-up, staging index steps and per-pixel window
// positions as the kernels (shared through sarbp_geom.h, instantiated with the
// host math policy), and checks every LDS window index and staging index against
// its range.  For nearest interpolation it also replays the fp32 bin decisions
// and the tie band, and compares the bins they keep with the definition's
// floor(u + 1/2) in double precision.
//
// The page "基于GPU的SAR后向投影成像优化与CUDA加速实践" (GPU-based SAR
// backprojection), section 4.4, names index errors that read outside the echo
// window as the usual source of a noisy image and recommends checking for them
// with a memory checker; this emulation is that check for the kernels' arithmetic,
// run on the host over a caller's own geometry.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "sarbp_geom.h"
#include "sarbp_internal.h"

namespace {

struct Checker {
    const sarbp_params& p;
    const BpLayout& L;
    BpArgs A;
    const double* pos;
    int n;
    const float* dem;
    sarbp_index_report* r;
    uint32_t flagged[BP_WAVES][BP_TX]; // per lane of the current chunk: its groups of pulses with a decision in the band
    std::vector<uint32_t> marked;      // the pulses the queued words mark (a bitmap over the call's pulses)

    // A queue resolution of qn words: whether the set-ups of the pulses its words mark
    // fit the kernels' table (the window LDS after the bitmap and its prefix counts,
    // and the queue's unused words), as the kernel decides it.
    void resolve_queue(int qn, bool dem) {
        int K = 0;
        for (uint32_t w : marked) K += __builtin_popcount(w);
        const int nbw = (int)marked.size();
        const int region = L.entries * entry_bytes<SARBP_NEAREST>();
        const int head = ((2 * nbw + 1) * 4 + 15) & ~15;
        const int te = (dem ? 3 : 2) * 16 + 4;
        const bool table = head <= region && K <= (region - head) / te + (L.tie_queue - qn) * 16 / te;
        ++(table ? r->tie_queue_tables : r->tie_queue_table_misses);
        std::fill(marked.begin(), marked.end(), 0u);
    }

    Checker(const sarbp_params& p_, const BpLayout& L_, const double* pos_, int n_, const float* dem_,
            sarbp_index_report* r_)
        : p(p_), L(L_), pos(pos_), n(n_), dem(dem_), r(r_) {
        sarbp_bp_args(p, L, &A);
        A.n = n;
        A.split_len = n;
    }

    // The definition's fractional bin u of pixel (i, j) at height z for pulse q.
    double def_bin(int q, int i, int j, double z) const {
        const double* a = pos + 3 * (size_t)q;
        return definition_bin<HostMath>(a[0], a[1], a[2], A.x0, A.y0, z, A.dx, A.dy, A.r0, A.dr, i, j);
    }

    void stage_check(const int* klo_s, int np, int win_c) {
        const int B = p.interp == SARBP_SINC8 ? 1 : 2;
        const int wu = win_c / B;
        const float rwu = 1.0f / (float)wu;
        if (win_c % B != 0 || win_c > A.win || np * win_c > A.entries) ++r->staging_violations;
        for (int u = 0; u < np * wu; ++u) {
            int pp, k;
            bool bad;
            if (B == 1)
                stage_step_f32<1>(klo_s, u, wu, rwu, &pp, &k, &bad);
            else
                stage_step_f32<2>(klo_s, u, wu, rwu, &pp, &k, &bad);
            bool ok = pp == u / wu && pp >= 0 && pp < np;
            if (ok) {
                const int ke = B == 1 ? carrier_index<1>(k, A.n_range, bad) : carrier_index<2>(k, A.n_range, bad);
                ok = ke >= 0 && ke + B - 1 <= A.n_range + 9;
                if (!bad) ok = ok && k - klo_s[pp] >= 0 && k - klo_s[pp] + B - 1 <= win_c - 1;
            }
            if (!ok) ++r->staging_violations;
        }
    }

    // One window position of a pixel: bin k (LDS entry) and fraction f.
    template <int MODE, bool DEM, bool F64>
    void locate(const float4* cst, int pl, float dxl, float dy, float dd, float dz, const double* pxd, int m,
                int ppt, uint32_t* k, float* f, double* ub) const {
        if (F64) {
            locate_f64<MODE, DEM>(cst, pl, pxd[0], pxd[1 + m], pxd[1 + ppt + m], pxd[1 + 2 * ppt + m], f, k);
            *ub = (double)*k + (double)*f;
        } else {
            const int CS = DEM ? 3 : 2;
            const float4 c0 = cst[CS * pl], c1 = cst[CS * pl + 1], c2 = DEM ? cst[CS * pl + 2] : c1;
            const float num = pixel_num(dxl, dy, dd, dz, c0, c2, DEM);
            const float u = bin_position<MODE, HostMath>(num, c0, c1);
            *f = HostMath::fract(u);
            *k = HostMath::to_u32(u);
            *ub = (double)u;
        }
    }

    template <int PPT, bool DEM, bool F64>
    void run() {
        const int CS = (DEM || F64) ? 3 : 2;
        const int P = A.chunk;
        std::vector<float4> cst((size_t)CS * P);
        std::vector<int> klo(P);
        std::vector<double> uc(P);
        const int nb = A.group_blocks;
        const bool nearest = p.interp == SARBP_NEAREST;
        const bool sinc8 = p.interp == SARBP_SINC8;
        for (int b = 0; b < nb; ++b) {
            const TileFrame T = tile_frame<PPT>(A, b);
            // Lane offsets, as in the kernel: lanes past the grid's edge repeat the last column or row.
            float dxl[BP_TX], dyv[BP_WAVES][PPT], ddv[BP_TX][BP_WAVES][PPT], dzv[BP_TX][BP_WAVES][PPT];
            double pxd[BP_TX][BP_WAVES][1 + 3 * PPT];
            float hv[BP_TX][BP_WAVES][PPT];
            double cz = T.zl, za = T.zl, zb = T.zl;
            bool bad_tile = false;
            double hc = 0.0;
            if (DEM) {
                float hmin = INFINITY, hmax = -INFINITY;
                for (int lane = 0; lane < BP_TX; ++lane)
                    for (int w = 0; w < BP_WAVES; ++w)
                        for (int m = 0; m < PPT; ++m) {
                            const int io = std::min(T.i0 + lane, T.i_last);
                            const int jo = std::min(T.j0 + w + BP_WAVES * m, T.j_last);
                            hv[lane][w][m] = dem[(size_t)jo * A.nx + io];
                            hmin = fminf(hmin, hv[lane][w][m]);
                            hmax = fmaxf(hmax, hv[lane][w][m]);
                        }
                bad_tile = !((double)hmax - (double)hmin <= A.dem_relief);
                hc = 0.5 * ((double)hmin + (double)hmax);
                cz = A.z0 + hc;
                za = A.z0 + (double)hmin;
                zb = A.z0 + (double)hmax;
            }
            const TileBox box = tile_box(A, T, za, zb);
            if (bad_tile) {
                ++r->nan_tiles;
                continue;
            }
            for (int lane = 0; lane < BP_TX; ++lane) {
                const int io = std::min(T.i0 + lane, T.i_last);
                const double ddx = ((double)io - T.cxp) * A.dx;
                dxl[lane] = (float)ddx;
                for (int w = 0; w < BP_WAVES; ++w)
                    for (int m = 0; m < PPT; ++m) {
                        const int jo = std::min(T.j0 + w + BP_WAVES * m, T.j_last);
                        const double ddy = ((double)jo - T.cyp) * A.dy;
                        const double ddz = DEM ? (double)hv[lane][w][m] - hc : 0.0;
                        dyv[w][m] = (float)ddy;
                        ddv[lane][w][m] = (float)(ddx * ddx + ddy * ddy + (DEM ? ddz * ddz : 0.0));
                        dzv[lane][w][m] = (float)ddz;
                        double* x = pxd[lane][w];
                        x[0] = ddx;
                        x[1 + m] = ddy;
                        x[1 + PPT + m] = ddx * ddx + ddy * ddy + (DEM ? ddz * ddz : 0.0);
                        x[1 + 2 * PPT + m] = ddz;
                    }
            }
            const int stagger = BP_STAGGER ? ((b / A.slots) ^ (b >> 3)) & 1 : 0;
            int queued = 0, tile_words = 0; // the deferred nearest rechecks' queue (one per workgroup)
            marked.assign((size_t)(n + 31) / 32, 0u);
            for (int n0 = 0, np = 0, c = 0; n0 < n; n0 += np, ++c) {
                // the set-up's candidates: constants, u_c and exact window of each; the
                // chunk's mode, tie-band size and in-record flag over all of them
                const int cand = std::min(P, n - n0);
                int cmode = 0, wmax = 0;
                float crho = 0.f;
                bool inside = A.fast_stage != 0;
                for (int t = 0; t < cand; ++t) {
                    const double* a = pos + 3 * (size_t)(n0 + t);
                    float rh = 0.f;
                    cmode |= F64 ? pulse_setup_f64(A, a[0], a[1], a[2], T.cx, T.cy, cz, &cst[(size_t)CS * t], &uc[t])
                                 : pulse_setup(A, a[0], a[1], a[2], T.cx, T.cy, cz, &cst[(size_t)CS * t], &uc[t],
                                               &rh, DEM);
                    wmax = std::max(wmax, pulse_window(A, a[0], a[1], a[2], box, &klo[t]));
                    if (!F64) crho = std::max(crho, rh);
                    inside = inside && (sinc8 ? window_in_record<SARBP_SINC8>(A, klo[t])
                                              : window_in_record<SARBP_LINEAR>(A, klo[t]));
                }
                const int win_c = chunk_window(wmax, sinc8 ? 1 : 2, A.win);
                np = chunk_length(cand, A.entries, win_c, c == 0 && stagger);
                for (int t = 0; t < np; ++t) pulse_finish(A, uc[t], klo[t], &cst[(size_t)CS * t], DEM, F64);
                const int mi = (cmode & 2) ? 2 : (cmode & 1);
                ++r->mode_chunks[mi];
                r->window_mean += win_c;
                ++r->chunks;
                stage_check(klo.data(), np, win_c);
                // the in-record staging path: taken when every candidate's window, with
                // what its staging reads, lies in the record; then every sample it reads
                // must be in the record
                if (inside) {
                    ++r->chunks_in_record;
                    for (int t = 0; t < np; ++t) {
                        const int lo = klo[t] - (sinc8 ? 3 : 0);
                        const int hi = klo[t] + win_c - 1 + (sinc8 ? 4 : (p.interp == SARBP_LINEAR ? 1 : 0));
                        const uint64_t last = ((uint64_t)t * (uint64_t)A.n_range + (uint64_t)hi) * 8u + 8u;
                        if (lo < 0 || hi > A.n_range - 1 || last >= (1ull << 32)) ++r->staging_violations;
                    }
                }
                // the tie band (twice the error bound of the chunk's window positions)
                const float band = fmaf(A.tie_rho[mi], crho, fmaf(A.tie_win, (float)win_c, A.tie_base[mi]));
                const float tie_lim = 0.5f - band;
                if (nearest) r->tie_band_max = std::max(r->tie_band_max, band);
                if (mi == 2)
                    pixels<2, PPT, DEM, F64>(T, np, n0, cst.data(), klo.data(), dxl, dyv, ddv, dzv, pxd, hv, hc,
                                             tie_lim, band, win_c);
                else if (mi == 1)
                    pixels<1, PPT, DEM, F64>(T, np, n0, cst.data(), klo.data(), dxl, dyv, ddv, dzv, pxd, hv, hc,
                                             tie_lim, band, win_c);
                else
                    pixels<0, PPT, DEM, F64>(T, np, n0, cst.data(), klo.data(), dxl, dyv, ddv, dzv, pxd, hv, hc,
                                             tie_lim, band, win_c);
                if (nearest && !F64 && BP_NEAREST_DEFER) {
                    // each lane with a decision in the band queues one word; between chunks
                    // the queue is resolved when it has no room for another chunk's words
                    int cnt = 0;
                    const int nf = np / BP_NEAREST_GROUP;
                    for (int w = 0; w < BP_WAVES; ++w)
                        for (int lane = 0; lane < BP_TX; ++lane) {
                            cnt += flagged[w][lane] != 0;
                            for (uint32_t g = flagged[w][lane]; g != 0; g &= g - 1) {
                                const int gi = __builtin_ctz(g);
                                const int p0 = gi < nf ? gi * BP_NEAREST_GROUP : nf * BP_NEAREST_GROUP + (gi - nf);
                                for (int q = 0; q < (gi < nf ? BP_NEAREST_GROUP : 1); ++q)
                                    marked[(n0 + p0 + q) >> 5] |= 1u << ((n0 + p0 + q) & 31);
                            }
                        }
                    queued += cnt;
                    tile_words += cnt;
                    r->tie_queue_words += cnt;
                    if (n0 + np < n && queued > L.tie_queue - BP_THREADS) {
                        ++r->tie_queue_drains;
                        resolve_queue(queued, DEM);
                        queued = 0;
                    }
                }
            }
            r->tie_queue_tile_max = std::max(r->tie_queue_tile_max, tile_words);
            if (nearest && !F64 && BP_NEAREST_DEFER && queued > 0) resolve_queue(queued, DEM);
        }
    }

    template <int MODE, int PPT, bool DEM, bool F64>
    void pixels(const TileFrame& T, int np, int n0, const float4* cst, const int* klo, const float* dxl,
                const float (*dyv)[PPT], const float (*ddv)[BP_WAVES][PPT], const float (*dzv)[BP_WAVES][PPT],
                const double (*pxd)[BP_WAVES][1 + 3 * PPT], const float (*hv)[BP_WAVES][PPT], double hc,
                float tie_lim, float band, int win_c) {
        const bool nearest = p.interp == SARBP_NEAREST;
        const double half = nearest ? 0.5 : 0.0;
        const float a_lim = nearest_tie_limit(A.kappa, tie_lim);
        for (int w = 0; w < BP_WAVES; ++w)
            for (int lane = 0; lane < BP_TX; ++lane) flagged[w][lane] = 0;
        for (int t = 0; t < np; ++t) {
            const bool bad = klo[t] == INT32_MIN;
            for (int lane = 0; lane < BP_TX; ++lane) {
                const int i = T.i0 + lane;
                for (int w = 0; w < BP_WAVES; ++w)
                    for (int m = 0; m < PPT; ++m) {
                        const int j = T.j0 + w + BP_WAVES * m;
                        uint32_t k;
                        float f;
                        double ub;
                        locate<MODE, DEM, F64>(cst, t, dxl[lane], dyv[w][m], ddv[lane][w][m], dzv[lane][w][m],
                                               pxd[lane][w], m, PPT, &k, &f, &ub);
                        ++r->decisions;
                        if (bad) continue;
                        if (!(ub >= 0.0) || !(k <= (uint32_t)(win_c - 1))) ++r->window_violations;
                        r->min_position = std::min(r->min_position, ub);
                        r->max_position_margin = std::max(r->max_position_margin, ub - (double)win_c);
                        if (i >= A.nx || j >= A.ny) continue; // lanes past the edge: results not stored
                        const double z = DEM ? A.z0 + (double)hv[lane][w][m] : T.zl;
                        const double u = def_bin(n0 + t, i, j, z);
                        const double want = u - (double)klo[t] + half; // the exact window position
                        const double err = fabs(ub - want);
                        r->max_position_error = std::max(r->max_position_error, err);
                        r->max_error_to_band = std::max(r->max_error_to_band, err / (0.5 * (double)band));
                        if (!nearest) continue;
                        const int kdef = (int)floor(u + 0.5);
                        if (fabsf(nearest_phase(A.kappa, f)) > a_lim) { // the kernel's tie test
                            ++r->nearest_rechecks;
                            {
                                const int nf = np / BP_NEAREST_GROUP; // the kernel's mark: one bit per group
                                flagged[w][lane] |= 1u << (t < nf * BP_NEAREST_GROUP ? t / BP_NEAREST_GROUP
                                                                                     : nf + (t - nf * BP_NEAREST_GROUP));
                            }
                            const int kr = kdef - klo[t];
                            if (kr < 0 || kr > win_c - 1) ++r->nearest_recheck_clamped;
                        } else if ((int)k + klo[t] != kdef) {
                            ++r->nearest_escapes;
                        }
                    }
            }
        }
        (void)hc;
    }
};

} // namespace

extern "C" int sarbp_check_indices(const sarbp_params* params, int32_t n_cu, const double* positions_h, int32_t n,
                                   const float* dem_h, sarbp_index_report* report) {
    if (report == nullptr || positions_h == nullptr || n < 1) return SARBP_EINVAL;
    memset(report, 0, sizeof(*report));
    int st = sarbp_validate(params);
    if (st != SARBP_OK) return st;
    if (n > params->n_pulses) return SARBP_EINVAL;
    if (dem_h != nullptr && !(params->dem_relief > 0.0)) return SARBP_EINVAL;
    BpLayout L;
    st = sarbp_plan_layout(*params, n_cu > 0 ? n_cu : 256, &L);
    if (st != SARBP_OK) return st;
    report->window = L.win;
    report->chunk = L.chunk;
    report->pixels_per_lane = L.ppt;
    report->fp64_ranges = L.f64;
    report->tie_queue_capacity = L.tie_queue;
    report->min_position = INFINITY;
    report->max_position_margin = -INFINITY;
    Checker c(*params, L, positions_h, n, dem_h, report);
    const bool dem = dem_h != nullptr;
    if (L.f64) {
        dem ? c.run<2, true, true>() : c.run<2, false, true>();
    } else if (L.ppt == 1) {
        dem ? c.run<1, true, false>() : c.run<1, false, false>();
    } else {
        dem ? c.run<2, true, false>() : c.run<2, false, false>();
    }
    if (report->chunks > 0) report->window_mean /= (double)report->chunks;
    return SARBP_OK;
}
