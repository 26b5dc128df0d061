// Internal declarations shared by the host side of the sarbp library.
// Not installed; the public interface is include/sarbp.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sarbp.h"

// Backprojection tiling (see sarbp_bp.hip): a workgroup of BP_WAVES wave64s
// owns a tile of BP_TX (along x) by BP_WAVES * ppt (along y) pixels; each lane
// keeps ppt pixels of one column in registers.  16 waves x 2 pixels (64 x 32
// tiles, 1024-lane workgroups) measured fastest on gfx950: the loop is bound by
// VALU issue and needs many waves per SIMD to hide LDS and transcendental
// latency.  Grids of fewer than two such tiles per CU use 1 pixel per lane
// (64 x 16 tiles) instead, so that two workgroups still share each CU.
#define BP_TX 64
#ifndef BP_WAVES
#define BP_WAVES 16
#endif
#define BP_THREADS (64 * BP_WAVES)
#ifndef BP_MAX_CHUNK
#define BP_MAX_CHUNK 224 // pulses staged in LDS per step, at most (the set-up takes one lane per pulse)
#endif
#ifndef BP_MAX_CHUNK_NEAREST
#define BP_MAX_CHUNK_NEAREST 112 // nearest: one tie-mark bit per group of pulses in a 32-bit word
#endif
// Pulses per unrolled hot-loop iteration (measured best: linear four, sinc8
// eight).  Nearest works on groups of pulses, with one tie branch per group.
#ifndef BP_PUNROLL_LINEAR
#define BP_PUNROLL_LINEAR 4
#endif
#ifndef BP_NEAREST_DEFER
#define BP_NEAREST_DEFER 1
#endif
#ifndef BP_TIE_QUEUE
#define BP_TIE_QUEUE 2048 // nearest (fp32 ranges): queued tie-recheck words per workgroup, at least (18 B each, in LDS)
#endif
#if BP_TIE_QUEUE < 2 * BP_THREADS || BP_TIE_QUEUE > 65536
#error "a chunk adds up to one tie-queue word per lane, and the queue is resolved when it holds more than BP_TIE_QUEUE - BP_THREADS"
#endif
#ifndef BP_NEAREST_GROUP
#define BP_NEAREST_GROUP 4
#endif
#ifndef BP_PUNROLL_F64
#define BP_PUNROLL_F64 1 // fp64-range kernels (measured: 1, 2 and 4 equal for linear and nearest; sinc8 5 % faster at 1)
#endif
#ifndef BP_PUNROLL_SINC8
#define BP_PUNROLL_SINC8 8
#endif
// Workgroups that share a CU start with a half-size pulse chunk on alternate
// slots, so their chunk barriers (pulse set-up and echo staging) do not line up.
#ifndef BP_STAGGER
#define BP_STAGGER 1
#endif
#ifndef BP_LDS_BUDGET
#define BP_LDS_BUDGET 80000 // bytes per workgroup: two 1024-lane workgroups per CU fit in 160 KiB
#endif

// Doubles kept per pulse beside its constants in a backprojection chunk's records:
// the tile centre's bin u_c, and for nearest with fp64 ranges (whose tie rechecks
// run inside the pulse loop) the antenna position.
__host__ __device__ constexpr int bp_ext_doubles(int interp, bool f64) {
    return (interp == SARBP_NEAREST && f64) ? 4 : 1;
}

// Backprojection launch geometry of a plan: a function of its parameters and
// the device's compute-unit count alone (sarbp_plan_layout), so that the host
// emulation of the kernels' index arithmetic (sarbp_check_indices) can build it
// without a device.
struct BpLayout {
    int n_cu;         // compute units the layout is for
    int tiles_x, tiles_y;
    int ppt;          // backprojection pixels per lane (1 or 2): tiles of 64 x 16 ppt
    int f64;          // 1: range differences in fp64 (windows of many carrier cycles; ppt = 2)
    int win;          // LDS window entries per pulse, at most (a chunk stages its pulses' exact extent)
    int margin_lo;    // bins below the tile's lowest range kept in the window
    int chunk;        // pulses per LDS step, at most (the per-pulse record capacity)
    int entries;      // LDS window entries per step, shared by the step's pulses
    int tie_queue;    // nearest (fp32 ranges): words of the workgroup's tie-recheck queue, else 0
    size_t lds_bytes; // dynamic LDS per workgroup
    double half_span; // half tile diagonal [m]
    // sinc8: monomial coefficients in g = f - 1/2 of the degree-7 interpolant of
    // tap t - 3 (t = 0..3) of the windowed sinc, coefficient j at [4 j + t]
    float sinc_poly[32];
};

struct sarbp_plan {
    sarbp_params p;
    int device;
    BpLayout L;
    // exp(+j 4 pi (r0 + k dr) / lambda) for k = -4 .. n_range + 3, stored at [k + 4]
    float2* phase_tab;
    int* progress;    // [2 * n_cu] per-workgroup pulse progress (scheduling hints only)
    void* scratch;    // device address of the library's static scratch on the plan's device (not owned)
    // range compression
    int rc_log2;       // log2(n_fast), 0 when disabled
    float2* rc_filter; // conj(FFT(ref)) * W / n_fast
};

// Argument block of the backprojection kernels (passed by value).
struct BpArgs {
    const double* pos;     // [n][3]
    const float2* echo;    // [n][n_range]
    float2* image;         // [ny][nx]
    const float2* phase;   // phase_tab
    int n, n_range, nx, ny;
    int tiles_x, ntiles;
    int nblocks;           // the launch's workgroups: group_blocks * pulse groups
    int group_blocks;      // ntiles * voxel layers: the workgroups of one pulse group
    int split_len;         // pulses per group (n when the pulses are not split)
    size_t split_stride;   // complex64 elements between the groups' partial images (0 unsplit)
    int win, margin_lo, chunk, accumulate; // win: the plan's (longest) window; chunk: pulses per step, at most
    int entries;           // LDS window entries per step (a step holds entries / its window pulses)
    int tie_queue;         // nearest (fp32 ranges): words of the workgroup's tie-recheck queue
    int fast_stage;        // 1: a chunk's records span less than 4 GiB, so staging may use 32-bit byte offsets
    int slots;             // compute units: workgroup b and b + slots usually share a CU
    int* progress;         // [2 * slots] pulse progress per workgroup, read by its CU partner
    double r0, dr, inv_dr, x0, y0, z0, dx, dy;
    double dz;             // voxel layer spacing (3-D images), else 0
    double half_span;      // half tile diagonal [m]
    double half_span_bins; // half_span / dr
    float sinc_poly[32];   // see sarbp_plan::sinc_poly
    const float* dem;      // [ny][nx] pixel heights above z0 (terrain kernels), else null
    double dem_relief;     // bound on one tile's height range (terrain kernels)
    float kappa;           // 2 dr / lambda: phase cycles per bin
    // nearest: fp64 recheck band around a rounding tie [bins], per accuracy mode:
    // tie_base[m] + tie_win * (the chunk's window) + tie_rho[m] * (its largest range-term size, in bins)
    float tie_base[3], tie_win, tie_rho[3];
    int round_half;        // nearest: window positions carry u + 1/2
};

// Largest nearest tie band [bins] the fp32 kernels accept on a 64 x 32 tile; a
// plan beyond it takes the fp64-range kernels, whose band is 1e-6 bins.  (The
// band's fp64 rechecks cost about 100 instructions each: at 2.5e-4 bins that is
// about one update in five.)
#ifndef BP_NEAREST_TIE_MAX
#define BP_NEAREST_TIE_MAX 2.5e-4
#endif

// Validate parameters (SARBP_OK, SARBP_EINVAL, SARBP_EUNSUPPORTED); no device use.
int sarbp_validate(const sarbp_params* p);
// The backprojection layout of p on a device of n_cu compute units (SARBP_OK or
// SARBP_EUNSUPPORTED); p must have passed sarbp_validate.
int sarbp_plan_layout(const sarbp_params& p, int n_cu, BpLayout* L);
// The launch-independent fields of the backprojection kernels' arguments
// (pointers, pulse counts and split fields are left for the launch).
void sarbp_bp_args(const sarbp_params& p, const BpLayout& L, BpArgs* A);

int sarbp_launch_bp(const sarbp_plan* plan, const double* pos, const float2* echo, const float* dem,
                    float2* image, int n, int accumulate, hipStream_t stream, float2* workspace = nullptr,
                    int nsplit = 1);
// Argument checks shared by the pulse-group entry points (SARBP_OK or SARBP_EINVAL).
int sarbp_split_check(const sarbp_plan* plan, const double* positions_d, const void* echo_d, const float* dem_d,
                      const void* image_d, int32_t n, int32_t accumulate);
// SARBP_OK when the current device is the plan's.
int sarbp_check_device(const sarbp_plan* plan);
// The device address of the static scratch array on `device` (the current device),
// looked up once per device and cached.
int sarbp_scratch_address(int device, void** out);
// Pulse groups of a split backprojection of n pulses (1: no split) and its workspace bytes.
int sarbp_split_count(const sarbp_plan* plan, int n);
int sarbp_launch_rc(const sarbp_plan* plan, const float2* raw, float2* out, int n, hipStream_t stream);
