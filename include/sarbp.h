/*
 * sarbp.h -- time-domain SAR backprojection on AMD Instinct MI355X (gfx950).
 *
 * The method is the one of the page "基于GPU的SAR后向投影成像优化与CUDA加速实践"
 * (GPU-based SAR backprojection imaging and CUDA acceleration):
 *
 *   I(x, y) = sum over pulses n of  interp(s_n, R_n(x, y)) * exp(+j 4 pi R_n / lambda)
 *
 * (section 1.1 for the coherent sum over pulses at each pixel's range history;
 * section 2.2 for the four per-pulse steps and the interpolation choices;
 * section 3.3 for the argument list: antenna X/Y/Z per pulse, the
 * range-compressed complex matrix indexed [pulse * n_range + bin], the range
 * axis r0 and dr, the pixel grid x = x0 + i dx, y = y0 + j dy, and the image
 * indexed [j * nx + i]; section 4.2 for the carrier wavelength in the phase).
 * Range compression (section 3.1) is an FFT matched filter with an optional
 * Hamming or Taylor window, batched over pulses.
 *
 * Conventions shared by every entry point:
 *   - Complex data are complex64: interleaved (re, im) float pairs.
 *   - Device pointers are caller-owned device memory on the plan's device;
 *     the library never frees or retains them.  Every pointer must be 8-byte
 *     aligned.  Array contents are not inspected: NaN in gives NaN out.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Argument checks are synchronous and return SARBP_EINVAL
 *     before anything is enqueued; a failed launch returns SARBP_EDEVICE.
 *   - A plan's parameters and device tables are immutable after creation,
 *     so calls with one plan on different streams may run concurrently.  The
 *     plan also owns a small progress array that backprojection workgroups
 *     write and read to balance issue priority between the two workgroups of
 *     a compute unit; it steers scheduling only, so overlapping calls that
 *     share it stay correct (they may run slightly slower).  Calls that write
 *     the same image must be ordered by the caller.  No entry point allocates
 *     device memory except sarbp_plan_create and sarbp_stream_create (the library's
 *     one static device array is described at sarbp_backproject_split_noalloc).
 */
#ifndef SARBP_H
#define SARBP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SARBP_OK 0
#define SARBP_EINVAL (-1)       /* an argument is out of range, null or misaligned */
#define SARBP_ENOMEM (-2)       /* a device or host allocation failed (plan creation only) */
#define SARBP_EDEVICE (-3)      /* a HIP runtime call or kernel launch failed */
#define SARBP_EUNSUPPORTED (-4) /* valid request the library cannot serve (e.g. LDS too small) */
#define SARBP_ESCRATCH (-5)     /* the call needs more than the library's static scratch (see below) */

/* Interpolation of the range-compressed echo at a fractional bin u (section 2.2):
 *   NEAREST: s[floor(u + 1/2)]
 *   LINEAR : (1 - f) s[k] + f s[k + 1],  k = floor(u), f = u - k
 *   SINC8  : sum_{m=-3..4} s[k + m] h(f - m),
 *            h(t) = sinc(t) (0.54 + 0.46 cos(pi t / 4)) for |t| < 4
 * Samples outside [0, n_range - 1] are zero. */
typedef enum { SARBP_NEAREST = 0, SARBP_LINEAR = 1, SARBP_SINC8 = 2 } sarbp_interp;

/* How the sum over pulses is accumulated (section 4.3 of the page: fp32 sums over
 * thousands of pulses lose precision; it offers a Kahan compensation term in the
 * kernel, or partial sums folded into double precision).  The image stays complex64.
 *   SARBP_ACC_FP32    fp32 registers (default, fastest)
 *   SARBP_ACC_KAHAN   fp32 with a Kahan compensation term per pixel, per pulse
 *   SARBP_ACC_CHUNK64 fp32 within each LDS pulse chunk (<= 224 pulses), chunk partial
 *                     sums added in fp64 (nearly free) */
typedef enum { SARBP_ACC_FP32 = 0, SARBP_ACC_KAHAN = 1, SARBP_ACC_CHUNK64 = 2 } sarbp_accum;

/* Plan parameters.  Lengths in metres, frequencies in Hz, times in seconds. */
typedef struct {
    int32_t n_pulses;   /* Na: the most pulses one sarbp_backproject call may take (>= 1)      */
    int32_t n_range;    /* Nr: bins per range-compressed pulse (>= 2; >= 8 for SINC8)           */
    double r0;          /* range of bin 0                                                       */
    double dr;          /* bin spacing (> 0): bin k lies at r0 + k * dr                         */
    int32_t nx, ny;     /* image size (>= 1 each); image[j * nx + i]                           */
    double x0, y0, z0;  /* centre of pixel (0, 0); every pixel lies in the plane z = z0          */
    double dx, dy;      /* pixel spacing (> 0): pixel (i, j) centre = (x0 + i dx, y0 + j dy, z0);
                         * a plan whose LDS echo window spans more than 4096 carrier cycles,
                         * (2 dr / lambda) x (window bins) ~ 4 x (tile half diagonal) / lambda
                         * for 64 dx x 32 dy tiles (relief included), takes range differences
                         * in fp64 (about 1.4x the time)                                      */
    double wavelength;  /* carrier wavelength lambda (> 0) of the phase term exp(+j 4 pi R / lambda);
                         * 2 dr / lambda, the carrier cycles per range bin, must be below 255
                         * (SARBP_EUNSUPPORTED otherwise): the kernels rotate each sample with
                         * hardware sine and cosine, whose argument is limited to 256 cycles */
    int32_t interp;     /* sarbp_interp                                                         */
    /* Range compression (sarbp_range_compress); n_fast = 0 disables it. */
    int32_t n_fast;     /* samples per raw pulse = FFT length: a power of two in [64, 16384]    */
    double fs;          /* fast-time sampling rate (> 0)                                        */
    double chirp_T;     /* LFM pulse length (> 0); round(chirp_T * fs) samples, <= n_fast      */
    double chirp_B;     /* LFM bandwidth (> 0), up-chirp exp(j pi (B/T) t^2), -T/2 <= t < T/2   */
    int32_t window;     /* weight w(f / B) over |f| <= B/2, zero outside the band:
                         *   0: none (w = 1 everywhere); 1: Hamming 0.54 + 0.46 cos(2 pi x);
                         *   2: Taylor, 1 + 2 sum_{m<nbar} F_m cos(2 pi m x) scaled to w(0) = 1
                         *      (the page's lower-widening alternative to Hamming, section 3.1) */
    int32_t taylor_nbar; /* Taylor: nearly equal sidelobes, 2..64 (0: 4)                        */
    double taylor_sll;   /* Taylor: design sidelobe level in dB below the peak, 13..150 (0: 35)  */
    int32_t accum;       /* sarbp_accum of sarbp_backproject (0: SARBP_ACC_FP32)                 */
    double dem_relief;   /* terrain (sarbp_backproject_dem): bound on the height range, max - min,
                          * within any 64 x 32-pixel block of the grid aligned to pixel (0, 0)
                          * (the whole map's range will do); 0 disables terrain.  The echo
                          * windows grow with it.                                            */
    /* 3-D imaging (section 5 of the page names backprojection onto a volume as the
     * next step): nz layers of the grid, layer l at height z0 + l dz; the image is
     * complex64 [nz][ny][nx].  nz = 0 or 1 is the plane z = z0.                    */
    int32_t nz;          /* voxel layers, 0..65535 (0 or 1: a 2-D image)                          */
    double dz;           /* layer spacing (> 0 when nz > 1)                                       */
} sarbp_params;

typedef struct sarbp_plan sarbp_plan; /* opaque */

/* Validate `params`, build the plan's device tables (read-only phase and
 * filter tables, plus the 2 x compute-unit progress array) on the current
 * HIP device and return the plan in *out (set to NULL on failure).
 * Returns SARBP_EINVAL for invalid parameters, SARBP_ENOMEM if an allocation
 * fails, SARBP_EDEVICE if the HIP runtime fails. */
int sarbp_plan_create(const sarbp_params* params, sarbp_plan** out);

/* Backproject n pulses into the image (sections 1.1, 2.2 and 3.3 of the page).
 *   positions_d : device, float64 [n][3] antenna phase centres (x, y, z)
 *   echo_d      : device, complex64 [n][n_range] range-compressed echo, bin fastest
 *   image_d     : device, complex64 [ny][nx], x fastest ([nz][ny][nx] for a volume);
 *                 written (accumulate = 0) or added to (accumulate = 1)
 *   n           : pulses in this call, 1 <= n <= plan n_pulses
 * Because the sum is linear in the echo, a long aperture can be streamed in
 * pulse chunks with accumulate = 1.  Returns SARBP_EINVAL (null plan or
 * pointer, misalignment, n out of range, accumulate not 0/1, or the current
 * device is not the plan's), SARBP_EDEVICE on a launch failure. */
int sarbp_backproject(const sarbp_plan* plan, const double* positions_d, const void* echo_d,
                      void* image_d, int32_t n, int32_t accumulate, void* stream);

/* Backproject onto terrain (section 3.3 of the page: the pixel height may have to
 * follow elevation data): as sarbp_backproject, with pixel (i, j) at
 * (x0 + i dx, y0 + j dy, z0 + dem[j * nx + i]).
 *   dem_d : device, float32 [ny][nx] heights above z0, 4-byte aligned
 * The plan must have dem_relief > 0 and nz <= 1.  Pixels of a 64 x 32 block whose heights
 * span more than dem_relief come out NaN, as does a pixel with a non-finite
 * height.  Returns SARBP_EINVAL (as sarbp_backproject, or a null or misaligned
 * dem, or a plan without terrain), SARBP_EDEVICE on a launch failure. */
int sarbp_backproject_dem(const sarbp_plan* plan, const double* positions_d, const void* echo_d, const float* dem_d,
                          void* image_d, int32_t n, int32_t accumulate, void* stream);

/* ---- Small grids: the pulses split over several workgroups per pixel tile. ----
 * A grid with fewer than two 64 x 32 (or 64 x 16) pixel tiles per compute unit
 * leaves most of the GPU idle in sarbp_backproject, whose workgroups each own one
 * tile for every pulse (the sum of section 1.1 runs over the pulses of one
 * pixel).  The sum is linear in the pulses, so it can run as S groups of
 * consecutive pulses, each into a partial image, followed by the sum of the
 * partials. */

/* Workspace for sarbp_backproject_split of n pulses with this plan: S partial
 * images of complex64 [nz][ny][nx], S = 2 .. 16 chosen so that the launch holds
 * about two workgroups per compute unit with at least 32 pulses per group.
 * Returns 0 when the plan's grid already fills the GPU (or for a null plan or n
 * out of range): such calls run unsplit and need no workspace. */
size_t sarbp_split_workspace_bytes(const sarbp_plan* plan, int32_t n);

/* As sarbp_backproject (dem_d = NULL) or sarbp_backproject_dem (dem_d not NULL),
 * with the pulses split into S groups as above.
 *   workspace_d     : device memory of at least sarbp_split_workspace_bytes(plan, n)
 *                     bytes, 8-byte aligned, not overlapping the image; caller-owned,
 *                     written by the call (its contents afterwards are unspecified).
 *                     May be NULL when that size is 0.
 * Each group sums its pulses as sarbp_backproject does (with the plan's
 * accumulator) into an fp32 partial image; a second kernel adds the S partials
 * in group order in fp64, plus the old image when accumulate = 1, and rounds once
 * to complex64.  The result equals sarbp_backproject's up to that summation order
 * (about 1e-7 relative).  Two calls must not share a workspace while both may
 * run.  Returns SARBP_EINVAL as sarbp_backproject / sarbp_backproject_dem, or for
 * a missing, short, misaligned or overlapping workspace; SARBP_EDEVICE on a launch
 * failure. */
int sarbp_backproject_split(const sarbp_plan* plan, const double* positions_d, const void* echo_d,
                            const float* dem_d, void* image_d, int32_t n, int32_t accumulate, void* workspace_d,
                            size_t workspace_bytes, void* stream);

/* ---- For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the pulse-group
 * backprojection with its partial images in a static device array of the library
 * instead of a caller workspace. ------------------------------------------------ */

/* Size of that array, per GPU: 8 MiB.  On a 256-CU MI355X every plan's pulse-group
 * workspace fits: at most 2 x 256 workgroups' tiles of up to 2048 pixels, 8 bytes
 * each. */
#define SARBP_STATIC_SCRATCH_BYTES (8u << 20)

/* As sarbp_backproject_split with no workspace argument: the S partial images go to
 * the library's static array on the plan's device (its address on each device is
 * taken once, by the first sarbp_plan_create there).  The call itself allocates
 * nothing and runs the same kernels, so its image equals sarbp_backproject_split's
 * bit for bit.  When sarbp_split_workspace_bytes(plan, n) is 0 it runs unsplit,
 * as sarbp_backproject does.  The array keeps the last call's partials; every
 * element is written before it is read, so no clearing is needed, but all calls on
 * one GPU share it: two calls that may run at the same time on one GPU (on
 * different streams or host threads) race and give wrong images -- order them.
 * Returns SARBP_ESCRATCH when the workspace would exceed
 * SARBP_STATIC_SCRATCH_BYTES (possible only on a GPU with more compute units), and
 * otherwise the codes of sarbp_backproject_split. */
int sarbp_backproject_split_noalloc(const sarbp_plan* plan, const double* positions_d, const void* echo_d,
                                    const float* dem_d, void* image_d, int32_t n, int32_t accumulate,
                                    void* stream);

/* Range-compress n raw pulses (section 3.1 of the page):
 *   out_n = IFFT( FFT(raw_n) * conj(FFT(ref)) * W ) with 1/n_fast on the inverse,
 *   ref[m mod n_fast] = p(m / fs), m = -L/2 .. L/2 - 1, L = round(chirp_T * fs).
 *   raw_d : device, complex64 [n][n_fast]
 *   out_d : device, complex64 [n][n_fast]; must not overlap raw_d
 * Output bin k corresponds to the range of raw sample k.  Returns
 * SARBP_EINVAL (as above, or the plan has n_fast = 0, or the buffers
 * overlap), SARBP_EDEVICE on a launch failure. */
int sarbp_range_compress(const sarbp_plan* plan, const void* raw_d, void* out_d, int32_t n,
                         void* stream);

/* Release the plan and its device tables.  NULL is a no-op.  The caller must
 * ensure no call using the plan is still running. */
void sarbp_destroy(sarbp_plan* plan);

/* ---- Antenna positions from navigation samples (section 3.3 of the page: in
 * practice the radar position of each pulse may have to be interpolated from the
 * flight track). -------------------------------------------------------------- */

/* Interpolate positions at n pulse times from n_nav navigation samples: per axis,
 * the cubic Lagrange polynomial through the 4 samples around the time (two on each
 * side where the record allows: samples j0 .. j0+3, j0 = clamp(i - 1, 0, n_nav - 4)
 * for the interval i with nav_t[i] <= t < nav_t[i+1]), in double precision.
 *   nav_t_d     : device, float64 [n_nav], strictly increasing sample times
 *   nav_xyz_d   : device, float64 [n_nav][3] sampled positions
 *   t_d         : device, float64 [n] pulse times
 *   positions_d : device, float64 [n][3] output, ready for sarbp_backproject; must
 *                 not overlap the inputs
 * A time outside [nav_t[0], nav_t[n_nav-1]], a non-finite time, or a stencil whose
 * times do not increase gives NaN for that pulse (which backprojection propagates).
 * Returns SARBP_EINVAL (null or misaligned pointer, n_nav < 4, n < 1, overlap),
 * SARBP_EDEVICE on a launch failure.  Asynchronous on `stream`. */
int sarbp_interpolate_track(const double* nav_t_d, const double* nav_xyz_d, int32_t n_nav, const double* t_d,
                            double* positions_d, int32_t n, void* stream);

/* ---- Streaming pulses from host memory (section 3.3 of the page: prefetch the
 * echo with streams so that copies overlap computation). --------------------- */

typedef struct sarbp_stream sarbp_stream; /* opaque */

/* Create a host-to-device pipeline for `plan` on the plan's device: two device
 * staging buffers of `chunk` pulses each, a copy stream and its events.
 *   chunk    : pulses per staged step, 1 <= chunk <= plan n_pulses
 *   compress : 0: host data is the range-compressed echo, [n][n_range];
 *              1: host data is raw pulses, [n][n_fast], range-compressed on the
 *                 device chunk by chunk (requires n_fast = n_range)
 * The plan must outlive the stream object.  Returns SARBP_EINVAL (bad chunk,
 * compress without a compatible plan, null pointers, wrong device),
 * SARBP_ENOMEM, SARBP_EDEVICE. */
int sarbp_stream_create(const sarbp_plan* plan, int32_t chunk, int32_t compress, sarbp_stream** out);

/* Backproject n pulses held in host memory into a device image.
 *   positions_h : host, float64 [n][3]
 *   data_h      : host, complex64 pulses (see compress above)
 *   image_d     : device, complex64 [ny][nx]; written (accumulate = 0) or added to
 *   n           : any count >= 1 (it may exceed the plan's n_pulses: the pulses
 *                 go through in chunks, each added to the image)
 * Chunk c is copied on the object's copy stream while chunk c - 1 is processed
 * on `stream`; the two staging buffers alternate, ordered by events.  Before
 * refilling a staging buffer the calling thread waits until the device has
 * finished with it, so the host runs at most two chunks ahead (and the call
 * cannot be captured into a HIP graph); it returns once the last chunk is
 * enqueued.  Synchronise `stream` before reading the
 * image or reusing the host buffers.  Overlap needs page-locked host memory
 * (hipHostMalloc); pageable memory still works but copies synchronously.  One
 * stream object must not be used by two threads at once; calls on it are
 * ordered through its buffers' events.  Returns SARBP_EINVAL (null pointer,
 * n < 1, accumulate not 0/1, wrong device), SARBP_EDEVICE. */
int sarbp_backproject_host(sarbp_stream* s, const double* positions_h, const void* data_h, void* image_d,
                           int32_t n, int32_t accumulate, void* stream);

/* Release the stream object after its work has finished.  NULL is a no-op. */
void sarbp_stream_destroy(sarbp_stream* s);

/* ---- Host-side check of the kernels' index arithmetic (section 4.4 of the page:
 * an index outside the staged echo window fills the image with noise, so index
 * bounds are worth checking with a memory checker).  No device is used. ------ */

typedef struct {
    int64_t decisions;               /* window positions evaluated: pixels x pulses, lanes past the grid's edge included */
    int64_t window_violations;       /* positions outside [0, W) of their pulse's LDS window (must be 0)               */
    int64_t staging_violations;      /* staging steps whose pulse, carrier-table index or window bin is out of range (must be 0) */
    int64_t nearest_rechecks;        /* nearest: decisions inside the fp64 tie band (rechecked in fp64)                */
    int64_t nearest_recheck_clamped; /* nearest: rechecked bins outside the window (must be 0)                         */
    int64_t nearest_escapes;         /* nearest: decisions outside the band whose bin differs from floor(u + 1/2) (must be 0) */
    int64_t nan_tiles;               /* terrain tiles beyond dem_relief (skipped; their pixels come out NaN)           */
    double max_position_error;       /* largest |window position - exact one| over in-grid pixels [bins]               */
    double max_error_to_band;        /* largest ratio of that error to the error bound of its chunk (half the tie band) */
    double min_position;             /* smallest window position (>= 0 required)                                        */
    double max_position_margin;      /* largest window position minus its chunk's window length (< 0 required)          */
    double window_mean;              /* mean window length of the chunks (each stages its pulses' exact extent)         */
    int64_t chunks;                  /* pulse chunks staged (all workgroups)                                            */
    int64_t chunks_in_record;        /* of which staged by the in-record path (every window and its taps in the record) */
    int32_t window;                  /* W: the plan's longest LDS window, entries per pulse                             */
    int32_t chunk;                   /* pulses per LDS chunk, at most (each holds what its exact windows let fit)       */
    int32_t pixels_per_lane;         /* 1 or 2 (tiles of 64 x 16 or 64 x 32 pixels)                                    */
    int32_t fp64_ranges;             /* 1: the plan runs the fp64-range kernels                                         */
    int32_t mode_chunks[3];          /* chunks whose window position used the two-term series, three terms, exact form */
    float tie_band_max;              /* the widest tie band of any chunk [bins] (the fp32 decision is rechecked within it) */
    int64_t tie_queue_words;         /* nearest, fp32 ranges: words queued for the deferred recheck, one per lane and chunk
                                        with a decision inside the band                                                 */
    int64_t tie_queue_drains;        /* the workgroups' queues resolved between chunks (more words than a chunk's room)  */
    int32_t tie_queue_tile_max;      /* the most words one workgroup (one tile) queued over the call                    */
    int32_t tie_queue_capacity;      /* words per workgroup the kernels' queue holds                                    */
    int64_t tie_queue_tables;        /* queue resolutions whose marked pulses' set-ups fit a table in LDS               */
    int64_t tie_queue_table_misses;  /* queue resolutions that repeat each word's set-ups instead (no table fits)        */
} sarbp_index_report;

/* Emulate on the host, for the plan `params` would create on a device of n_cu
 * compute units (0: 256, one MI355X), the backprojection kernels' index and
 * window-position arithmetic for n pulses (one call, unsplit): each workgroup's
 * tile frame and lane offsets, each pulse chunk's fp64 set-up, staging steps and
 * accuracy mode, and every lane's fp32 (or fp64-range) window position, with the
 * kernels' own source code (the only difference: the exact form's fp32 square
 * root and reciprocal are correctly rounded on the host, within about one ulp of
 * the device's).  Counts out-of-range indices and, for nearest interpolation,
 * bin decisions that would differ from the double-precision definition.
 *   positions_h : host, float64 [n][3]; 1 <= n <= params->n_pulses
 *   dem_h       : host, float32 [ny][nx] terrain heights (the sarbp_backproject_dem
 *                 kernels), or NULL (sarbp_backproject; required NULL when
 *                 dem_relief = 0)
 * Cost: about the kernel's work per pixel and pulse on one host thread (a few
 * tens of nanoseconds each).  Returns SARBP_OK with *report filled, SARBP_EINVAL
 * or SARBP_EUNSUPPORTED as sarbp_plan_create would, or SARBP_EINVAL for a null
 * pointer or n out of range. */
int sarbp_check_indices(const sarbp_params* params, int32_t n_cu, const double* positions_h, int32_t n,
                        const float* dem_h, sarbp_index_report* report);

/* Static description of a status code (never NULL). */
const char* sarbp_status_string(int status);

/* Library version as 10000 * major + 100 * minor + patch. */
int sarbp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SARBP_H */
