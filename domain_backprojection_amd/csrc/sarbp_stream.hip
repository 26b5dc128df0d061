// Host-to-device pulse pipeline of the sarbp C ABI (see include/sarbp.h): two
// device staging buffers alternate between a copy stream (host -> device) and
// the caller's compute stream (optional range compression, then
// backprojection), ordered by events, so the copy of one chunk overlaps the
// processing of the previous one.
#include <stdint.h>
#include <string.h>

#include <new>

#include "sarbp_internal.h"

struct sarbp_stream {
    const sarbp_plan* plan;
    int device;
    int chunk;
    int compress;
    size_t row;                // complex64 samples per staged pulse
    hipStream_t copy;          // host -> device copies
    hipEvent_t copied[2];      // staging buffer b holds its chunk
    hipEvent_t released[2];    // the last kernel reading staging buffer b has run
    double* pos_d[2];          // [chunk][3]
    float2* data_d[2];         // [chunk][row]: echo, or raw pulses when compressing
    float2* rc_d;              // [chunk][row]: compressed chunk (compress = 1)
    hipEvent_t rc_free;        // the last kernel reading rc_d has run
};

namespace {

void release(sarbp_stream* s) {
    if (s == nullptr) return;
    int cur = -1;
    const bool switch_dev = hipGetDevice(&cur) == hipSuccess && cur != s->device;
    if (switch_dev) (void)hipSetDevice(s->device);
    for (int b = 0; b < 2; ++b) {
        if (s->pos_d[b]) (void)hipFree(s->pos_d[b]);
        if (s->data_d[b]) (void)hipFree(s->data_d[b]);
        if (s->copied[b]) (void)hipEventDestroy(s->copied[b]);
        if (s->released[b]) (void)hipEventDestroy(s->released[b]);
    }
    if (s->rc_d) (void)hipFree(s->rc_d);
    if (s->rc_free) (void)hipEventDestroy(s->rc_free);
    if (s->copy) (void)hipStreamDestroy(s->copy);
    if (switch_dev) (void)hipSetDevice(cur);
    delete s;
}

bool aligned8(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

} // namespace

extern "C" int sarbp_stream_create(const sarbp_plan* plan, int32_t chunk, int32_t compress, sarbp_stream** out) {
    if (out == nullptr) return SARBP_EINVAL;
    *out = nullptr;
    if (plan == nullptr || chunk < 1 || chunk > plan->p.n_pulses || (compress != 0 && compress != 1))
        return SARBP_EINVAL;
    if (compress && (plan->p.n_fast == 0 || plan->p.n_fast != plan->p.n_range)) return SARBP_EINVAL;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SARBP_EDEVICE;
    if (cur != plan->device) return SARBP_EINVAL;

    sarbp_stream* s = new (std::nothrow) sarbp_stream();
    if (s == nullptr) return SARBP_ENOMEM;
    memset(s, 0, sizeof(*s));
    s->plan = plan;
    s->device = plan->device;
    s->chunk = chunk;
    s->compress = compress;
    s->row = (size_t)plan->p.n_range;
    if (hipStreamCreateWithFlags(&s->copy, hipStreamNonBlocking) != hipSuccess) {
        release(s);
        return SARBP_EDEVICE;
    }
    for (int b = 0; b < 2; ++b) {
        if (hipEventCreateWithFlags(&s->copied[b], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&s->released[b], hipEventDisableTiming) != hipSuccess) {
            release(s);
            return SARBP_EDEVICE;
        }
        if (hipMalloc(reinterpret_cast<void**>(&s->pos_d[b]), (size_t)chunk * 3 * sizeof(double)) != hipSuccess ||
            hipMalloc(reinterpret_cast<void**>(&s->data_d[b]), (size_t)chunk * s->row * sizeof(float2)) !=
                hipSuccess) {
            release(s);
            return SARBP_ENOMEM;
        }
    }
    if (compress) {
        if (hipEventCreateWithFlags(&s->rc_free, hipEventDisableTiming) != hipSuccess) {
            release(s);
            return SARBP_EDEVICE;
        }
        if (hipMalloc(reinterpret_cast<void**>(&s->rc_d), (size_t)chunk * s->row * sizeof(float2)) != hipSuccess) {
            release(s);
            return SARBP_ENOMEM;
        }
    }
    *out = s;
    return SARBP_OK;
}

extern "C" int sarbp_backproject_host(sarbp_stream* s, const double* positions_h, const void* data_h,
                                      void* image_d, int32_t n, int32_t accumulate, void* stream) {
    if (s == nullptr || positions_h == nullptr || data_h == nullptr || !aligned8(image_d) || n < 1 ||
        (accumulate != 0 && accumulate != 1))
        return SARBP_EINVAL;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SARBP_EDEVICE;
    if (cur != s->device) return SARBP_EINVAL;
    const hipStream_t work = static_cast<hipStream_t>(stream);
    const char* host = static_cast<const char*>(data_h);
    const size_t row_bytes = s->row * sizeof(float2);

    for (int64_t n0 = 0, c = 0; n0 < n; n0 += s->chunk, ++c) {
        const int b = (int)(c & 1);
        const int np = (int)((int64_t)n - n0 < s->chunk ? (int64_t)n - n0 : s->chunk);
        // The host waits until staging buffer b is free before queueing its next
        // fill, so it runs at most two chunks ahead of the device.  Unbounded
        // run-ahead queued hundreds of cross-stream waits, and the runtime then
        // stalled the calling thread for 10-40 ms at a time, long enough to leave
        // the device idle.  The device still orders the copy by the event below.
        if (hipEventSynchronize(s->released[b]) != hipSuccess) return SARBP_EDEVICE;
        // copy stream: wait until the kernels that last read buffer b have run, then fill it.
        // The pulses go first: the runtime moves large copies with the DMA engines, which
        // run beside the kernel of the previous chunk, but small ones (here the positions,
        // below ~16 KiB) with a copy kernel that must wait for free compute units; queued
        // first, it would hold the large copy back until that kernel had finished.
        if (hipStreamWaitEvent(s->copy, s->released[b], 0) != hipSuccess ||
            hipMemcpyAsync(s->data_d[b], host + (size_t)n0 * row_bytes, (size_t)np * row_bytes,
                           hipMemcpyHostToDevice, s->copy) != hipSuccess ||
            hipMemcpyAsync(s->pos_d[b], positions_h + 3 * n0, (size_t)np * 3 * sizeof(double),
                           hipMemcpyHostToDevice, s->copy) != hipSuccess ||
            hipEventRecord(s->copied[b], s->copy) != hipSuccess)
            return SARBP_EDEVICE;
        // compute stream: wait for the copy, (compress,) backproject, release buffer b
        if (hipStreamWaitEvent(work, s->copied[b], 0) != hipSuccess) return SARBP_EDEVICE;
        const float2* echo = s->data_d[b];
        if (s->compress) {
            // rc_d is shared by all chunks: a call on another stream waits for its last reader
            if (hipStreamWaitEvent(work, s->rc_free, 0) != hipSuccess) return SARBP_EDEVICE;
            const int st = sarbp_launch_rc(s->plan, s->data_d[b], s->rc_d, np, work);
            if (st != SARBP_OK) return st;
            echo = s->rc_d;
        }
        const int st = sarbp_launch_bp(s->plan, s->pos_d[b], echo, nullptr, static_cast<float2*>(image_d), np,
                                       (c == 0) ? accumulate : 1, work);
        if (st != SARBP_OK) return st;
        if (hipEventRecord(s->released[b], work) != hipSuccess) return SARBP_EDEVICE;
        if (s->compress && hipEventRecord(s->rc_free, work) != hipSuccess) return SARBP_EDEVICE;
    }
    return SARBP_OK;
}

extern "C" void sarbp_stream_destroy(sarbp_stream* s) { release(s); }
