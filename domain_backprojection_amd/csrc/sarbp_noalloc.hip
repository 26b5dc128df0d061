// The pulse-group backprojection (sarbp_backproject_split) without a caller
// workspace: its partial images live in a file-scope device array owned by the
// library, so the call allocates nothing.  It is meant for callers that cannot
// allocate device memory: code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc.
//
// The array is a static __device__ object: every GPU the library runs on holds
// its own copy of it from the time the code object loads there until the process
// ends.  In host code the name `scratch` is a host-side stand-in, not a device
// address; its device address on each GPU comes from hipGetSymbolAddress, taken
// once per device (with that device current) when the first plan is created there
// and cached per device.  Kernels receive that address as their workspace
// argument, exactly as sarbp_backproject_split passes a caller's workspace.
//
// Every call on one GPU shares that GPU's array and leaves its contents behind.
// The pulse-group kernels write every partial-image element before the partial sum
// reads it, so nothing needs clearing; but two calls that may run at the same time
// on one GPU (different streams, or different host threads) race on the array.
#include <mutex>

#include "sarbp_internal.h"

static __device__ __align__(256) char scratch[SARBP_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];
} // namespace

int sarbp_scratch_address(int device, void** out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return SARBP_EUNSUPPORTED;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_scratch[device] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SARBP_EDEVICE;
        g_scratch[device] = p;
    }
    *out = g_scratch[device];
    return SARBP_OK;
}

extern "C" int sarbp_backproject_split_noalloc(const sarbp_plan* plan, const double* positions_d, const void* echo_d,
                                               const float* dem_d, void* image_d, int32_t n, int32_t accumulate,
                                               void* stream) {
    int st = sarbp_split_check(plan, positions_d, echo_d, dem_d, image_d, n, accumulate);
    if (st != SARBP_OK) return st;
    const size_t need = sarbp_split_workspace_bytes(plan, n);
    if (need > (size_t)SARBP_STATIC_SCRATCH_BYTES) return SARBP_ESCRATCH;
    st = sarbp_check_device(plan);
    if (st != SARBP_OK) return st;
    if (need > 0 && plan->scratch == nullptr) return SARBP_EDEVICE;
    return sarbp_launch_bp(plan, positions_d, static_cast<const float2*>(echo_d), dem_d,
                           static_cast<float2*>(image_d), n, accumulate, static_cast<hipStream_t>(stream),
                           need > 0 ? static_cast<float2*>(plan->scratch) : nullptr,
                           need > 0 ? sarbp_split_count(plan, n) : 1);
}
