// Range compression for gfx950: one workgroup per pulse, the whole record
// resident in LDS.  Computes
//   y = IFFT( FFT(x) * H ),  H = conj(FFT(ref)) * W / N,
// the FFT matched filter with a Hamming window of the page
// "基于GPU的SAR后向投影成像优化与CUDA加速实践" (GPU-based SAR backprojection),
// section 3.1: pulses are independent, so the batch is one launch with one
// workgroup per pulse.
//
// Both transforms are radix-8 Stockham passes (radix 4 or 2 for the remaining
// factor) over a single LDS buffer: each pass loads its butterfly inputs into
// registers, synchronises, and stores the outputs in autosorted order.  The
// first pass reads the raw record straight from global memory, the matched
// filter multiply is fused into the first pass of the inverse transform
// (computed as conj(FFT(conj(X H)))), and the last pass writes the conjugated
// result straight to global memory, so the record crosses HBM once each way.
#include "sarbp_internal.h"

#pragma clang fp contract(off)

namespace {

constexpr int RC_THREADS = 256;
constexpr int RC_MAX_N = 16384;

struct RcArgs {
    const float2* raw;
    float2* out;
    const float2* filt; // H[m], 1/N included
    const float2* tw;   // exp(-2 pi i t / N)
    int log2n;
};

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
// multiply by -i
__device__ __forceinline__ float2 cmul_mi(float2 a) { return make_float2(a.y, -a.x); }

// Forward DFT of R points in natural order (exp(-2 pi i n k / R)).
template <int R>
__device__ __forceinline__ void dft(float2* v) {
    if constexpr (R == 2) {
        const float2 t = csub(v[0], v[1]);
        v[0] = cadd(v[0], v[1]);
        v[1] = t;
    } else if constexpr (R == 4) {
        const float2 a0 = cadd(v[0], v[2]), a1 = csub(v[0], v[2]);
        const float2 b0 = cadd(v[1], v[3]), b1 = cmul_mi(csub(v[1], v[3]));
        v[0] = cadd(a0, b0);
        v[2] = csub(a0, b0);
        v[1] = cadd(a1, b1);
        v[3] = csub(a1, b1);
    } else {
        // split into even outputs (DFT4 of x_n + x_{n+4}) and odd outputs
        // (DFT4 of (x_n - x_{n+4}) W8^n), W8 = exp(-2 pi i / 8)
        constexpr float h = 0.70710678118654752f;
        float2 a[4], b[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            a[n] = cadd(v[n], v[n + 4]);
            b[n] = csub(v[n], v[n + 4]);
        }
        b[1] = make_float2(h * (b[1].x + b[1].y), h * (b[1].y - b[1].x));
        b[2] = cmul_mi(b[2]);
        b[3] = make_float2(h * (b[3].y - b[3].x), -h * (b[3].x + b[3].y));
        dft<4>(a);
        dft<4>(b);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = a[k];
            v[2 * k + 1] = b[k];
        }
    }
}

enum Src { SRC_LDS = 0, SRC_RAW = 1, SRC_LDS_FILTER = 2 };
enum Dst { DST_LDS = 0, DST_OUT_CONJ = 1 };

// One Stockham pass of radix R over N points with current sub-transform length
// Ns: butterfly j reads x[j + r N/R], twiddles input r by exp(-2 pi i k r/(Ns R))
// (k = j mod Ns) and writes output r to (j / Ns) Ns R + k + r Ns.
template <int R, int SRC, int DST>
__device__ __forceinline__ void pass(const RcArgs& A, float2* buf, const float2* rin, float2* rout, int N, int Ns) {
    constexpr int BMAX = RC_MAX_N / (R * RC_THREADS);
    const int nb = N / R;
    const int stride = N / R;
    float2 v[BMAX][R];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
        const int j = threadIdx.x + b * RC_THREADS;
        if (j < nb) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int idx = j + r * stride;
                float2 x;
                if constexpr (SRC == SRC_RAW) {
                    x = rin[idx];
                } else if constexpr (SRC == SRC_LDS_FILTER) {
                    x = cconj(cmul(buf[idx], A.filt[idx]));
                } else {
                    x = buf[idx];
                }
                v[b][r] = x;
            }
        }
    }
    __syncthreads();
    const int twstep = N / (Ns * R);
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
        const int j = threadIdx.x + b * RC_THREADS;
        if (j < nb) {
            const int k = j & (Ns - 1);
#pragma unroll
            for (int r = 1; r < R; ++r) v[b][r] = cmul(v[b][r], A.tw[k * r * twstep]);
            dft<R>(v[b]);
            const int base = (j / Ns) * Ns * R + k;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if constexpr (DST == DST_OUT_CONJ) {
                    rout[base + r * Ns] = cconj(v[b][r]);
                } else {
                    buf[base + r * Ns] = v[b][r];
                }
            }
        }
    }
    __syncthreads();
}

// One full transform: radix-8 passes, then a radix-4 or radix-2 pass for the
// remaining factor.  The first pass reads SRC0, the last writes DST_LAST.
template <int SRC0, int DST_LAST>
__device__ void fft(const RcArgs& A, float2* buf, const float2* rin, float2* rout) {
    const int N = 1 << A.log2n;
    int rem = A.log2n, Ns = 1;
    bool first = true;
    while (rem > 0) {
        const int lr = rem >= 3 ? 3 : rem;
        const bool last = (rem == lr);
#define RC_PASS(R)                                                                  \
    if (first && last) pass<R, SRC0, DST_LAST>(A, buf, rin, rout, N, Ns);          \
    else if (first) pass<R, SRC0, DST_LDS>(A, buf, rin, rout, N, Ns);              \
    else if (last) pass<R, SRC_LDS, DST_LAST>(A, buf, rin, rout, N, Ns);           \
    else pass<R, SRC_LDS, DST_LDS>(A, buf, rin, rout, N, Ns);
        if (lr == 3) {
            RC_PASS(8)
        } else if (lr == 2) {
            RC_PASS(4)
        } else {
            RC_PASS(2)
        }
#undef RC_PASS
        Ns <<= lr;
        rem -= lr;
        first = false;
    }
}

__global__ __launch_bounds__(RC_THREADS) void rc_kernel(RcArgs A) {
    extern __shared__ __align__(16) float2 rc_buf[];
    const size_t N = (size_t)1 << A.log2n;
    const float2* rin = A.raw + (size_t)blockIdx.x * N;
    float2* rout = A.out + (size_t)blockIdx.x * N;
    fft<SRC_RAW, DST_LDS>(A, rc_buf, rin, rout);        // X = FFT(x)       -> LDS
    fft<SRC_LDS_FILTER, DST_OUT_CONJ>(A, rc_buf, rin, rout); // y = conj(FFT(conj(X H)))
}

} // namespace

int sarbp_rc_prepare_device() {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(rc_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               RC_MAX_N * (int)sizeof(float2)) == hipSuccess
               ? SARBP_OK
               : SARBP_EDEVICE;
}

int sarbp_launch_rc(const sarbp_plan* plan, const float2* raw, float2* out, int n, hipStream_t stream) {
    RcArgs A;
    A.raw = raw;
    A.out = out;
    A.filt = plan->rc_filter;
    A.tw = plan->rc_twiddle;
    A.log2n = plan->rc_log2;
    const size_t lds = ((size_t)1 << plan->rc_log2) * sizeof(float2);
    hipLaunchKernelGGL(rc_kernel, dim3(n), dim3(RC_THREADS), lds, stream, A);
    return hipGetLastError() == hipSuccess ? SARBP_OK : SARBP_EDEVICE;
}
