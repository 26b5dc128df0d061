// Range compression for gfx950: one workgroup per pulse, the whole record
// resident in LDS.  Computes
//   y = IFFT( FFT(x) * H ),  H = conj(FFT(ref)) * W / N,
// the FFT matched filter with a Hamming or Taylor window W (built into the
// plan's table H) of the page
// "基于GPU的SAR后向投影成像优化与CUDA加速实践" (GPU-based SAR backprojection),
// section 3.1: pulses are independent, so the batch is one launch with one
// workgroup per pulse.
//
// Both transforms are Stockham autosort passes of radix 8 or 16 over a single
// LDS buffer, specialised at compile time for each record length N = 2^L
// (64 .. 16384) with N/16 lanes, so a lane holds exactly one radix-16 butterfly
// (or two radix-8 ones) in registers.  Twiddles exp(-2 pi i k r / (Ns R)) come
// from v_sin_f32 / v_cos_f32, whose inputs are in revolutions: the dyadic angle
// k r / (Ns R) is exact in fp32, so no table is read.  The first pass reads the
// raw record straight from global memory, and the last pass writes the
// conjugated result straight to global memory, so the record crosses HBM once
// each way.  The inverse (computed as conj(FFT(conj(X H)))) runs the forward's
// radices in reverse order, so its first butterfly takes the points the forward's
// last butterfly produced: those two passes and the matched-filter multiply run
// as one, in registers (fused_pass).
//
// LDS layout: a pass with Ns < 32 writes each lane's outputs Ns apart, so the
// lanes of a wave would land on a few banks.  Its output buffer is padded by Ns
// entries after every group of Ns R (entry i is stored at i + Ns floor(i / (Ns R))):
// R + 1 is odd, so the lanes' groups then start on distinct banks, and both the
// writer's and the next reader's pad is one per-lane term plus compile-time
// constants.  The padded buffer holds N (1 + 1/8) entries.
#include "sarbp_internal.h"

#pragma clang fp contract(fast)

namespace {

struct RcArgs {
    const float2* raw;
    float2* out;
    const float2* filt; // H[m], 1/N included
    int n;              // records
};

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cmul_mi(float2 a) { return make_float2(a.y, -a.x); } // times -i

// In-register forward DFT of R points in natural order (exp(-2 pi i n k / R)).
template <int R>
__device__ __forceinline__ void dft(float2* v);

template <>
__device__ __forceinline__ void dft<4>(float2* v) {
    const float2 a0 = cadd(v[0], v[2]), a1 = csub(v[0], v[2]);
    const float2 b0 = cadd(v[1], v[3]), b1 = cmul_mi(csub(v[1], v[3]));
    v[0] = cadd(a0, b0);
    v[2] = csub(a0, b0);
    v[1] = cadd(a1, b1);
    v[3] = csub(a1, b1);
}

template <>
__device__ __forceinline__ void dft<8>(float2* v) {
    // even outputs: DFT4 of x_n + x_{n+4}; odd outputs: DFT4 of (x_n - x_{n+4}) W8^n
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

template <>
__device__ __forceinline__ void dft<16>(float2* v) {
    // n = 4 n1 + n2, k = k1 + 4 k2:  X[k] = sum_n2 W4^{n2 k2} W16^{n2 k1} sum_n1 x[4 n1 + n2] W4^{n1 k1}
    constexpr float c1 = 0.92387953251128674f, s1 = 0.38268343236508978f, h = 0.70710678118654752f;
    float2 y[4][4]; // y[n2][k1]
#pragma unroll
    for (int n2 = 0; n2 < 4; ++n2) {
        float2 t[4] = {v[n2], v[4 + n2], v[8 + n2], v[12 + n2]};
        dft<4>(t);
#pragma unroll
        for (int k1 = 0; k1 < 4; ++k1) y[n2][k1] = t[k1];
    }
    // twiddles W16^{n2 k1}, W16 = exp(-2 pi i / 16)
    y[1][1] = cmul(y[1][1], make_float2(c1, -s1));
    y[1][2] = cmul(y[1][2], make_float2(h, -h));
    y[1][3] = cmul(y[1][3], make_float2(s1, -c1));
    y[2][1] = cmul(y[2][1], make_float2(h, -h));
    y[2][2] = cmul_mi(y[2][2]);
    y[2][3] = cmul(y[2][3], make_float2(-h, -h));
    y[3][1] = cmul(y[3][1], make_float2(s1, -c1));
    y[3][2] = cmul(y[3][2], make_float2(-h, -h));
    y[3][3] = cmul(y[3][3], make_float2(-c1, s1));
#pragma unroll
    for (int k1 = 0; k1 < 4; ++k1) {
        float2 t[4] = {y[0][k1], y[1][k1], y[2][k1], y[3][k1]};
        dft<4>(t);
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) v[k1 + 4 * k2] = t[k2];
    }
}

enum Src { SRC_LDS = 0, SRC_RAW = 1, SRC_REG = 2 };
enum Dst { DST_LDS = 0, DST_OUT_CONJ = 1 };

constexpr int rc_threads(int log2n) {
    return (1 << log2n) / 16 < 64 ? 64 : ((1 << log2n) / 16 > 1024 ? 1024 : (1 << log2n) / 16);
}

// Radix of pass `p` for a transform of 2^L points: passes of 16 and up to three
// of 8 so that every pass is radix 8 or 16.  The forward transform runs them in
// this order and the inverse in the reverse order (INV), so that the inverse's
// first butterfly j takes the very points j + r N/R the forward's last butterfly j
// produced (see fused_pass).
constexpr int rc_radix(int L, int p) {
    const int n8 = (L % 4 == 1) ? 3 : (L % 4 == 2 ? 2 : (L % 4 == 3 ? 1 : 0));
    return p < n8 ? 8 : 16;
}
constexpr int rc_passes(int L) {
    return (L % 4 == 1) ? 3 + (L - 9) / 4 : (L % 4 == 2 ? 2 + (L - 6) / 4 : (L % 4 == 3 ? 1 + (L - 3) / 4 : L / 4));
}
constexpr int rc_radix_dir(int L, bool inv, int p) { return inv ? rc_radix(L, rc_passes(L) - 1 - p) : rc_radix(L, p); }
// Ns of pass p: the product of the radices before it.
constexpr int rc_ns(int L, bool inv, int p) { return p == 0 ? 1 : rc_ns(L, inv, p - 1) * rc_radix_dir(L, inv, p - 1); }
// The pad unit of pass p's writes (passes with Ns < 32 pad their output, except a
// transform's last).
constexpr int rc_pad(int L, bool inv, int p) {
    return (p < rc_passes(L) - 1 && rc_ns(L, inv, p) < 32) ? rc_ns(L, inv, p) : 0;
}

// One Stockham pass: butterfly j reads x[j + r N/R], twiddles input r by
// exp(-2 pi i k r/(Ns R)) (k = j mod Ns) and writes output r to
// (j / Ns) Ns R + k + r Ns.  PADR is the pad unit of the previous pass's writes
// (0: unpadded), PADW this pass's (see the LDS layout above).
template <int L, int R, int NS, int SRC, int DST, int PADR, int PADW>
__device__ __forceinline__ void pass(float2* buf, const float2* rin, float2* rout, int tx, const float2* vreg = nullptr) {
    constexpr int N = 1 << L, T = rc_threads(L), NB = N / R, BPT = (NB + T - 1) / T;
    static_assert(NB % NS == 0, "group size divides the butterfly stride");
    float2 v[BPT][R];
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        const int j = tx + b * T;
        if (NB % T == 0 || j < NB) {
            // (j + r NB) / Ns = j / Ns + r NB / Ns: the previous writer's pad
            const int rpad = PADR ? PADR * (j / NS) : 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int idx = j + r * NB;
                const int phys = idx + rpad + PADR * (r * NB / NS);
                if constexpr (SRC == SRC_RAW) {
                    v[b][r] = rin[idx];
                } else if constexpr (SRC == SRC_REG) {
                    v[b][r] = vreg[b * R + r]; // the inputs, already loaded (load_record)
                } else {
                    v[b][r] = buf[phys];
                }
            }
        }
    }
    // every lane must have read its inputs before any output overwrites them
    if constexpr (SRC == SRC_LDS && DST == DST_LDS) __syncthreads();
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        const int j = tx + b * T;
        if (NB % T == 0 || j < NB) {
            const int k = j & (NS - 1);
            if constexpr (NS > 1) {
                const float step = (float)k * (1.0f / (float)(NS * R)); // revolutions per input index
#pragma unroll
                for (int r = 1; r < R; ++r) {
                    const float ang = step * (float)r; // exact: k r < 2^14, power-of-two divisor
                    v[b][r] = cmul(v[b][r], make_float2(__builtin_amdgcn_cosf(ang), -__builtin_amdgcn_sinf(ang)));
                }
            }
            dft<R>(v[b]);
            // (base + r Ns) / (Ns R) = j / Ns: this pass's pad
            const int base = (j / NS) * NS * R + k + (PADW ? PADW * (j / NS) : 0);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if constexpr (DST == DST_OUT_CONJ) {
                    rout[base + r * NS] = cconj(v[b][r]);
                } else {
                    buf[base + r * NS] = v[b][r];
                }
            }
        }
    }
    if constexpr (DST == DST_LDS) __syncthreads();
}

// Passes P .. PEND - 1 of one transform (forward, or inverse with INV); the first
// of them reads from SRC0 (or LDS), the transform's last writes to DST_LAST.
template <int L, bool INV, int P, int PEND, int SRC0, int DST_LAST>
__device__ __forceinline__ void fft_range(const RcArgs& A, float2* buf, const float2* rin, float2* rout, int tx) {
    if constexpr (P < PEND) {
        constexpr int R = rc_radix_dir(L, INV, P), NS = rc_ns(L, INV, P);
        constexpr bool last = (P == rc_passes(L) - 1);
        pass<L, R, NS, P == 0 ? SRC0 : SRC_LDS, last ? DST_LAST : DST_LDS, P == 0 ? 0 : rc_pad(L, INV, P - 1),
             rc_pad(L, INV, P)>(buf, rin, rout, tx);
        fft_range<L, INV, P + 1, PEND, SRC0, DST_LAST>(A, buf, rin, rout, tx);
    }
}

// The forward transform's last pass, the matched-filter multiply and the inverse
// transform's first pass in one: forward butterfly j (radix R, Ns = N/R) reads
// LDS, twiddles and transforms its R points, whose outputs are X[j + r N/R]; each
// is multiplied by H and conjugated (the inverse is computed as conj(FFT(conj(.))));
// the inverse's first pass (radix R, Ns = 1, no twiddles) transforms the same R
// values and writes them, padded, for its next pass.  One LDS round trip and its
// barriers fewer than running the two passes apart.
template <int L>
__device__ __forceinline__ void fused_pass(const RcArgs& A, float2* buf, int tx) {
    constexpr int PF = rc_passes(L) - 1; // the forward's last pass
    constexpr int N = 1 << L, R = rc_radix_dir(L, false, PF), NS = rc_ns(L, false, PF);
    constexpr int T = rc_threads(L), NB = N / R, BPT = (NB + T - 1) / T, PADR = PF == 0 ? 0 : rc_pad(L, false, PF - 1);
    constexpr int PADW = rc_pad(L, true, 0);
    static_assert(R == rc_radix_dir(L, true, 0) && NS == NB, "the two passes meet on the same points");
    float2 v[BPT][R];
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        const int j = tx + b * T;
        if (NB % T == 0 || j < NB) {
            const int rpad = PADR ? PADR * (j / NS) : 0;
#pragma unroll
            for (int r = 0; r < R; ++r) v[b][r] = buf[j + r * NB + rpad + PADR * (r * NB / NS)];
        }
    }
    __syncthreads(); // every lane has read its inputs before any output overwrites them
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        const int j = tx + b * T;
        if (NB % T == 0 || j < NB) {
            const float step = (float)j * (1.0f / (float)(NS * R)); // k = j (j < Ns)
#pragma unroll
            for (int r = 1; r < R; ++r) {
                const float ang = step * (float)r;
                v[b][r] = cmul(v[b][r], make_float2(__builtin_amdgcn_cosf(ang), -__builtin_amdgcn_sinf(ang)));
            }
            dft<R>(v[b]);
#pragma unroll
            for (int r = 0; r < R; ++r) v[b][r] = cconj(cmul(v[b][r], A.filt[j + r * NS]));
            dft<R>(v[b]);
            const int base = j * R + (PADW ? PADW * j : 0);
#pragma unroll
            for (int r = 0; r < R; ++r) buf[base + r] = v[b][r];
        }
    }
    __syncthreads();
}

constexpr size_t rc_lds_bytes(int L) { return ((size_t)1 << L) / 8 * 9 * sizeof(float2); }

// The first pass's inputs of one record: butterfly j's points j + r N/R.
template <int L>
__device__ __forceinline__ void load_record(const float2* rin, float2* v, int tx) {
    constexpr int N = 1 << L, R = rc_radix_dir(L, false, 0), T = rc_threads(L), NB = N / R, BPT = (NB + T - 1) / T;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        const int j = tx + b * T;
        if (NB % T == 0 || j < NB) {
#pragma unroll
            for (int r = 0; r < R; ++r) v[b * R + r] = rin[j + r * NB];
        }
    }
}

// One record per workgroup (LOOP false), or (LOOP true) records blockIdx.x,
// blockIdx.x + gridDim.x, ..., each workgroup loading the next record's
// first-pass inputs into registers before it transforms the current one, so that
// record's HBM latency overlaps the LDS passes.  The launch takes the loop when a
// single record fills a CU's LDS: then nothing else on the CU hides its loads.
template <int L, bool LOOP>
__global__ __launch_bounds__(rc_threads(L)) void rc_kernel(RcArgs A) {
    extern __shared__ __align__(16) float2 rc_buf[];
    constexpr size_t N = (size_t)1 << L;
    constexpr int P = rc_passes(L);
    static_assert(P >= 2, "the fused pass joins two transforms of at least two passes");
    if constexpr (!LOOP) {
        const int tx = (int)threadIdx.x;
        const float2* rin = A.raw + (size_t)blockIdx.x * N;
        float2* rout = A.out + (size_t)blockIdx.x * N;
        fft_range<L, false, 0, P - 1, SRC_RAW, DST_LDS>(A, rc_buf, rin, rout, tx); // X = FFT(x), all but its last pass
        fused_pass<L>(A, rc_buf, tx);                                           // ... its last, * H, conj, inverse first
        fft_range<L, true, 1, P, SRC_LDS, DST_OUT_CONJ>(A, rc_buf, rin, rout, tx); // y = conj(FFT(conj(X H)))
    } else {
        constexpr int R0 = rc_radix_dir(L, false, 0), T = rc_threads(L), NB0 = (int)(N / R0),
                      BPT0 = (NB0 + T - 1) / T;
        float2 pre[BPT0 * R0];
        int rec = blockIdx.x;
        load_record<L>(A.raw + (size_t)rec * N, pre, (int)threadIdx.x);
        for (;;) {
            // the lane index, opaque to the compiler on each record, so that it does
            // not keep every pass's twiddles in registers across records
            int tx = (int)threadIdx.x;
            asm volatile("" : "+v"(tx));
            float2 v[BPT0 * R0];
#pragma unroll
            for (int i = 0; i < BPT0 * R0; ++i) v[i] = pre[i];
            const int next = rec + (int)gridDim.x;
            if (next < A.n) load_record<L>(A.raw + (size_t)next * N, pre, tx);
            float2* rout = A.out + (size_t)rec * N;
            pass<L, R0, 1, SRC_REG, DST_LDS, 0, rc_pad(L, false, 0)>(rc_buf, nullptr, rout, tx, v);
            fft_range<L, false, 1, P - 1, SRC_LDS, DST_LDS>(A, rc_buf, nullptr, rout, tx);
            fused_pass<L>(A, rc_buf, tx);
            fft_range<L, true, 1, P, SRC_LDS, DST_OUT_CONJ>(A, rc_buf, nullptr, rout, tx);
            if (next >= A.n) break;
            rec = next;
            __syncthreads(); // the last pass has read the LDS before the next record's first pass writes it
        }
    }
}

// Workgroups of the one-record kernel resident per CU (bound by LDS for the long
// records), looked up once.
template <int L>
int rc_per_cu() {
    static const int per_cu = [] {
        int b = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, rc_kernel<L, false>, rc_threads(L), rc_lds_bytes(L)) ==
                           hipSuccess &&
                       b > 0
                   ? b
                   : 1;
    }();
    return per_cu;
}

template <int L>
int launch(const RcArgs& A, int n, int n_cu, hipStream_t stream) {
    if (rc_per_cu<L>() == 1 && n_cu > 0 && n > n_cu)
        hipLaunchKernelGGL((rc_kernel<L, true>), dim3(n_cu), dim3(rc_threads(L)), rc_lds_bytes(L), stream, A);
    else
        hipLaunchKernelGGL((rc_kernel<L, false>), dim3(n), dim3(rc_threads(L)), rc_lds_bytes(L), stream, A);
    return hipGetLastError() == hipSuccess ? SARBP_OK : SARBP_EDEVICE;
}

template <int L>
int allow_lds() {
    const int bytes = (int)rc_lds_bytes(L);
    return hipFuncSetAttribute(reinterpret_cast<const void*>(rc_kernel<L, false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess &&
                   hipFuncSetAttribute(reinterpret_cast<const void*>(rc_kernel<L, true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess
               ? SARBP_OK
               : SARBP_EDEVICE;
}

} // namespace

int sarbp_rc_prepare_device() {
    // the 8192- and 16384-point records need more than the default 64 KiB of dynamic LDS
    const int st = allow_lds<13>();
    return st == SARBP_OK ? allow_lds<14>() : st;
}

int sarbp_launch_rc(const sarbp_plan* plan, const float2* raw, float2* out, int n, hipStream_t stream) {
    RcArgs A;
    A.raw = raw;
    A.out = out;
    A.filt = plan->rc_filter;
    A.n = n;
    const int cu = plan->L.n_cu;
    switch (plan->rc_log2) {
        case 6: return launch<6>(A, n, cu, stream);
        case 7: return launch<7>(A, n, cu, stream);
        case 8: return launch<8>(A, n, cu, stream);
        case 9: return launch<9>(A, n, cu, stream);
        case 10: return launch<10>(A, n, cu, stream);
        case 11: return launch<11>(A, n, cu, stream);
        case 12: return launch<12>(A, n, cu, stream);
        case 13: return launch<13>(A, n, cu, stream);
        case 14: return launch<14>(A, n, cu, stream);
        default: return SARBP_EINVAL;
    }
}
