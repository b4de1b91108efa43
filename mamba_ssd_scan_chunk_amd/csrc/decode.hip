// decode.hip -- fused single-token decode step on the O(1) cache (gfx950).
//
// One step of the recurrence of arXiv 2603.09555 (Santoni), in the form of
// the bqwf.cn article on its compiler-first implementation, §2.1-§2.2: roll
// the depthwise-conv input window by one token, then
//     state[p,n] <- exp(dt*A_h) * state[p,n] + dt * x[p] * B[n]
//     y[p]        = sum_n C[n] * state[p,n] + D_h * x[p].
//
// The step is bound by HBM bandwidth: the fp32 state (P*N*4 bytes per head)
// is read and written once, everything else is tiny.  A workgroup owns one
// (batch, head, block of PBLK state rows).  Each state row of N floats is
// covered by N/4 consecutive lanes with one float4 each, so a wavefront
// reads and writes 1 KiB contiguous per row pass; the readout sum over n is
// a butterfly over those N/4 lanes.  The convolution of the PBLK x-channels
// of the block and of the 2N B/C channels of its group is recomputed per
// workgroup (a few hundred FMAs) so that no second kernel or grid-wide sync
// is needed; the shifted windows go to a separate output buffer, written for
// the x-channels by their owner and for the B/C channels by the first
// block of the group's first head.
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 8;

template <int N>
struct DecodeShape {
    static constexpr int LPR = N / 4;                  // lanes per state row
    static constexpr int ROWS_PER_PASS = kThreads / LPR;
    static constexpr int PBLK = ROWS_PER_PASS >= 16 ? ROWS_PER_PASS : 16;
    static constexpr int RPT = PBLK / ROWS_PER_PASS;   // rows per thread
};

template <typename T, int N, bool CONV>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(DecodeArgs a) {
    using S = DecodeShape<N>;
    __shared__ float xs[S::PBLK];
    __shared__ float Bs[N];
    __shared__ float Cs[N];

    const int npb = (a.P + S::PBLK - 1) / S::PBLK;
    int bid = blockIdx.x;
    const int pb = bid % npb;
    bid /= npb;
    const int h = bid % a.H;
    const int b = bid / a.H;
    const int hpg = a.H / a.G;
    const int g = h / hpg;
    const int P = a.P;
    const int p0 = pb * S::PBLK;
    const int prows = min(S::PBLK, P - p0);
    const long HP = (long)a.H * P, GN = (long)a.G * N;
    const long xstride = a.in_stride ? a.in_stride : HP;
    const long bcstride = a.in_stride ? a.in_stride : GN;
    const T *xin = (const T *)a.x_t + b * xstride + (long)h * P + p0;
    const T *Bin = (const T *)a.B_t + b * bcstride + (long)g * N;
    const T *Cin = (const T *)a.C_t + b * bcstride + (long)g * N;

    // ---- stage this block's x, B, C (through the conv window if any)
    const int nch = prows + 2 * N;
    for (int i = threadIdx.x; i < nch; i += kThreads) {
        long cidx;
        float raw;
        float *dst;
        if (i < prows) {
            cidx = (long)h * P + p0 + i;
            raw = ld(xin + i);
            dst = &xs[i];
        } else if (i < prows + N) {
            const int n = i - prows;
            cidx = HP + (long)g * N + n;
            raw = ld(Bin + n);
            dst = &Bs[n];
        } else {
            const int n = i - prows - N;
            cidx = HP + GN + (long)g * N + n;
            raw = ld(Cin + n);
            dst = &Cs[n];
        }
        float v = raw;
        if (CONV) {
            const int K = a.K;
            const long C = HP + 2 * GN;
            const T *cin = (const T *)a.conv_in + ((long)b * C + cidx) * (K - 1);
            const T *w = (const T *)a.conv_w + cidx * K;
            float win[kMaxK];
#pragma unroll
            for (int k = 0; k < kMaxK; ++k)
                win[k] = (k < K - 1) ? ld(cin + k) : (k == K - 1 ? raw : 0.0f);
            float acc = a.conv_b ? ld((const T *)a.conv_b + cidx) : 0.0f;
#pragma unroll
            for (int k = 0; k < kMaxK; ++k)
                if (k < K) acc = fmaf(ld(w + k), win[k], acc);
            v = a.activation ? silu(acc) : acc;
            if (i < prows || ((h % hpg) == 0 && pb == 0)) {
                T *cout = (T *)a.conv_out + ((long)b * C + cidx) * (K - 1);
#pragma unroll
                for (int k = 0; k < kMaxK - 1; ++k)
                    if (k < K - 1) st(cout + k, win[k + 1]);
            }
        }
        *dst = v;
    }
    __syncthreads();

    // ---- state update and readout
    // The update is evaluated as h + (expm1(dt*A) * h + dt*x*B), rounding the
    // state once per step.  Two forms that look equivalent drift over long
    // runs when the decay is within a few ulp of 1: exp(dt*A) * h (the fp32
    // value of exp(dt*A) carries a fixed relative error, repeated every step)
    // and fma(expm1, h, h + dt*x*B) (the nearly constant decrement is rounded
    // against the fp32 grid the same way every step).  Here the only
    // state-sized rounding is of h plus a random increment.
    const float A = -expf(a.A_log[h]);
    const float dtv = a.dt_t[(long)b * a.H + h];
    const float dm1 = expm1f(dtv * A);
    const float Dh = a.D ? a.D[h] : 0.0f;
    const int lr = threadIdx.x % S::LPR;
    const int row0 = threadIdx.x / S::LPR;
    const int n0 = lr * 4;
    const float4 Bv = make_float4(Bs[n0], Bs[n0 + 1], Bs[n0 + 2], Bs[n0 + 3]);
    const float4 Cv = make_float4(Cs[n0], Cs[n0 + 1], Cs[n0 + 2], Cs[n0 + 3]);
    float *sbase = a.state + (((long)b * a.H + h) * P + p0) * N + n0;

    float4 hv[S::RPT];
#pragma unroll
    for (int r = 0; r < S::RPT; ++r) {
        const int pr = row0 + r * S::ROWS_PER_PASS;
        hv[r] = pr < prows ? *(const float4 *)(sbase + (long)pr * N) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    T *yout = (T *)a.y_t + ((long)b * a.H + h) * P + p0;
#pragma unroll
    for (int r = 0; r < S::RPT; ++r) {
        const int pr = row0 + r * S::ROWS_PER_PASS;
        const bool valid = pr < prows;
        const float xv = valid ? xs[pr] : 0.0f;
        const float coef = dtv * xv;
        float4 v = hv[r];
        v.x += fmaf(dm1, v.x, coef * Bv.x);
        v.y += fmaf(dm1, v.y, coef * Bv.y);
        v.z += fmaf(dm1, v.z, coef * Bv.z);
        v.w += fmaf(dm1, v.w, coef * Bv.w);
        float part = Cv.x * v.x;
        part = fmaf(Cv.y, v.y, part);
        part = fmaf(Cv.z, v.z, part);
        part = fmaf(Cv.w, v.w, part);
        part = group_sum<S::LPR>(part);
        if (valid) {
            *(float4 *)(sbase + (long)pr * N) = v;
            if (lr == 0) st(yout + pr, fmaf(Dh, xv, part));
        }
    }
}

template <typename T, int N>
hipError_t launch_n(const DecodeArgs &a, hipStream_t s) {
    using S = DecodeShape<N>;
    const long npb = (a.P + S::PBLK - 1) / S::PBLK;
    const long blocks = (long)a.B * a.H * npb;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (a.conv_in)
        hipLaunchKernelGGL((decode_step_kernel<T, N, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((decode_step_kernel<T, N, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s) {
    switch (a.N) {
        case 16: return launch_n<T, 16>(a, s);
        case 32: return launch_n<T, 32>(a, s);
        case 64: return launch_n<T, 64>(a, s);
        case 128: return launch_n<T, 128>(a, s);
        case 256: return launch_n<T, 256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int dtype, hipStream_t s) {
    return dtype == DT_BF16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace ssd
