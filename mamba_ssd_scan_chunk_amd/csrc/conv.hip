// conv.hip -- depthwise causal convolution over T tokens with the
// (K-1)-token window cache (bqwf.cn article on the compiler-first Mamba-2
// implementation of arXiv 2603.09555, §2.1-§2.2: a fixed-size input cache per
// channel, rolled by one with the newest token written last).
//
// out[b,t,c] = act(bias[c] + sum_k w[c,k] * hist[t+k]),
// where hist = (cache[b,c,0..K-2], xBC[b,0..T-1,c]) and hist[t+K-1] is token t.
// The convolution has no recurrence, so tokens are split into blocks of TB
// that run in parallel; a thread keeps a K-wide sliding window in registers
// and reads each token once (consecutive threads = consecutive channels, so
// every load and store is coalesced).  Only the thread of token block 0 reads
// the old cache, and the same thread writes the new cache after that read,
// which makes the in-place update race free.
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 8;
constexpr int kTB = 16;  // tokens per thread (>= kMaxK - 1)

template <typename T>
__global__ __launch_bounds__(kThreads) void conv_update_kernel(ConvArgs a) {
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= a.C) return;
    const int tb = blockIdx.y;
    const int b = blockIdx.z;
    const int K = a.K, T_ = a.T;
    const long C = a.C;
    const int t0 = tb * kTB;
    const int t1 = min(T_, t0 + kTB);
    T *stp = (T *)a.state + ((long)b * C + c) * (K - 1);
    const T *xp = (const T *)a.xBC + (long)b * T_ * C + c;  // token t at xp[t * C]
    const T *wp = (const T *)a.w + (long)c * K;

    float w[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) w[k] = (k < K - 1) ? ld(wp + k) : 0.0f;
    const float wlast = ld(wp + K - 1);
    const float bias = a.bias ? ld((const T *)a.bias + c) : 0.0f;

    // window[0..K-2]: the K-1 inputs before token t0
    float win[kMaxK];
    if (tb == 0) {
#pragma unroll
        for (int j = 0; j < kMaxK - 1; ++j) win[j] = (j < K - 1) ? ld(stp + j) : 0.0f;
    } else {
#pragma unroll
        for (int j = 0; j < kMaxK - 1; ++j)
            win[j] = (j < K - 1) ? ld(xp + (long)(t0 + j - (K - 1)) * C) : 0.0f;
    }

    T *op = a.out ? (T *)a.out + (long)b * T_ * C + c : nullptr;
    for (int t = t0; t < t1; ++t) {
        const float u = ld(xp + (long)t * C);
        float acc = bias;
#pragma unroll
        for (int k = 0; k < kMaxK - 1; ++k)
            if (k < K - 1) acc = fmaf(w[k], win[k], acc);
        acc = fmaf(wlast, u, acc);
        if (op) st(op + (long)t * C, a.activation ? silu(acc) : acc);
#pragma unroll
        for (int k = 0; k < kMaxK - 1; ++k)
            win[k] = (k < K - 2) ? win[k + 1] : (k == K - 2 ? u : win[k]);
    }

    if (tb == 0) {
        // new cache = hist[T .. T+K-2]
        if (T_ >= K - 1) {
#pragma unroll
            for (int j = 0; j < kMaxK - 1; ++j)
                if (j < K - 1) st(stp + j, ld(xp + (long)(T_ - (K - 1) + j) * C));
        } else {
            // a single token block covered every token: win already is the new cache
#pragma unroll
            for (int j = 0; j < kMaxK - 1; ++j)
                if (j < K - 1) st(stp + j, win[j]);
        }
    }
}

}  // namespace

hipError_t launch_conv_update(const ConvArgs &a, int dtype, hipStream_t s) {
    if (a.T == 0 || a.B == 0) return hipSuccess;
    const long tblocks = (a.T + kTB - 1) / kTB;
    if (tblocks > 65535 || a.B > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((a.C + kThreads - 1) / kThreads, (unsigned)tblocks, a.B);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(conv_update_kernel<bf16_t>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(conv_update_kernel<float>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ssd
