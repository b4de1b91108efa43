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
// which makes the in-place update race free.  Two forms: one channel per
// thread (any C and alignment), and V channels per thread with 16-byte
// accesses (C % V == 0, 16-byte aligned tensors), the one the 2.7B shape uses.
// For sequences packed without padding the channel-group form takes its
// token blocks (sequence, block, first row, tokens) from a slot table built
// on the device (chunk_table.hip), each sequence starting from its own cache.
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kThreads = 256;  // one-channel form
constexpr int kVThreads = 64;  // channel-group form: one wave per workgroup (fewer idle lanes at the ragged end)
constexpr int kMaxK = 8;
constexpr int kTB = 16;  // tokens per thread, one-channel form (>= kMaxK - 1)
constexpr int kTBV = 8;  // tokens per thread, channel-group form
// a token block other than the first reads its window from the tokens before
// it, never from the cache that the first block rewrites
static_assert(kTB >= kMaxK - 1 && kTBV >= kMaxK - 1, "token blocks must cover a window");
static_assert(kTBV == kConvSlotTokens, "slot table of packed sequences");

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

// Vector form, for C a multiple of V = 16 / sizeof(T) and 16-byte aligned
// tensors (workgroups of one wave): a thread owns V consecutive channels, so every token load and
// output store is 16 bytes per lane (1 KiB per wave instruction) and the
// taps, bias and cache of its channels are a few 16-byte loads.  K is a
// template argument, so the window lives in registers.  The SiLU of the bf16
// output uses the hardware exp2 and reciprocal (relative error ~1e-7, far
// below the output's bf16 rounding); fp32 keeps expf and IEEE division.
template <typename T, int K>
__global__ __launch_bounds__(kVThreads) void conv_update_vec(ConvArgs a) {
    using VT = Vec16<T>;
    constexpr int V = VT::V;
    const long ngrp = a.C / V;
    // grid (channel blocks, token blocks, B), or (slots, channel blocks) for
    // packed sequences
    const long grp = (long)(a.blocks ? blockIdx.y : blockIdx.x) * kVThreads + threadIdx.x;
    if (grp >= ngrp) return;
    // sequence b, its token block tb (tokens t0 .. t1 - 1 of the sequence),
    // and the token row of the sequence's first token
    int b, tb, t1;
    long row0;
    if (a.blocks) {
        const ChunkEntry e = a.blocks[blockIdx.x];
        if (e.Qc <= 0) return;  // unused slot
        b = e.seq;
        tb = e.c;
        row0 = (long)e.tok0 - (long)e.c * kTBV;
        t1 = e.c * kTBV + e.Qc;
    } else {
        b = blockIdx.z;
        tb = blockIdx.y;
        row0 = (long)b * a.T;
        t1 = min(a.T, tb * kTBV + kTBV);
    }
    const long C = a.C, c0 = grp * V;
    const int t0 = tb * kTBV;
    // tap k of channel c0 + i is element i * K + k of the V*K taps of the group
    float w[V][K];
    {
        constexpr int NW = V * K * (int)sizeof(T) / 16;
        const uint4 *wp = (const uint4 *)((const T *)a.w + c0 * K);
        float f[NW][V];
#pragma unroll
        for (int j = 0; j < NW; ++j) VT::unpack(wp[j], f[j]);
#pragma unroll
        for (int e = 0; e < V * K; ++e) w[e / K][e % K] = f[e / V][e % V];
    }
    float bias[V];
    if (a.bias) {
        VT::unpack(*(const uint4 *)((const T *)a.bias + c0), bias);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) bias[i] = 0.0f;
    }
    T *stp = (T *)a.state + ((long)b * C + c0) * (K - 1);  // V channels x (K-1), contiguous
    const uint4 *xp = (const uint4 *)((const T *)a.xBC + row0 * C + c0);  // token t at xp[t * C / V]
    const long xs = C / V;
    // win[j][i]: input j of the K-1 before token t0, channel c0 + i; old:
    // the old cache (token block 0 only)
    float win[K][V], old[K - 1][V];
    // the group's cache is V * (K-1) elements = K-1 whole 16-byte words
    constexpr int NS = V * (K - 1) * (int)sizeof(T);
    static_assert(NS == 16 * (K - 1), "cache of a channel group is whole 16-byte words");
    if (tb == 0) {
        float f[K - 1][V];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) VT::unpack(((const uint4 *)stp)[j], f[j]);
        // element e: channel e / (K-1), slot e % (K-1)
#pragma unroll
        for (int e = 0; e < V * (K - 1); ++e) win[e % (K - 1)][e / (K - 1)] = f[e / V][e % V];
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
#pragma unroll
            for (int i = 0; i < V; ++i) old[j][i] = win[j][i];
    } else {
#pragma unroll
        for (int j = 0; j < K - 1; ++j) VT::unpack(xp[(long)(t0 + j - (K - 1)) * xs], win[j]);
    }
    // tokens of the block: all loads first
    uint4 raw[kTBV];
#pragma unroll
    for (int t = 0; t < kTBV; ++t) raw[t] = t0 + t < t1 ? xp[(long)(t0 + t) * xs] : make_uint4(0, 0, 0, 0);
    uint4 *op = a.out ? (uint4 *)((T *)a.out + row0 * C + c0) : nullptr;
#pragma unroll
    for (int t = 0; t < kTBV; ++t) {
        if (t0 + t >= t1) break;
        VT::unpack(raw[t], win[K - 1]);
        float o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float acc = bias[i];
#pragma unroll
            for (int k = 0; k < K; ++k) acc = fmaf(w[i][k], win[k][i], acc);
            o[i] = a.activation ? VT::act(acc) : acc;
        }
        if (op) op[(long)(t0 + t) * xs] = VT::pack(o);
#pragma unroll
        for (int k = 0; k < K - 1; ++k)
#pragma unroll
            for (int i = 0; i < V; ++i) win[k][i] = win[k + 1][i];
    }
    if (tb == 0) {
        // new cache = hist[T .. T+K-2] with hist = (old cache, tokens): the
        // last K-1 tokens, preceded by the end of the old cache (read by this
        // thread into `old` before it is overwritten) when T < K-1
        const int T_ = a.blocks ? a.seqs[b].len : a.T;
        float nc[K - 1][V];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            const int hj = T_ + j;  // index into hist
            if (hj >= K - 1) {
                VT::unpack(xp[(long)(hj - (K - 1)) * xs], nc[j]);
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) nc[j][i] = old[hj][i];
            }
        }
        // back to [channel][K-1] order, 16 bytes at a time
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            float f[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int e = j * V + i;  // element e of the group's cache: channel e / (K-1), slot e % (K-1)
                f[i] = nc[e % (K - 1)][e / (K - 1)];
            }
            ((uint4 *)stp)[j] = VT::pack(f);
        }
    }
}

template <typename T>
hipError_t launch_vec(const ConvArgs &a, dim3 grid, hipStream_t s) {
    switch (a.K) {
        case 2: hipLaunchKernelGGL((conv_update_vec<T, 2>), grid, dim3(kVThreads), 0, s, a); break;
        case 3: hipLaunchKernelGGL((conv_update_vec<T, 3>), grid, dim3(kVThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL((conv_update_vec<T, 4>), grid, dim3(kVThreads), 0, s, a); break;
        case 5: hipLaunchKernelGGL((conv_update_vec<T, 5>), grid, dim3(kVThreads), 0, s, a); break;
        case 6: hipLaunchKernelGGL((conv_update_vec<T, 6>), grid, dim3(kVThreads), 0, s, a); break;
        case 7: hipLaunchKernelGGL((conv_update_vec<T, 7>), grid, dim3(kVThreads), 0, s, a); break;
        case 8: hipLaunchKernelGGL((conv_update_vec<T, 8>), grid, dim3(kVThreads), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

hipError_t launch_conv_update(const ConvArgs &a, int dtype, hipStream_t s) {
    if (a.T == 0 || a.B == 0) return hipSuccess;
    if (a.blocks) {
        // packed sequences: channel-group form only (checked by the caller)
        const long gblocks = (a.C / (dtype == DT_BF16 ? 8 : 4) + kVThreads - 1) / kVThreads;
        if (gblocks > 65535) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)a.nslots, (unsigned)gblocks, 1);
        return dtype == DT_BF16 ? launch_vec<bf16_t>(a, grid, s) : launch_vec<float>(a, grid, s);
    }
    if (a.B > 65535) return hipErrorInvalidConfiguration;
    const int V = dtype == DT_BF16 ? 8 : 4;
    const long vblocks = (a.T + kTBV - 1) / kTBV;
    if (a.C % V == 0 && vblocks <= 65535 && aligned16(a.state) && aligned16(a.xBC) && aligned16(a.w) &&
        aligned16(a.bias) && aligned16(a.out)) {
        const long tblocks = vblocks;
        const long ngrp = a.C / V;
        const long gblocks = (ngrp + kVThreads - 1) / kVThreads;
        if (gblocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)gblocks, (unsigned)tblocks, a.B);
        return dtype == DT_BF16 ? launch_vec<bf16_t>(a, grid, s) : launch_vec<float>(a, grid, s);
    }
    const long tblocks = (a.T + kTB - 1) / kTB;
    if (tblocks > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((a.C + kThreads - 1) / kThreads, (unsigned)tblocks, a.B);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(conv_update_kernel<bf16_t>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(conv_update_kernel<float>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ssd
