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
// (batch, group, block of PBLK consecutive state rows); the rows of a group
// are the flattened (head, p) pairs, contiguous in the state, x and y.  Each
// state row of N floats is covered by N/4 consecutive lanes with one float4
// each, so a wavefront reads and writes 1 KiB contiguous per row pass.
//
// Order of work in a workgroup:
//  1. the small operands are loaded: per-row step constants and the conv
//     operands (cached window, taps, bias, new input) of the PBLK x-channels
//     of the block and the 2N B/C channels of its group;
//  2. the state rows are loaded.  Vector-memory loads retire in issue
//     order, so step 3 waits only for the loads of step 1 while the state
//     is still on its way from HBM;
//  3. the convolution is finished and its results go to LDS (the B/C
//     channels are recomputed by every block of the group, a few hundred
//     FMAs, so that no second kernel or grid-wide sync is needed); the
//     shifted windows go to the separate output buffer, for the x-channels
//     by their owner and for the B/C channels by the group's first block;
//  4. each state row is updated and stored as soon as it arrives, and its
//     partial readout sum kept; the RPT partial sums of a lane are reduced
//     over the N/4 lanes of the row with a transposing butterfly (half of
//     the rows move at each lane bit while more than one row is left), so a
//     lane moves RPT - 1 + log2(N/4 / RPT) values instead of
//     RPT * log2(N/4).
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 8;

template <int N, int RPT>
struct DecodeShape {
    static constexpr int LPR = N / 4;                  // lanes per state row
    static constexpr int ROWS_PER_PASS = kThreads / LPR;
    static constexpr int PBLK = ROWS_PER_PASS * RPT;   // state rows per workgroup
    static constexpr int NCH = PBLK + 2 * N;           // conv channels per workgroup (at most)
    static constexpr int CH_ROUNDS = (NCH + kThreads - 1) / kThreads;
};

// ---- convolution of one channel, split into its loads and its arithmetic

// The loads of step 1 must not be waited for before the state loads are
// issued.  Any arithmetic on a loaded value placed above them (the compiler
// is free to: a bf16 widening, a half-word extraction from a merged load, a
// packing of two window values for one store) makes them wait.  So
//  - window elements are loaded and stored one by one (no_merge keeps the
//    compiler from fusing neighbours into one access that then needs
//    extraction or packing), as raw bits;
//  - after the state loads every loaded register passes through `settle`,
//    which the compiler must treat as producing it there, so all the
//    arithmetic comes after.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw bits of one element (bf16 zero-extended, fp32 as is) and their value.
template <typename T> __device__ __forceinline__ uint32_t ld_bits(const T *p);
template <> __device__ __forceinline__ uint32_t ld_bits<float>(const float *p) { return __float_as_uint(*p); }
template <> __device__ __forceinline__ uint32_t ld_bits<bf16_t>(const bf16_t *p) { return *p; }
// An empty statement that may touch memory: accesses are not merged across it.
__device__ __forceinline__ void no_merge() { asm volatile("" ::: "memory"); }
template <typename T> __device__ __forceinline__ float widen(uint32_t v);
template <> __device__ __forceinline__ float widen<float>(uint32_t v) { return __uint_as_float(v); }
template <> __device__ __forceinline__ float widen<bf16_t>(uint32_t v) { return __uint_as_float(v << 16); }
template <typename T> __device__ __forceinline__ void st_bits(T *p, uint32_t v);
template <> __device__ __forceinline__ void st_bits<float>(float *p, uint32_t v) { *p = __uint_as_float(v); }
template <> __device__ __forceinline__ void st_bits<bf16_t>(bf16_t *p, uint32_t v) { *p = (bf16_t)v; }

// Operands of one conv channel at this step, as loaded: the K-1 cached
// inputs and the new input (win[K-1]), the K taps and the bias.
template <int KM>
struct ConvIn {
    uint32_t win[KM];
    uint32_t w[KM];
    uint32_t bias;
};

// KT is the kernel width when fixed at compile time, 0 when it is taken from
// the arguments (up to kMaxK).  With KT = 4 the taps of a channel are one
// 8-byte (bf16) or 16-byte (fp32) load, in w[0..1] as bf16 pairs or in
// w[0..3]; the launcher takes this path only for taps aligned to that size.
// Loads are unconditional (the caller clamps the channel index): a load
// under a branch is waited for at the end of the branch.
template <typename T, bool CONV, int KT, int KM>
__device__ __forceinline__ void conv_load(const DecodeArgs &a, long C, int b, long cidx, const T *raw,
                                          ConvIn<KM> &in) {
    if (!CONV) {
        in.win[0] = ld_bits(raw);
        return;
    }
    const int K = KT ? KT : a.K;
    const T *cin = (const T *)a.conv_in + ((long)b * C + cidx) * (K - 1);
    const T *w = (const T *)a.conv_w + cidx * K;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        in.win[k] = (k < K - 1) ? ld_bits(cin + k) : (k == K - 1 ? ld_bits(raw) : 0u);
        no_merge();
    }
    if constexpr (KT == 4 && sizeof(T) == 2) {
        const u32x2 p = *(const u32x2 *)w;
        in.w[0] = p.x;
        in.w[1] = p.y;
    } else if constexpr (KT == 4) {
        const u32x4 p = *(const u32x4 *)w;
        in.w[0] = p.x; in.w[1] = p.y; in.w[2] = p.z; in.w[3] = p.w;
    } else {
#pragma unroll
        for (int k = 0; k < KM; ++k) in.w[k] = k < K ? ld_bits(w + k) : 0u;
    }
    // the bias is read from the taps when there is none, and not used
    in.bias = ld_bits(a.conv_b ? (const T *)a.conv_b + cidx : w);
}

// The registers of the first nwin window values and nw tap words become the
// outputs of an empty statement placed here.
template <int KM>
__device__ __forceinline__ void settle(ConvIn<KM> &in, int nwin, int nw) {
#pragma unroll
    for (int k = 0; k < KM; ++k)
        if (k < nwin) asm volatile("" : "+v"(in.win[k]));
#pragma unroll
    for (int k = 0; k < KM; ++k)
        if (k < nw) asm volatile("" : "+v"(in.w[k]));
    asm volatile("" : "+v"(in.bias));
}

// Convolved value of the channel; its shifted window goes to conv_out when
// `write_out`.
template <typename T, bool CONV, int KT, int KM>
__device__ __forceinline__ float conv_finish(const DecodeArgs &a, long C, int b, long cidx, const ConvIn<KM> &in,
                                             bool write_out) {
    if (!CONV) return widen<T>(in.win[0]);
    const int K = KT ? KT : a.K;
    float acc = a.conv_b ? widen<T>(in.bias) : 0.0f;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        float wk;
        if constexpr (KT == 4 && sizeof(T) == 2)
            wk = __uint_as_float((k & 1) ? (in.w[k / 2] & 0xffff0000u) : (in.w[k / 2] << 16));
        else
            wk = widen<T>(in.w[k]);
        if (k < K) acc = fmaf(wk, widen<T>(in.win[k]), acc);
    }
    if (write_out) {
        // the window moves by one token: raw bits, no rounding
        T *cout = (T *)a.conv_out + ((long)b * C + cidx) * (K - 1);
#pragma unroll
        for (int k = 0; k < KM - 1; ++k)
            if (k < K - 1) {
                st_bits(cout + k, in.win[k + 1]);
                no_merge();
            }
    }
    return a.activation ? silu(acc) : acc;
}

// ---- readout reduction

// The value that lane l receives from its partner across lane bit BIT, the
// partner being l ^ 1, l ^ 2 (quad permutations), l ^ 7, l ^ 15 (the
// half-row and row mirrors), l ^ 16, l ^ 32 (the permlane swaps).  The
// mirrors also flip the lower bits; the reduction below only needs a
// partner whose bit BIT differs and whose higher bits agree, and the masks
// 1, 2, 7, 15, 16, 32 are independent, so every lane of a group is summed
// exactly once.
template <int BIT>
__device__ __forceinline__ float lane_partner(float v, int lane) {
    const int u = __float_as_int(v);
    if constexpr (BIT == 0) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0xb1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
    } else if constexpr (BIT == 1) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0x4e, 0xf, 0xf, false));  // quad_perm 2,3,0,1
    } else if constexpr (BIT == 2) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0x141, 0xf, 0xf, false));  // row_half_mirror
    } else if constexpr (BIT == 3) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0x140, 0xf, 0xf, false));  // row_mirror
    } else if constexpr (BIT == 4) {
        // element 0: rows 0 and 2 in both rows of each pair; element 1: rows 1 and 3
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __int_as_float((lane & 16) ? r[0] : r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __int_as_float((lane & 32) ? r[0] : r[1]);
    }
}

// Sums v[j] (row pass j of this lane) over the lanes that share bits above
// BIT + 1 of the lane index, from lane bit BIT down to 0.  While M > 1 rows
// are live, each step keeps the half of them selected by the lane's bit and
// adds the partner's values of the same rows; `first` accumulates the first
// live row.  On return v[0..M_end) hold totals of rows first .. first+M_end-1.
template <int BIT, int M, int RPT>
__device__ __forceinline__ void reduce_rows(float (&v)[RPT], int &first, int lane) {
    if constexpr (BIT >= 0) {
        if constexpr (M > 1) {
            constexpr int HALF = M / 2;
            const bool upper = (lane >> BIT) & 1;
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                const float keep = upper ? v[j + HALF] : v[j];
                const float send = upper ? v[j] : v[j + HALF];
                v[j] = keep + lane_partner<BIT>(send, lane);
            }
            first += upper ? HALF : 0;
            reduce_rows<BIT - 1, HALF, RPT>(v, first, lane);
        } else {
            v[0] += lane_partner<BIT>(v[0], lane);
            reduce_rows<BIT - 1, 1, RPT>(v, first, lane);
        }
    }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

template <typename T, int N, bool CONV, int RPT, int KT>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(DecodeArgs a) {
    using S = DecodeShape<N, RPT>;
    static_assert(S::PBLK <= kThreads, "one thread per row of the block for the row constants");
    constexpr int KM = KT ? KT : kMaxK;
    __shared__ float2 rowc[S::PBLK];  // per row: dt * x, expm1(dt * A)
    __shared__ float rowdx[S::PBLK];  // per row: D * x
    __shared__ float Bs[N];
    __shared__ float Cs[N];

    const int P = a.P, H = a.H;
    const int hpg = H / a.G;
    const int GR = hpg * P;                      // state rows per (batch, group)
    const int npb = (GR + S::PBLK - 1) / S::PBLK;
    // 32-bit quotients (the grid is below 2^31 workgroups): a 64-bit one
    // costs the scalar unit about a hundred instructions before the first
    // state load can be addressed
    const int pb = (int)blockIdx.x % npb;
    const int bg = (int)blockIdx.x / npb;        // b * G + g
    const int g = bg % a.G;
    const int b = bg / a.G;
    const int r0 = pb * S::PBLK;                 // first row within the group
    const int prows = min(S::PBLK, GR - r0);
    const long HP = (long)H * P, GN = (long)a.G * N, C = HP + 2 * GN;
    const long xstride = a.in_stride ? a.in_stride : HP;
    const long bcstride = a.in_stride ? a.in_stride : GN;
    const long row_base = (long)b * HP + (long)g * GR + r0;  // row index in [B*H*P)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lr = tid % S::LPR;
    const int row0 = tid / S::LPR;
    const int n0 = lr * 4;

    // ---- 1. small operands
    // row constants: thread t for row t of the block (clamped)
    const int trow = min(tid, prows - 1);
    const int th = g * hpg + (r0 + trow) / P;
    const float t_dtv = a.dt_t[(long)b * H + th];  // raw value when dt is preprocessed here (below)
    const float t_bias = a.dtp.dt_bias ? a.dtp.dt_bias[th] : 0.0f;
    const float t_alog = a.A_log[th];
    const float t_Dv = a.D ? a.D[th] : 0.0f;
    // conv channels: the block's x rows, then B, then C; thread tid takes
    // channels tid + k * kThreads (clamped, the duplicates write nothing)
    const bool bc_writer = pb == 0;
    const long xch0 = (long)g * GR + r0;  // conv channel of the block's first row
    const T *xin = (const T *)a.x_t + b * xstride + xch0;
    const T *Bin = (const T *)a.B_t + b * bcstride + (long)g * N;
    const T *Cin = (const T *)a.C_t + b * bcstride + (long)g * N;
    const int nch = prows + 2 * N;
    ConvIn<KM> cin[S::CH_ROUNDS];
    long cidx[S::CH_ROUNDS];
#pragma unroll
    for (int k = 0; k < S::CH_ROUNDS; ++k) {
        const int i = min(tid + k * kThreads, nch - 1);
        const T *raw;
        if (i < prows) {
            cidx[k] = xch0 + i;
            raw = xin + i;
        } else if (i < prows + N) {
            cidx[k] = HP + (long)g * N + (i - prows);
            raw = Bin + (i - prows);
        } else {
            cidx[k] = HP + GN + (long)g * N + (i - prows - N);
            raw = Cin + (i - prows - N);
        }
        conv_load<T, CONV, KT, KM>(a, C, b, cidx[k], raw, cin[k]);
    }

    // ---- 2. state rows (clamped; rows past the block are not stored)
    float *sbase = a.state + row_base * N + n0;
    float4 hv[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int pr = min(row0 + r * S::ROWS_PER_PASS, prows - 1);
        hv[r] = *(const float4 *)(sbase + (long)pr * N);
    }
    // nothing may be scheduled above this point that uses a step-1 value
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kWinRegs = CONV ? KM : 1;
    constexpr int kTapRegs = !CONV ? 0 : (KT == 4 && sizeof(T) == 2) ? 2 : KM;
#pragma unroll
    for (int k = 0; k < S::CH_ROUNDS; ++k) settle(cin[k], kWinRegs, kTapRegs);
    float t_dtv_s = t_dtv, t_bias_s = t_bias, t_alog_s = t_alog, t_Dv_s = t_Dv;
    asm volatile("" : "+v"(t_dtv_s), "+v"(t_bias_s), "+v"(t_alog_s), "+v"(t_Dv_s));

    // ---- 3. convolution results and row constants to LDS
#pragma unroll
    for (int k = 0; k < S::CH_ROUNDS; ++k) {
        const int i = tid + k * kThreads;
        const bool valid = i < nch;
        const bool is_x = i < prows;
        const float v = conv_finish<T, CONV, KT, KM>(a, C, b, cidx[k], cin[k], valid && (is_x || bc_writer));
        if (k == 0 && is_x) {
            // thread t = row t: the channel just finished is x of row t
            const float t_dt =
                a.dtp.dt_raw ? dt_softplus_clamp(t_dtv_s + t_bias_s, a.dtp.dt_min, a.dtp.dt_max) : t_dtv_s;
            rowc[i] = make_float2(t_dt * v, expm1f(t_dt * -expf(t_alog_s)));
            rowdx[i] = t_Dv_s * v;
        } else if (valid && !is_x) {
            if (i < prows + N) Bs[i - prows] = v;
            else Cs[i - prows - N] = v;
        }
    }
    __syncthreads();

    // ---- 4. state update, stores and readout
    // The update is evaluated as h + (expm1(dt*A) * h + dt*x*B), rounding the
    // state once per step.  Two forms that look equivalent drift over long
    // runs when the decay is within a few ulp of 1: exp(dt*A) * h (the fp32
    // value of exp(dt*A) carries a fixed relative error, repeated every step)
    // and fma(expm1, h, h + dt*x*B) (the nearly constant decrement is rounded
    // against the fp32 grid the same way every step).  Here the only
    // state-sized rounding is of h plus a random increment.
    const float4 Bv = make_float4(Bs[n0], Bs[n0 + 1], Bs[n0 + 2], Bs[n0 + 3]);
    const float4 Cv = make_float4(Cs[n0], Cs[n0 + 1], Cs[n0 + 2], Cs[n0 + 3]);
    float part[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int pr = row0 + r * S::ROWS_PER_PASS;
        const float2 rc = rowc[min(pr, prows - 1)];
        const float coef = rc.x, dm1 = rc.y;
        float4 v = hv[r];
        v.x += fmaf(dm1, v.x, coef * Bv.x);
        v.y += fmaf(dm1, v.y, coef * Bv.y);
        v.z += fmaf(dm1, v.z, coef * Bv.z);
        v.w += fmaf(dm1, v.w, coef * Bv.w);
        float p = Cv.x * v.x;
        p = fmaf(Cv.y, v.y, p);
        p = fmaf(Cv.z, v.z, p);
        p = fmaf(Cv.w, v.w, p);
        part[r] = p;
        if (pr < prows) *(float4 *)(sbase + (long)pr * N) = v;
    }
    constexpr int LB = ilog2(S::LPR);
    constexpr int HALVINGS = ilog2(RPT) < LB ? ilog2(RPT) : LB;
    constexpr int M_END = RPT >> HALVINGS;
    int first = 0;
    reduce_rows<LB - 1, RPT, RPT>(part, first, lane);
    // lanes that differ only in the fully reduced low bits hold the same
    // totals; the one with those bits zero writes
    constexpr int LOW = LB - HALVINGS;
    if ((lr & ((1 << LOW) - 1)) == 0) {
        T *yout = (T *)a.y_t + row_base;
#pragma unroll
        for (int j = 0; j < M_END; ++j) {
            const int pr = row0 + (first + j) * S::ROWS_PER_PASS;
            if (pr < prows) st(yout + pr, part[j] + rowdx[pr]);
        }
    }
}

template <typename T, int N, int RPT>
hipError_t launch_nr(const DecodeArgs &a, hipStream_t s) {
    using S = DecodeShape<N, RPT>;
    const long GR = (long)(a.H / a.G) * a.P;
    const long npb = (GR + S::PBLK - 1) / S::PBLK;
    const long blocks = (long)a.B * a.G * npb;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    const bool taps_aligned = ((uintptr_t)a.conv_w & (4 * sizeof(T) - 1)) == 0;
    if (a.conv_in && a.K == 4 && taps_aligned)
        hipLaunchKernelGGL((decode_step_kernel<T, N, true, RPT, 4>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else if (a.conv_in)
        hipLaunchKernelGGL((decode_step_kernel<T, N, true, RPT, 0>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((decode_step_kernel<T, N, false, RPT, 0>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// Rows per workgroup, from the number of workgroups the largest blocks
// (4x the smallest) would make: the smallest blocks below 64 such
// workgroups (more workgroups in flight), twice the smallest below 128, the
// largest from there.  Measured per step in a HIP graph, conv on, P = 64,
// N = 128 (16-, 32- and 64-row blocks), at B = 1 .. 32 on the 2.7B-shaped
// (H = 80) and 130M-shaped (H = 24) layers: e.g. H = 80, B = 1 (80):
// 3.99 / 3.81 / 3.98 us; B = 8 (640): 9.53 / 7.90 / 7.53 us; H = 24, B = 2
// (48): 3.57 / 3.64 / 3.87 us; B = 4 (96): 4.33 / 3.84 / 4.06 us.
template <typename T, int N>
hipError_t launch_n(const DecodeArgs &a, hipStream_t s) {
    constexpr int base = DecodeShape<N, 1>::ROWS_PER_PASS >= 16 ? 1 : 16 / DecodeShape<N, 1>::ROWS_PER_PASS;
    const long big = (long)a.B * a.H * ((a.P + DecodeShape<N, 4 * base>::PBLK - 1) / DecodeShape<N, 4 * base>::PBLK);
    if (big >= 128) return launch_nr<T, N, 4 * base>(a, s);
    if (big >= 64) return launch_nr<T, N, 2 * base>(a, s);
    return launch_nr<T, N, base>(a, s);
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
