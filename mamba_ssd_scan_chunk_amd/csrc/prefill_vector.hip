// prefill_vector.hip -- chunked SSD prefill on the fp32 vector units.
//
// The chunked form of the scan (bqwf.cn article on the compiler-first Mamba-2
// implementation of arXiv 2603.09555, §1.1 and §1.2).  Per chunk c of Q
// tokens and head h, with a_l = dt_l * A_h and cs_l = sum_{j<=l} a_j:
//   S_c      = sum_s exp(cs_last - cs_s) dt_s x_s (outer) B_s     (chunk state)
//   h_c      = exp(cs_last) h_{c-1} + S_c                          (state pass)
//   y_l      = sum_{s<=l} (C_l . B_s) exp(cs_l - cs_s) dt_s x_s
//              + exp(cs_l) C_l . h_{c-1} + D x_l                    (output)
// Three kernels: chunk states, the state pass (prefill_state_pass.hip) and
// the output.  Used for fp32 activations and for any bf16 shape the MFMA
// path does not cover.  All arithmetic is fp32 except the in-chunk cumsum,
// which is kept in fp64 so that differences cs_l - cs_s stay exact to fp32
// rounding even when |cs| reaches a few hundred.
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kTpt = 4;                    // chunk tokens per thread in the chunk-state kernel
constexpr int kMaxQ = kThreads * kTpt;     // largest chunk this path takes
static_assert(kMaxQ == kPrefillMaxQ, "chunk limit of the vector path");

__device__ __forceinline__ double wave_inclusive_sum_f64(double v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        double o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

// Grid (nchunks, H, B).  Writes the in-chunk cumsum, the chunk decay and S_c.
// A thread owns kTpt consecutive tokens of the chunk (Q <= kThreads * kTpt):
// it sums them in order, a block scan of the thread totals gives each
// thread's offset.
template <typename T>
__global__ __launch_bounds__(kThreads) void chunk_state_vec(PrefillArgs a) {
    __shared__ double wsum[kThreads / 64];
    __shared__ float wgt[kMaxQ];
    __shared__ double cs_last_sh;
    const int h = blockIdx.y;
    const long f = (long)blockIdx.z * a.nchunks + blockIdx.x;
    const ChunkEntry ch = chunk_at(a, f);
    const int Qc = ch.Qc;
    if (Qc <= 0) return;  // unused slot of a packed prefill
    const long tok0 = ch.tok0;
    const int g = h / (a.H / a.G);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const double A = -exp((double)a.A_log[h]);
    const float Af = (float)A;
    const int tpt = (Qc + kThreads - 1) / kThreads;  // tokens per thread, 1 .. kTpt

    float dtv[kTpt];
    double loc[kTpt];
    double run = 0.0;
#pragma unroll
    for (int k = 0; k < kTpt; ++k) {
        const int t = tid * tpt + k;
        dtv[k] = 0.0f;
        if (k < tpt && t < Qc) {
            dtv[k] = dt_value(a.dt[(tok0 + t) * a.H + h], a.dtp.dt_raw, a.dtp.dt_bias, h,
                              a.dtp.dt_min, a.dtp.dt_max);
            run += (double)(dtv[k] * Af);
        }
        loc[k] = run;
    }
    double inc = wave_inclusive_sum_f64(run);
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    double base = inc - run;  // exclusive offset of this thread
    for (int w = 0; w < wid; ++w) base += wsum[w];
    const long hc = f * a.H + h;
#pragma unroll
    for (int k = 0; k < kTpt; ++k) {
        const int t = tid * tpt + k;
        if (k < tpt && t == Qc - 1) cs_last_sh = base + loc[k];
    }
    __syncthreads();
    const double cs_last = cs_last_sh;
#pragma unroll
    for (int k = 0; k < kTpt; ++k) {
        const int t = tid * tpt + k;
        if (k < tpt && t < Qc) {
            const double cs = base + loc[k];
            wgt[t] = expf((float)(cs_last - cs)) * dtv[k];
            a.ws_cs[hc * a.Q + t] = cs;
        }
    }
    if (tid == 0) a.ws_dec[hc] = expm1f((float)cs_last);
    __syncthreads();

    const int P = a.P, N = a.N;
    const long HP = (long)a.H * P, GN = (long)a.G * N;
    const T *xp = (const T *)a.x + (tok0 * a.H + h) * P;
    const T *Bp = (const T *)a.Bm + (tok0 * a.G + g) * N;
    float *Sp = a.ws_S + hc * P * N;
    for (int o = tid; o < P * N; o += kThreads) {
        const int p = o / N, n = o - (o / N) * N;
        float acc = 0.0f;
        for (int s = 0; s < Qc; ++s)
            acc = fmaf(wgt[s] * ld(xp + s * HP + p), ld(Bp + s * GN + n), acc);
        Sp[o] = acc;
    }
}

constexpr int LT = 16;   // output rows per workgroup
constexpr int ST = 16;   // source tokens per step
constexpr int MAXD = 256;

// Grid (nchunks * ceil(Q/LT), H, B).  Reads the carried-in state h_{c-1}
// that the state pass left in ws_S.
template <typename T>
__global__ __launch_bounds__(kThreads) void chunk_out_vec(PrefillArgs a) {
    __shared__ float Cl[LT][MAXD + 1];
    __shared__ float Bs[ST][MAXD + 1];
    __shared__ float Xs[ST][MAXD + 1];
    __shared__ float Gt[LT][ST + 1];
    __shared__ double csl[LT], css[ST];
    __shared__ float dts[ST];

    const int nlt = (a.Q + LT - 1) / LT;
    const int c = blockIdx.x / nlt, lt = blockIdx.x - (blockIdx.x / nlt) * nlt;
    const int h = blockIdx.y;
    const long f = (long)blockIdx.z * a.nchunks + c;
    const ChunkEntry ch = chunk_at(a, f);
    const int Qc = ch.Qc;
    const long tok0 = ch.tok0;
    const int l0 = lt * LT;
    if (l0 >= Qc) return;
    const int lrows = min(LT, Qc - l0);
    const int g = h / (a.H / a.G);
    const int P = a.P, N = a.N;
    const long HP = (long)a.H * P, GN = (long)a.G * N;
    const int tid = threadIdx.x;
    const long hc = f * a.H + h;
    const double *cs = a.ws_cs + hc * a.Q;
    const T *xp = (const T *)a.x + (tok0 * a.H + h) * P;
    const T *Bp = (const T *)a.Bm + (tok0 * a.G + g) * N;
    const T *Cp = (const T *)a.Cm + (tok0 * a.G + g) * N;

    for (int i = tid; i < LT * N; i += kThreads) {
        const int r = i / N, n = i - (i / N) * N;
        Cl[r][n] = r < lrows ? ld(Cp + (l0 + r) * GN + n) : 0.0f;
    }
    if (tid < LT) csl[tid] = tid < lrows ? cs[l0 + tid] : 0.0;

    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.0f;

    const int send = l0 + lrows;  // sources s < send
    for (int s0 = 0; s0 < send; s0 += ST) {
        const int srows = min(ST, send - s0);
        __syncthreads();
        for (int i = tid; i < ST * N; i += kThreads) {
            const int r = i / N, n = i - (i / N) * N;
            Bs[r][n] = r < srows ? ld(Bp + (s0 + r) * GN + n) : 0.0f;
        }
        for (int i = tid; i < ST * P; i += kThreads) {
            const int r = i / P, p = i - (i / P) * P;
            Xs[r][p] = r < srows ? ld(xp + (s0 + r) * HP + p) : 0.0f;
        }
        if (tid < ST) {
            css[tid] = tid < srows ? cs[s0 + tid] : 0.0;
            dts[tid] = tid < srows ? dt_value(a.dt[(tok0 + s0 + tid) * a.H + h], a.dtp.dt_raw,
                                              a.dtp.dt_bias, h, a.dtp.dt_min, a.dtp.dt_max)
                                   : 0.0f;
        }
        __syncthreads();
        {
            const int i = tid / ST, j = tid - (tid / ST) * ST;
            float gv = 0.0f;
            if (i < lrows && j < srows && l0 + i >= s0 + j) {
                float d = 0.0f;
                for (int n = 0; n < N; ++n) d = fmaf(Cl[i][n], Bs[j][n], d);
                gv = d * expf((float)(csl[i] - css[j])) * dts[j];
            }
            Gt[i][j] = gv;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int o = tid + k * kThreads;
            if (o < LT * P) {
                const int i = o / P, p = o - (o / P) * P;
                float sacc = acc[k];
                for (int j = 0; j < srows; ++j) sacc = fmaf(Gt[i][j], Xs[j][p], sacc);
                acc[k] = sacc;
            }
        }
    }

    const float *hin = a.ws_S + hc * P * N;
    const float Dh = a.D ? a.D[h] : 0.0f;
    T *yp = (T *)a.y + (tok0 * a.H + h) * P;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int o = tid + k * kThreads;
        if (o < LT * P) {
            const int i = o / P, p = o - (o / P) * P;
            if (i < lrows) {
                float off = 0.0f;
                const float *hr = hin + (long)p * N;
                for (int n = 0; n < N; ++n) off = fmaf(Cl[i][n], hr[n], off);
                const float xv = ld(xp + (l0 + i) * HP + p);
                const float yv = acc[k] + expf((float)csl[i]) * off + Dh * xv;
                st(yp + (l0 + i) * HP + p, yv);
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill_vector(const PrefillArgs &a, int dtype, hipStream_t s) {
    const int gridB = a.chunks ? 1 : a.B;  // packed sequences: nchunks slots in all
    if (gridB > 65535 || a.H > 65535) return hipErrorInvalidConfiguration;
    stage_begin();
    dim3 g1(a.nchunks, a.H, gridB);
    hipError_t e = dtype == DT_BF16
                       ? launch_stage("chunk_state_vec", chunk_state_vec<bf16_t>, g1, dim3(kThreads), 0, s, a)
                       : launch_stage("chunk_state_vec", chunk_state_vec<float>, g1, dim3(kThreads), 0, s, a);
    if (e != hipSuccess) return e;
    e = launch_state_pass(a, s);
    if (e != hipSuccess) return e;
    const long nlt = (a.Q + LT - 1) / LT;
    dim3 g3((unsigned)(a.nchunks * nlt), a.H, gridB);
    return dtype == DT_BF16 ? launch_stage("chunk_out_vec", chunk_out_vec<bf16_t>, g3, dim3(kThreads), 0, s, a)
                            : launch_stage("chunk_out_vec", chunk_out_vec<float>, g3, dim3(kThreads), 0, s, a);
}

}  // namespace ssd
