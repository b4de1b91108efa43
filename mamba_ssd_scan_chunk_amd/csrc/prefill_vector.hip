// prefill_vector.hip -- chunked SSD prefill on the fp32 vector units.
//
// The chunked form of the scan (bqwf.cn article on the compiler-first Mamba-2
// implementation of arXiv 2603.09555, §1.1 and §1.2).  Per chunk c of Q
// tokens and head h, with a_l = dt_l * A_h and cs_l = sum_{j<=l} a_j:
//   S_c      = sum_s exp(cs_last - cs_s) dt_s x_s (outer) B_s     (chunk state)
//   h_c      = exp(cs_last) h_{c-1} + S_c                          (state pass)
//   y_l      = sum_{s<=l} (C_l . B_s) exp(cs_l - cs_s) dt_s x_s
//              + exp(cs_l) C_l . h_{c-1} + D x_l                    (output)
// Four kernels: chunk states, the masked C . B products (once per chunk and
// group, shared by the group's heads), the state pass
// (prefill_state_pass.hip) and the output.  Used for fp32 activations and
// for any bf16 shape the MFMA path does not cover (P, N <= 256, Q <= 1024).
// All arithmetic is fp32 except the in-chunk cumsum, which is kept in fp64
// so that differences cs_l - cs_s stay exact to fp32 rounding even when |cs|
// reaches a few hundred.  Chunks come from chunk_at, so packed sequences use
// the same kernels.
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kTpt = 4;                    // chunk tokens per thread in the chunk-state kernel
constexpr int kSP = 64, kSN = 128, kST = 16;  // chunk-state output pass (16 x 16 threads of 4 x 8) and token step
constexpr int kMaxQ = kThreads * kTpt;     // largest chunk this path takes
constexpr int CBT = 64, CBN = 32;  // C B^T kernel: 64 x 64 tiles, 32 columns of n per step
constexpr int LTO = 64;   // output rows per workgroup of the output kernel
constexpr int ST = 16;    // source tokens per step of the output kernel
constexpr int MAXD = 256;  // largest P and N
static_assert(kMaxQ == kPrefillMaxQ, "chunk limit of the vector path");
static_assert(CBT * CBT == 16 * kThreads, "C B^T kernel: 4 x 4 outputs per thread");
static_assert(LTO * 4 == kThreads && (LTO * ST) % kThreads == 0 && 4 * 64 == MAXD,
              "output kernel: 16 threads per four output rows, 64 features per pass");

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
    __shared__ __attribute__((aligned(16))) float xs[kST][kSP];
    __shared__ __attribute__((aligned(16))) float bs[kST][kSN];
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

    // S[p][n] = sum_s wgt_s x_s[p] B_s[n], in passes of kSP x kSN outputs:
    // thread (tp, tn) accumulates a 4 x 8 tile; kST tokens of x' = wgt x and
    // of B are staged in LDS per step.
    const int P = a.P, N = a.N;
    const long HP = (long)a.H * P, GN = (long)a.G * N;
    const T *xp = (const T *)a.x + (tok0 * a.H + h) * P;
    const T *Bp = (const T *)a.Bm + (tok0 * a.G + g) * N;
    float *Sp = a.ws_S + hc * P * N;
    const int tp = tid >> 4, tn = tid & 15;
    for (int p0 = 0; p0 < P; p0 += kSP) {
        for (int n0 = 0; n0 < N; n0 += kSN) {
            float acc[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
            for (int s0 = 0; s0 < Qc; s0 += kST) {
                __syncthreads();  // the previous step's tiles are consumed
                for (int i = tid; i < kST * kSP; i += kThreads) {
                    const int r = i / kSP, c = i - r * kSP, sx = s0 + r, px = p0 + c;
                    xs[r][c] = (sx < Qc && px < P) ? wgt[sx] * ld(xp + sx * HP + px) : 0.0f;
                }
                for (int i = tid; i < kST * kSN; i += kThreads) {
                    const int r = i / kSN, c = i - r * kSN, sx = s0 + r, nx = n0 + c;
                    bs[r][c] = (sx < Qc && nx < N) ? ld(Bp + sx * GN + nx) : 0.0f;
                }
                __syncthreads();
#pragma unroll
                for (int r = 0; r < kST; ++r) {
                    const float4 av = *(const float4 *)&xs[r][4 * tp];
                    const float4 b0 = *(const float4 *)&bs[r][8 * tn];
                    const float4 b1 = *(const float4 *)&bs[r][8 * tn + 4];
                    const float xa[4] = {av.x, av.y, av.z, av.w};
                    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xa[i], bb[j], acc[i][j]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pp = p0 + 4 * tp + i;
                if (pp >= P) continue;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int nn = n0 + 8 * tn + j;
                    if (nn < N) Sp[(long)pp * N + nn] = acc[i][j];
                }
            }
        }
    }
}

// Grid (nchunks * T(T+1)/2, G, B) with T = ceil(Q/CBT).  The causal masked
// product of the chunk, G[l][s] = C_l . B_s for s <= l (0 above the
// diagonal), once per (chunk, group) for every head of the group: one
// workgroup per CBT x CBT tile on or below the diagonal, each thread a
// 4 x 4 register tile.  C and B
// are staged transposed ([n][row]) CBN columns of n at a time, so a step of n
// is two 16-byte LDS reads for 16 FMAs.
template <typename T>
__global__ __launch_bounds__(kThreads) void chunk_cb_vec(PrefillArgs a) {
    // rows padded by 4 floats: the transposing stores spread over 8 banks,
    // the 16-byte reads stay aligned
    __shared__ __attribute__((aligned(16))) float Ct[CBN][CBT + 4];
    __shared__ __attribute__((aligned(16))) float Bt[CBN][CBT + 4];
    const int nlt = (a.Q + CBT - 1) / CBT, ntile = nlt * (nlt + 1) / 2;
    const int c = blockIdx.x / ntile, tix = blockIdx.x - (blockIdx.x / ntile) * ntile;
    int lt = 0;
    while ((lt + 1) * (lt + 2) / 2 <= tix) ++lt;
    const int st = tix - lt * (lt + 1) / 2;  // source tile, st <= lt
    const int g = blockIdx.y;
    const long f = (long)blockIdx.z * a.nchunks + c;
    const ChunkEntry ch = chunk_at(a, f);
    const int Qc = ch.Qc;
    const int l0 = lt * CBT;
    if (l0 >= Qc) return;
    const int N = a.N;
    const long GN = (long)a.G * N;
    const long tok0 = ch.tok0;
    const T *Bp = (const T *)a.Bm + (tok0 * a.G + g) * N;
    const T *Cp = (const T *)a.Cm + (tok0 * a.G + g) * N;
    float *Gp = a.ws_cb + (f * a.G + g) * a.Q * a.Q;
    const int tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;  // rows 4ti.., columns 4tj..
    {
        const int s0 = st * CBT;
        float acc[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[r][q] = 0.0f;
        for (int n0 = 0; n0 < N; n0 += CBN) {
            __syncthreads();  // the previous step is consumed
            for (int e = tid; e < CBN * CBT; e += kThreads) {  // element (row, nn), nn fastest for coalescing
                const int row = e / CBN, nn = e - (e / CBN) * CBN, n = n0 + nn;
                Ct[nn][row] = (l0 + row < Qc && n < N) ? ld(Cp + (l0 + row) * GN + n) : 0.0f;
                Bt[nn][row] = (s0 + row < Qc && n < N) ? ld(Bp + (s0 + row) * GN + n) : 0.0f;
            }
            __syncthreads();
#pragma unroll 8
            for (int nn = 0; nn < CBN; ++nn) {
                const float4 cv = *(const float4 *)&Ct[nn][4 * ti];
                const float4 bv = *(const float4 *)&Bt[nn][4 * tj];
                const float cr[4] = {cv.x, cv.y, cv.z, cv.w}, bq[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[r][q] = fmaf(cr[r], bq[q], acc[r][q]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int l = l0 + 4 * ti + r;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int sx = s0 + 4 * tj + q;
                if (l < Qc && sx < Qc && sx <= l0 + CBT - 1) Gp[(long)l * a.Q + sx] = sx <= l ? acc[r][q] : 0.0f;
            }
        }
    }
}

// Grid (nchunks * ceil(Q/LTO), H, B).  Reads the masked C B^T of the chunk
// and group (chunk_cb_vec) and the carried-in state h_{c-1} that the state
// pass left in ws_S.  A workgroup forms LTO output rows; thread (i, q) owns
// rows l0 + 4i .. 4i+3 and the features 4q + 64m .. +3 (m < MQ): per source
// token four LDS reads of G' and one 16-byte read of x per m feed 16 FMAs per m.
template <typename T, int MQ>
__global__ __launch_bounds__(kThreads) void chunk_out_vec(PrefillArgs a) {
    // x rows of a source step in the main loop, then h columns in the state
    // term: one LDS array for both
    __shared__ __attribute__((aligned(16))) float XHs[ST][MAXD];
    float (*Xs)[MAXD] = XHs;
    float (*Hs)[MAXD] = XHs;
    __shared__ float Gt[LTO][ST + 1];
    __shared__ float Cl[LTO][ST + 1];
    __shared__ double css[kMaxQ];  // cumsum of the chunk's sources s < l0 + LTO
    __shared__ float dts[kMaxQ];   // their steps

    const int nlt = (a.Q + LTO - 1) / LTO;
    const int c = blockIdx.x / nlt, lt = blockIdx.x - (blockIdx.x / nlt) * nlt;
    const int h = blockIdx.y;
    const long f = (long)blockIdx.z * a.nchunks + c;
    const ChunkEntry ch = chunk_at(a, f);
    const int Qc = ch.Qc;
    const long tok0 = ch.tok0;
    const int l0 = lt * LTO;
    if (l0 >= Qc) return;
    const int lrows = min(LTO, Qc - l0);
    const int g = h / (a.H / a.G);
    const int P = a.P, N = a.N;
    const long HP = (long)a.H * P, GN = (long)a.G * N;
    const int tid = threadIdx.x;
    const int oi = tid >> 4, oq = tid & 15;  // output row quad, feature quad within 64
    const long hc = f * a.H + h;
    const double *cs = a.ws_cs + hc * a.Q;
    const T *xp = (const T *)a.x + (tok0 * a.H + h) * P;
    const T *Cp = (const T *)a.Cm + (tok0 * a.G + g) * N;
    const float *Gp = a.ws_cb + (f * a.G + g) * a.Q * a.Q;

    float acc[4][MQ][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int m = 0; m < MQ; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r][m][e] = 0.0f;

    const int send = l0 + lrows;  // sources s < send
    for (int sx = tid; sx < send; sx += kThreads) {
        css[sx] = cs[sx];
        dts[sx] = dt_value(a.dt[(tok0 + sx) * a.H + h], a.dtp.dt_raw, a.dtp.dt_bias, h, a.dtp.dt_min, a.dtp.dt_max);
    }
    // the product G of a LTO x ST tile, four elements per thread, read one
    // step ahead (its scattered 64-byte rows are the longest wait of a step)
    constexpr int GPT = LTO * ST / kThreads;
    float gnext[GPT];
    auto load_g = [&](int s0) {
#pragma unroll
        for (int k = 0; k < GPT; ++k) {
            const int e = tid + k * kThreads;
            const int gi = e / ST, gj = e - (e / ST) * ST, sx = s0 + gj;
            gnext[k] = (gi < lrows && sx < send && l0 + gi >= sx) ? Gp[(long)(l0 + gi) * a.Q + sx] : 0.0f;
        }
    };
    load_g(0);
    __syncthreads();  // css, dts
    for (int s0 = 0; s0 < send; s0 += ST) {
        __syncthreads();  // the previous step is consumed
        // G' = G * exp(cs_l - cs_s) * dt_s, and the step's x rows
#pragma unroll
        for (int k = 0; k < GPT; ++k) {
            const int e = tid + k * kThreads;
            const int gi = e / ST, gj = e - (e / ST) * ST, sx = s0 + gj;
            Gt[gi][gj] = (gi < lrows && sx < send && l0 + gi >= sx)
                             ? gnext[k] * expf((float)(css[l0 + gi] - css[sx])) * dts[sx]
                             : 0.0f;
        }
        if (s0 + ST < send) load_g(s0 + ST);
        for (int e = tid; e < ST * P; e += kThreads) {
            const int r = e / P, p = e - (e / P) * P;
            Xs[r][p] = s0 + r < send ? ld(xp + (s0 + r) * HP + p) : 0.0f;
        }
        __syncthreads();
        const int srows = min(ST, send - s0);
        for (int j = 0; j < srows; ++j) {
            float gg[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) gg[r] = Gt[4 * oi + r][j];
#pragma unroll
            for (int m = 0; m < MQ; ++m) {
                const float4 x4 = *(const float4 *)&Xs[j][64 * m + 4 * oq];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[r][m][0] = fmaf(gg[r], x4.x, acc[r][m][0]);
                    acc[r][m][1] = fmaf(gg[r], x4.y, acc[r][m][1]);
                    acc[r][m][2] = fmaf(gg[r], x4.z, acc[r][m][2]);
                    acc[r][m][3] = fmaf(gg[r], x4.w, acc[r][m][3]);
                }
            }
        }
    }

    // carried-in state: off = C_l . h[p], ST columns of n at a time
    const float *hin = a.ws_S + hc * P * N;
    float off[4][MQ][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int m = 0; m < MQ; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) off[r][m][e] = 0.0f;
    for (int n0 = 0; n0 < N; n0 += ST) {
        const int ncols = min(ST, N - n0);
        __syncthreads();
        for (int e = tid; e < ST * P; e += kThreads) {  // Hs[nn][p] = h[p][n0 + nn]
            const int p = e / ST, nn = e - (e / ST) * ST;
            Hs[nn][p] = nn < ncols ? hin[(long)p * N + n0 + nn] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < LTO * ST / kThreads; ++k) {
            const int e = tid + k * kThreads;
            const int r = e / ST, nn = e - (e / ST) * ST;
            Cl[r][nn] = (r < lrows && nn < ncols) ? ld(Cp + (l0 + r) * GN + n0 + nn) : 0.0f;
        }
        __syncthreads();
        for (int nn = 0; nn < ncols; ++nn) {
            float cv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) cv[r] = Cl[4 * oi + r][nn];
#pragma unroll
            for (int m = 0; m < MQ; ++m) {
                const float4 h4 = *(const float4 *)&Hs[nn][64 * m + 4 * oq];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    off[r][m][0] = fmaf(cv[r], h4.x, off[r][m][0]);
                    off[r][m][1] = fmaf(cv[r], h4.y, off[r][m][1]);
                    off[r][m][2] = fmaf(cv[r], h4.z, off[r][m][2]);
                    off[r][m][3] = fmaf(cv[r], h4.w, off[r][m][3]);
                }
            }
        }
    }

    const float Dh = a.D ? a.D[h] : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 4 * oi + r;
        if (i >= lrows) break;
        const float el = expf((float)css[l0 + i]);
        const T *xl = xp + (l0 + i) * HP;
        T *yl = (T *)a.y + (tok0 + l0 + i) * HP + (long)h * P;
#pragma unroll
        for (int m = 0; m < MQ; ++m) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = 64 * m + 4 * oq + e;
                if (p < P) st(yl + p, acc[r][m][e] + el * off[r][m][e] + Dh * ld(xl + p));
            }
        }
    }
}

template <typename T, int MQ>
hipError_t launch_out(const PrefillArgs &a, dim3 grid, hipStream_t s) {
    return launch_stage("chunk_out_vec", chunk_out_vec<T, MQ>, grid, dim3(kThreads), 0, s, a);
}

// MQ = ceil(P / 64): 1, 2 or 4 (P <= 256)
template <typename T>
hipError_t launch_out_p(const PrefillArgs &a, dim3 grid, hipStream_t s) {
    const int mq = (a.P + 63) / 64;
    if (mq <= 1) return launch_out<T, 1>(a, grid, s);
    if (mq <= 2) return launch_out<T, 2>(a, grid, s);
    return launch_out<T, 4>(a, grid, s);
}

}  // namespace

hipError_t launch_prefill_vector(const PrefillArgs &a, int dtype, hipStream_t s) {
    const int gridB = a.chunks ? 1 : a.B;  // packed sequences: nchunks slots in all
    if (gridB > 65535 || a.H > 65535) return hipErrorInvalidConfiguration;
    dim3 g1(a.nchunks, a.H, gridB);
    hipError_t e = dtype == DT_BF16
                       ? launch_stage("chunk_state_vec", chunk_state_vec<bf16_t>, g1, dim3(kThreads), 0, s, a)
                       : launch_stage("chunk_state_vec", chunk_state_vec<float>, g1, dim3(kThreads), 0, s, a);
    if (e != hipSuccess) return e;
    if (a.G > 65535) return hipErrorInvalidConfiguration;
    const long ncb = (a.Q + CBT - 1) / CBT;
    if ((long)a.nchunks * (ncb * (ncb + 1) / 2) > 0x7fffffffL) return hipErrorInvalidConfiguration;
    dim3 g2((unsigned)(a.nchunks * (ncb * (ncb + 1) / 2)), a.G, gridB);
    e = dtype == DT_BF16 ? launch_stage("chunk_cb_vec", chunk_cb_vec<bf16_t>, g2, dim3(kThreads), 0, s, a)
                         : launch_stage("chunk_cb_vec", chunk_cb_vec<float>, g2, dim3(kThreads), 0, s, a);
    if (e != hipSuccess) return e;
    e = launch_state_pass(a, s);
    if (e != hipSuccess) return e;
    const long nlto = (a.Q + LTO - 1) / LTO;
    dim3 g3((unsigned)(a.nchunks * nlto), a.H, gridB);
    return dtype == DT_BF16 ? launch_out_p<bf16_t>(a, g3, s) : launch_out_p<float>(a, g3, s);
}

}  // namespace ssd
