// prefill_mfma.hip -- chunked SSD prefill on bf16 MFMA (gfx950),
// P = 64, N = 128, chunk Q = 256.
//
// The chunked form of the scan of arXiv 2603.09555 as laid out in the bqwf.cn
// article on its compiler-first Mamba-2 implementation: §1.1 (fixed chunks,
// dense work inside a chunk, a light sequential state scan between chunks,
// decay matrix tril(exp(segsum))) and §1.2 (intra-chunk product of C B^T
// masked by the decay with the discretised input).  For chunk c, head h,
// tokens l, s in [0, Q) and cs the in-chunk inclusive cumsum of dt*A:
//
//   S_c[p,n]  = sum_s exp(cs_last - cs_s) dt_s x_s[p] B_s[n]       (K1)
//   h_c       = exp(cs_last) h_{c-1} + S_c                          (K2)
//   y_l[p]    = sum_{s<=l} (C_l . B_s) exp(cs_l - cs_s) dt_s x_s[p]
//               + exp(cs_l) sum_n C_l[n] h_{c-1}[p,n] + D x_l[p]     (K3)
//
// K0 runs once per (batch, chunk, group): it forms G^T = B C^T (the only
// part of the masked product that does not depend on the head, shared by all
// heads of the group), applies the causal mask, and stores it as bf16 in the
// exact register order of the 32x32x16 MFMA accumulator; it also stores B in
// the order of the MFMA B operand for the token contraction of K1.  K1 and K3
// then run one workgroup per (batch, chunk, head) with small LDS footprints,
// several per CU, and read those packed operands straight from L2.
//
// Contractions over tokens need 8 consecutive tokens per lane in an operand,
// while x is stored token-major: K1 and K3 transpose their x chunk through
// registers into LDS once, folding in a per-token scale.  The decay of K3 is
// factored per 32x32 tile (si, lt) of G^T as
//     exp(cs_l - cs_s) dt_s = exp(cs_l - cs_end(si)) * [exp(cs_end(si) - cs_s) dt_s]
// with cs_end(si) the cumsum at the end of token tile si: the bracket depends
// on s only and is folded into x; the first factor is one value per lane
// (its column l).  Off the diagonal tile both factors are <= 1; on it the
// first is at most exp(32 max|dt*A|), finite in fp32, and the product is <= 1.
// The accumulator order of a 32x32 tile (lane i: column i%32, rows
// 8q + 4(i/32) + r) is a valid K order of 16 tokens for each pair of q, so G^T
// tiles feed the A operand directly and x is read from LDS in that order.
// D x is added through the diagonal of the masked product: with x' = v x and
// M = u G^T, adding D / dt_l to G^T[l,l] before the scale by u_l adds
// u_l v_l D/dt_l x_l = D x_l (u_l v_l = dt_l).
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 256, kP = 64, kN = 128, kThreads = 256;
constexpr int kTiles = kQ / 32;                      // token tiles per chunk
constexpr int kGTiles = kTiles * (kTiles + 1) / 2;   // causal 32x32 tiles of G^T
constexpr long kGTChunk = (long)kGTiles * 64 * 16;   // bf16 per chunk (64 lanes x 16)
constexpr long kBTChunk = (long)kQ * kN;             // bf16 per chunk

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// Byte offset of 16-byte chunk `ch` of row `r`, XOR-swizzled so that the 32
// rows one MFMA operand read touches land in distinct LDS banks.
__device__ __forceinline__ int sw16(int r, int ch) { return r * 256 + ((ch ^ (r & 15)) << 4); }  // 128-bf16 rows
__device__ __forceinline__ int sw32(int r, int ch) { return r * 512 + ((ch ^ (r & 31)) << 4); }  // 256-bf16 rows

__device__ __forceinline__ u32x4 lds16(const char *base, int off) { return *(const u32x4 *)(base + off); }
__device__ __forceinline__ u32x2 lds8(const char *base, int off) { return *(const u32x2 *)(base + off); }

__device__ __forceinline__ float lo_bf16(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}

// index of causal tile (token tile si, column tile lt), si <= lt
__device__ __forceinline__ int gt_index(int si, int lt) { return lt * (lt + 1) / 2 + si; }

__device__ __forceinline__ double wave_inclusive_sum_f64(double v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        double o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

// In-chunk inclusive cumsum of dt*A over the Q tokens of (b, chunk, h), in
// fp64 so that differences cs_l - cs_s keep full fp32 accuracy.  Token t is
// thread t; padded tokens (t >= Qc) get dt = 0.  Writes cs[] and dt[].
__device__ __forceinline__ void chunk_cumsum(const PrefillArgs &a, int b, int t0, int Qc, int h, double *cs,
                                             float *dts, double *wsum) {
    const int t = threadIdx.x;
    const float dtv = t < Qc ? a.dt[((long)b * a.L + t0 + t) * a.H + h] : 0.0f;
    const float Af = -expf(a.A_log[h]);
    double inc = wave_inclusive_sum_f64((double)(dtv * Af));
    if ((t & 63) == 63) wsum[t >> 6] = inc;
    __syncthreads();
    for (int w = 0; w < (t >> 6); ++w) inc += wsum[w];
    cs[t] = inc;
    dts[t] = dtv;
}

// Load the x chunk of head h ([Q tokens][P] bf16, row stride H*P): thread t
// owns the 8x8 block of tokens 8*(t/8).. and features 8*(t%8)..
__device__ __forceinline__ void load_x_raw(const PrefillArgs &a, int b, int t0, int Qc, int h, u32x4 (&raw)[8]) {
    const int t = threadIdx.x;
    const int sb = t >> 3, pb = t & 7;
    const bf16_t *xg = (const bf16_t *)a.x + (((long)b * a.L + t0) * a.H + h) * kP + pb * 8;
    const int rs = a.H * kP;  // in-chunk row offsets fit in 32 bits (Q * H * P < 2^31)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int s = sb * 8 + r;
        raw[r] = s < Qc ? *(const u32x4 *)(xg + s * rs) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Scale token s of the thread's block by scale(s) and store the block
// transposed ([P][Q], swizzled) in LDS.
template <typename ScaleFn>
__device__ __forceinline__ void store_x_transposed(const u32x4 (&raw)[8], char *xt, ScaleFn scale) {
    const int t = threadIdx.x;
    const int sb = t >> 3, pb = t & 7;
    float v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = scale(sb * 8 + r);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned w0 = raw[2 * e][j >> 1], w1 = raw[2 * e + 1][j >> 1];
            const float f0 = (j & 1) ? hi_bf16(w0) : lo_bf16(w0);
            const float f1 = (j & 1) ? hi_bf16(w1) : lo_bf16(w1);
            o[e] = pack_bf16(f0 * v[2 * e], f1 * v[2 * e + 1]);
        }
        *(u32x4 *)(xt + sw32(pb * 8 + j, sb)) = o;
    }
}

// ------------------------------------------------------------------------
// K0: per (batch, chunk, group, part): masked G^T tiles of the column-tile
// pair (part, 7-part), and the part-th 32-wide slice of B in K1's operand
// order.  Grid (nchunks, 4 * G, B).
// ------------------------------------------------------------------------
constexpr int K0_LDS = 2 * kQ * kN * 2;  // B and C of the chunk

__global__ __launch_bounds__(kThreads) void chunk_pack_mfma(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *bl = smem;
    char *cl = smem + kQ * kN * 2;
    const int c = blockIdx.x, b = blockIdx.z;
    const int part = blockIdx.y & 3, g = blockIdx.y >> 2;
    const int t0 = c * kQ;
    const int Qc = min(kQ, a.L - t0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    const long cg = ((long)b * a.nchunks + c) * a.G + g;  // (batch, chunk, group) index
    {
        const bf16_t *bg = (const bf16_t *)a.Bm + (((long)b * a.L + t0) * a.G + g) * kN;
        const bf16_t *cgp = (const bf16_t *)a.Cm + (((long)b * a.L + t0) * a.G + g) * kN;
        const int rs = a.G * kN;
#pragma unroll
        for (int k = 0; k < (kQ * kN / 8) / kThreads; ++k) {
            const int idx = tid + k * kThreads;
            const int r = idx >> 4, ch = idx & 15;
            u32x4 vb = {0u, 0u, 0u, 0u}, vc = {0u, 0u, 0u, 0u};
            if (r < Qc) {
                vb = *(const u32x4 *)(bg + r * rs + ch * 8);
                vc = *(const u32x4 *)(cgp + r * rs + ch * 8);
            }
            *(u32x4 *)(bl + sw16(r, ch)) = vb;
            *(u32x4 *)(cl + sw16(r, ch)) = vc;
        }
    }
    __syncthreads();

    // G^T tiles: slot k -> (si, lt); slots 0..part belong to column tile
    // `part`, slots part+1..8 to column tile 7-part.  Wave w takes slots
    // w, w+4, w+8.
    u32x4 *gt = (u32x4 *)(a.ws_gt + cg * kGTChunk);
    for (int k = wave; k <= kTiles; k += 4) {
        const int si = k <= part ? k : k - part - 1;
        const int lt = k <= part ? part : kTiles - 1 - part;
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < kN / 16; ++kk) {
            const u32x4 av = lds16(bl, sw16(si * 32 + li, kk * 2 + lh));
            const u32x4 bv = lds16(cl, sw16(lt * 32 + li, kk * 2 + lh));
            acc = mfma32(av, bv, acc);
        }
        if (si == lt) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if ((v >> 2) * 8 + lh * 4 + (v & 3) > li) acc[v] = 0.0f;  // token s after token l
        }
        u32x4 o0, o1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o0[e] = pack_bf16(acc[e * 2], acc[e * 2 + 1]);
            o1[e] = pack_bf16(acc[8 + e * 2], acc[8 + e * 2 + 1]);
        }
        u32x4 *dst = gt + ((long)gt_index(si, lt) * 64 + lane) * 2;
        dst[0] = o0;
        dst[1] = o1;
    }

    // B in K1's operand order: [nt][kk][lane] 16 bytes = B[kk*16 + lh*8 + j][nt*32 + li]
    u32x4 *bt = (u32x4 *)(a.ws_bt + cg * kBTChunk);
    const int nt = part;
    for (int idx = tid; idx < (kQ / 16) * 64; idx += kThreads) {
        const int kk = idx >> 6, ln = idx & 63;
        const int n = nt * 32 + (ln & 31), s0 = kk * 16 + (ln >> 5) * 8;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned short lo = *(const unsigned short *)(bl + sw16(s0 + 2 * e, n >> 3) + (n & 7) * 2);
            const unsigned short hi = *(const unsigned short *)(bl + sw16(s0 + 2 * e + 1, n >> 3) + (n & 7) * 2);
            o[e] = (unsigned)lo | ((unsigned)hi << 16);
        }
        bt[(nt * (kQ / 16) + kk) * 64 + ln] = o;
    }
}

// ------------------------------------------------------------------------
// K1: chunk states S_c = (w o X)^T B, w_s = exp(cs_last - cs_s) dt_s.
// Grid (nchunks * H, 1, B), one workgroup per (batch, chunk, head).
// Wave w computes the 64 x 32 slice of S for state columns 32w..32w+31.
// ------------------------------------------------------------------------
constexpr int K1_XT = 0;
constexpr int K1_CS = K1_XT + kP * kQ * 2;
constexpr int K1_DT = K1_CS + kQ * 8;
constexpr int K1_WS = K1_DT + kQ * 4;
constexpr int K1_LDS = K1_WS + 64;

__global__ __launch_bounds__(kThreads) void chunk_state_mfma(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *xt = smem + K1_XT;
    double *cs = (double *)(smem + K1_CS);
    float *dts = (float *)(smem + K1_DT);
    double *wsum = (double *)(smem + K1_WS);
    const int c = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H, b = blockIdx.z;
    const int t0 = c * kQ;
    const int Qc = min(kQ, a.L - t0);
    const int g = h / (a.H / a.G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;

    // every global load of this workgroup is issued before the cumsum
    u32x4 raw[8];
    load_x_raw(a, b, t0, Qc, h, raw);
    const long cg = ((long)b * a.nchunks + c) * a.G + g;
    const u32x4 *bt = (const u32x4 *)(a.ws_bt + cg * kBTChunk) + (wave * (kQ / 16)) * 64 + lane;
    u32x4 bq[kQ / 16];
#pragma unroll
    for (int kk = 0; kk < kQ / 16; ++kk) bq[kk] = bt[kk * 64];

    chunk_cumsum(a, b, t0, Qc, h, cs, dts, wsum);
    __syncthreads();
    const double cs_last = cs[kQ - 1];
    store_x_transposed(raw, xt, [&](int s) { return expf((float)(cs_last - cs[s])) * dts[s]; });
    __syncthreads();

    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int kk = 0; kk < kQ / 16; ++kk) {
        const u32x4 bv = bq[kk];
        const u32x4 a0 = lds16(xt, sw32(li, kk * 2 + lh));
        const u32x4 a1 = lds16(xt, sw32(32 + li, kk * 2 + lh));
        acc0 = mfma32(a0, bv, acc0);
        acc1 = mfma32(a1, bv, acc1);
    }
    const long hc = ((long)b * a.nchunks + c) * a.H + h;
    float *Sg = a.ws_S + hc * kP * kN + wave * 32 + li;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int p = (v >> 2) * 8 + lh * 4 + (v & 3);
        Sg[p * kN] = acc0[v];
        Sg[(32 + p) * kN] = acc1[v];
    }
    if (tid == 0) a.ws_dec[hc] = expm1f((float)cs_last);
}

// ------------------------------------------------------------------------
// K3: outputs.  Grid (nchunks * H, 1, B), one workgroup per (batch, chunk,
// head).  Wave w owns token tiles w and 7-w (balanced causal work) and both
// 32-wide feature tiles of P.
// ------------------------------------------------------------------------
constexpr int K3_XT = 0;                       // x'^T [P][Q] bf16, later y staging [Q][P] bf16
constexpr int K3_H = K3_XT + kP * kQ * 2;      // h [P][N] bf16
constexpr int K3_CS = K3_H + kP * kN * 2;      // cs [Q] f64
constexpr int K3_EL = K3_CS + kQ * 8;          // exp(cs) [Q]
constexpr int K3_DT = K3_EL + kQ * 4;          // dt [Q]
constexpr int K3_WS = K3_DT + kQ * 4;
constexpr int K3_LDS = K3_WS + 64;

// One G^T tile (si, lt) applied to x'^T: unpack, add D/dt on the diagonal,
// scale by the lane's column factor, repack as the bf16 A operand, then two
// K=16 MFMAs per 32-wide feature tile.
__device__ __forceinline__ void intra_tile(const u32x4 g0, const u32x4 g1, f32x16 (&Y)[2], const char *xt,
                                           const double *cs, const float *dts, float Dh, int si, int lt, int li,
                                           int lh) {
    float gv[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        gv[e * 2] = lo_bf16(g0[e]);
        gv[e * 2 + 1] = hi_bf16(g0[e]);
        gv[8 + e * 2] = lo_bf16(g1[e]);
        gv[8 + e * 2 + 1] = hi_bf16(g1[e]);
    }
    const int l = lt * 32 + li;
    if (si == lt) {
        // this lane holds G^T[l, l] iff bit 2 of l matches its row half
        const float dtl = dts[l];
        const float add = (((li >> 2) & 1) == lh && dtl > 0.0f) ? Dh / dtl : 0.0f;
        const int vd = ((li >> 3) << 2) | (li & 3);
#pragma unroll
        for (int v = 0; v < 16; ++v) gv[v] += (v == vd) ? add : 0.0f;
    }
    const float u = expf((float)(cs[l] - cs[si * 32 + 31]));
    u32x4 f[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 4; ++e) f[hf][e] = pack_bf16(gv[hf * 8 + e * 2] * u, gv[hf * 8 + e * 2 + 1] * u);
#pragma unroll
    for (int ptile = 0; ptile < 2; ++ptile) {
        const int p = ptile * 32 + li;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int ch = si * 4 + hf * 2;
            const u32x2 xa = lds8(xt, sw32(p, ch) + lh * 8);
            const u32x2 xb = lds8(xt, sw32(p, ch + 1) + lh * 8);
            const u32x4 bv = {xa[0], xa[1], xb[0], xb[1]};
            Y[ptile] = mfma32(f[hf], bv, Y[ptile]);
        }
    }
}

__global__ __launch_bounds__(kThreads) void chunk_out_mfma(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *xt = smem + K3_XT;
    char *hl = smem + K3_H;
    double *cs = (double *)(smem + K3_CS);
    float *el = (float *)(smem + K3_EL);
    float *dts = (float *)(smem + K3_DT);
    double *wsum = (double *)(smem + K3_WS);

    const int c = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H, b = blockIdx.z;
    const int t0 = c * kQ;
    const int Qc = min(kQ, a.L - t0);
    const int g = h / (a.H / a.G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    const int ltA = wave, ltB = kTiles - 1 - wave;
    const long hc = ((long)b * a.nchunks + c) * a.H + h;
    const long cg = ((long)b * a.nchunks + c) * a.G + g;

    // x and the first two G^T tiles of this wave are requested before the
    // cumsum; the other tiles are requested two slots ahead of their use.
    // Slot k of wave w: k <= w -> (token tile k, column tile w),
    // k > w -> (token tile k-w-1, column tile 7-w).
    u32x4 raw[8];
    load_x_raw(a, b, t0, Qc, h, raw);
    const u32x4 *gt = (const u32x4 *)(a.ws_gt + cg * kGTChunk) + lane * 2;
    auto slot_src = [&](int k) {
        const int si = k <= wave ? k : k - wave - 1;
        const int lt = k <= wave ? ltA : ltB;
        return gt + gt_index(si, lt) * 128;
    };
    u32x4 gq[3][2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        gq[k][0] = slot_src(k)[0];
        gq[k][1] = slot_src(k)[1];
    }

    chunk_cumsum(a, b, t0, Qc, h, cs, dts, wsum);
    el[tid] = expf((float)cs[tid]);
    __syncthreads();
    store_x_transposed(raw, xt, [&](int s) {
        const double ce = cs[(s & ~31) + 31];
        return expf((float)(ce - cs[s])) * dts[s];
    });
    {
        const bf16_t *hg = a.ws_hb + hc * kP * kN;
#pragma unroll
        for (int k = 0; k < (kP * kN / 8) / kThreads; ++k) {
            const int idx = tid + k * kThreads;
            const int r = idx >> 4, ch = idx & 15;
            *(u32x4 *)(hl + sw16(r, ch)) = *(const u32x4 *)(hg + r * kN + ch * 8);
        }
    }
    __syncthreads();

    // ---- inter-chunk term: Y = exp(cs_l) * C h^T   (K = N); C read from L2
    const bf16_t *cgp = (const bf16_t *)a.Cm + (((long)b * a.L + t0) * a.G + g) * kN;
    const int rs_c = a.G * kN;
    f32x16 Y[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int lt = s2 ? ltB : ltA;
        const int l = lt * 32 + li;
        const bf16_t *crow = cgp + l * rs_c + lh * 8;
        const bool lv = l < Qc;
        f32x16 y0 = {}, y1 = {};
#pragma unroll
        for (int kk = 0; kk < kN / 16; ++kk) {
            const u32x4 av = lv ? *(const u32x4 *)(crow + kk * 16) : u32x4{0u, 0u, 0u, 0u};
            const u32x4 b0 = lds16(hl, sw16(li, kk * 2 + lh));
            const u32x4 b1 = lds16(hl, sw16(32 + li, kk * 2 + lh));
            y0 = mfma32(av, b0, y0);
            y1 = mfma32(av, b1, y1);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float e = el[lt * 32 + (v >> 2) * 8 + lh * 4 + (v & 3)];
            y0[v] *= e;
            y1[v] *= e;
        }
        Y[s2][0] = y0;
        Y[s2][1] = y1;
    }

    // ---- intra-chunk term and D x: Y += (G^T o decay + D/dt on the diagonal)^T x'
    const float Dh = a.D ? a.D[h] : 0.0f;
#pragma unroll
    for (int k = 0; k <= kTiles; ++k) {
        if (k + 2 <= kTiles) {
            gq[(k + 2) % 3][0] = slot_src(k + 2)[0];
            gq[(k + 2) % 3][1] = slot_src(k + 2)[1];
        }
        if (k <= wave)
            intra_tile(gq[k % 3][0], gq[k % 3][1], Y[0], xt, cs, dts, Dh, k, ltA, li, lh);
        else
            intra_tile(gq[k % 3][0], gq[k % 3][1], Y[1], xt, cs, dts, Dh, k - wave - 1, ltB, li, lh);
    }

    // ---- epilogue: stage y (bf16) through LDS, then 16-byte coalesced stores
    __syncthreads();  // every wave is done reading x'^T
    char *ys = xt;    // [Q][P] bf16, rows of 128 bytes, 8 chunks, swizzled by row
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int lt = s2 ? ltB : ltA;
#pragma unroll
        for (int ptile = 0; ptile < 2; ++ptile) {
            const int p = ptile * 32 + li;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int l = lt * 32 + (v >> 2) * 8 + lh * 4 + (v & 3);
                *(bf16_t *)(ys + l * 128 + (((p >> 3) ^ (l & 7)) << 4) + (p & 7) * 2) = f32_to_bf16(Y[s2][ptile][v]);
            }
        }
    }
    __syncthreads();
    bf16_t *yg = (bf16_t *)a.y + (((long)b * a.L + t0) * a.H + h) * kP;
    const int rs_y = a.H * kP;
#pragma unroll
    for (int k = 0; k < (kQ * kP / 8) / kThreads; ++k) {
        const int idx = tid + k * kThreads;
        const int l = idx >> 3, ch = idx & 7;
        if (l < Qc) *(u32x4 *)(yg + l * rs_y + ch * 8) = *(const u32x4 *)(ys + l * 128 + ((ch ^ (l & 7)) << 4));
    }
}

// ------------------------------------------------------------------------
// K2: the state pass.  Reads S_c (fp32), keeps h in fp32, writes the
// carried-in state h_{c-1} as bf16 (the MFMA operand of C h) and the final
// state in fp32.  h + (dm1 * h + S) rounds the state once per chunk.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void state_pass_bf16(PrefillArgs a, long total) {
    const long e = (long)blockIdx.x * kThreads + threadIdx.x;  // float4 index
    if (e >= total) return;
    const long PN4 = (long)kP * kN / 4;
    const long bh = e / PN4;
    const long pn = e - bh * PN4;
    const int h = (int)(bh % a.H);
    const long b = bh / a.H;
    float4 hv = a.init_state ? ((const float4 *)a.init_state)[bh * PN4 + pn] : make_float4(0.f, 0.f, 0.f, 0.f);
    const int nch = a.nchunks;
    constexpr int kB = 8;
    for (int c0 = 0; c0 < nch; c0 += kB) {
        float4 sv[kB];
        float dv[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            if (c0 + j < nch) {
                const long hc = (b * nch + c0 + j) * a.H + h;
                sv[j] = ((const float4 *)(a.ws_S + hc * kP * kN))[pn];
                dv[j] = a.ws_dec[hc];
            }
        }
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            if (c0 + j < nch) {
                const long hc = (b * nch + c0 + j) * a.H + h;
                u32x2 o = {pack_bf16(hv.x, hv.y), pack_bf16(hv.z, hv.w)};
                ((u32x2 *)(a.ws_hb + hc * kP * kN))[pn] = o;
                const float d = dv[j];
                hv.x += fmaf(d, hv.x, sv[j].x);
                hv.y += fmaf(d, hv.y, sv[j].y);
                hv.z += fmaf(d, hv.z, sv[j].z);
                hv.w += fmaf(d, hv.w, sv[j].w);
            }
        }
    }
    if (a.final_state) ((float4 *)a.final_state)[bh * PN4 + pn] = hv;
}

bool g_attr_set = false;

}  // namespace

long prefill_mfma_gt_elems_per_chunk() { return kGTChunk; }
long prefill_mfma_bt_elems_per_chunk() { return kBTChunk; }

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t s) {
    if (!g_attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)chunk_pack_mfma, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           K0_LDS);
        if (e != hipSuccess) return e;
        g_attr_set = true;
    }
    if ((long)a.nchunks * a.H > 0x7fffffffL || a.G * 4 > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_pack_mfma, dim3(a.nchunks, 4 * a.G, a.B), dim3(kThreads), K0_LDS, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(a.nchunks * a.H), 1, a.B);
    hipLaunchKernelGGL(chunk_state_mfma, grid, dim3(kThreads), K1_LDS, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long total = (long)a.B * a.H * (kP * kN / 4);
    hipLaunchKernelGGL(state_pass_bf16, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                       a, total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_out_mfma, grid, dim3(kThreads), K3_LDS, s, a);
    return hipGetLastError();
}

}  // namespace ssd
