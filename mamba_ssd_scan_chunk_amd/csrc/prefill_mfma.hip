// prefill_mfma.hip -- chunked SSD prefill on bf16 MFMA (gfx950),
// P = 64, N = 128, chunks of 256 tokens (a longer chunk, a multiple of 256,
// runs as 256-token sub-chunks linked by the state pass).
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
// the order of the MFMA B operand for the token contraction of K1 (the state
// pass K2, a streaming kernel with spare issue slots, stores C in the order
// of the B operand of h C^T in K3).  K1 and K3 then run one
// workgroup per (batch, chunk, head) with small LDS footprints, several per
// CU, and read those packed operands straight from L2, 1 KiB contiguous per
// load instruction.
//
// Contractions over tokens need 8 consecutive tokens per lane in an operand,
// while x is stored token-major: K1 and K3 transpose their x chunk through
// registers into LDS once, folding in a per-token scale.  K3 factors the
// decay exp(cs_l - cs_s) dt_s through a reference cumsum R_k per 32-token
// tile (a Horner scheme over token tiles, described at K3), so the masked
// C B^T tiles enter the MFMA exactly as K0 stored them.  The accumulator
// order of a 32x32 tile (lane i: column i%32, rows 8q + 4(i/32) + r) is a
// valid K order of 16 tokens for each pair of q, so a G^T tile is the B
// operand of K3's MFMA as it stands and x'^T is read from LDS in that order.
// D x is added through the diagonal of the masked product: with x' = v x and
// the output scaled by u, adding D / dt_l to G^T[l,l] adds
// u_l v_l D/dt_l x_l = D x_l (u_l v_l = dt_l).
#include <algorithm>

#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = kMfmaQ, kP = 64, kN = 128, kThreads = 256;
constexpr int kTiles = kQ / 32;                      // token tiles per chunk
constexpr int kGTiles = kTiles * (kTiles + 1) / 2;   // causal 32x32 tiles of G^T
constexpr long kGTChunk = (long)kGTiles * 64 * 16;   // bf16 per chunk (64 lanes x 16)
constexpr long kBTChunk = (long)kQ * kN;             // bf16 per chunk

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ float lo_bf16(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup i to XCD i % 8),
// each XCD with its own L2.  This maps workgroup i to an item so that every
// XCD gets one contiguous range of items: the heads of a chunk then share one
// L2 for the chunk's packed operands (B for K1; C and the G^T tiles for K3)
// instead of each of the 8 L2s fetching them.
__device__ __forceinline__ int xcd_item(int i, int total) {
    const int x = i & 7, j = i >> 3;
    const int q = total >> 3, r = total & 7;
    return x * q + min(x, r) + j;
}

// index of causal tile (token tile si, column tile lt), si <= lt
__device__ __forceinline__ int gt_index(int si, int lt) { return lt * (lt + 1) / 2 + si; }

// Buffer resource over `bytes` bytes from p: loads at or past the end
// return zeros, which is how the ragged last chunk reads its missing tokens.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Load the x chunk of head h ([Q tokens][P] bf16, row stride H*P) whose
// first token is row tok0: thread t owns the 8x8 block of tokens 8*(t/8)..
// and features 8*(t%8)..; tokens at or past Qc read as zero.
__device__ __forceinline__ void load_x_raw(const PrefillArgs &a, long tok0, int Qc, int h, u32x4 (&raw)[8], int t) {
    const int sb = t >> 3, pb = t & 7;
    const unsigned rs = (unsigned)a.H * kP * 2;  // row stride in bytes
    const bf16_t *x0 = (const bf16_t *)a.x + (tok0 * a.H + h) * kP;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(x0, (unsigned)(Qc - 1) * rs + kP * 2);
#pragma unroll
    for (int k = 0; k < 8; ++k) raw[k] = buf_load16(r, (unsigned)(sb * 8 + k) * rs + pb * 16);
}

// dt of token tid of the chunk (0 at or past Qc), after the optional
// preprocessing of the raw value.
__device__ __forceinline__ float load_dt(const PrefillArgs &a, long tok0, int Qc, int h, int t) {
    const float *d0 = a.dt + tok0 * a.H + h;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(d0, (unsigned)((Qc - 1) * a.H + 1) * 4);
    const float v = buf_load_f32(r, (unsigned)t * a.H * 4);
    if (!a.dtp.dt_raw) return v;
    return t < Qc ? dt_value(v, 1, a.dtp.dt_bias, h, a.dtp.dt_min, a.dtp.dt_max) : 0.0f;
}

constexpr int kXRow = kQ * 2 + 16;        // x'^T row stride in LDS (bytes), padded against bank conflicts
constexpr int K3_XT = 0;                  // x'^T [P][Q] bf16, tokens in MFMA K order
constexpr int K3_H = K3_XT + kP * kXRow;  // h_{c-1} [P][N] bf16, 16-byte chunks XOR-swizzled by row
constexpr int K3_V = K3_H + kP * kN * 2;  // x' scale per token (fast path) or cs (exact path)
constexpr int K3_U = K3_V + kQ * 4;       // u_l
constexpr int K3_DT = K3_U + kQ * 4;      // dt
constexpr int K3_W = K3_DT + kQ * 4;      // per wave: cumsum at tokens 15, 47, 63; Q_k
constexpr int K3_LDS = K3_W + 32 * 4;
constexpr int kYRow = kP * 2 + 16;        // output staging row stride (bytes), after the main phase
static_assert(4 * 2 * 32 * kYRow <= K3_V, "output staging must fit in the x'^T and h areas");

__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// Byte offset in x'^T of the 16 bytes that lane (row p, half lh) feeds to the
// MFMA for token tile si, K half hf.  Within every 16-token group the four
// 4-token runs are stored in the order 0, 2, 1, 3, so that the tokens
// {0-3, 8-11} (lh = 0) and {4-7, 12-15} (lh = 1) -- the K order in which a
// G^T accumulator tile is consumed -- are contiguous.
__device__ __forceinline__ int xt_operand(int p, int lh, int si, int hf) {
    return p * kXRow + 32 * (2 * si + hf) + 16 * lh;
}

// Scale token s of the thread's 8x8 block (tokens 8*(t/8).., features
// 8*(t%8)..) by sc[s] and store it transposed into x'^T.
__device__ __forceinline__ void store_xt_korder(const u32x4 (&raw)[8], const float (&sc)[8], char *xt, int t) {
    const int sb = t >> 3, pb = t & 7;
    // tokens 8sb..8sb+3 and 8sb+4..8sb+7 are runs 2(sb&1) and 2(sb&1)+1 of
    // group sb/2, stored at positions (sb&1) and 2+(sb&1)
    char *dst = xt + (pb * 8) * kXRow + 32 * (sb >> 1) + 8 * (sb & 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        unsigned o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned w0 = raw[2 * e][j >> 1], w1 = raw[2 * e + 1][j >> 1];
            const float f0 = (j & 1) ? hi_bf16(w0) : lo_bf16(w0);
            const float f1 = (j & 1) ? hi_bf16(w1) : lo_bf16(w1);
            o[e] = pack_bf16(f0 * sc[2 * e], f1 * sc[2 * e + 1]);
        }
        *(u32x2 *)(dst + j * kXRow) = u32x2{o[0], o[1]};
        *(u32x2 *)(dst + j * kXRow + 16) = u32x2{o[2], o[3]};
    }
}

// ------------------------------------------------------------------------
// K0: per (batch, chunk, group), shared by every head of the group.  Grid
// (nchunks, 13 * G, B).  Blocks y % 13 < 9 form the 36 causal 32x32 tiles of
// G^T = B C^T, one per wave, masked (s > l -> 0) and stored as bf16 in the
// exact register order of the MFMA accumulator; blocks y % 13 >= 9 write the
// 32-column slice y % 13 - 9 of B in the order of K1's MFMA B operand.  The
// operands are read straight from L2; tokens past the end read as zero.
// ------------------------------------------------------------------------
constexpr int kK0Tiles = kGTiles / 4;         // workgroups forming G^T tiles
constexpr int kK0Blocks = kK0Tiles + kN / 32;  // plus one per 32 columns of B

__global__ __launch_bounds__(kThreads) void chunk_pack_mfma(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) char bl[kQ * 64];  // B[:, 32 columns] as [token][32] bf16
    const long f = (long)blockIdx.z * a.nchunks + blockIdx.x;
    const ChunkEntry ch = chunk_at(a, f);
    const int Qc = ch.Qc;
    if (Qc <= 0) return;  // unused slot of a packed prefill
    const int part = blockIdx.y % kK0Blocks, g = blockIdx.y / kK0Blocks;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    const long cg = f * a.G + g;
    const unsigned rs = (unsigned)a.G * kN * 2;  // token stride of B and C in bytes
    const long base = ((long)ch.tok0 * a.G + g) * kN;
    const unsigned bytes = (unsigned)(Qc - 1) * rs + kN * 2;
    const __amdgpu_buffer_rsrc_t brs = make_rsrc((const bf16_t *)a.Bm + base, bytes);

    if (part < kK0Tiles) {
        const __amdgpu_buffer_rsrc_t crs = make_rsrc((const bf16_t *)a.Cm + base, bytes);
        const int tix = part * 4 + wave;  // = gt_index(si, lt)
        int lt = 0;
        while ((lt + 1) * (lt + 2) / 2 <= tix) ++lt;
        const int si = tix - lt * (lt + 1) / 2;
        const unsigned oa = (unsigned)(si * 32 + li) * rs + 16 * lh;
        const unsigned ob = (unsigned)(lt * 32 + li) * rs + 16 * lh;
        u32x4 av[8], bv[8];
#pragma unroll
        for (int kk = 0; kk < kN / 16; ++kk) {
            av[kk] = buf_load16(brs, oa + 32 * kk);
            bv[kk] = buf_load16(crs, ob + 32 * kk);
        }
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < kN / 16; ++kk) acc = mfma32(av[kk], bv[kk], acc);
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
        // [tile][half][lane]: each half of a tile is 1 KiB contiguous, one
        // load instruction of K3
        u32x4 *dst = (u32x4 *)(a.ws_gt + cg * kGTChunk) + (long)tix * 128 + lane;
        dst[0] = o0;
        dst[64] = o1;
        return;
    }

    // B columns 32 nt .. 32 nt + 31 into LDS, then K1's operand order:
    // [nt][group gg of 16 tokens][lane] 16 bytes = B[s_j][32 nt + li] with
    // s_j = 16 gg + 4 lh + (j & 3) + 8 (j >> 2), the token order of x'^T.
    const int nt = part - kK0Tiles;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + k * kThreads;
        const int s = idx >> 2, q = idx & 3;
        *(u32x4 *)(bl + s * 64 + q * 16) = buf_load16(brs, (unsigned)s * rs + nt * 64 + q * 16);
    }
    __syncthreads();
    u32x4 *bt = (u32x4 *)(a.ws_bt + cg * kBTChunk) + nt * (kQ / 16) * 64;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + k * kThreads;
        const int gg = idx >> 6, ln = idx & 63;
        const int s0 = 16 * gg + 4 * (ln >> 5);
        const char *col = bl + (ln & 31) * 2;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int sa = s0 + 2 * (e & 1) + 8 * (e >> 1);
            const unsigned lo = *(const unsigned short *)(col + sa * 64);
            const unsigned hi = *(const unsigned short *)(col + (sa + 1) * 64);
            o[e] = lo | (hi << 16);
        }
        bt[gg * 64 + ln] = o;
    }
}

// ------------------------------------------------------------------------
// K1: chunk states.  Grid (B * nchunks * H), workgroup = item (b, c, h) in
// the XCD-aware order:
//   S_c[p, n] = sum_s exp(cs_last - cs_s) dt_s x_s[p] B_s[n]
// with x'' = exp(cs_last - cs_s) dt_s x_s <= dt_s folded into x in LDS.
// Wave w computes the 64 x 32 slice of S for columns n in [32w, 32w + 32).
// Also writes exp(cs_last) - 1 for the state pass.
// ------------------------------------------------------------------------
constexpr int K1_XT = 0;
constexpr int K1_V = K1_XT + kP * kXRow;
constexpr int K1_W = K1_V + kQ * 4;
constexpr int K1_LDS = K1_W + 16 * 4;

__global__ __launch_bounds__(kThreads) void chunk_state_mfma(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *xt = smem + K1_XT;
    float *vt = (float *)(smem + K1_V);
    float *wv = (float *)(smem + K1_W);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    const int item = xcd_item(blockIdx.x, gridDim.x);  // grid = one workgroup per item
    const int h = item % a.H, bc = item / a.H;
    const ChunkEntry ch = chunk_at(a, bc);
    const int Qc = ch.Qc;
    if (Qc <= 0) return;  // unused slot of a packed prefill
    const long tok0 = ch.tok0;
    const int g = h / (a.H / a.G);
    const long cg = (long)bc * a.G + g;

    // every global load of this workgroup is issued before the cumsum, dt
    // first: loads retire in issue order, so the cumsum waits for dt only
    const float dtv = load_dt(a, tok0, Qc, h, tid);
    u32x4 raw[8];
    load_x_raw(a, tok0, Qc, h, raw, tid);
    const u32x4 *bt = (const u32x4 *)(a.ws_bt + cg * kBTChunk) + (wave * (kQ / 16)) * 64 + lane;
    u32x4 bq[kQ / 16];
#pragma unroll
    for (int gg = 0; gg < kQ / 16; ++gg) bq[gg] = bt[gg * 64];

    // cumsum within each 64-token wave (fp32); cs_last - cs_t from the wave totals
    const float loc = wave_inclusive_sum(dtv * -expf(a.A_log[h]));
    if (lane == 63) wv[wave] = loc;
    __syncthreads();
    float after = 0.0f, total = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float tw = wv[w];
        total += tw;
        after += w > wave ? tw : 0.0f;
    }
    vt[tid] = exp_fast(wv[wave] - loc + after) * dtv;  // dt = 0 past Qc
    if (tid == 0) a.ws_dec[item] = expm1f(total);
    __syncthreads();
    {
        const float4 s0 = *(const float4 *)(vt + (tid >> 3) * 8);
        const float4 s1 = *(const float4 *)(vt + (tid >> 3) * 8 + 4);
        const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        store_xt_korder(raw, sc, xt, tid);
    }
    __syncthreads();

    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int gg = 0; gg < kQ / 16; ++gg) {
        const u32x4 a0 = *(const u32x4 *)(xt + xt_operand(li, lh, gg >> 1, gg & 1));
        const u32x4 a1 = *(const u32x4 *)(xt + xt_operand(32 + li, lh, gg >> 1, gg & 1));
        acc0 = mfma32(a0, bq[gg], acc0);
        acc1 = mfma32(a1, bq[gg], acc1);
    }
    float *Sg = a.ws_S + (long)item * kP * kN + wave * 32 + li;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int p = (v >> 2) * 8 + lh * 4 + (v & 3);
        Sg[p * kN] = acc0[v];
        Sg[(32 + p) * kN] = acc1[v];
    }
}

// ------------------------------------------------------------------------
// K3: outputs.  Grid (B * nchunks * H), one workgroup per item (batch,
// chunk, head), in the XCD-aware order.  The output is formed transposed,
// Y^T [P x Q]; wave w owns the column (token) tiles w and 7-w and both
// 32-row feature tiles.
//
// Decay bookkeeping.  R_k is the cumsum at the 16th token of token tile k.
// With
//   x'_s = exp(R_k(s) - cs_s) dt_s x_s      (folded into x in LDS)
//   Q_k  = exp(R_k - R_{k-1}),  R_{-1} = 0   (one scalar per tile)
//   u_l  = exp(cs_l - R_k(l))               (one scalar per output column)
// column tile lt is accumulated tile by tile as a Horner scheme,
//   acc <- h_{c-1} C^T,   acc <- Q_si acc + x'^T_si G^T_(si,lt)   (si = 0..lt),
// and Y^T = u_l acc: the intra-chunk term gets exp(cs_l - cs_s) dt_s and the
// carried-in state exp(cs_l).  G^T tiles enter the MFMA as K0 stored them; the
// only per-element work on them is D x, added as D / dt_l on the diagonal of
// the diagonal tile (u_l v_l = dt_l).  The fast path needs every token within
// 60 of its tile reference in cumsum and consecutive references at most 80
// apart, so that no factor leaves the normal fp32 range; a workgroup whose
// chunk breaks that, or has dt <= 0 or |D/dt| > 1e30, takes the exact path
// instead: x' = x, Q = u = 1, h C^T scaled by exp(cs_l), each G^T element
// scaled by exp(min(cs_l - cs_s, 0)) dt_s, and D added on the diagonal after
// that scaling.
// ------------------------------------------------------------------------
// Exact path: scale the G^T tile (si, lt) held by this lane (column l, rows
// s = 32 si + 8q + 4 lh + r in register 4q + r) by exp(min(cs_l - cs_s, 0)) dt_s.
__device__ __forceinline__ void scale_tile_exact(u32x4 (&gt)[2], const float *cst, const float *dtt, float csl,
                                                 int si, int lh) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int s0 = 32 * si + 8 * q + 4 * lh;
        const float4 cs4 = *(const float4 *)(cst + s0);
        const float4 dt4 = *(const float4 *)(dtt + s0);
        const float f[4] = {exp_fast(fminf(csl - cs4.x, 0.f)) * dt4.x, exp_fast(fminf(csl - cs4.y, 0.f)) * dt4.y,
                            exp_fast(fminf(csl - cs4.z, 0.f)) * dt4.z, exp_fast(fminf(csl - cs4.w, 0.f)) * dt4.w};
        const int i0 = 2 * (q & 1);
        const unsigned w0 = gt[q >> 1][i0], w1 = gt[q >> 1][i0 + 1];
        gt[q >> 1][i0] = pack_bf16(lo_bf16(w0) * f[0], hi_bf16(w0) * f[1]);
        gt[q >> 1][i0 + 1] = pack_bf16(lo_bf16(w1) * f[2], hi_bf16(w1) * f[3]);
    }
}

// Add dl to G^T[l, l] of the diagonal tile.  Lane (li, lh) holds it iff bit 2
// of li equals lh, in register 4(li>>3) + (li&3): word widx of the two u32x4.
__device__ __forceinline__ void add_diagonal(u32x4 (&gt)[2], float dl, int li, int lh) {
    const int widx = ((li >> 4) << 2) | (((li >> 3) & 1) << 1) | ((li & 3) >> 1);
    const bool hi = li & 1;
    unsigned w = gt[0][0];
#pragma unroll
    for (int k = 1; k < 8; ++k) w = (widx == k) ? gt[k >> 2][k & 3] : w;
    const float f = (hi ? hi_bf16(w) : lo_bf16(w)) + ((((li >> 2) & 1) == lh) ? dl : 0.0f);
    const unsigned nb = f32_to_bf16(f);
    const unsigned w2 = hi ? ((w & 0xffffu) | (nb << 16)) : ((w & 0xffff0000u) | nb);
#pragma unroll
    for (int k = 0; k < 8; ++k) gt[k >> 2][k & 3] = (widx == k) ? w2 : gt[k >> 2][k & 3];
}

// Item (b, c, h), h fastest, from xcd_item.  Wave w owns column tiles
// ltA = w and ltB = 7 - w and processes them side by side:
// step k applies token tile k to both (while k <= lt), so the two Horner
// chains of a wave (four accumulators) hide each other's MFMA -> VALU -> MFMA
// latency, and the x'^T operands of token tile k are read once for both.
__global__ __launch_bounds__(kThreads) void chunk_out_mfma(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *xt = smem + K3_XT;
    char *hl = smem + K3_H;
    float *vt = (float *)(smem + K3_V);
    float *ut = (float *)(smem + K3_U);
    float *dtt = (float *)(smem + K3_DT);
    float *wv = (float *)(smem + K3_W);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    const int ltA = wave, ltB = kTiles - 1 - wave;
    const int item = xcd_item(blockIdx.x, gridDim.x);  // grid = one workgroup per item
    const int h = item % a.H, bc = item / a.H;
    const ChunkEntry ch = chunk_at(a, bc);
    const int Qc = ch.Qc;
    if (Qc <= 0) return;  // unused slot of a packed prefill
    const long tok0 = ch.tok0;
    const int g = h / (a.H / a.G);
    const long cg = (long)bc * a.G + g;

    // ---- global loads, all issued before the cumsum: dt, x, h_{c-1}, the C
    // operands of column tile ltA and the first G^T tiles
    // dt first: loads retire in issue order, so the cumsum waits for dt only
    const float dtv = load_dt(a, tok0, Qc, h, tid);
    u32x4 raw[8], hv[4];
    load_x_raw(a, tok0, Qc, h, raw, tid);
    {
        const bf16_t *hg = a.ws_hb + (long)item * kP * kN;
#pragma unroll
        for (int k = 0; k < 4; ++k) hv[k] = *(const u32x4 *)(hg + (tid + k * kThreads) * 8);
    }
    // C operands as K0 packed them: 1 KiB contiguous per load instruction
    const u32x4 *ctp = (const u32x4 *)(a.ws_ct + cg * kBTChunk) + lane;
    auto load_c = [&](int lt, u32x4 (&cop)[8]) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) cop[kk] = ctp[(lt * 8 + kk) * 64];
    };
    u32x4 cop[8];
    load_c(ltA, cop);
    const u32x4 *gtp = (const u32x4 *)(a.ws_gt + cg * kGTChunk) + lane;
    auto tile_ptr = [&](int si, int lt) { return gtp + gt_index(si, lt) * 128; };  // halves at [0] and [64]
    // G^T tiles in flight: steps k, k+1 for column tile ltA (at most 4 steps),
    // k .. k+2 for ltB (5 to 8 steps; one step ahead leaves the L2 latency
    // exposed on the longer chain)
    u32x4 gA[2][2], gB[3][2];
    {
        const u32x4 *pa = tile_ptr(0, ltA);
        const u32x4 *pb = tile_ptr(0, ltB);
        gA[0][0] = pa[0];
        gA[0][1] = pa[64];
        gB[0][0] = pb[0];
        gB[0][1] = pb[64];
        const u32x4 *pb1 = tile_ptr(1, ltB);  // ltB >= 4
        gB[1][0] = pb1[0];
        gB[1][1] = pb1[64];
    }

    // ---- cumsum of dt*A within each 64-token wave (fp32), per-token factors
    const float Af = -expf(a.A_log[h]);
    const float loc = wave_inclusive_sum(dtv * Af);
    const float r15 = __shfl(loc, 15, 64), r47 = __shfl(loc, 47, 64);
    const float e = loc - ((lane & 32) ? r47 : r15);  // cs_t - R_k(t)
    if (lane == 63) {
        wv[3 * wave] = r15;
        wv[3 * wave + 1] = r47;
        wv[3 * wave + 2] = loc;
    }
    __syncthreads();
    // R_k - R_{k-1}: within a wave r47 - r15; across waves total - r47 + r15
    float dq = 0.0f;
    if (tid < kTiles) {
        const int w = tid >> 1;
        dq = (tid & 1) ? wv[3 * w + 1] - wv[3 * w]
                       : (w == 0 ? wv[0] : wv[3 * (w - 1) + 2] - wv[3 * (w - 1) + 1] + wv[3 * w]);
    }
    const float Dh = a.D ? a.D[h] : 0.0f;
    const bool valid = tid < Qc;
    const float dl_fast = dtv > 0.0f ? Dh / dtv : 0.0f;
    const bool ok = (!valid || (fabsf(e) <= 60.0f && dtv > 0.0f && fabsf(dl_fast) <= 1e30f)) &&
                    (tid >= kTiles || fabsf(dq) <= 80.0f);
    const bool exact = __syncthreads_or(!ok);
    if (!exact) {
        vt[tid] = exp_fast(-e) * dtv;
        ut[tid] = exp_fast(e);
    } else {
        float pre = 0.0f;
        for (int w = 0; w < wave; ++w) pre += wv[3 * w + 2];
        vt[tid] = pre + loc;  // cs
        ut[tid] = 1.0f;
    }
    dtt[tid] = dtv;
    if (tid < kTiles) wv[16 + tid] = exact ? 1.0f : exp_fast(dq);
    __syncthreads();

    // ---- x' into LDS (tokens in K order), h_{c-1} into LDS
    {
        float sc[8];
        if (!exact) {
            const float4 s0 = *(const float4 *)(vt + (tid >> 3) * 8);
            const float4 s1 = *(const float4 *)(vt + (tid >> 3) * 8 + 4);
            sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
            sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) sc[r] = 1.0f;
        }
        store_xt_korder(raw, sc, xt, tid);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int idx = tid + k * kThreads;
            const int r = idx >> 4, ch = idx & 15;
            *(u32x4 *)(hl + r * 256 + ((ch ^ (r & 15)) << 4)) = hv[k];
        }
    }
    __syncthreads();

    const float *cst = vt;  // cs on the exact path
    const int hrow = li * 256;
    const int hsw = li & 15;

    // carried-in state: acc = h_{c-1} C^T (K = N) for both column tiles
    auto state_term = [&](const u32x4 (&cp)[8], f32x16 &y0, f32x16 &y1) {
        y0 = f32x16{};
        y1 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int off = hrow + (((2 * kk + lh) ^ hsw) << 4);
            const u32x4 a0 = *(const u32x4 *)(hl + off);
            const u32x4 a1 = *(const u32x4 *)(hl + off + 32 * 256);
            y0 = mfma32(a0, cp[kk], y0);
            y1 = mfma32(a1, cp[kk], y1);
        }
    };
    f32x16 yA0, yA1, yB0, yB1;
    state_term(cop, yA0, yA1);
    load_c(ltB, cop);
    state_term(cop, yB0, yB1);
    const int lA = ltA * 32 + li, lB = ltB * 32 + li;
    if (exact) {
        const float eA = exp_fast(cst[lA]), eB = exp_fast(cst[lB]);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            yA0[v] *= eA;
            yA1[v] *= eA;
            yB0[v] *= eB;
            yB1[v] *= eB;
        }
    }
    const float dlA = exact ? Dh : (dtt[lA] > 0.0f ? Dh / dtt[lA] : 0.0f);
    const float dlB = exact ? Dh : (dtt[lB] > 0.0f ? Dh / dtt[lB] : 0.0f);
    const float cslA = exact ? cst[lA] : 0.0f, cslB = exact ? cst[lB] : 0.0f;

    // Y^T = u_l acc, staged through LDS as bf16 rows [l][P] (144-byte stride:
    // 2-way bank conflicts at most) so that each global store instruction
    // writes eight whole 128-byte rows of y.
    auto stage_tile = [&](char *st, int l, const f32x16 &y0, const f32x16 &y1) {
        const float u = ut[l];
        char *row = st + li * kYRow + 8 * lh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *(u32x2 *)(row + 16 * q) = u32x2{pack_bf16(y0[4 * q] * u, y0[4 * q + 1] * u),
                                             pack_bf16(y0[4 * q + 2] * u, y0[4 * q + 3] * u)};
            *(u32x2 *)(row + 64 + 16 * q) = u32x2{pack_bf16(y1[4 * q] * u, y1[4 * q + 1] * u),
                                                  pack_bf16(y1[4 * q + 2] * u, y1[4 * q + 3] * u)};
        }
    };
    auto store_tile = [&](const char *st, int lt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + (lane >> 3);
            const u32x4 v = *(const u32x4 *)(st + r * kYRow + 16 * (lane & 7));
            const int l = lt * 32 + r;
            if (l < Qc) *(u32x4 *)((bf16_t *)a.y + ((tok0 + l) * a.H + h) * kP + 8 * (lane & 7)) = v;
        }
    };

    // ---- intra-chunk term: step k applies token tile k to both column tiles
#pragma unroll
    for (int k = 0; k < kTiles; ++k) {
        if (k <= ltB) {
            if (k + 2 <= ltB) {
                const u32x4 *pb = tile_ptr(k + 2, ltB);
                gB[(k + 2) % 3][0] = pb[0];
                gB[(k + 2) % 3][1] = pb[64];
            }
            if (k + 1 <= ltA) {
                const u32x4 *pa = tile_ptr(k + 1, ltA);
                gA[(k + 1) & 1][0] = pa[0];
                gA[(k + 1) & 1][1] = pa[64];
            }
            u32x4 xa[2][2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                xa[0][hf] = *(const u32x4 *)(xt + xt_operand(li, lh, k, hf));
                xa[1][hf] = *(const u32x4 *)(xt + xt_operand(32 + li, lh, k, hf));
            }
            const float qv = wv[16 + k];
            if (k <= ltA) {
                u32x4 g2[2] = {gA[k & 1][0], gA[k & 1][1]};
                if (exact) scale_tile_exact(g2, cst, dtt, cslA, k, lh);
                if (k == ltA) add_diagonal(g2, dlA, li, lh);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    yA0[v] *= qv;
                    yA1[v] *= qv;
                }
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    yA0 = mfma32(xa[0][hf], g2[hf], yA0);
                    yA1 = mfma32(xa[1][hf], g2[hf], yA1);
                }
            }
            {
                u32x4 g2[2] = {gB[k % 3][0], gB[k % 3][1]};
                if (exact) scale_tile_exact(g2, cst, dtt, cslB, k, lh);
                if (k == ltB) add_diagonal(g2, dlB, li, lh);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    yB0[v] *= qv;
                    yB1[v] *= qv;
                }
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    yB0 = mfma32(xa[0][hf], g2[hf], yB0);
                    yB1 = mfma32(xa[1][hf], g2[hf], yB1);
                }
            }
        }
    }

    // ---- outputs: every wave is done with x'^T and h; reuse their LDS
    __syncthreads();
    char *st = smem + wave * 2 * 32 * kYRow;
    stage_tile(st, lA, yA0, yA1);
    stage_tile(st + 32 * kYRow, lB, yB0, yB1);
    store_tile(st, ltA);
    store_tile(st + 32 * kYRow, ltB);
}

// ------------------------------------------------------------------------
// K2: the state pass.  Reads S_c (fp32), keeps h in fp32, writes the
// carried-in state h_{c-1} as bf16 (the MFMA operand of C h) and the final
// state in fp32.  h + (dm1 * h + S) rounds the state once per chunk.
// ------------------------------------------------------------------------
// Blocks past the state blocks pack C for K3: block (b, c, g, q) writes token
// tiles 2q, 2q+1 as [lt][kk][lane] 16 bytes = C[32 lt + li][16 kk + 8 lh ..
// + 8] (tokens past the end as zero).
__device__ __forceinline__ void pack_c(const PrefillArgs &a, long blk) {
    const int q = (int)(blk % (kTiles / 2));
    const long cg = blk / (kTiles / 2);  // slot * G + g
    const int g = (int)(cg % a.G);
    const ChunkEntry ch = chunk_at(a, cg / a.G);
    const int Qc = ch.Qc;
    if (Qc <= 0) return;  // unused slot of a packed prefill
    const unsigned rs = (unsigned)a.G * kN * 2;
    const __amdgpu_buffer_rsrc_t crs =
        make_rsrc((const bf16_t *)a.Cm + ((long)ch.tok0 * a.G + g) * kN, (unsigned)(Qc - 1) * rs + kN * 2);
    u32x4 *ct = (u32x4 *)(a.ws_ct + cg * kBTChunk);
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = threadIdx.x + k * kThreads;
        const int lt = 2 * q + (idx >> 9), kk = (idx >> 6) & 7, ln = idx & 63;
        v[k] = buf_load16(crs, (unsigned)(lt * 32 + (ln & 31)) * rs + 32 * kk + 16 * (ln >> 5));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) ct[2 * q * 8 * 64 + threadIdx.x + k * kThreads] = v[k];
}

__global__ __launch_bounds__(kThreads) void state_pass_bf16(PrefillArgs a, long total, long state_blocks) {
    if ((long)blockIdx.x >= state_blocks) {
        pack_c(a, (long)blockIdx.x - state_blocks);
        return;
    }
    const long e = (long)blockIdx.x * kThreads + threadIdx.x;  // float4 index
    if (e >= total) return;
    const long PN4 = (long)kP * kN / 4;
    const long bh = e / PN4;
    const long pn = e - bh * PN4;
    const int h = (int)(bh % a.H);
    const SeqEntry sq = seq_chunks(a, bh / a.H);
    float4 hv = a.init_state ? ((const float4 *)a.init_state)[bh * PN4 + pn] : make_float4(0.f, 0.f, 0.f, 0.f);
    const int nch = sq.n;
    constexpr int kB = 8;
    for (int c0 = 0; c0 < nch; c0 += kB) {
        float4 sv[kB];
        float dv[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            if (c0 + j < nch) {
                const long hc = ((long)sq.f0 + c0 + j) * a.H + h;
                sv[j] = ((const float4 *)(a.ws_S + hc * kP * kN))[pn];
                dv[j] = a.ws_dec[hc];
            }
        }
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            if (c0 + j < nch) {
                const long hc = ((long)sq.f0 + c0 + j) * a.H + h;
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



}  // namespace

long prefill_mfma_gt_elems_per_chunk() { return kGTChunk; }
long prefill_mfma_bt_elems_per_chunk() { return kBTChunk; }

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t s) {
    const int gridB = a.chunks ? 1 : a.B;  // packed sequences: nchunks slots in all
    const long nitems = (long)gridB * a.nchunks * a.H;
    if (nitems > 0x7fffffffL || (long)a.G * kK0Blocks > 65535 || a.nchunks > 0x7fffffff) return hipErrorInvalidConfiguration;
    stage_begin();
    hipError_t e = launch_stage("chunk_pack_mfma", chunk_pack_mfma, dim3(a.nchunks, kK0Blocks * a.G, gridB),
                                dim3(kThreads), 0, s, a);
    if (e != hipSuccess) return e;
    e = launch_stage("chunk_state_mfma", chunk_state_mfma, dim3((unsigned)nitems), dim3(kThreads), K1_LDS, s, a);
    if (e != hipSuccess) return e;
    const long total = (long)a.B * a.H * (kP * kN / 4);
    const long state_blocks = (total + kThreads - 1) / kThreads;
    const long pack_blocks = (long)gridB * a.nchunks * a.G * (kTiles / 2);
    if (state_blocks + pack_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    e = launch_stage("state_pass_bf16", state_pass_bf16, dim3((unsigned)(state_blocks + pack_blocks)),
                     dim3(kThreads), 0, s, a, total, state_blocks);
    if (e != hipSuccess) return e;
    return launch_stage("chunk_out_mfma", chunk_out_mfma, dim3((unsigned)nitems), dim3(kThreads), K3_LDS, s, a);
}

}  // namespace ssd
