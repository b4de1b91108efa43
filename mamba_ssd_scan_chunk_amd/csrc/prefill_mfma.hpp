// prefill_mfma.hpp -- device helpers of the bf16 MFMA prefill kernels
// (gfx950; P = 64, N = 128, 256-token chunks): operand types, loads, the x
// chunk transposition into LDS, the in-chunk decay bookkeeping and the
// output phase.  Included by prefill_mfma.hip (the four-kernel form) and
// prefill_chain.hip (the chained single-pass form); the scheme itself is
// described at the top of prefill_mfma.hip.
#pragma once

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

// Cache-policy operand of the buffer builtins marking an access non-temporal.
constexpr int kCacheNonTemporal = 2;

// x (and so y) larger than the Infinity Cache (256 MB on MI355X) cannot stay
// cached for the operation after the prefill anyway: the kernels then read x
// and write y with non-temporal accesses, so that they do not push the
// chunks' shared operand tiles out of the L2s.
constexpr double kStreamBytes = 256.0 * (1 << 20);
__host__ __device__ inline bool prefill_streams(const PrefillArgs &a) {
    return (double)a.T * a.H * kP * 2 >= kStreamBytes;  // T token rows: B L, or the packed total
}

// Packed sequences where the chunk table chooses the form: whether the
// chained form runs the call, so that the four-kernel form's workgroups exit
// at once (one scalar load, before any store of the kernel).
__device__ __forceinline__ bool chained_runs(const PrefillArgs &a) {
    return a.ws_items && a.ws_items[kItemForm] == 1u;
}

// Buffer resource over `bytes` bytes from p: loads at or past the end
// return zeros, which is how the ragged last chunk reads its missing tokens.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Non-temporal form (the line is a candidate for early eviction): for data
// read once that should not push reused operand tiles out of the L2.
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCacheNonTemporal));
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Load the x chunk of head h ([Q tokens][P] bf16, row stride H*P) whose
// first token is row tok0: thread t owns the 8x8 block of tokens 8*(t/8)..
// and features 8*(t%8)..; tokens at or past Qc read as zero.  kNt: with
// non-temporal loads.
template <bool kNt = false>
__device__ __forceinline__ void load_x_raw(const PrefillArgs &a, long tok0, int Qc, int h, u32x4 (&raw)[8], int t) {
    const int sb = t >> 3, pb = t & 7;
    const unsigned rs = (unsigned)a.H * kP * 2;  // row stride in bytes
    const bf16_t *x0 = (const bf16_t *)a.x + (tok0 * a.H + h) * kP;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(x0, (unsigned)(Qc - 1) * rs + kP * 2);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const unsigned off = (unsigned)(sb * 8 + k) * rs + pb * 16;
        raw[k] = kNt ? buf_load16_nt(r, off) : buf_load16(r, off);
    }
}

// What the chunk's decay tables are made of: the step of token t as stored
// (0 at or past Qc), A_log[h], D[h] and the step bias of head h (0 without
// one).  An item requests these before any other global load: vector loads
// retire in issue order, so the cumsum, which needs all four, then waits for
// them alone while x and the operand tiles are still on their way (a per-head
// value loaded after x makes the cumsum wait for x as well).  No arithmetic
// is done on them here: that too would wait, and delay the loads after it.
struct DecayIn {
    float dt, alog, D, bias;
};
__device__ __forceinline__ DecayIn load_decay_in(const PrefillArgs &a, long tok0, int Qc, int h, int t) {
    DecayIn d;
    const float *d0 = a.dt + tok0 * a.H + h;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(d0, (unsigned)((Qc - 1) * a.H + 1) * 4);
    d.dt = buf_load_f32(r, (unsigned)t * a.H * 4);
    d.alog = a.A_log[h];
    d.D = a.D ? a.D[h] : 0.0f;
    d.bias = a.dtp.dt_raw && a.dtp.dt_bias ? a.dtp.dt_bias[h] : 0.0f;
    return d;
}
// The step of token t the scan uses: the stored value, or with a raw step
// softplus(raw + bias) clipped to [dt_min, dt_max] (0 at or past Qc).
__device__ __forceinline__ float step_of(const PrefillArgs &a, const DecayIn &d, int Qc, int t) {
    if (!a.dtp.dt_raw) return d.dt;
    return t < Qc ? dt_softplus_clamp(d.dt + d.bias, a.dtp.dt_min, a.dtp.dt_max) : 0.0f;
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

// ------------------------------------------------------------------------
// In-chunk decay bookkeeping of one item (the output kernel and the chained
// kernel).  R_k is the cumsum of dt*A at the 16th token of token tile k.
// With
//   x'_s = exp(R_k(s) - cs_s) dt_s x_s      (folded into x in LDS)
//   Q_k  = exp(R_k - R_{k-1}),  R_{-1} = 0   (one scalar per tile)
//   u_l  = exp(cs_l - R_k(l))               (one scalar per output column)
// the masked product term of column l is u_l sum_k (prod of Q over the tiles
// after k up to l's tile) x'^T_k G^T_k.  The fast path needs every token
// within 60 of its tile reference in cumsum and consecutive references at
// most 80 apart, so that no factor leaves the normal fp32 range; a chunk that
// breaks that, or has dt <= 0 or |D/dt| > 1e30, takes the exact path: x' = x,
// Q = u = 1, and cs itself in vt for per-element factors.
//
// Thread t owns token t.  Fills vt (x' scale, or cs on the exact path), ut
// (u_l), dtt (dt) and wv[16 + k] (Q_k, 1 on the exact path); wv[3w ..]
// keep each wave's cumsum at its tokens 15, 47 and 63.  Returns whether the
// chunk takes the exact path; *total receives the chunk's sum of dt*A.
// Contains two workgroup barriers.
// ------------------------------------------------------------------------
constexpr int K3_WQ = 16;  // wv[K3_WQ + k] = Q_k

__device__ __forceinline__ bool chunk_decay(float dtv, float Af, float Dh, int Qc, float *vt, float *ut, float *dtt,
                                            float *wv, int tid, int lane, int wave, float *total) {
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
    const bool valid = tid < Qc;
    const float dl_fast = dtv > 0.0f ? Dh / dtv : 0.0f;
    const bool ok = (!valid || (fabsf(e) <= 60.0f && dtv > 0.0f && fabsf(dl_fast) <= 1e30f)) &&
                    (tid >= kTiles || fabsf(dq) <= 80.0f);
    const bool exact = __syncthreads_or(!ok);
    float pre = 0.0f, tot = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        pre += w < wave ? wv[3 * w + 2] : 0.0f;
        tot += wv[3 * w + 2];
    }
    if (!exact) {
        vt[tid] = exp_fast(-e) * dtv;
        ut[tid] = exp_fast(e);
    } else {
        vt[tid] = pre + loc;  // cs
        ut[tid] = 1.0f;
    }
    dtt[tid] = dtv;
    if (tid < kTiles) wv[K3_WQ + tid] = exact ? 1.0f : exp_fast(dq);
    *total = tot;
    __syncthreads();
    return exact;
}

// The per-token scales of this thread's 8 tokens (8 * (t / 8) ..) from
// vt: the x' scale on the fast path, 1 on the exact path.
__device__ __forceinline__ void x_scales(const float *vt, bool exact, int tid, float (&sc)[8]) {
    if (!exact) {
        const float4 s0 = *(const float4 *)(vt + (tid >> 3) * 8);
        const float4 s1 = *(const float4 *)(vt + (tid >> 3) * 8 + 4);
        sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
        sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) sc[r] = 1.0f;
    }
}

// ------------------------------------------------------------------------
// Output phase of one item (the output kernel and the chained kernel), after
// x'^T and h_{c-1} (bf16, [P][N], 16-byte chunks XOR-swizzled by row) are
// in LDS and chunk_decay has run.  The output is formed transposed, Y^T
// [P x Q]; wave w owns the column (token) tiles ltA = w and ltB = 7 - w and
// both 32-row feature tiles.  Column tile lt is accumulated tile by tile as
// a Horner scheme,
//   acc <- h_{c-1} C^T,   acc <- Q_si acc + x'^T_si G^T_(si,lt)   (si = 0..lt),
// and Y^T = u_l acc: the intra-chunk term gets exp(cs_l - cs_s) dt_s and the
// carried-in state exp(cs_l).  G^T tiles enter the MFMA as the pack kernel
// stored them; the only per-element work on them is D x, added as D / dt_l
// on the diagonal of the diagonal tile (u_l v_l = dt_l); on the exact path
// each G^T element is scaled by exp(min(cs_l - cs_s, 0)) dt_s, h C^T by
// exp(cs_l), and D added on the diagonal after that scaling.
// Step k applies token tile k to both column tiles (while k <= lt), so the
// two Horner chains of a wave (four accumulators) hide each other's MFMA ->
// VALU -> MFMA latency, and the x'^T operands of token tile k are read once
// for both.  `cop` and `copB` hold the C operands of column tiles ltA and
// ltB, already requested.
// ------------------------------------------------------------------------
struct OutItem {
    const u32x4 *ctp;  // C operands of the chunk and group (this lane's)
    __amdgpu_buffer_rsrc_t gtr;  // G^T tiles of the chunk and group
    unsigned lane16;             // this lane's byte offset in a tile
    long tok0;
    int Qc, h;
    float Dh;
    bool exact;
};

// The G^T tiles of a chunk and group: per tile two 1 KiB halves of 16 bytes
// per lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gt_rsrc(const PrefillArgs &a, long cg) {
    return make_rsrc(a.ws_gt + cg * kGTChunk, (unsigned)(kGTChunk * 2));
}
// G^T tile (si, lt) into g.  With `use` false the two loads are still issued,
// past the end of the tiles: they return zeros without a memory access.  A
// loop that requests tiles under conditions then issues the same loads in the
// same order on every path, and as vector loads retire in issue order, each
// step waits for its own tiles only, not for the ones requested after them.
__device__ __forceinline__ void load_gt(const OutItem &it, int si, int lt, bool use, u32x4 (&g)[2]) {
    const unsigned off = use ? (unsigned)gt_index(si, lt) * 2048u + it.lane16 : 0x40000000u;
    g[0] = buf_load16(it.gtr, off);
    g[1] = buf_load16(it.gtr, off + 1024u);
}
__device__ __forceinline__ void load_c_tile(const OutItem &it, int lt, u32x4 (&cop)[8]) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) cop[kk] = it.ctp[(lt * 8 + kk) * 64];
}
// Requests of the first operands of wave `wave`: the C operands of its
// column tiles ltA and ltB.
__device__ __forceinline__ void out_first_loads(const OutItem &it, int wave, u32x4 (&cop)[8], u32x4 (&copB)[8]) {
    load_c_tile(it, wave, cop);
    load_c_tile(it, kTiles - 1 - wave, copB);
}

// kNtY: the y rows are written with non-temporal stores.
// kIssueAll: every G^T request of the loops is issued on every path (empty
// where not needed, see load_gt); otherwise only the needed ones are.  The
// output kernel runs faster with the former (B = 1, L = 4096 2.7B-shaped
// layer: 64.3 -> 63.4 us per call), the chained kernel with the latter
// (B = 8, L = 16384: 1271 against 1285 us).
template <bool kNtY, bool kIssueAll>
__device__ __forceinline__ void out_tiles(const PrefillArgs &a, const OutItem &it, char *smem, u32x4 (&cop)[8],
                                          u32x4 (&copB)[8], int tid) {
    const char *xt = smem + K3_XT;
    const char *hl = smem + K3_H;
    const float *vt = (const float *)(smem + K3_V);
    const float *ut = (const float *)(smem + K3_U);
    const float *dtt = (const float *)(smem + K3_DT);
    const float *wv = (const float *)(smem + K3_W);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    const int ltA = wave, ltB = kTiles - 1 - wave;
    // A short last chunk: column tiles past its last token are neither
    // formed nor stored (a wave whose tile ltB is past it forms ltA alone;
    // token tiles past it add only zeros to the tiles that are formed, which
    // run every Horner step as in a full chunk)
    const int ntl = (it.Qc + 31) >> 5;
    const bool doA = ltA < ntl, doB = ltB < ntl;  // doB implies doA
    const bool exact = it.exact;
    const float *cst = vt;  // cs on the exact path
    const int hrow = li * 256;
    const int hsw = li & 15;

    // carried-in state: acc = h_{c-1} C^T (K = N) for both feature tiles of
    // column tile ltA, and of ltB as well when `both` (each h_{c-1} operand
    // is read once for the two column tiles).  The G^T tiles of the first
    // steps (0 for ltA, 0 and 1 for ltB) are requested during it.
    // ltB's tiles are requested DB steps ahead
    constexpr int DB = kIssueAll ? 2 : 1;
    u32x4 gA[2][2], gB[DB + 1][2];
    auto want = [&](int si, int lt, bool use, u32x4 (&g)[2]) {
        if (kIssueAll)
            load_gt(it, si, lt, use, g);
        else if (use)
            load_gt(it, si, lt, true, g);
    };
    auto state_term = [&](bool both, f32x16 &y0, f32x16 &y1, f32x16 &z0, f32x16 &z1) {
        y0 = f32x16{};
        y1 = f32x16{};
        z0 = f32x16{};
        z1 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            if (kk == 4) {
                want(0, ltA, true, gA[0]);
                want(0, ltB, both, gB[0]);
                if (DB == 2) want(1, ltB, both, gB[1 % (DB + 1)]);
            }
            const int off = hrow + (((2 * kk + lh) ^ hsw) << 4);
            const u32x4 a0 = *(const u32x4 *)(hl + off);
            const u32x4 a1 = *(const u32x4 *)(hl + off + 32 * 256);
            y0 = mfma32(a0, cop[kk], y0);
            y1 = mfma32(a1, cop[kk], y1);
            if (both) {
                z0 = mfma32(a0, copB[kk], z0);
                z1 = mfma32(a1, copB[kk], z1);
            }
        }
    };
    const int lA = ltA * 32 + li, lB = ltB * 32 + li;
    const float Dh = it.Dh;
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
            if (l < it.Qc) {
                u32x4 *dst = (u32x4 *)((bf16_t *)a.y + ((it.tok0 + l) * a.H + it.h) * kP + 8 * (lane & 7));
                if (kNtY)
                    __builtin_nontemporal_store(v, dst);
                else
                    *dst = v;
            }
        }
    };

    f32x16 yA0 = {}, yA1 = {}, yB0 = {}, yB1 = {};
    if (doB) {
        state_term(true, yA0, yA1, yB0, yB1);
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
        // ---- intra-chunk term: step k applies token tile k to both column tiles
#pragma unroll
        for (int k = 0; k < kTiles; ++k) {
            // G^T tiles DB steps (ltB) and one step (ltA) ahead
            want(k + DB, ltB, k + DB <= ltB, gB[(k + DB) % (DB + 1)]);
            want(k + 1, ltA, k + 1 <= ltA, gA[(k + 1) & 1]);
            if (k <= ltB) {
                u32x4 xa[2][2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    xa[0][hf] = *(const u32x4 *)(xt + xt_operand(li, lh, k, hf));
                    xa[1][hf] = *(const u32x4 *)(xt + xt_operand(32 + li, lh, k, hf));
                }
                const float qv = wv[K3_WQ + k];
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
                    u32x4 g2[2] = {gB[k % (DB + 1)][0], gB[k % (DB + 1)][1]};
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
    } else if (doA) {
        // column tile ltA alone (its tile ltB is past the chunk's last token)
        state_term(false, yA0, yA1, yB0, yB1);
        if (exact) {
            const float eA = exp_fast(cst[lA]);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                yA0[v] *= eA;
                yA1[v] *= eA;
            }
        }
#pragma unroll
        for (int k = 0; k < kTiles; ++k) {
            want(k + 1, ltA, k + 1 <= ltA, gA[(k + 1) & 1]);
            if (k <= ltA) {
                u32x4 xa[2][2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    xa[0][hf] = *(const u32x4 *)(xt + xt_operand(li, lh, k, hf));
                    xa[1][hf] = *(const u32x4 *)(xt + xt_operand(32 + li, lh, k, hf));
                }
                const float qv = wv[K3_WQ + k];
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
        }
    }

    // ---- outputs: every wave is done with x'^T and h; reuse their LDS
    __syncthreads();
    char *st = smem + wave * 2 * 32 * kYRow;
    if (doA) stage_tile(st, lA, yA0, yA1);
    if (doB) stage_tile(st + 32 * kYRow, lB, yB0, yB1);
    if (doA) store_tile(st, ltA);
    if (doB) store_tile(st + 32 * kYRow, ltB);
}

}  // namespace
}  // namespace ssd
