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

#include "prefill_mfma.hpp"

namespace ssd {
namespace {

constexpr int kCBlocks = kTiles / 2;  // C packing: two token tiles per workgroup
constexpr long kDualStateBlocks = 4096;  // state-pass grid after the chained launch of packed sequences

// C in the order of the output kernel's operand: block (b, c, g, q) writes
// token tiles 2q, 2q+1 as [lt][kk][lane] 16 bytes = C[32 lt + li][16 kk +
// 8 lh .. + 8] (tokens past the end as zero).
__device__ __forceinline__ void pack_c(const PrefillArgs &a, long blk) {
    const int q = (int)(blk % kCBlocks);
    const long cg = blk / kCBlocks;  // slot * G + g
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

// ------------------------------------------------------------------------
// K0: per (batch, chunk, group), shared by every head of the group.  Grid
// (nchunks, kb * G, B), kb = 13 (four-kernel form) or 17 (chained form).
// Blocks y % kb < 9 form the 36 causal 32x32 tiles of G^T = B C^T, one per
// wave, masked (s > l -> 0) and stored as bf16 in the exact register order
// of the MFMA accumulator; blocks 9 .. 12 write the 32-column slice
// y % kb - 9 of B in the order of K1's MFMA B operand; blocks 13 .. 16 (the
// chained form; the four-kernel form has the state pass do it) write C in
// the order of the output kernel's operand.  The operands are read straight
// from L2; tokens past the end read as zero.  With `ctl` (the chained
// form's hand-off control block) the first chunk's blocks clear it.
// ------------------------------------------------------------------------
constexpr int kK0Tiles = kGTiles / 4;         // workgroups forming G^T tiles
constexpr int kK0Blocks = kK0Tiles + kN / 32;  // plus one per 32 columns of B

template <bool kPacked>
__global__ __launch_bounds__(kThreads) void chunk_pack_mfma(PrefillArgs a, int kb, int *ctl) {
    __shared__ __attribute__((aligned(16))) char bl[kQ * 64];  // B[:, 32 columns] as [token][32] bf16
    const long f = (long)blockIdx.z * a.nchunks + blockIdx.x;
    const int part = blockIdx.y % kb, g = blockIdx.y / kb;
    if (ctl && blockIdx.y == 0) {
        // hand-off control block of the chained form: ticket and error word
        // (once), then the published-chunk counter of each (b, h) chain: the
        // H of batch element z by block (0, 0, z); for packed sequences (one
        // grid row) the B * H counters spread over the slots' first blocks
        if (blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x < kChainCtlHeader) ctl[threadIdx.x] = 0;
        long lo = 0, hi = 0;
        if (a.chunks) {
            const long n = (long)a.B * a.H, per = (n + a.nchunks - 1) / a.nchunks;
            lo = min(n, (long)blockIdx.x * per);
            hi = min(n, lo + per);
        } else if (blockIdx.x == 0) {
            lo = (long)blockIdx.z * a.H;
            hi = lo + a.H;
        }
        for (long j = lo + threadIdx.x; j < hi; j += kThreads) ctl[kChainCtlHeader + j] = 0;
    }
    const ChunkEntry ch = chunk_at(a, f);
    const int Qc = ch.Qc;
    if (Qc <= 0) return;  // unused slot of a packed prefill
    if (part >= kK0Blocks) {
        pack_c(a, (f * a.G + g) * kCBlocks + (part - kK0Blocks));
        return;
    }
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
        // packed sequences (most chunks short in a batch of short prompts):
        // a column tile past the chunk's last token is never read
        if (kPacked && lt * 32 >= Qc) return;
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

template <bool kNt>
__global__ __launch_bounds__(kThreads) void chunk_state_mfma(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *xt = smem + K1_XT;
    float *vt = (float *)(smem + K1_V);
    float *wv = (float *)(smem + K1_W);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    if (chained_runs(a)) return;
    const int item = xcd_item(blockIdx.x, gridDim.x);  // grid = one workgroup per item
    const int h = item % a.H, bc = item / a.H;
    const ChunkEntry ch = chunk_at(a, bc);
    const int Qc = ch.Qc;
    if (Qc <= 0) return;  // unused slot of a packed prefill
    const long tok0 = ch.tok0;
    const int g = h / (a.H / a.G);
    const long cg = (long)bc * a.G + g;

    // every global load of this workgroup is issued before the cumsum, the
    // step and A_log first: loads retire in issue order, so the cumsum waits
    // for those only
    const DecayIn din = load_decay_in(a, tok0, Qc, h, tid);
    u32x4 raw[8];
    load_x_raw<kNt>(a, tok0, Qc, h, raw, tid);
    const u32x4 *bt = (const u32x4 *)(a.ws_bt + cg * kBTChunk) + (wave * (kQ / 16)) * 64 + lane;
    u32x4 bq[kQ / 16];
#pragma unroll
    for (int gg = 0; gg < kQ / 16; ++gg) bq[gg] = bt[gg * 64];

    // cumsum within each 64-token wave (fp32); cs_last - cs_t from the wave totals
    const float dtv = step_of(a, din, Qc, tid);
    const float loc = wave_inclusive_sum(dtv * -expf(din.alog));
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
// chunk, head) in the XCD-aware order, h fastest: the decay bookkeeping of
// chunk_decay, x' and h_{c-1} into LDS, then out_tiles.
// ------------------------------------------------------------------------
template <bool kNt>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void chunk_out_mfma(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *xt = smem + K3_XT;
    char *hl = smem + K3_H;
    float *vt = (float *)(smem + K3_V);
    float *ut = (float *)(smem + K3_U);
    float *dtt = (float *)(smem + K3_DT);
    float *wv = (float *)(smem + K3_W);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (chained_runs(a)) return;
    const int item = xcd_item(blockIdx.x, gridDim.x);  // grid = one workgroup per item
    const int h = item % a.H, bc = item / a.H;
    const ChunkEntry ch = chunk_at(a, bc);
    const int Qc = ch.Qc;
    if (Qc <= 0) return;  // unused slot of a packed prefill
    const long tok0 = ch.tok0;
    const int g = h / (a.H / a.G);
    const long cg = (long)bc * a.G + g;

    // ---- global loads, all issued before the cumsum: the step, A_log and D,
    // x, h_{c-1} and the C operands of both column tiles.
    // The step, A_log and D first: loads retire in issue order, so the cumsum
    // waits for those only
    const DecayIn din = load_decay_in(a, tok0, Qc, h, tid);
    u32x4 raw[8], hv[4];
    load_x_raw<kNt>(a, tok0, Qc, h, raw, tid);
    {
        const bf16_t *hg = a.ws_hb + (long)item * kP * kN;
#pragma unroll
        for (int k = 0; k < 4; ++k) hv[k] = *(const u32x4 *)(hg + (tid + k * kThreads) * 8);
    }
    OutItem it;
    it.ctp = (const u32x4 *)(a.ws_ct + cg * kBTChunk) + lane;
    it.gtr = gt_rsrc(a, cg);
    it.lane16 = (unsigned)lane * 16u;
    it.tok0 = tok0;
    it.Qc = Qc;
    it.h = h;
    it.Dh = din.D;
    u32x4 cop[8], copB[8];
    out_first_loads(it, wave, cop, copB);

    float total;
    const float dtv = step_of(a, din, Qc, tid);
    it.exact = chunk_decay(dtv, -expf(din.alog), it.Dh, Qc, vt, ut, dtt, wv, tid, lane, wave, &total);

    // ---- x' into LDS (tokens in K order), h_{c-1} into LDS
    {
        float sc[8];
        x_scales(vt, it.exact, tid, sc);
        store_xt_korder(raw, sc, xt, tid);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int idx = tid + k * kThreads;
            const int r = idx >> 4, ch = idx & 15;
            *(u32x4 *)(hl + r * 256 + ((ch ^ (r & 15)) << 4)) = hv[k];
        }
    }
    __syncthreads();
    out_tiles<kNt, true>(a, it, smem, cop, copB, tid);
}

// ------------------------------------------------------------------------
// K2: the state pass.  Reads S_c (fp32), keeps h in fp32, writes the
// carried-in state h_{c-1} as bf16 (the MFMA operand of C h) and the final
// state in fp32.  h + (dm1 * h + S) rounds the state once per chunk.  Blocks
// past the state blocks pack C for K3 (pack_c).
// ------------------------------------------------------------------------
// The chunks of one (b, h) chain for state float4 e (of B * H * P * N / 4).
__device__ __forceinline__ void state_walk(const PrefillArgs &a, long e) {
    const long PN4 = (long)kP * kN / 4;
    const long bh = e / PN4;
    const long pn = e - bh * PN4;
    const int h = (int)(bh % a.H);
    const SeqEntry sq = seq_chunks(a, bh / a.H);
    float4 hv = a.init_state ? ((const float4 *)a.init_state)[bh * PN4 + pn] : make_float4(0.f, 0.f, 0.f, 0.f);
    const int nch = sq.n;
    // 16 chunks of states and decays requested at once (a 4096-token
    // sequence in one round trip), with the same loads on every path (past
    // the last chunk the last chunk again, not used): vector loads retire in
    // issue order, so each chunk's update waits for its own operands only
    constexpr int kB = 16;
    for (int c0 = 0; c0 < nch; c0 += kB) {
        float4 sv[kB];
        float dv[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const long hc = ((long)sq.f0 + min(c0 + j, nch - 1)) * a.H + h;
            sv[j] = ((const float4 *)(a.ws_S + hc * kP * kN))[pn];
            dv[j] = a.ws_dec[hc];
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

__global__ __launch_bounds__(kThreads) void state_pass_bf16(PrefillArgs a, long total, long state_blocks) {
    if (chained_runs(a)) return;
    if ((long)blockIdx.x >= state_blocks) {
        pack_c(a, (long)blockIdx.x - state_blocks);
        return;
    }
    // one float4 of state per thread; a grid capped below total / kThreads
    // (the call of packed sequences that launches both forms) loops
    for (long e = (long)blockIdx.x * kThreads + threadIdx.x; e < total; e += state_blocks * kThreads)
        state_walk(a, e);
}




}  // namespace

long prefill_mfma_gt_elems_per_chunk() { return kGTChunk; }
long prefill_mfma_bt_elems_per_chunk() { return kBTChunk; }

hipError_t launch_chunk_pack(const PrefillArgs &a, bool with_c, int *ctl, hipStream_t s) {
    const int gridB = a.chunks ? 1 : a.B;  // packed sequences: nchunks slots in all
    const int kb = kK0Blocks + (with_c ? kCBlocks : 0);
    if ((long)a.G * kb > 65535 || a.nchunks > 0x7fffffff) return hipErrorInvalidConfiguration;
    return launch_stage("chunk_pack_mfma", a.chunks ? chunk_pack_mfma<true> : chunk_pack_mfma<false>,
                        dim3(a.nchunks, kb * a.G, gridB), dim3(kThreads), 0, s,
                        a, kb, ctl);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t s, bool after_chain) {
    const int gridB = a.chunks ? 1 : a.B;  // packed sequences: nchunks slots in all
    const long nitems = (long)gridB * a.nchunks * a.H;
    if (nitems > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipError_t e = hipSuccess;
    if (!after_chain) {  // else the chained launch has packed the operands, C included
        e = launch_chunk_pack(a, false, nullptr, s);
        if (e != hipSuccess) return e;
    }
    // streamed x and y (prefill_streams): at B = 1, L = 65536 and B = 2,
    // L = 32768 (x 671 MB) 959 and 951 us against 971 and 964 with cached x and y
    const bool stream = prefill_streams(a);
    e = launch_stage("chunk_state_mfma", stream ? chunk_state_mfma<true> : chunk_state_mfma<false>, dim3((unsigned)nitems), dim3(kThreads), K1_LDS, s, a);
    if (e != hipSuccess) return e;
    const long total = (long)a.B * a.H * (kP * kN / 4);
    // After the chained launch of packed sequences the chained form usually
    // runs the call and the state pass's workgroups exit at once; its grid is
    // then capped (each thread loops), which keeps skipping it cheap for many
    // sequences: 512 sequences of the 2.7B-shaped layer need 327 680 blocks,
    // 68 us to dispatch and skip.  (The chunk-state and output kernels keep
    // one workgroup per item: looping there costs registers, spills in the
    // output kernel.)
    const long state_blocks = std::min((total + kThreads - 1) / kThreads, after_chain ? kDualStateBlocks : total);
    const long pack_blocks = after_chain ? 0 : (long)gridB * a.nchunks * a.G * kCBlocks;
    if (state_blocks + pack_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    e = launch_stage("state_pass_bf16", state_pass_bf16, dim3((unsigned)(state_blocks + pack_blocks)),
                     dim3(kThreads), 0, s, a, total, state_blocks);
    if (e != hipSuccess) return e;
    return launch_stage("chunk_out_mfma", stream ? chunk_out_mfma<true> : chunk_out_mfma<false>, dim3((unsigned)nitems), dim3(kThreads), K3_LDS, s, a);
}

}  // namespace ssd
