// prefill_chain.hip -- chained single-pass SSD prefill on bf16 MFMA (gfx950),
// P = 64, N = 128, 256-token chunks, uniform batches and packed sequences.
//
// The chunked scan of arXiv 2603.09555 as the bqwf.cn article on its
// compiler-first Mamba-2 implementation lays it out: §1.1 (dense work inside
// fixed chunks, a light sequential scan of the state between chunks) and
// §1.2 (the intra-chunk product and its fusion into one kernel, which keeps
// intermediate results out of memory).  The four-kernel form
// (prefill_mfma.hip) writes every chunk state S_c and every carried state
// h_{c-1} to memory and reads x twice.  Here one workgroup per item (b, c, h)
// does all of the item's work in one pass:
//
//   1. takes the next item from a ticket counter (items in chunk-major
//      order, so chunk c of a chain is always taken after chunk c-1).  The
//      chains are split into eight contiguous shares, one per XCD, each
//      with its own counter: a workgroup takes from the share of the XCD it
//      runs on (the heads of a chunk then share one L2 for the chunk's
//      packed operands), and from the next shares once its own is used up.
//      Packed sequences: the chunk-table kernel deals the sequences (by
//      chunk count, snake order) to the shares and lists each share's items
//      round by round, one 16-byte record per chunk; a chunk's heads take
//      consecutive tickets.  The grid is then an upper bound of the items,
//      and the workgroups past the item count exit without a ticket;
//   2. loads x and dt once, forms x' in LDS, and the chunk state
//        S_c = exp(cs_last - R_7) sum_k (prod_{j > k} Q_j) x'^T_k B_k
//      on MFMA (the same tile references R_k and ratios Q_k as the outputs
//      use: the Horner scheme run to the chunk's end);
//   3. waits until chunk c-1 of its (b, h) chain has published
//      h_{c-1}, reads it, forms h_c = h_{c-1} + (expm1(cs_last) h_{c-1} + S_c)
//      in fp32 and publishes h_c for chunk c+1 (or writes the final state).
//      The chain's counter is read once at the start as well: when chunk c-1
//      has already published (the usual case with many chains in flight),
//      h_{c-1} is requested right away and arrives during the chunk state;
//   4. forms the outputs from x' (still in LDS), h_{c-1} and the packed
//      operands exactly as the output kernel does (out_tiles).
// When x exceeds the Infinity Cache (prefill_streams), x is read and y
// written with non-temporal accesses: the chunks' packed operands, which the
// heads of a chunk share, then stay in the L2 (one instantiation per
// policy).
//
// Only the carried state travels between workgroups, through two slots per
// chain (chunk c reads slot (c-1) % 2 and writes slot c % 2): 32 KB written
// and 32 KB read per item, against 96 KB of chunk and carried states plus a
// second read of x in the four-kernel form.
//
// Hand-off protocol.  The slot is written with agent-scope coherent stores
// (the cache-policy bits the compiler uses for agent-scope atomic stores, so
// the data goes past the XCD's own L2), each thread waits for its stores to
// complete, the workgroup synchronises, and thread 0 then sets the chain's
// counter to c + 1 with an agent-scope atomic store.  The successor's thread
// 0 polls the counter with agent-scope atomic loads, the workgroup
// synchronises, and every thread reads the slot with agent-scope coherent
// loads, which do not hit a stale line of the reader's L1 or L2 (loads with
// workgroup-scope or no cache-policy bits were seen to return the reader's
// stale L1 copy for milliseconds after another CU had rewritten the line).
// Slot reuse is
// safe: chunk c+2 writes slot c % 2 only after it has seen the counter of
// chunk c+1, which chunk c+1 sets after its reads of slot c % 2 returned.
// No deadlock: tickets are taken by running workgroups only, and an item
// waits only on chunk c-1 of its chain, which has a smaller ticket of the
// same counter and so is held by a running or finished workgroup; the
// unfinished item of smallest chunk index therefore always progresses.
// Every workgroup takes exactly one item: the grid has one workgroup per
// item (packed sequences: exactly as many workgroups as items try), and a
// workgroup moves on to another share only when its counter has handed out
// all of that share.  Packed sequences launch the four-kernel form after this
// kernel as well; the chunk table chooses which of the two does the work,
// and the other's workgroups exit at once.  Every wait is bounded (by default 0.2 s of
// the 100 MHz wall clock, far beyond the microseconds a hand-off takes; the
// bound is a kernel argument that ssd_debug_handoff_ticks sets per host
// thread for tests): on expiry the workgroup sets the control block's error
// word and carries NaN, so a broken hand-off shows as NaN outputs instead of
// a hang.  It also sets a sticky bit in the chain's counter (counters are
// only raised: publishing is an atomic max), and every later chunk of the
// chain that sees the bit carries NaN as well, whatever its slot holds: a
// late predecessor may still overwrite a slot after its successor gave up.
// The pack kernel clears the control block at the start of every call.
#include "prefill_mfma.hpp"

namespace ssd {
namespace {

// Cache-policy bits of an agent-scope coherent access (sc1), as the compiler
// emits them for agent-scope atomic loads and stores on gfx950.
constexpr int kScopeAgent = 16;
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).
constexpr int kWaitVmcnt0 = 0x0F70;
// Bit of a chain's counter set when one of its waits expired (sticky: the
// counter is only ever raised, by atomic max and OR).
constexpr int kChainPoison = 1 << 30;

constexpr int CH_TK = K3_LDS;       // the item, early counter, wait result
constexpr int CH_LDS = CH_TK + 48;

// Byte offset in a hand-off slot of the 16 bytes (registers 4q .. 4q+3 of
// accumulator `acc`) that lane `lane` of wave `wave` holds: 1 KiB contiguous
// per store instruction.
__device__ __forceinline__ unsigned slot_off(int wave, int acc, int q, int lane) {
    return (unsigned)((((wave * 2 + acc) * 4 + q) * 64 + lane) * 16);
}

__device__ __forceinline__ void buf_store16(u32x4 v, __amdgpu_buffer_rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kScopeAgent);
}

// XCD of the executing workgroup (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ int xcd_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (kChainXcds - 1); }

// Chains [lo, hi) of XCD share x of a uniform batch: eight contiguous ranges
// of the B*H chains.
__device__ __forceinline__ void xcd_share(int x, long BH, int &lo, int &hi) {
    lo = (int)(x * BH / kChainXcds);
    hi = (int)((x + 1) * BH / kChainXcds);
}

// Testing aid (ssd_debug_handoff_jitter): a delay of 0 .. a.handoff_jitter
// rounds of s_sleep 8, from a hash of `seed`; the seed is uniform, so the
// whole workgroup sleeps alike.
__device__ __forceinline__ void jitter_sleep(const PrefillArgs &a, unsigned seed) {
    if (!a.handoff_jitter) return;
    unsigned v = seed * 2654435761u;
    v ^= v >> 15;
    v *= 2246822519u;
    v ^= v >> 13;
    const unsigned n = v % (a.handoff_jitter + 1);
    for (unsigned i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
}

// Feature row of register v of accumulator acc (lane half lh): the
// accumulator order of a 32x32 MFMA tile.
__device__ __forceinline__ int acc_row(int acc, int v, int lh) { return 32 * acc + (v >> 2) * 8 + lh * 4 + (v & 3); }

template <bool kNtX, bool kNtY, bool kPacked>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void chunk_chain_mfma(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *xt = smem + K3_XT;
    char *hl = smem + K3_H;
    float *vt = (float *)(smem + K3_V);
    float *ut = (float *)(smem + K3_U);
    float *dtt = (float *)(smem + K3_DT);
    float *wv = (float *)(smem + K3_W);
    int *tk = (int *)(smem + CH_TK);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    int *ctl = a.ws_ctl;

    // ---- the item: the next ticket of this XCD's share, else of the next
    // shares.  Uniform batches: shares of the (b, h) chains, tickets
    // chunk-major over the share's chains.  Packed sequences: shares of the
    // sequences (the chunk table deals them out), tickets over the share's
    // item order (round c: chunk c of each of its sequences with more than c
    // chunks) times the H heads, so a chunk's heads follow each other.
    // Thread 0 hands the item to the workgroup through LDS: slot, head,
    // flags (last chunk, empty sequence), sequence, first token row, chunk
    // index and length.
    if (tid == 0) {
        int fi = -1, hh = 0, seq = 0, tok = 0, cc = 0, qc = 0;
        unsigned fl = 0;
        const int x0 = xcd_id();
        constexpr bool packed = kPacked;
        // packed: the header (groups and list start of each share), in flight
        // with the first ticket
        u32x4 hdr[5] = {};
        if (packed)
#pragma unroll
            for (int q = 0; q < 5; ++q) hdr[q] = ((const u32x4 *)a.ws_items)[q];
        static_assert(kItemForm == 16, "the form is the first int of the header's fifth 16 bytes");
        // The grid of packed sequences is an upper bound of the items.  Exactly
        // as many workgroups as there are items take tickets (each then gets
        // one): those below ceil(T / Q) * H always (every sequence has at least
        // ceil(its length / Q) chunks), the rest only below the header's total
        // (the last share's list start plus its groups, times H).  The rest exit
        // without touching the ticket counters, which every real item contends for.
        // With packed sequences the four-kernel form may run the call instead
        // (the chunk table's choice): then no workgroup takes a ticket.
        bool take = true;
        if (packed && (long)blockIdx.x >= ((long)a.T + a.Q - 1) / a.Q * a.H)
            take = (long)blockIdx.x < ((long)hdr[3][3] + hdr[1][3]) * a.H;
        if (packed && hdr[4][0] != 1u) take = false;
        for (int i = 0; take && i < kChainXcds && fi < 0; ++i) {
            const int x = (x0 + i) & (kChainXcds - 1);
            int lo = 0, hi = a.H;
            if (!packed) {
                xcd_share(x, (long)a.B * a.H, lo, hi);
                if (hi == lo) continue;
            }
            const long k = __hip_atomic_fetch_add(ctl + kChainTicket + x, 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
            const long groups = packed ? (long)hdr[x >> 2][x & 3] : a.nchunks;
            if (k < (long)(hi - lo) * groups) {
                const long u = k / (hi - lo);
                const int unit = lo + (int)(k - u * (hi - lo));
                if (packed) {
                    const unsigned start = hdr[2 + (x >> 2)][x & 3];
                    const u32x4 r = ((const u32x4 *)(a.ws_items + kItemHeader))[start + u];
                    fi = (int)(r[0] & kItemIndex);
                    fl = (r[0] & kItemLast) | (r[1] & kItemEmpty);
                    seq = (int)(r[1] & kItemIndex);
                    tok = (int)r[2];
                    cc = (int)(r[3] >> kItemQcBits);
                    qc = (int)(r[3] & ((1u << kItemQcBits) - 1));
                    hh = unit;
                } else {
                    const int b = unit / a.H;
                    fi = (int)((long)b * a.nchunks + u);
                    fl = u + 1 == a.nchunks ? kItemLast : 0u;
                    seq = b;
                    tok = (int)((long)b * a.L + u * a.Q);
                    cc = (int)u;
                    qc = min((long)a.Q, a.L - u * a.Q);
                    hh = unit - b * a.H;
                }
            }
        }
        if (packed && fi >= 0 && (seq >= a.B || (!(fl & kItemEmpty) && fi >= a.nchunks))) {
            // never for a table the chunk-table kernel wrote
            __hip_atomic_fetch_or(ctl + kChainError, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            fi = -1;
        }
        tk[0] = fi;
        tk[1] = hh;
        tk[4] = (int)fl;
        tk[5] = seq;
        tk[6] = tok;
        tk[7] = cc;
        tk[8] = qc;
    }
    __syncthreads();
    const int fi = __builtin_amdgcn_readfirstlane(tk[0]);
    const int h = __builtin_amdgcn_readfirstlane(tk[1]);
    const unsigned fl = (unsigned)__builtin_amdgcn_readfirstlane(tk[4]);
    const int b = __builtin_amdgcn_readfirstlane(tk[5]);
    if (fi < 0) return;  // every share handed out
    if (fl & kItemEmpty) {
        // an empty sequence: its state is carried over unchanged
        if (a.final_state) {
            const long o = ((long)b * a.H + h) * kP * kN;
            const float4 *src = (const float4 *)(a.init_state + o);
            float4 *dst = (float4 *)(a.final_state + o);
            for (int i = tid; i < kP * kN / 4; i += kThreads) dst[i] = a.init_state ? src[i] : make_float4(0, 0, 0, 0);
        }
        return;
    }
    const bool last = (fl & kItemLast) != 0;
    const long f = fi;
    const int c = __builtin_amdgcn_readfirstlane(tk[7]);
    const int Qc = __builtin_amdgcn_readfirstlane(tk[8]);
    const long tok0 = __builtin_amdgcn_readfirstlane(tk[6]);
    const int bh = b * a.H + h;
    const int g = h / (a.H / a.G);
    const long cg = f * a.G + g;

    jitter_sleep(a, (unsigned)bh * 131u + (unsigned)c * 7u + 1u);

    // ---- loads: the chain's counter (thread 0), the step, A_log and D (the
    // cumsum waits for these only), x, the B operands
    int *counter = ctl + kChainCtlHeader + bh;
    int early = 0;
    if (tid == 0 && c > 0) early = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const DecayIn din = load_decay_in(a, tok0, Qc, h, tid);
    u32x4 raw[8];
    load_x_raw<kNtX>(a, tok0, Qc, h, raw, tid);
    // B operands of the first token tile (the rest are streamed one tile
    // ahead: B = 8, L = 16384 1259 -> 1245 us against two tiles ahead; the
    // kernel does better with fewer loads in flight)
    const u32x4 *bt = (const u32x4 *)(a.ws_bt + cg * kBTChunk) + (wave * (kQ / 16)) * 64 + lane;
    u32x4 bq[4];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) bq[gg] = bt[gg * 64];
    // packed sequences: a tile past the chunk's last token is requested past
    // the end of this resource (zeros, no memory access), so that every path
    // issues the same loads
    const __amdgpu_buffer_rsrc_t btr = make_rsrc(bt - lane, (unsigned)(kQ / 16) * 64 * 16);
    const float Dh = din.D;
    if (tid == 0) tk[2] = early;
    float total;
    const float dtv = step_of(a, din, Qc, tid);
    const bool exact = chunk_decay(dtv, -expf(din.alog), Dh, Qc, vt, ut, dtt, wv, tid, lane, wave, &total);

    // ---- h_{c-1} requested now if chunk c-1 had published by the start
    // (the counter was read before the barriers above).  The loads are issued
    // on every path, against an empty range when chunk c-1 had not published
    // (they then return zeros without touching memory): loads retire in issue
    // order, and with the same loads in the same order on every path the
    // waits before the x' store and the chunk state need not cover them.
    const bool ready = c > 0 && tk[2] >= c;
    const bool early_poison = (tk[2] & kChainPoison) != 0;
    float hp[2][16];
    const float *slot = a.ws_ring + ((long)bh * 2 + ((c - 1) & 1)) * kP * kN;
    auto load_h = [&](__amdgpu_buffer_rsrc_t hrs) {
#pragma unroll
        for (int acc = 0; acc < 2; ++acc)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 v = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(hrs, slot_off(wave, acc, q, lane), 0, kScopeAgent));
#pragma unroll
                for (int r = 0; r < 4; ++r) hp[acc][4 * q + r] = __uint_as_float(v[r]);
            }
    };
    load_h(make_rsrc(slot, ready ? kP * kN * 4 : 0));

    // ---- x' into LDS: the outputs' x' on the fast path; on the exact path
    // first x'' = exp(cs_last - cs_s) dt_s x_s for the chunk state
    {
        float sc[8];
        if (!exact) {
            x_scales(vt, false, tid, sc);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int s = (tid >> 3) * 8 + r;
                sc[r] = exp_fast(total - vt[s]) * dtt[s];
            }
        }
        store_xt_korder(raw, sc, xt, tid);
    }
    __syncthreads();

    // ---- chunk state S_c, wave w: columns n in [32w, 32w + 32), both
    // 32-row feature tiles; Horner over the token tiles (Q = 1 and no final
    // factor on the exact path)
    // Packed sequences (most chunks short in a batch of short prompts): the
    // loop stops at the last token tile K = ntl - 1 (the tiles after it hold
    // no token) and the closing factor is exp(cs_last - R_K).  A uniform batch
    // runs all eight tiles (at most its last chunk is short), which keeps its
    // loop free of the extra branches.
    const int ntl = kPacked ? (Qc + 31) >> 5 : kTiles;
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int k = 0; k < kTiles; ++k) {
        if (kPacked && k + 1 < kTiles) {  // token tile k + 1, one step ahead
            const unsigned off = k + 1 < ntl ? (unsigned)((2 * k + 2) * 64 + lane) * 16u : 0x40000000u;
            bq[(2 * k + 2) & 3] = buf_load16(btr, off);
            bq[(2 * k + 3) & 3] = buf_load16(btr, off + 1024u);
        }
        if (k < ntl) {
            if (k > 0) {
                const float q = wv[K3_WQ + k];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    s0[v] *= q;
                    s1[v] *= q;
                }
            }
            if (!kPacked && k + 1 < kTiles) {  // token tile k + 1, one step ahead
                bq[(2 * k + 2) & 3] = bt[(2 * k + 2) * 64];
                bq[(2 * k + 3) & 3] = bt[(2 * k + 3) * 64];
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const u32x4 a0 = *(const u32x4 *)(xt + xt_operand(li, lh, k, hf));
                const u32x4 a1 = *(const u32x4 *)(xt + xt_operand(32 + li, lh, k, hf));
                s0 = mfma32(a0, bq[(2 * k + hf) & 3], s0);
                s1 = mfma32(a1, bq[(2 * k + hf) & 3], s1);
            }
        }
    }
    {
        float rest = wv[3 * 3 + 2] - wv[3 * 3 + 1];  // cs_last - R_7
        if (kPacked && ntl < kTiles) {
            // cs_last - R_K: the rest of R_K's wave after it, then the later
            // waves' totals
            const int kw = (ntl - 1) >> 1;
            rest = wv[3 * kw + 2] - wv[3 * kw + ((ntl - 1) & 1)];
#pragma unroll
            for (int w = 0; w < 4; ++w) rest += w > kw ? wv[3 * w + 2] : 0.0f;
        }
        const float fin = exact ? 1.0f : exp_fast(rest);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            s0[v] *= fin;
            s1[v] *= fin;
        }
    }
    if (exact) {
        // the outputs' exact path takes x' = x
        __syncthreads();
        load_x_raw<kNtX>(a, tok0, Qc, h, raw, tid);
        float sc[8];
        x_scales(vt, true, tid, sc);
        store_xt_korder(raw, sc, xt, tid);
    }

    // ---- h_{c-1}: the initial state, or chunk c-1's hand-off
    jitter_sleep(a, (unsigned)bh * 131u + (unsigned)c * 7u + 2u);
    if (c == 0) {
        const float *init = a.init_state ? a.init_state + (long)bh * kP * kN : nullptr;
#pragma unroll
        for (int acc = 0; acc < 2; ++acc)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                hp[acc][v] = init ? init[acc_row(acc, v, lh) * kN + 32 * wave + li] : 0.0f;
    } else if (!ready) {
        if (tid == 0) {
            const unsigned long long t0 = wall_clock64();
            int ok = 1, seen;
            while ((seen = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < c) {
                __builtin_amdgcn_s_sleep(2);
                if (wall_clock64() - t0 > a.handoff_ticks) {
                    // expired: mark the chain, so that every later chunk takes
                    // NaN as well (a late predecessor may still write its slot)
                    ok = 0;
                    __hip_atomic_fetch_or(counter, kChainPoison, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_fetch_or(ctl + kChainError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            tk[3] = ok && !(seen & kChainPoison);
        }
        __syncthreads();
        load_h(make_rsrc(slot, kP * kN * 4));
        if (!tk[3]) {
#pragma unroll
            for (int acc = 0; acc < 2; ++acc)
#pragma unroll
                for (int v = 0; v < 16; ++v) hp[acc][v] = __builtin_nanf("");
        }
    }

    if (ready && early_poison) {  // an earlier chunk of the chain expired
#pragma unroll
        for (int acc = 0; acc < 2; ++acc)
#pragma unroll
            for (int v = 0; v < 16; ++v) hp[acc][v] = __builtin_nanf("");
    }

    // ---- first operands of the output phase, the C operands of both column
    // tiles (not hoisted above the chunk state), requested after every load
    // of h_{c-1} on every path: the combine below then waits for h_{c-1}
    // alone, and these arrive while h_c is formed and published
    __builtin_amdgcn_sched_barrier(0);
    OutItem it;
    it.ctp = (const u32x4 *)(a.ws_ct + cg * kBTChunk) + lane;
    it.gtr = gt_rsrc(a, cg);
    it.lane16 = (unsigned)lane * 16u;
    it.tok0 = tok0;
    it.Qc = Qc;
    it.h = h;
    it.Dh = Dh;
    it.exact = exact;
    u32x4 cop[8], copB[8];
    out_first_loads(it, wave, cop, copB);

    // ---- h_c, rounded once: h + (expm1(cs_last) h + S); h_{c-1} into LDS
    // as bf16 ([P][N], 16-byte chunks XOR-swizzled by row) for the outputs
    const float dm1 = expm1f(total);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        s0[v] = hp[0][v] + fmaf(dm1, hp[0][v], s0[v]);
        s1[v] = hp[1][v] + fmaf(dm1, hp[1][v], s1[v]);
    }
#pragma unroll
    for (int acc = 0; acc < 2; ++acc)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int p = acc_row(acc, v, lh), n = 32 * wave + li;
            *(bf16_t *)(hl + p * 256 + (((n >> 3) ^ (p & 15)) << 4) + (n & 7) * 2) = f32_to_bf16(hp[acc][v]);
        }
    if (!last) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.ws_ring + ((long)bh * 2 + (c & 1)) * kP * kN, kP * kN * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            buf_store16(u32x4{__float_as_uint(s0[4 * q]), __float_as_uint(s0[4 * q + 1]),
                              __float_as_uint(s0[4 * q + 2]), __float_as_uint(s0[4 * q + 3])},
                        rs, slot_off(wave, 0, q, lane));
            buf_store16(u32x4{__float_as_uint(s1[4 * q]), __float_as_uint(s1[4 * q + 1]),
                              __float_as_uint(s1[4 * q + 2]), __float_as_uint(s1[4 * q + 3])},
                        rs, slot_off(wave, 1, q, lane));
        }
        jitter_sleep(a, (unsigned)bh * 131u + (unsigned)c * 7u + 3u);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this thread's slot stores are complete
        __syncthreads();                          // ... and every other thread's
        // the counter only grows: a predecessor that publishes after this
        // chunk's wait expired cannot move it back
        if (tid == 0) __hip_atomic_fetch_max(counter, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (a.final_state) {
        float *fs = a.final_state + (long)bh * kP * kN + 32 * wave + li;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            fs[acc_row(0, v, lh) * kN] = s0[v];
            fs[acc_row(1, v, lh) * kN] = s1[v];
        }
    }

    __syncthreads();
    out_tiles<kNtY, false>(a, it, smem, cop, copB, tid);
}

}  // namespace

// The chained form needs enough (b, h) chains to keep the machine busy while
// each chain waits on its hand-offs.
bool prefill_uses_chain(int B, int L, int H) { return L > 0 && (long)B * H >= kChainMinChains; }

hipError_t launch_prefill_chain(const PrefillArgs &a, hipStream_t s) {
    // one workgroup per item: B * nchunks * H for a uniform batch; for packed
    // sequences at most (slots + sequences) * H (an empty sequence counts as
    // one chunk), and the workgroups past the actual items exit at once
    const long nitems = (a.chunks ? (long)a.nchunks + a.B : (long)a.B * a.nchunks) * a.H;
    if (nitems > 0x7fffffffL || (a.chunks && !a.ws_items)) return hipErrorInvalidConfiguration;
    hipError_t e = launch_chunk_pack(a, true, a.ws_ctl, s);
    if (e != hipSuccess) return e;
    // streamed x and y (prefill_streams).  Measured on the 2.7B-shaped layer
    // at B = 8, L = 16384 (x and y 1.34 GB each): 1405 us with cached x and
    // y, 1355 with non-temporal x loads, 1375 with non-temporal y stores,
    // 1316 with both
    const bool stream = prefill_streams(a);
    auto kernel = a.chunks ? (stream ? chunk_chain_mfma<true, true, true> : chunk_chain_mfma<false, false, true>)
                           : (stream ? chunk_chain_mfma<true, true, false> : chunk_chain_mfma<false, false, false>);
    return launch_stage("chunk_chain_mfma", kernel, dim3((unsigned)nitems), dim3(kThreads), CH_LDS, s, a);
}

}  // namespace ssd
