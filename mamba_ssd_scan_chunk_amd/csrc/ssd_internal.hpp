// ssd_internal.hpp -- launch interface between the C ABI layer and kernels.
// Arguments reaching these launchers have already been validated.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

enum { DT_F32 = 0, DT_BF16 = 1 };

// dt preprocessing: dt as given (dt_raw = 0), or dt = clamp(softplus(dt +
// dt_bias[h]), dt_min, dt_max) computed where dt is read (dt_raw = 1).
struct DtPrep {
    int dt_raw;
    const float *dt_bias;  // [H] or null (0)
    float dt_min, dt_max;
};

// Chunks are addressed by a flat slot f.  Uniform batch [B, L]: f = b *
// nchunks + c.  Packed sequences (cu_seqlens): nchunks slots in all (B = 1 in
// the grids), described by the table that build_chunk_table writes into the
// workspace; a slot past the last chunk has Qc = 0.
struct ChunkEntry {
    int seq;   // sequence (batch element)
    int c;     // chunk within the sequence
    int tok0;  // token row of the chunk's first token in x / y / dt / Bm / Cm
    int Qc;    // tokens in the chunk (0: unused slot)
};
struct SeqEntry {
    int f0;    // slot of the sequence's first chunk
    int n;     // chunks of the sequence
    int tok0;  // token row of the sequence's first token
    int len;   // tokens of the sequence
};

struct PrefillArgs {
    int B, L, H, P, G, N, Q, nchunks;
    int T;                    // token rows of x (B * L, or the packed total)
    const int *cu_seqlens;    // packed sequences: [B + 1] token offsets; null: uniform
    const ChunkEntry *chunks; // packed sequences: [nchunks] slot table
    const SeqEntry *seqs;     // packed sequences: [B]
    const void *x;
    const float *dt, *A_log;
    DtPrep dtp;
    const void *Bm, *Cm;
    const float *D, *init_state;
    void *y;
    float *final_state;
    // workspace views
    float *ws_S;    // [B, nchunks, H, P, N]: chunk states, then carried-in states
    float *ws_dec;  // [B, nchunks, H]: exp(sum of dt*A over the chunk) - 1
    double *ws_cs;  // [B, nchunks, H, Q]: in-chunk inclusive cumsum of dt*A (vector path)
    uint16_t *ws_hb;  // [B, nchunks, H, P, N] bf16: carried-in states (MFMA path)
    uint16_t *ws_gt;  // [B, nchunks, G, tiles, 2, lanes, 8] bf16: masked C B^T (MFMA path)
    uint16_t *ws_bt;  // [B, nchunks, G, Q*N] bf16: B in MFMA operand order (MFMA path)
    uint16_t *ws_ct;  // [B, nchunks, G, Q*N] bf16: C in MFMA operand order (MFMA path)
    float *ws_cb;     // [B, nchunks, G, Q, Q] fp32: C B^T masked to s <= l (vector path)
    int *ws_ctl;      // chained MFMA path: control block (ticket, error word, per-chain counters)
    float *ws_ring;   // chained MFMA path: [B*H, 2, P*N] fp32 hand-off slots of the carried state
    unsigned long long handoff_ticks;  // chained MFMA path: bound of each hand-off wait (100 MHz ticks)
    unsigned handoff_jitter;           // chained MFMA path, testing: most s_sleep(8) rounds added per point
    const unsigned *ws_items;  // chained MFMA path over packed sequences: header + ItemEntry records (chunk-table kernel)
    int packed_form;           // packed sequences, testing: -1 = the chunk table chooses, 0 = four-kernel, 1 = chained
};

// Item order of the chained MFMA path over packed sequences, written by the
// chunk-table kernel.  The sequences, in order of decreasing chunk count, are
// dealt to the kChainXcds shares in snake order (0..7, 7..0, ...).  Header:
// items[x] = item groups of share x, items[kChainXcds + x] = where its list
// starts among the ItemEntry records that follow the header, items[kItemForm]
// = 1 when the chained form runs the call and 0 when the four-kernel form
// does (both are launched; the other one's workgroups exit at once).  Record
// R_x[c] + j of share x's list is chunk c of the share's j-th sequence
// (R_x[c]: groups in the share's rounds before c); an empty sequence counts as
// one chunk.
constexpr unsigned kItemLast = 1u << 31;   // in ItemEntry::f: the sequence's last chunk
constexpr unsigned kItemEmpty = 1u << 30;  // in ItemEntry::seq: an empty sequence (no slot)
constexpr unsigned kItemIndex = kItemEmpty - 1;
constexpr int kItemHeader = 32;            // header ints: 2 kChainXcds, the form, reserved
constexpr int kItemForm = 16;
constexpr int kItemQcBits = 9;             // ItemEntry::cq = c << kItemQcBits | Qc, Qc <= 256
constexpr long kItemMaxSlots = 1L << (31 - kItemQcBits);
// One item group, read with one 16-byte load: chunk c of sequence seq, in
// slot f, from token row tok0, Qc tokens.
struct ItemEntry {
    unsigned f;    // slot | kItemLast
    unsigned seq;  // sequence | kItemEmpty
    int tok0;
    int cq;
};

// Default bound of a hand-off wait of the chained MFMA path: 0.2 s of the
// 100 MHz device clock, far beyond the microseconds a hand-off takes.
constexpr unsigned long long kHandoffTicks = 20000000ull;

// Control block of the chained MFMA path: kChainCtlHeader ints (one item
// ticket counter per XCD, the hand-off error word), then one published-chunk
// counter per (b, h) chain.  Cleared by the pack kernel at the start of every
// call.
constexpr int kChainCtlHeader = 64;
constexpr int kChainXcds = 8;      // ticket counters: one per XCD of the MI355X
static_assert(kItemForm >= 2 * kChainXcds && kItemForm < kItemHeader && kItemHeader % 4 == 0,
              "item header: groups and list start of each share, then the form");
// Chains needed before the chained form pays.  Measured on one MI355X
// against the four-kernel form: 192 chains (B = 8 of the 130M-shaped layer,
// H = 24) 160 vs 176 us; 240 (B = 3, H = 80, L = 4096 / 16384) 176 vs 196 and
// 603 vs 723 us; 320 and more 17-31% faster chained; 160 and fewer 2-80%
// slower (B = 2, H = 80, L = 8192: 271 vs 251 us), because each chain's
// hand-offs are serial and too few chains leave them exposed.  For packed
// sequences the chunk-table kernel applies the same bound to the effective
// chains H * (sum of chunks) / (most chunks of one sequence).
constexpr long kChainMinChains = 192;
constexpr int kChainTicket = 0;    // ctl[kChainTicket + x]: tickets taken from XCD x's share
constexpr int kChainError = 8;     // bit 0: a hand-off wait expired; bit 1: an item index out of range

struct WorkspaceLayout {
    size_t off_S, off_dec, off_cs, off_hb, off_gt, off_bt, off_ct, off_tab, off_ctl, off_ring, off_items, total;
};
constexpr int kPrefillMaxQ = 1024;  // largest chunk
constexpr int kMfmaQ = 256;         // chunk of the MFMA kernels
long prefill_mfma_gt_elems_per_chunk();
long prefill_mfma_bt_elems_per_chunk();
// Workspace for `slots` chunk slots of H heads (and G groups), plus the slot
// and sequence tables of packed sequences when nseq > 0.  `chains` > 0
// selects the chained MFMA path with that many (b, h) chains: control block,
// hand-off slots and the packed operands, no per-chunk states.
WorkspaceLayout prefill_workspace_layout(long slots, int H, int P, int N, int Q, int G, bool mfma, int nseq,
                                         long chains = 0);
// Chunk slots of a packed prefill of T tokens in B sequences: an upper bound
// of sum over sequences of ceil(L_b / Q).
inline long varlen_slots(long T, int B, int Q) { return T / Q + B; }
// `items` (nullable): also the item order of the chained path, built with
// `scratch` (chunk_table_scratch_ints(slots, nseq) ints).  `timed`: a
// prefill's table, recorded by the stage timing.
hipError_t launch_chunk_table(const PrefillArgs &a, ChunkEntry *chunks, SeqEntry *seqs, hipStream_t s,
                              unsigned *items = nullptr, int *scratch = nullptr, bool timed = false);
inline long chunk_table_item_ints(long slots, long nseq) { return kItemHeader + 4 * (slots + nseq); }
inline long chunk_table_scratch_ints(long slots, long nseq) { return (2 + 2 * kChainXcds) * (slots + 2) + nseq; }
bool prefill_uses_mfma(int P, int N, int Q, int dtype);

// Stage timing (profiling aid, per host thread).  stage_begin starts a new
// record for one ssd_prefill call (the API calls it once per call, before
// the call's first kernel); stage_events hands out the start/stop
// events of its next kernel (false when timing is off or the record is
// full), which launch_stage passes to hipExtLaunchKernelGGL so that they
// are stamped when that kernel's dispatch starts and ends.
void stage_begin();
bool stage_events(const char *kernel, hipEvent_t *start, hipEvent_t *stop);

template <typename Kernel, typename... Args>
hipError_t launch_stage(const char *name, Kernel kernel, dim3 grid, dim3 block, size_t shm, hipStream_t s,
                        Args... args) {
    hipEvent_t e0, e1;
    if (stage_events(name, &e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, shm, s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
    return hipGetLastError();
}

hipError_t launch_prefill_vector(const PrefillArgs &a, int dtype, hipStream_t s);
// `after_chain`: the call of packed sequences where the chunk table chooses
// the form; the chained launch before it has run the pack kernel (with C).
hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t s, bool after_chain = false);
// The pack kernel alone: G^T tiles and B operands, plus C operands with
// `with_c`; clears the chained path's control block when `ctl` is given.
hipError_t launch_chunk_pack(const PrefillArgs &a, bool with_c, int *ctl, hipStream_t s);
// Chained single-pass MFMA prefill (the MFMA shape; for packed sequences
// followed by launch_prefill_mfma(..., true)).
hipError_t launch_prefill_chain(const PrefillArgs &a, hipStream_t s);
// Whether a batch of the MFMA shape runs the chained path (packed sequences:
// may run it, the chunk table decides).  L: tokens per sequence or the packed total.
bool prefill_uses_chain(int B, int L, int H);
hipError_t launch_state_pass(const PrefillArgs &a, hipStream_t s);
hipError_t launch_state_copy(const float *src, float *dst, size_t n, hipStream_t s);

struct DecodeArgs {
    int B, H, P, G, N, K, activation;
    long in_stride;
    const void *x_t;
    const float *dt_t, *A_log;
    DtPrep dtp;
    const void *B_t, *C_t;
    const float *D;
    float *state;
    void *y_t;
    const void *conv_in;
    void *conv_out;
    const void *conv_w, *conv_b;
};
hipError_t launch_decode(const DecodeArgs &a, int dtype, hipStream_t s);

struct ConvArgs {
    int B, T, C, K, activation;
    void *state;
    const void *xBC, *w, *bias;
    void *out;
    // packed sequences (xBC and out [T, C], T the packed total): a slot table
    // of kConvSlotTokens-token blocks; null for a uniform batch [B, T, C]
    const ChunkEntry *blocks;
    const SeqEntry *seqs;
    int nslots;
};
constexpr int kConvSlotTokens = 8;  // tokens per thread of the channel-group conv kernel
hipError_t launch_conv_update(const ConvArgs &a, int dtype, hipStream_t s);

struct NormArgs {
    long rows;
    int D, group;
    long z_stride;
    const void *y, *z;  // z null: no gate
    const float *w;     // null: weight 1
    float eps;
    void *out;
};
// Largest row the one-wave-per-row kernel takes, in 16-byte vectors.
constexpr int kNormMaxVecs = 64 * 32;
hipError_t launch_gated_rmsnorm(const NormArgs &a, int dtype, hipStream_t s);

}  // namespace ssd
