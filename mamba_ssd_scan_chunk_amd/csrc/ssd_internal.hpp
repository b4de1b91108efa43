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
};

struct WorkspaceLayout {
    size_t off_S, off_dec, off_cs, off_hb, off_gt, off_bt, off_ct, off_tab, total;
};
constexpr int kPrefillMaxQ = 1024;  // largest chunk
constexpr int kMfmaQ = 256;         // chunk of the MFMA kernels
long prefill_mfma_gt_elems_per_chunk();
long prefill_mfma_bt_elems_per_chunk();
// Workspace for `slots` chunk slots of H heads (and G groups), plus the slot
// and sequence tables of packed sequences when nseq > 0.
WorkspaceLayout prefill_workspace_layout(long slots, int H, int P, int N, int Q, int G, bool mfma, int nseq);
// Chunk slots of a packed prefill of T tokens in B sequences: an upper bound
// of sum over sequences of ceil(L_b / Q).
inline long varlen_slots(long T, int B, int Q) { return T / Q + B; }
hipError_t launch_chunk_table(const PrefillArgs &a, ChunkEntry *chunks, SeqEntry *seqs, hipStream_t s);
bool prefill_uses_mfma(int P, int N, int Q, int dtype);

// Stage timing (profiling aid, per host thread).  stage_begin starts a new
// record for one ssd_prefill call; stage_events hands out the start/stop
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
hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t s);
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
