// ssd_api.hip -- the C ABI declared in include/ssd.h: host-side argument
// checks, workspace layout and kernel dispatch.  Every check runs before the
// first HIP call, so a rejected call launches nothing.
#include "../../include/ssd.h"

#include <stdint.h>

#include <mutex>

#include "ssd_internal.hpp"

#define SSD_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;
// Bound of the chained prefill's hand-off waits for calls of this thread
// (ssd_debug_handoff_ticks); negative = the default.
thread_local long long g_handoff_ticks = -1;
// Random delays at the chained prefill's hand-off points for calls of this
// thread (ssd_debug_handoff_jitter); 0 = none.
thread_local unsigned g_handoff_jitter = 0;
// Form of a packed prefill on the chained path, for this host thread
// (ssd_debug_packed_form): -1 = the chunk table chooses, 0 = four-kernel, 1 = chained.
thread_local int g_packed_form = -1;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return SSD_OK;
    g_last_hip_error = (int)e;
    return SSD_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// [p, p + n) and [q, q + m) share a byte (null or empty never overlaps).
bool overlap(const void *p, size_t n, const void *q, size_t m) {
    if (!p || !q || n == 0 || m == 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + m && b < a + n;
}

bool valid_dtype(int d) { return d == SSD_F32 || d == SSD_BF16; }
size_t esize(int d) { return d == SSD_BF16 ? 2 : 4; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Product of non-negative factors, or SIZE_MAX on overflow.
size_t mul(size_t a, size_t b) {
    if (a != 0 && b > SIZE_MAX / a) return SIZE_MAX;
    return a * b;
}

// L: tokens per sequence (uniform batch) or the packed total T (varlen).
struct PrefillShape {
    int B, L, H, P, G, N, Q, dtype;
    bool varlen;
};

int check_prefill_shape(const PrefillShape &s) {
    if (!valid_dtype(s.dtype)) return SSD_ERR_INVALID_ARG;
    if (s.B < 1 || s.L < 0 || s.H < 1 || s.P < 1 || s.G < 1 || s.N < 1 || s.Q < 1) return SSD_ERR_INVALID_ARG;
    if (s.H % s.G != 0) return SSD_ERR_INVALID_ARG;
    if (s.P > 256 || s.N > 256 || s.Q > ssd::kPrefillMaxQ) return SSD_ERR_UNSUPPORTED;
    if (s.B > 65535 || s.H > 65535) return SSD_ERR_UNSUPPORTED;
    // in-chunk row offsets are 32-bit: Q * H * P and Q * G * N below 2^31
    if ((long)s.Q * s.H * s.P >= (1L << 31) || (long)s.Q * s.G * s.N >= (1L << 31)) return SSD_ERR_UNSUPPORTED;
    // token rows index with 32 bits; every element index must fit
    // comfortably in 63 bits
    const size_t rows = s.varlen ? (size_t)s.L : (size_t)s.B * s.L;
    if (rows >= ((size_t)1 << 31)) return SSD_ERR_UNSUPPORTED;
    if (mul(mul(rows + (size_t)s.B * s.Q, (size_t)s.H), (size_t)s.P * s.N) >= ((size_t)1 << 60))
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

}  // namespace

namespace ssd {

// The MFMA kernels run 256-token chunks.  A chunk of any multiple of 256
// tokens runs as 256-token sub-chunks whose hand-off goes through the state
// pass: the chunked form gives the same scan for any chunk length (up to
// rounding), so the sub-chunks are an evaluation order, not an approximation.
bool prefill_uses_mfma(int P, int N, int Q, int dtype) {
    return dtype == SSD_BF16 && P == 64 && N == 128 && Q % kMfmaQ == 0;
}

WorkspaceLayout prefill_workspace_layout(long slots, int H, int P, int N, int Q, int G, bool mfma, int nseq,
                                         long chains) {
    WorkspaceLayout w{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    if (slots <= 0) return w;
    const size_t heads = (size_t)slots * H;
    const size_t groups = (size_t)slots * G;
    const bool chain = mfma && chains > 0;
    // packed sequences on the chained path: the chunk table chooses the form
    // on the device, so the four-kernel form's per-chunk states are there too
    const bool four = !chain || nseq > 0;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    // chained MFMA path: control block and two hand-off slots per chain
    // instead of per-chunk states
    w.off_ctl = take(chain ? (size_t)(kChainCtlHeader + chains) * sizeof(int) : 0);
    w.off_ring = take(chain ? (size_t)chains * 2 * P * N * sizeof(float) : 0);
    w.off_S = take(four ? heads * P * N * sizeof(float) : 0);
    w.off_dec = take(four ? heads * sizeof(float) : 0);
    w.off_cs = take(mfma ? 0 : heads * Q * sizeof(double));
    w.off_hb = take(mfma && four ? heads * P * N * sizeof(uint16_t) : 0);
    // MFMA path: G^T tiles in bf16; vector path: the Q x Q masked C B^T in fp32
    w.off_gt = take(mfma ? groups * prefill_mfma_gt_elems_per_chunk() * sizeof(uint16_t)
                         : groups * (size_t)Q * Q * sizeof(float));
    const size_t bt_bytes = mfma ? groups * prefill_mfma_bt_elems_per_chunk() * sizeof(uint16_t) : 0;
    w.off_bt = take(bt_bytes);
    w.off_ct = take(bt_bytes);  // C packed like B
    w.off_tab = take(nseq > 0 ? (size_t)slots * sizeof(ChunkEntry) + (size_t)nseq * sizeof(SeqEntry) : 0);
    // chained path over packed sequences: the item order, then the chunk-table
    // kernel's scratch for building it
    w.off_items = take(chain && nseq > 0 ? (size_t)(chunk_table_item_ints(slots, nseq) +
                                                    chunk_table_scratch_ints(slots, nseq)) * sizeof(int)
                                         : 0);
    w.total = off;
    return w;
}

}  // namespace ssd

namespace {
// Chunk length the kernels run: 256 on the MFMA path (see prefill_uses_mfma),
// Q on the vector path.
int run_q(const PrefillShape &s) { return ssd::prefill_uses_mfma(s.P, s.N, s.Q, s.dtype) ? ssd::kMfmaQ : s.Q; }
// Chunk slots of a prefill: B * ceil(L / q) for a uniform batch, the bound
// varlen_slots(T, B, q) for packed sequences (0 when there are no tokens),
// q = run_q.
long prefill_slots(const PrefillShape &s) {
    if (s.L <= 0) return 0;
    const int q = run_q(s);
    return s.varlen ? ssd::varlen_slots(s.L, s.B, q) : (long)s.B * ((s.L + q - 1) / q);
}
// (b, h) chains of the chained MFMA path, 0 when the call takes another path.
long prefill_chains(const PrefillShape &s) {
    bool chain = ssd::prefill_uses_mfma(s.P, s.N, s.Q, s.dtype) && ssd::prefill_uses_chain(s.B, s.L, s.H);
    // packed sequences: the item records hold a slot below kItemMaxSlots and a
    // sequence index below kItemIndex; beyond that the four-kernel form runs
    if (chain && s.varlen && (prefill_slots(s) >= ssd::kItemMaxSlots || (long)s.B >= (long)ssd::kItemIndex))
        chain = false;
    return chain ? (long)s.B * s.H : 0;
}
ssd::WorkspaceLayout workspace_layout_for(const PrefillShape &s) {
    return ssd::prefill_workspace_layout(prefill_slots(s), s.H, s.P, s.N, run_q(s), s.G,
                                         ssd::prefill_uses_mfma(s.P, s.N, s.Q, s.dtype), s.varlen ? s.B : 0,
                                         prefill_chains(s));
}
size_t workspace_bytes_for(const PrefillShape &s) { return workspace_layout_for(s).total; }
}  // namespace

SSD_API size_t ssd_prefill_workspace_bytes(int B, int L, int H, int P, int G, int N, int Q, int dtype) {
    const PrefillShape s{B, L, H, P, G, N, Q, dtype, false};
    if (check_prefill_shape(s) != SSD_OK) return (size_t)-1;
    return workspace_bytes_for(s);
}

SSD_API size_t ssd_prefill_varlen_workspace_bytes(int B, int T, int H, int P, int G, int N, int Q, int dtype) {
    const PrefillShape s{B, T, H, P, G, N, Q, dtype, true};
    if (check_prefill_shape(s) != SSD_OK) return (size_t)-1;
    return workspace_bytes_for(s);
}

namespace {

// dt preprocessing arguments: dt_bias may be null; 0 <= dt_min <= dt_max
// (dt_max may be +inf); no NaN.
bool valid_dt_prep(float dt_min, float dt_max, const float *dt_bias) {
    if (!(dt_min >= 0.0f) || !(dt_max >= dt_min)) return false;  // also rejects NaN
    return aligned(dt_bias, 4);
}

// ---- the fixed scratch of ssd_prefill_noalloc
// One copy per GPU, held until the process ends.  On the host, `scratch` is
// a stand-in for the symbol, not a device address: host code only ever uses
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // per device, set on its first call

// Device address of the current device's scratch (looked up once per device,
// with that device current).  `stream` must belong to the current device.
int noalloc_scratch(hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (stream) {
        hipDevice_t sdev = 0;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return hip_status(e);
        if ((int)sdev != dev) return SSD_ERR_INVALID_ARG;
    }
    if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p || !aligned(p, 256)) return SSD_ERR_ALIGNMENT;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSD_OK;
}

// L is the per-sequence length, or with cu_seqlens (packed sequences, a
// device array of B + 1 token offsets) the packed total T.  With `noalloc`
// the workspace arguments are ignored and the scratch is the fixed buffer
// above (after every argument check, so a rejected call makes no HIP call).
int prefill_impl(int B, int L, int H, int P, int G, int N, int Q, int dtype, const int *cu_seqlens,
                 const void *x, const float *dt, const float *A_log,
                 const void *Bm, const void *Cm, const float *D,
                 const float *init_state, void *y, float *final_state,
                 void *workspace, size_t workspace_bytes, hipStream_t stream, const ssd::DtPrep &dtp,
                 bool varlen = false, bool noalloc = false) {
    const PrefillShape s{B, L, H, P, G, N, Q, dtype, varlen};
    int rc = check_prefill_shape(s);
    if (rc != SSD_OK) return rc;
    if (!A_log || (varlen && !cu_seqlens)) return SSD_ERR_INVALID_ARG;
    if (L > 0 && (!x || !dt || !Bm || !Cm || !y)) return SSD_ERR_INVALID_ARG;
    if (!aligned(cu_seqlens, 4)) return SSD_ERR_ALIGNMENT;

    const size_t es = esize(dtype);
    const size_t rows = varlen ? (size_t)L : (size_t)B * L;  // token rows of x, y, dt, Bm, Cm
    const size_t n_x = rows * H * P, n_bc = rows * G * N;
    const size_t n_dt = rows * H, n_state = (size_t)B * H * P * N;
    const size_t b_x = n_x * es, b_bc = n_bc * es, b_dt = n_dt * 4, b_state = n_state * 4;

    if (!aligned(x, 16) || !aligned(Bm, 16) || !aligned(Cm, 16) || !aligned(y, 16) ||
        !aligned(init_state, 16) || !aligned(final_state, 16) || !aligned(dt, 4) ||
        !aligned(A_log, 4) || !aligned(D, 4) || !aligned(workspace, 256))
        return SSD_ERR_ALIGNMENT;

    const bool mfma = ssd::prefill_uses_mfma(P, N, Q, dtype);
    const int q = run_q(s);
    const long slots = prefill_slots(s);
    const bool chain = prefill_chains(s) > 0;
    const ssd::WorkspaceLayout wl = workspace_layout_for(s);
    const size_t b_ws = wl.total;

    // outputs may not overlap inputs, workspace or each other
    // (final_state == init_state exactly is allowed)
    struct R { const void *p; size_t n; };
    const R ins[] = {{x, b_x}, {dt, b_dt}, {A_log, (size_t)H * 4}, {Bm, b_bc}, {Cm, b_bc}, {D, D ? (size_t)H * 4 : 0},
                     {dtp.dt_bias, dtp.dt_bias ? (size_t)H * 4 : 0},
                     {cu_seqlens, cu_seqlens ? (size_t)(B + 1) * 4 : 0}};
    if (L > 0) {
        for (const R &r : ins) if (overlap(y, b_x, r.p, r.n)) return SSD_ERR_INVALID_ARG;
        if (overlap(y, b_x, init_state, b_state) || overlap(y, b_x, final_state, b_state) ||
            overlap(y, b_x, workspace, b_ws))
            return SSD_ERR_INVALID_ARG;
    }
    if (final_state) {
        for (const R &r : ins) if (overlap(final_state, b_state, r.p, r.n)) return SSD_ERR_INVALID_ARG;
        if (overlap(final_state, b_state, workspace, b_ws)) return SSD_ERR_INVALID_ARG;
        if (final_state != init_state && overlap(final_state, b_state, init_state, b_state)) return SSD_ERR_INVALID_ARG;
    }
    if (noalloc) {
        if (b_ws > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_TOO_LARGE;
    } else if (b_ws > 0) {
        if (!workspace || workspace_bytes < b_ws) return SSD_ERR_WORKSPACE;
        for (const R &r : ins) if (overlap(workspace, b_ws, r.p, r.n)) return SSD_ERR_INVALID_ARG;
        if (overlap(workspace, b_ws, init_state, b_state)) return SSD_ERR_INVALID_ARG;
    }

    ssd::stage_begin();  // a new stage record for this call (empty when no kernel is timed)
    if (L == 0) {
        if (!final_state) return SSD_OK;
        return hip_status(ssd::launch_state_copy(init_state, final_state, n_state, stream));
    }
    if (noalloc && b_ws > 0) {
        rc = noalloc_scratch(stream, &workspace);
        if (rc != SSD_OK) return rc;
    }

    ssd::PrefillArgs a;
    a.B = B; a.L = varlen ? 0 : L; a.H = H; a.P = P; a.G = G; a.N = N; a.Q = q;
    a.nchunks = varlen ? (int)slots : (L + q - 1) / q;
    a.T = (int)rows;
    a.cu_seqlens = varlen ? cu_seqlens : nullptr;
    a.x = x; a.dt = dt; a.A_log = A_log; a.Bm = Bm; a.Cm = Cm; a.D = D;
    a.dtp = dtp;
    a.init_state = init_state; a.y = y; a.final_state = final_state;
    char *ws = (char *)workspace;
    const bool four = !chain || varlen;  // packed sequences: either form may run
    a.ws_S = four ? (float *)(ws + wl.off_S) : nullptr;
    a.ws_dec = four ? (float *)(ws + wl.off_dec) : nullptr;
    a.ws_cs = mfma ? nullptr : (double *)(ws + wl.off_cs);
    a.ws_hb = mfma && four ? (uint16_t *)(ws + wl.off_hb) : nullptr;
    a.ws_ctl = chain ? (int *)(ws + wl.off_ctl) : nullptr;
    a.ws_ring = chain ? (float *)(ws + wl.off_ring) : nullptr;
    a.handoff_ticks = g_handoff_ticks < 0 ? ssd::kHandoffTicks : (unsigned long long)g_handoff_ticks;
    a.handoff_jitter = g_handoff_jitter;
    a.packed_form = g_packed_form;
    a.ws_gt = mfma ? (uint16_t *)(ws + wl.off_gt) : nullptr;
    a.ws_bt = mfma ? (uint16_t *)(ws + wl.off_bt) : nullptr;
    a.ws_ct = mfma ? (uint16_t *)(ws + wl.off_ct) : nullptr;
    a.ws_cb = mfma ? nullptr : (float *)(ws + wl.off_gt);
    a.chunks = nullptr;
    a.seqs = nullptr;
    a.ws_items = nullptr;
    if (varlen) {
        ssd::ChunkEntry *chunks = (ssd::ChunkEntry *)(ws + wl.off_tab);
        ssd::SeqEntry *seqs = (ssd::SeqEntry *)(ws + wl.off_tab + (size_t)slots * sizeof(ssd::ChunkEntry));
        unsigned *items = chain ? (unsigned *)(ws + wl.off_items) : nullptr;
        int *scratch = chain ? (int *)(items + ssd::chunk_table_item_ints(slots, B)) : nullptr;
        hipError_t e = ssd::launch_chunk_table(a, chunks, seqs, stream, items, scratch, true);
        if (e != hipSuccess) return hip_status(e);
        a.chunks = chunks;
        a.seqs = seqs;
        a.ws_items = items;
    }
    hipError_t e;
    if (chain && varlen) {
        // both forms; the chunk table's choice runs, the other exits at once
        e = ssd::launch_prefill_chain(a, stream);
        if (e == hipSuccess) e = ssd::launch_prefill_mfma(a, stream, true);
    } else {
        e = chain  ? ssd::launch_prefill_chain(a, stream)
            : mfma ? ssd::launch_prefill_mfma(a, stream)
                   : ssd::launch_prefill_vector(a, dtype, stream);
    }
    return hip_status(e);
}

int decode_impl(int B, int H, int P, int G, int N, int dtype,
                const void *x_t, const float *dt_t, const float *A_log,
                const void *B_t, const void *C_t, const float *D,
                float *ssm_state, void *y_t, long in_stride,
                const void *conv_state_in, void *conv_state_out,
                const void *conv_w, const void *conv_b, int K,
                int activation, hipStream_t stream, const ssd::DtPrep &dtp) {
    if (!valid_dtype(dtype)) return SSD_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || P < 1 || G < 1 || N < 1 || H % G != 0 || in_stride < 0) return SSD_ERR_INVALID_ARG;
    if (!x_t || !dt_t || !A_log || !B_t || !C_t || !ssm_state || !y_t) return SSD_ERR_INVALID_ARG;
    if (!(N == 16 || N == 32 || N == 64 || N == 128 || N == 256) || P > 1024) return SSD_ERR_UNSUPPORTED;
    const long HP = (long)H * P, GN = (long)G * N, C = HP + 2 * GN;
    if (in_stride != 0 && (in_stride < HP || in_stride < GN)) return SSD_ERR_INVALID_ARG;
    const bool conv = conv_state_in != nullptr;
    if (conv) {
        if (!conv_state_out || !conv_w) return SSD_ERR_INVALID_ARG;
        if (K < 2 || K > 8 || (activation != 0 && activation != 1)) return SSD_ERR_INVALID_ARG;
    }
    const size_t es = esize(dtype);
    if (!aligned(ssm_state, 16) || !aligned(x_t, es) || !aligned(B_t, es) || !aligned(C_t, es) ||
        !aligned(y_t, es) || !aligned(dt_t, 4) || !aligned(A_log, 4) || !aligned(D, 4))
        return SSD_ERR_ALIGNMENT;
    if (conv && (!aligned(conv_state_in, es) || !aligned(conv_state_out, es) || !aligned(conv_w, es) ||
                 !aligned(conv_b, es)))
        return SSD_ERR_ALIGNMENT;

    const long xs = in_stride ? in_stride : HP, bs = in_stride ? in_stride : GN;
    const size_t b_x = ((size_t)(B - 1) * xs + HP) * es, b_bc = ((size_t)(B - 1) * bs + GN) * es;
    const size_t b_state = (size_t)B * H * P * N * 4, b_y = (size_t)B * HP * es;
    const size_t b_conv = conv ? (size_t)B * C * (K - 1) * es : 0;
    struct R { const void *p; size_t n; };
    const R ins[] = {{x_t, b_x}, {B_t, b_bc}, {C_t, b_bc}, {dt_t, (size_t)B * H * 4}, {A_log, (size_t)H * 4},
                     {D, D ? (size_t)H * 4 : 0}, {dtp.dt_bias, dtp.dt_bias ? (size_t)H * 4 : 0}, {conv_state_in, b_conv},
                     {conv ? conv_w : nullptr, conv ? (size_t)C * K * es : 0},
                     {conv ? conv_b : nullptr, (conv && conv_b) ? (size_t)C * es : 0}};
    for (const R &r : ins) {
        if (overlap(y_t, b_y, r.p, r.n) || overlap(ssm_state, b_state, r.p, r.n)) return SSD_ERR_INVALID_ARG;
        if (conv && overlap(conv_state_out, b_conv, r.p, r.n)) return SSD_ERR_INVALID_ARG;
    }
    if (overlap(y_t, b_y, ssm_state, b_state)) return SSD_ERR_INVALID_ARG;
    if (conv && (overlap(conv_state_out, b_conv, y_t, b_y) || overlap(conv_state_out, b_conv, ssm_state, b_state)))
        return SSD_ERR_INVALID_ARG;

    ssd::DecodeArgs a;
    a.B = B; a.H = H; a.P = P; a.G = G; a.N = N; a.K = K; a.activation = activation;
    a.in_stride = in_stride;
    a.x_t = x_t; a.dt_t = dt_t; a.A_log = A_log; a.B_t = B_t; a.C_t = C_t; a.D = D;
    a.dtp = dtp;
    a.state = ssm_state; a.y_t = y_t;
    a.conv_in = conv ? conv_state_in : nullptr;
    a.conv_out = conv ? conv_state_out : nullptr;
    a.conv_w = conv ? conv_w : nullptr;
    a.conv_b = conv ? conv_b : nullptr;
    return hip_status(ssd::launch_decode(a, dtype, stream));
}

}  // namespace

SSD_API int ssd_prefill(int B, int L, int H, int P, int G, int N, int Q, int dtype,
                        const void *x, const float *dt, const float *A_log,
                        const void *Bm, const void *Cm, const float *D,
                        const float *init_state, void *y, float *final_state,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return prefill_impl(B, L, H, P, G, N, Q, dtype, nullptr, x, dt, A_log, Bm, Cm, D, init_state, y, final_state,
                        workspace, workspace_bytes, stream, ssd::DtPrep{0, nullptr, 0.0f, 0.0f});
}

SSD_API int ssd_prefill_noalloc(int B, int L, int H, int P, int G, int N, int Q, int dtype,
                                const void *x, const float *dt, const float *A_log,
                                const void *Bm, const void *Cm, const float *D,
                                const float *init_state, void *y, float *final_state, hipStream_t stream) {
    return prefill_impl(B, L, H, P, G, N, Q, dtype, nullptr, x, dt, A_log, Bm, Cm, D, init_state, y, final_state,
                        nullptr, 0, stream, ssd::DtPrep{0, nullptr, 0.0f, 0.0f}, false, true);
}

SSD_API int ssd_prefill_varlen(int B, int T, int H, int P, int G, int N, int Q, int dtype, const int *cu_seqlens,
                               const void *x, const float *dt, const float *A_log,
                               const void *Bm, const void *Cm, const float *D,
                               const float *init_state, void *y, float *final_state,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return prefill_impl(B, T, H, P, G, N, Q, dtype, cu_seqlens, x, dt, A_log, Bm, Cm, D, init_state, y,
                        final_state, workspace, workspace_bytes, stream, ssd::DtPrep{0, nullptr, 0.0f, 0.0f}, true);
}

SSD_API int ssd_prefill_varlen_dt_raw(int B, int T, int H, int P, int G, int N, int Q, int dtype,
                                      const int *cu_seqlens, const void *x, const float *dt_raw,
                                      const float *dt_bias, float dt_min, float dt_max, const float *A_log,
                                      const void *Bm, const void *Cm, const float *D,
                                      const float *init_state, void *y, float *final_state,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dt_prep(dt_min, dt_max, dt_bias)) return aligned(dt_bias, 4) ? SSD_ERR_INVALID_ARG : SSD_ERR_ALIGNMENT;
    return prefill_impl(B, T, H, P, G, N, Q, dtype, cu_seqlens, x, dt_raw, A_log, Bm, Cm, D, init_state, y,
                        final_state, workspace, workspace_bytes, stream, ssd::DtPrep{1, dt_bias, dt_min, dt_max},
                        true);
}

SSD_API int ssd_prefill_dt_raw(int B, int L, int H, int P, int G, int N, int Q, int dtype,
                               const void *x, const float *dt_raw, const float *dt_bias, float dt_min,
                               float dt_max, const float *A_log, const void *Bm, const void *Cm,
                               const float *D, const float *init_state, void *y, float *final_state,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dt_prep(dt_min, dt_max, dt_bias)) return aligned(dt_bias, 4) ? SSD_ERR_INVALID_ARG : SSD_ERR_ALIGNMENT;
    return prefill_impl(B, L, H, P, G, N, Q, dtype, nullptr, x, dt_raw, A_log, Bm, Cm, D, init_state, y,
                        final_state, workspace, workspace_bytes, stream, ssd::DtPrep{1, dt_bias, dt_min, dt_max});
}

SSD_API int ssd_decode_step(int B, int H, int P, int G, int N, int dtype,
                            const void *x_t, const float *dt_t, const float *A_log,
                            const void *B_t, const void *C_t, const float *D,
                            float *ssm_state, void *y_t, long in_stride,
                            const void *conv_state_in, void *conv_state_out,
                            const void *conv_w, const void *conv_b, int K,
                            int activation, hipStream_t stream) {
    return decode_impl(B, H, P, G, N, dtype, x_t, dt_t, A_log, B_t, C_t, D, ssm_state, y_t, in_stride,
                       conv_state_in, conv_state_out, conv_w, conv_b, K, activation, stream,
                       ssd::DtPrep{0, nullptr, 0.0f, 0.0f});
}

SSD_API int ssd_decode_step_dt_raw(int B, int H, int P, int G, int N, int dtype,
                                   const void *x_t, const float *dt_raw, const float *dt_bias, float dt_min,
                                   float dt_max, const float *A_log, const void *B_t, const void *C_t,
                                   const float *D, float *ssm_state, void *y_t, long in_stride,
                                   const void *conv_state_in, void *conv_state_out,
                                   const void *conv_w, const void *conv_b, int K,
                                   int activation, hipStream_t stream) {
    if (!valid_dt_prep(dt_min, dt_max, dt_bias)) return aligned(dt_bias, 4) ? SSD_ERR_INVALID_ARG : SSD_ERR_ALIGNMENT;
    return decode_impl(B, H, P, G, N, dtype, x_t, dt_raw, A_log, B_t, C_t, D, ssm_state, y_t, in_stride,
                       conv_state_in, conv_state_out, conv_w, conv_b, K, activation, stream,
                       ssd::DtPrep{1, dt_bias, dt_min, dt_max});
}

SSD_API int conv_state_update(int B, int T, int C, int K, int dtype, void *conv_state,
                              const void *xBC, const void *conv_w, const void *conv_b,
                              int activation, void *out, hipStream_t stream) {
    if (!valid_dtype(dtype)) return SSD_ERR_INVALID_ARG;
    if (B < 1 || T < 0 || C < 1 || K < 2 || K > 8 || (activation != 0 && activation != 1)) return SSD_ERR_INVALID_ARG;
    if (!conv_state || !conv_w || (T > 0 && !xBC)) return SSD_ERR_INVALID_ARG;
    if (B > 65535 || ((long)T + 15) / 16 > 65535) return SSD_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    if (!aligned(conv_state, es) || !aligned(xBC, es) || !aligned(conv_w, es) || !aligned(conv_b, es) ||
        !aligned(out, es))
        return SSD_ERR_ALIGNMENT;
    const size_t b_state = (size_t)B * C * (K - 1) * es, b_x = (size_t)B * T * C * es;
    const size_t b_w = (size_t)C * K * es, b_b = conv_b ? (size_t)C * es : 0;
    if (overlap(conv_state, b_state, xBC, b_x) || overlap(conv_state, b_state, conv_w, b_w) ||
        overlap(conv_state, b_state, conv_b, b_b))
        return SSD_ERR_INVALID_ARG;
    if (out && (overlap(out, b_x, xBC, b_x) || overlap(out, b_x, conv_state, b_state) ||
                overlap(out, b_x, conv_w, b_w) || overlap(out, b_x, conv_b, b_b)))
        return SSD_ERR_INVALID_ARG;
    if (T == 0) return SSD_OK;
    ssd::ConvArgs a;
    a.B = B; a.T = T; a.C = C; a.K = K; a.activation = activation;
    a.state = conv_state; a.xBC = xBC; a.w = conv_w; a.bias = conv_b; a.out = out;
    a.blocks = nullptr; a.seqs = nullptr; a.nslots = 0;
    return hip_status(ssd::launch_conv_update(a, dtype, stream));
}

namespace {
size_t conv_varlen_ws(int B, int T) {
    const long slots = ssd::varlen_slots(T, B, ssd::kConvSlotTokens);
    return T > 0 ? align_up((size_t)slots * sizeof(ssd::ChunkEntry) + (size_t)B * sizeof(ssd::SeqEntry), 256) : 0;
}
}  // namespace

SSD_API size_t conv_state_update_varlen_workspace_bytes(int B, int T) {
    if (B < 1 || T < 0) return (size_t)-1;
    return conv_varlen_ws(B, T);
}

SSD_API int conv_state_update_varlen(int B, int T, int C, int K, int dtype, const int *cu_seqlens, void *conv_state,
                                     const void *xBC, const void *conv_w, const void *conv_b, int activation,
                                     void *out, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(dtype)) return SSD_ERR_INVALID_ARG;
    if (B < 1 || T < 0 || C < 1 || K < 2 || K > 8 || (activation != 0 && activation != 1)) return SSD_ERR_INVALID_ARG;
    if (!cu_seqlens || !conv_state || !conv_w || (T > 0 && !xBC)) return SSD_ERR_INVALID_ARG;
    const size_t es = esize(dtype);
    const int V = (int)(16 / es);
    if (C % V != 0 || (long)C / V > 65535L * 64) return SSD_ERR_UNSUPPORTED;
    if (!aligned(cu_seqlens, 4) || !aligned(conv_state, 16) || !aligned(xBC, 16) || !aligned(conv_w, 16) ||
        !aligned(conv_b, 16) || !aligned(out, 16) || !aligned(workspace, 256))
        return SSD_ERR_ALIGNMENT;
    const size_t b_state = (size_t)B * C * (K - 1) * es, b_x = (size_t)T * C * es;
    const size_t b_w = (size_t)C * K * es, b_b = conv_b ? (size_t)C * es : 0, b_cu = (size_t)(B + 1) * 4;
    const size_t b_ws = conv_varlen_ws(B, T);
    struct R { const void *p; size_t n; };
    const R ins[] = {{xBC, b_x}, {conv_w, b_w}, {conv_b, b_b}, {cu_seqlens, b_cu}};
    for (const R &r : ins) {
        if (overlap(conv_state, b_state, r.p, r.n) || overlap(out, b_x, r.p, r.n)) return SSD_ERR_INVALID_ARG;
        if (overlap(workspace, b_ws, r.p, r.n)) return SSD_ERR_INVALID_ARG;
    }
    if (overlap(out, b_x, conv_state, b_state) || overlap(workspace, b_ws, conv_state, b_state) ||
        overlap(workspace, b_ws, out, b_x))
        return SSD_ERR_INVALID_ARG;
    if (T == 0) return SSD_OK;
    if (!workspace || workspace_bytes < b_ws) return SSD_ERR_WORKSPACE;
    // the slot table of kConvSlotTokens-token blocks, built on the device
    ssd::PrefillArgs t{};
    t.B = B; t.T = T; t.Q = ssd::kConvSlotTokens; t.cu_seqlens = cu_seqlens;
    t.nchunks = (int)ssd::varlen_slots(T, B, ssd::kConvSlotTokens);
    ssd::ChunkEntry *blocks = (ssd::ChunkEntry *)workspace;
    ssd::SeqEntry *seqs = (ssd::SeqEntry *)((char *)workspace + (size_t)t.nchunks * sizeof(ssd::ChunkEntry));
    hipError_t e = ssd::launch_chunk_table(t, blocks, seqs, stream);
    if (e != hipSuccess) return hip_status(e);
    ssd::ConvArgs a;
    a.B = B; a.T = T; a.C = C; a.K = K; a.activation = activation;
    a.state = conv_state; a.xBC = xBC; a.w = conv_w; a.bias = conv_b; a.out = out;
    a.blocks = blocks; a.seqs = seqs; a.nslots = t.nchunks;
    return hip_status(ssd::launch_conv_update(a, dtype, stream));
}

SSD_API int ssd_gated_rmsnorm(long rows, int D, int group, int dtype, const void *y, const void *z, long z_stride,
                              const float *norm_w, float eps, void *out, hipStream_t stream) {
    if (!valid_dtype(dtype)) return SSD_ERR_INVALID_ARG;
    if (rows < 0 || D < 1 || group < 1 || D % group != 0 || !(eps >= 0.0f && eps < 1e30f)) return SSD_ERR_INVALID_ARG;
    if (rows > 0 && (!y || !out)) return SSD_ERR_INVALID_ARG;
    if (z && z_stride < D) return SSD_ERR_INVALID_ARG;
    const size_t es = esize(dtype);
    const int V = (int)(16 / es), gv = group / V;
    if (group % V != 0 || D / V > ssd::kNormMaxVecs || rows > 0x7fffffffL) return SSD_ERR_UNSUPPORTED;
    if (gv <= 64 ? (gv & (gv - 1)) != 0 : gv % 64 != 0) return SSD_ERR_UNSUPPORTED;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(z, 16) || !aligned(norm_w, 16) || (z && z_stride % V != 0))
        return SSD_ERR_ALIGNMENT;
    // out is y itself or disjoint from every input
    const size_t b_y = mul(mul((size_t)rows, (size_t)D), es);
    const size_t b_z = z && rows > 0 ? mul(mul((size_t)(rows - 1), (size_t)z_stride) + (size_t)D, es) : 0;
    const size_t b_w = norm_w ? (size_t)D * sizeof(float) : 0;
    if ((out != y && overlap(out, b_y, y, b_y)) || overlap(out, b_y, z, b_z) || overlap(out, b_y, norm_w, b_w))
        return SSD_ERR_INVALID_ARG;
    if (rows == 0) return SSD_OK;
    ssd::NormArgs a;
    a.rows = rows; a.D = D; a.group = group; a.z_stride = z_stride;
    a.y = y; a.z = z; a.w = norm_w; a.eps = eps; a.out = out;
    return hip_status(ssd::launch_gated_rmsnorm(a, dtype, stream));
}

// ---- stage timing (per host thread)
namespace {
constexpr int kMaxStages = 8;
struct StageTimer {
    bool on = false, have_events = false;
    int n = 0;  // kernels recorded for the last call
    hipEvent_t start[kMaxStages], stop[kMaxStages];
    const char *name[kMaxStages];
};
thread_local StageTimer g_timer;
}  // namespace

void ssd::stage_begin() { g_timer.n = 0; }

bool ssd::stage_events(const char *kernel, hipEvent_t *start, hipEvent_t *stop) {
    if (!g_timer.on || g_timer.n >= kMaxStages) return false;
    *start = g_timer.start[g_timer.n];
    *stop = g_timer.stop[g_timer.n];
    g_timer.name[g_timer.n++] = kernel;
    return true;
}

SSD_API int ssd_stage_timing(int enable) {
    if (enable && !g_timer.have_events) {
        int made = 0;
        hipError_t e = hipSuccess;
        for (; made < 2 * kMaxStages; ++made) {
            e = hipEventCreate(made < kMaxStages ? &g_timer.start[made] : &g_timer.stop[made - kMaxStages]);
            if (e != hipSuccess) break;
        }
        if (e != hipSuccess) {
            for (int j = 0; j < made; ++j)
                (void)hipEventDestroy(j < kMaxStages ? g_timer.start[j] : g_timer.stop[j - kMaxStages]);
            return hip_status(e);
        }
        g_timer.have_events = true;
    }
    g_timer.on = enable != 0;
    g_timer.n = 0;
    return SSD_OK;
}

SSD_API int ssd_stage_times(float *ms, int capacity, int *count) {
    if (!count || capacity < 0 || (capacity > 0 && !ms)) return SSD_ERR_INVALID_ARG;
    const int n = g_timer.n;
    *count = n;
    for (int i = 0; i < n && i < capacity; ++i) {
        hipError_t e = hipEventSynchronize(g_timer.stop[i]);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], g_timer.start[i], g_timer.stop[i]);
        if (e != hipSuccess) return hip_status(e);
    }
    return SSD_OK;
}

SSD_API int ssd_debug_handoff_ticks(long long ticks) {
    g_handoff_ticks = ticks < 0 ? -1 : ticks;
    return SSD_OK;
}

SSD_API int ssd_debug_handoff_jitter(int max_rounds) {
    if (max_rounds < 0 || max_rounds > 100000) return SSD_ERR_INVALID_ARG;
    g_handoff_jitter = (unsigned)max_rounds;
    return SSD_OK;
}

SSD_API int ssd_debug_packed_form(int form) {
    if (form < -1 || form > 1) return SSD_ERR_INVALID_ARG;
    g_packed_form = form;
    return SSD_OK;
}

SSD_API const char *ssd_stage_name(int index) {
    return (index >= 0 && index < g_timer.n) ? g_timer.name[index] : nullptr;
}

SSD_API const char *ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "success";
        case SSD_ERR_INVALID_ARG: return "invalid argument (null pointer, bad dimension, G not dividing H, bad K or overlapping buffers)";
        case SSD_ERR_UNSUPPORTED: return "unsupported shape or dtype (no kernel in this library)";
        case SSD_ERR_ALIGNMENT: return "pointer or stride breaks the required alignment";
        case SSD_ERR_WORKSPACE: return "workspace missing or too small";
        case SSD_ERR_HIP: return "HIP call failed (see ssd_last_hip_error)";
        case SSD_ERR_TOO_LARGE: return "the call needs more scratch than the fixed no-allocation buffer holds";
        default: return "unknown status";
    }
}

SSD_API int ssd_last_hip_error(void) { return g_last_hip_error; }
