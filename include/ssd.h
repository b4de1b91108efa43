/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD layer scan library.
 *
 * The operation is the state space duality (SSD) scan of Mamba-2 as stated in
 * arXiv 2603.09555 (C. Santoni, "Compiler-First State Space Duality and
 * Portable O(1) Autoregressive Caching for Inference"), abstract, and in the
 * bqwf.cn article on its compiler-first implementation (§1.1 diagonal
 * per-head decay and fixed-size chunks, §1.2 intra-chunk einsum, §2.1-§2.2
 * the constant-size cache and its update).  For every batch element b and
 * head h, with A_h = -exp(A_log[h]) and g = h / (H / G):
 *
 *     state_t = exp(dt[b,t,h] * A_h) * state_{t-1}
 *               + dt[b,t,h] * x[b,t,h,:] (outer) Bm[b,t,g,:]      [P x N]
 *     y[b,t,h,p] = sum_n Cm[b,t,g,n] * state_t[p,n] + D[h] * x[b,t,h,p]
 *
 * ssd_prefill evaluates it over a whole sequence in chunks of Q tokens;
 * ssd_decode_step advances it by one token from a cached state, optionally
 * after one step of the depthwise causal convolution whose (K-1)-token input
 * window is the other half of the cache; conv_state_update runs that
 * convolution over T tokens.  Around them:
 *   - ssd_prefill_dt_raw / ssd_decode_step_dt_raw form the step from its raw
 *     projection inside the kernels (softplus, bias, clip; §1.2);
 *   - ssd_prefill_varlen (and its _dt_raw form) / conv_state_update_varlen
 *     take sequences of different lengths packed without padding;
 *   - ssd_gated_rmsnorm is the normalisation that closes the layer (the
 *     output gated by the z branch, then RMS-normalised per group, §3.2).
 *
 * Conventions shared by every entry point
 *   - Layouts: dense, row-major (C-contiguous) in the shapes given, unless a
 *     row stride argument says otherwise.
 *   - Ownership: every pointer is a device pointer owned by the caller.  The
 *     library allocates nothing, frees nothing and keeps no pointer after the
 *     call returns.  Scratch memory is the caller's `workspace` (except for
 *     ssd_prefill_noalloc, which uses a fixed buffer of the library's own).
 *   - Asynchrony: calls only enqueue kernels on `stream` (0 = the null
 *     stream) and return without synchronising.  Results are valid once the
 *     caller has synchronised with the stream.
 *   - Errors: 0 on success, a negative SSD_ERR_* code otherwise.  All
 *     argument checks run on the host before any HIP call, so a rejected call
 *     launches nothing and leaves every output untouched.  A failed launch
 *     returns SSD_ERR_HIP; its hipError_t is kept per host thread and read by
 *     ssd_last_hip_error().  Faults inside a kernel surface at the caller's
 *     next synchronisation, as for any HIP library.  No C++ exception crosses
 *     this interface.
 *   - Re-entrancy: no global mutable state apart from two per-host-thread
 *     records (the last HIP error and the optional stage timing below) and
 *     the per-GPU scratch address of ssd_prefill_noalloc (set once per GPU
 *     under a lock); calls on different streams may run concurrently as long
 *     as their buffers do not overlap (ssd_prefill_noalloc: see there).
 *   - dtype: SSD_F32 or SSD_BF16, the storage type of the activations named
 *     "void*" below (x, Bm, Cm, y and the conv data).  dt, A_log, D and the
 *     SSM state are always fp32; all arithmetic accumulates in fp32 (the
 *     in-chunk cumsum of the fp32 vector path in fp64).
 */
#ifndef MAMBA_SSD_H
#define MAMBA_SSD_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SSD_F32 = 0,
    SSD_BF16 = 1,
};

enum {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARG = -1, /* null required pointer, bad dimension, G not dividing H, K < 2, aliasing */
    SSD_ERR_UNSUPPORTED = -2, /* shape / dtype combination the library has no kernel for */
    SSD_ERR_ALIGNMENT = -3,   /* a pointer or row stride breaks the documented alignment */
    SSD_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the query returned */
    SSD_ERR_HIP = -5,         /* a HIP call failed; see ssd_last_hip_error() */
    SSD_ERR_TOO_LARGE = -6,   /* ssd_prefill_noalloc: the call needs more scratch than its fixed buffer */
};

/* Size of the fixed per-GPU scratch buffer of ssd_prefill_noalloc. */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * ssd_prefill -- chunked SSD scan over a whole sequence.
 * Source: bqwf.cn article §1.1 (sequence split into fixed-size chunks; dense
 * matrix work inside a chunk, a light sequential scan of the state between
 * chunks; decay matrix tril(exp(segsum(dt*A)))) and §1.2 (intra-chunk
 * product C B^T masked by the decay, applied to the discretised input).
 *
 *   x      [B,L,H,P]  dtype       input of every head
 *   dt     [B,L,H]    fp32        discretisation step, already positive (the
 *                                 caller applies softplus / clipping)
 *   A_log  [H]        fp32        A_h = -exp(A_log[h])
 *   Bm, Cm [B,L,G,N]  dtype       input and output projections per group
 *   D      [H]        fp32        skip weight; NULL means 0
 *   init_state  [B,H,P,N] fp32    state before token 0; NULL means zeros
 *   y      [B,L,H,P]  dtype       output; must not overlap any input
 *   final_state [B,H,P,N] fp32    state after token L-1; NULL to skip; may be
 *                                 the same buffer as init_state
 *   workspace, workspace_bytes    device scratch of at least
 *                                 ssd_prefill_workspace_bytes(...) bytes,
 *                                 256-byte aligned (NULL allowed if that is 0)
 *
 * Q is the chunk length (the last chunk may be shorter: L need not be a
 * multiple of Q).  L = 0 is allowed: y is untouched and final_state receives
 * init_state (or zeros).  Alignment: x, Bm, Cm, y, init_state, final_state
 * 16-byte aligned.  Limits: 1 <= P <= 256, 1 <= N <= 256, 1 <= Q <= 1024
 * (Q = 512 is the chunk suggested for contexts beyond 8k tokens, bqwf.cn
 * article §6.3).  bf16 with (P, N) = (64, 128) and Q a multiple of 256 runs
 * on MFMA (bf16 operands, fp32 accumulation, decay factors in fp32) in
 * 256-token sub-chunks linked by the state pass: the chunked scan is the same
 * for any chunk length up to rounding, and 256 is the chunk these kernels are
 * built for.  Every other shape runs on the fp32 vector path with chunks of
 * exactly Q tokens.  The MFMA path factors the decay
 * exp(cs_l - cs_s) per 32-token tile; a chunk whose factors would leave the
 * normal fp32 range (a token more than 60 from its tile reference in cumsum
 * of dt*A, tile references more than 80 apart, dt <= 0, or |D/dt| > 1e30)
 * is computed on an exact per-element path instead, automatically.
 */
int ssd_prefill(int B, int L, int H, int P, int G, int N, int Q, int dtype,
                const void *x, const float *dt, const float *A_log,
                const void *Bm, const void *Cm, const float *D,
                const float *init_state, void *y, float *final_state,
                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_prefill_dt_raw -- ssd_prefill with the step computed from its raw
 * value inside the kernels, dt = clamp(softplus(dt_raw + dt_bias[h]),
 * dt_min, dt_max) with softplus(u) = log(1 + exp(u)), in fp32.
 * Source: bqwf.cn article §1.2 (the softplus and clipping of the step fused
 * into the kernels that consume it instead of a separate elementwise pass).
 *
 *   dt_raw [B,L,H]  fp32   raw step (any real value)
 *   dt_bias [H]     fp32   added before softplus; NULL means 0
 *   dt_min, dt_max         0 <= dt_min <= dt_max (dt_max may be +inf); NaN is
 *                          rejected (SSD_ERR_INVALID_ARG); an unaligned
 *                          dt_bias gives SSD_ERR_ALIGNMENT
 * Every other argument, limit and error is as for ssd_prefill, and the
 * workspace size is the same.
 */
int ssd_prefill_dt_raw(int B, int L, int H, int P, int G, int N, int Q, int dtype,
                       const void *x, const float *dt_raw, const float *dt_bias,
                       float dt_min, float dt_max, const float *A_log,
                       const void *Bm, const void *Cm, const float *D,
                       const float *init_state, void *y, float *final_state,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_prefill_noalloc -- ssd_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.  It takes no workspace: the scratch is a buffer of
 * SSD_NOALLOC_SCRATCH_BYTES that the library holds in a static device array,
 * one copy per GPU (each GPU the library runs on holds it until the process
 * ends).  Its device address is looked up once per GPU, on the first call
 * made while that GPU is current; no call allocates or frees anything.
 *
 * Every argument, limit and result is as for ssd_prefill (same kernels, same
 * bits).  `stream` must belong to the current device (else
 * SSD_ERR_INVALID_ARG).  A call whose ssd_prefill_workspace_bytes(...)
 * exceeds SSD_NOALLOC_SCRATCH_BYTES returns SSD_ERR_TOO_LARGE before any HIP
 * call (the 2.7B-shaped layer at B = 1, L = 4096 needs 63.2 MiB and fits).
 * The buffer keeps the last call's contents; nothing in it needs to start at
 * zero.  All calls on one GPU share the one buffer: calls that overlap in
 * time on one GPU (different streams, or different host threads without
 * ordering between their streams) race on it and give undefined results.
 */
int ssd_prefill_noalloc(int B, int L, int H, int P, int G, int N, int Q, int dtype,
                        const void *x, const float *dt, const float *A_log,
                        const void *Bm, const void *Cm, const float *D,
                        const float *init_state, void *y, float *final_state,
                        hipStream_t stream);

/* Bytes of workspace ssd_prefill needs for these arguments (0 if none).
 * Returns (size_t)-1 for arguments ssd_prefill would reject. */
size_t ssd_prefill_workspace_bytes(int B, int L, int H, int P, int G, int N,
                                   int Q, int dtype);

/*
 * ssd_prefill_varlen -- ssd_prefill over B sequences of different lengths
 * packed one after another (no padding): sequence b is the token rows
 * [cu_seqlens[b], cu_seqlens[b + 1]) of
 *
 *   x [T,H,P], dt [T,H], Bm [T,G,N], Cm [T,G,N], y [T,H,P]
 *
 * and its scan starts from init_state[b] (or zeros) and leaves
 * final_state[b] ([B,H,P,N] as in ssd_prefill).  Each sequence is chunked
 * from its own first token (its last chunk may be short), so the result for
 * a sequence equals ssd_prefill on that sequence alone.  Source: the
 * chunked scan of bqwf.cn article §1.1-§1.2, applied per sequence.
 *
 *   cu_seqlens [B+1] int32, DEVICE memory, 4-byte aligned: 0 = cu_seqlens[0]
 *                <= cu_seqlens[1] <= ... <= cu_seqlens[B] = T.  The library
 *                reads it on the device only (no host synchronisation), so it
 *                cannot check it: offsets that break this contract give
 *                unspecified outputs but never an access outside x, y, dt,
 *                Bm, Cm or the workspace (offsets are clamped to [0, T]).
 *   T            total tokens (0 allowed: final_state receives init_state)
 * Empty sequences are allowed (their final state is their initial state).
 * The workspace (ssd_prefill_varlen_workspace_bytes) also holds the chunk
 * table the library builds on the device.  For the chained shape (bf16,
 * P = 64, N = 128, Q a multiple of 256, B*H >= 192, and fewer than 2^22 chunk
 * slots T/256 + B) the call launches both
 * prefill forms and that table's kernel picks, from the lengths, the one
 * that does the work (see ssd_debug_packed_form); the workspace then holds
 * both forms' buffers.  Every other argument, limit, alignment rule and
 * error is as for ssd_prefill; T < 2^31.
 */
int ssd_prefill_varlen(int B, int T, int H, int P, int G, int N, int Q, int dtype,
                       const int *cu_seqlens, const void *x, const float *dt, const float *A_log,
                       const void *Bm, const void *Cm, const float *D,
                       const float *init_state, void *y, float *final_state,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_prefill_varlen_dt_raw -- ssd_prefill_varlen with the step computed from
 * its raw value inside the kernels, as in ssd_prefill_dt_raw (dt_raw [T,H],
 * dt_bias [H] or NULL, 0 <= dt_min <= dt_max).  Same workspace size as
 * ssd_prefill_varlen.
 */
int ssd_prefill_varlen_dt_raw(int B, int T, int H, int P, int G, int N, int Q, int dtype,
                              const int *cu_seqlens, const void *x, const float *dt_raw,
                              const float *dt_bias, float dt_min, float dt_max, const float *A_log,
                              const void *Bm, const void *Cm, const float *D,
                              const float *init_state, void *y, float *final_state,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace ssd_prefill_varlen needs (0 if none); (size_t)-1 for
 * arguments it would reject. */
size_t ssd_prefill_varlen_workspace_bytes(int B, int T, int H, int P, int G, int N,
                                          int Q, int dtype);

/*
 * ssd_decode_step -- one token of the recurrence on the O(1) cache, fused
 * with one step of the depthwise convolution.
 * Source: bqwf.cn article §2.1 (state of shape [H,P,N] per layer plus a
 * (K-1)-token input window per conv channel) and §2.2 (cache update: roll
 * the window by one and write the new token last; state = state * A_bar +
 * B_bar * input).
 *
 *   x_t    [B, H*P]   dtype   this token's x (row stride in_stride)
 *   dt_t   [B, H]     fp32    step, already positive
 *   A_log  [H], D [H] fp32    as in ssd_prefill (D may be NULL)
 *   B_t, C_t [B, G*N] dtype   this token's Bm / Cm (row stride in_stride)
 *   ssm_state [B,H,P,N] fp32  read and updated in place; 16-byte aligned
 *   y_t    [B, H, P]  dtype   output
 *   in_stride                 elements between rows b and b+1 of x_t, B_t
 *                             and C_t; 0 means dense (H*P and G*N).  Pass
 *                             C = H*P + 2*G*N with x_t, B_t, C_t pointing
 *                             into one [B, C] token row ordered x | B | C.
 *   conv_state_in [B,C,K-1]   dtype; NULL means x_t, B_t, C_t are already
 *                             convolved (conv arguments are then ignored).
 *                             Otherwise x_t, B_t, C_t are the raw inputs of
 *                             the C = H*P + 2*G*N conv channels, in the
 *                             order x | B | C; index 0 of the window is the
 *                             oldest token, K-2 the newest.
 *   conv_state_out [B,C,K-1]  dtype; receives the window shifted by one with
 *                             the raw new token last.  Must not overlap
 *                             conv_state_in (every head reads the shared B/C
 *                             channels of the input window while the update
 *                             is written), so callers alternate two buffers.
 *   conv_w [C,K] dtype, conv_b [C] dtype (NULL means 0)
 *                             v = conv_b + sum_k conv_w[c,k] * window[k],
 *                             window[K-1] the new token; then SiLU
 *                             v / (1 + exp(-v)) if activation == 1.
 *   K                         2 <= K <= 8
 * Limits: 1 <= P <= 1024; N in {16, 32, 64, 128, 256}.
 */
int ssd_decode_step(int B, int H, int P, int G, int N, int dtype,
                    const void *x_t, const float *dt_t, const float *A_log,
                    const void *B_t, const void *C_t, const float *D,
                    float *ssm_state, void *y_t, long in_stride,
                    const void *conv_state_in, void *conv_state_out,
                    const void *conv_w, const void *conv_b, int K,
                    int activation, hipStream_t stream);

/*
 * ssd_decode_step_dt_raw -- ssd_decode_step with dt = clamp(softplus(
 * dt_raw[b,h] + dt_bias[h]), dt_min, dt_max) computed in the kernel, as in
 * ssd_prefill_dt_raw (same source, same argument rules for dt_raw [B,H],
 * dt_bias, dt_min and dt_max); everything else as for ssd_decode_step.
 */
int ssd_decode_step_dt_raw(int B, int H, int P, int G, int N, int dtype,
                           const void *x_t, const float *dt_raw, const float *dt_bias,
                           float dt_min, float dt_max, const float *A_log,
                           const void *B_t, const void *C_t, const float *D,
                           float *ssm_state, void *y_t, long in_stride,
                           const void *conv_state_in, void *conv_state_out,
                           const void *conv_w, const void *conv_b, int K,
                           int activation, hipStream_t stream);

/*
 * conv_state_update -- depthwise causal convolution over T new tokens with
 * the (K-1)-token window cache (bqwf.cn article §2.1-§2.2).  T = 1 is one
 * decode step; T = L from a zeroed cache is the convolution of a prompt,
 * which also leaves the cache ready for decoding.
 *
 *   conv_state [B,C,K-1] dtype  updated in place (index K-2 newest)
 *   xBC   [B,T,C]  dtype        raw inputs
 *   conv_w [C,K], conv_b [C] (NULL means 0)  dtype, as in ssd_decode_step
 *   out   [B,T,C]  dtype        convolved (and SiLU'd if activation) values;
 *                               NULL to update the cache only.  Must not
 *                               overlap xBC or conv_state.
 * T = 0 is allowed and changes nothing.  2 <= K <= 8.
 */
int conv_state_update(int B, int T, int C, int K, int dtype, void *conv_state,
                      const void *xBC, const void *conv_w, const void *conv_b,
                      int activation, void *out, hipStream_t stream);

/*
 * conv_state_update_varlen -- conv_state_update over B sequences packed
 * without padding, as ssd_prefill_varlen packs them: sequence b is the token
 * rows [cu_seqlens[b], cu_seqlens[b + 1]) of xBC [T,C] and out [T,C], and its
 * window starts from conv_state[b] ([B,C,K-1], updated in place to the
 * sequence's last K-1 inputs; an empty sequence keeps its cache).
 * Source: bqwf.cn article §2.1-§2.2, per sequence.
 *
 *   cu_seqlens [B+1] int32, DEVICE memory, contract as in ssd_prefill_varlen
 *   workspace  conv_state_update_varlen_workspace_bytes(B, T) bytes, 256-byte
 *              aligned (the block table the library builds on the device)
 * Requirements beyond conv_state_update's: C a multiple of 16 bytes of
 * elements (8 bf16, 4 fp32) else SSD_ERR_UNSUPPORTED; conv_state, xBC,
 * conv_w, conv_b and out 16-byte aligned else SSD_ERR_ALIGNMENT.  T = 0 is a
 * no-op.  out may be NULL (caches only).
 */
int conv_state_update_varlen(int B, int T, int C, int K, int dtype, const int *cu_seqlens, void *conv_state,
                             const void *xBC, const void *conv_w, const void *conv_b, int activation, void *out,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace conv_state_update_varlen needs; (size_t)-1 if B < 1 or
 * T < 0. */
size_t conv_state_update_varlen_workspace_bytes(int B, int T);

/*
 * ssd_gated_rmsnorm -- the normalisation that closes the layer, in the gated
 * RMS form of the Mamba-2 mixer (bqwf.cn article §3.2: normalisation fused
 * with its neighbours; §4.1: its variance in fp32 even for bf16 inputs).
 * For each of `rows` rows and each group of `group` consecutive channels:
 *
 *   g   = y * silu(z)                           (g = y when z is NULL)
 *   out = g / sqrt(mean over the group of g^2 + eps) * norm_w
 *
 * Sums, the gate and the scaling are fp32; out is rounded once to dtype.
 *
 *   y     [rows, D] dtype       the scan output (ssd_prefill's y as
 *                               [B*L, H*P], ssd_decode_step's y_t as [B, H*P])
 *   z     [rows, D] dtype or NULL, row stride z_stride elements (>= D), so z
 *                               may be a column slice of a wider projection
 *   norm_w [D] fp32 or NULL (weight 1)
 *   out   [rows, D] dtype       may be y itself (in place); otherwise it must
 *                               not overlap y, z or norm_w
 * group divides D; with V = 16 / sizeof(dtype) (8 for bf16, 4 for fp32),
 * group / V must be a power of two up to 64 or a multiple of 64 (for bf16:
 * group = 8, 16, ..., 512 or a multiple of 512 -- one head of P = 64, or
 * d_inner / ngroups of the Mamba-2 sizes), and D <= 2048 * V, else
 * SSD_ERR_UNSUPPORTED.  y, z, out and norm_w must be 16-byte aligned and
 * z_stride a multiple of V (SSD_ERR_ALIGNMENT).  eps >= 0.  rows = 0 is a
 * no-op.  Errors: SSD_ERR_INVALID_ARG for bad sizes, eps, null y/out or
 * overlapping buffers.
 */
int ssd_gated_rmsnorm(long rows, int D, int group, int dtype, const void *y, const void *z, long z_stride,
                      const float *norm_w, float eps, void *out, hipStream_t stream);

/*
 * Stage timing -- a profiling aid, kept per host thread.
 * ssd_stage_timing(1) makes the following prefill calls (ssd_prefill,
 * ssd_prefill_varlen and their raw-step forms; for packed sequences the
 * chunk-table kernel comes first) of the calling thread launch each kernel
 * with a pair of HIP events stamped when that
 * kernel's dispatch starts and ends (events created once, on the device
 * current at this call); ssd_stage_timing(0) stops it.  ssd_stage_times
 * waits for the last such call, stores in *count the number of kernels it
 * ran, and writes up to `capacity` of their durations in milliseconds, in
 * launch order; ssd_stage_name(i) names kernel i of that call (NULL out of
 * range).  Do not enable it while the stream is being captured into a graph.
 */
int ssd_stage_timing(int enable);
int ssd_stage_times(float *ms, int capacity, int *count);
const char *ssd_stage_name(int index);

/*
 * Testing aid, kept per host thread: the bound of each hand-off wait of the
 * chained single-pass prefill (the path ssd_prefill takes for bf16, P = 64,
 * N = 128, Q a multiple of 256 and B*H >= 192 chains, and packed sequences
 * of that shape whose lengths give enough chains, where chunk c of a
 * (batch, head) chain waits for chunk c-1 to publish its carried state), in
 * ticks of the 100 MHz device clock, for the calling thread's later calls.
 * ticks < 0 restores the default, 0.2 s (20 000 000 ticks).  A wait that
 * expires sets an error word in the workspace's control block and carries
 * NaN as the state, so that chunk's outputs and every later chunk of its
 * chain come out NaN: a broken hand-off shows in the results instead of
 * hanging the device.  A bound of 0 makes every wait that does not find its
 * predecessor already published expire, which is how the tests force that
 * path.  Returns SSD_OK.
 */
int ssd_debug_handoff_ticks(long long ticks);

/*
 * Testing aid, kept per host thread: delays at the chained prefill's
 * hand-off points, to shuffle the order in which workgroups reach them.  For
 * the calling thread's later calls each workgroup of the chained pass sleeps,
 * at its start, before it reads the carried state and between writing its
 * own and publishing it, for a pseudo-random number (a hash of its item) of
 * rounds of s_sleep 8 (about 0.2 us each) between 0 and max_rounds.  The
 * results do not depend on the timing, so they must not change.  0 (the
 * default) turns it off.  Errors: SSD_ERR_INVALID_ARG for max_rounds outside
 * [0, 100000].
 */
int ssd_debug_handoff_jitter(int max_rounds);

/*
 * Testing aid, kept per host thread: the form of a packed prefill
 * (ssd_prefill_varlen, ssd_prefill_varlen_dt_raw) that would take the
 * chained single pass (bf16, P = 64, N = 128, Q a multiple of 256,
 * B * H >= 192).  Such a call launches both forms and the chunk-table kernel
 * chooses on the device, from the sequence lengths, which one does the work:
 * the chained pass when H * (total chunks) / (most chunks of one sequence)
 * >= 192, else the four-kernel form (a batch dominated by one long sequence
 * would expose that sequence's hand-offs).  form = -1 (the default) keeps
 * that choice; 0 forces the four-kernel form and 1 the chained pass, for the
 * calling thread's later calls.  Both give results within the same bound of
 * the exact scan; which form ran shows in the output bits only.  Errors:
 * SSD_ERR_INVALID_ARG for form outside [-1, 1].
 */
int ssd_debug_packed_form(int form);

/* Static, human-readable text for a status code. */
const char *ssd_status_string(int status);

/* hipError_t of the last failed HIP call made by this library on the
 * calling host thread (0 if none). */
int ssd_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SSD_H */
