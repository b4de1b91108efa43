// chunk_table.hip -- chunk slots of a prefill over packed sequences.
//
// Sequence b is the token rows [cu_seqlens[b], cu_seqlens[b + 1]) of x, dt,
// Bm, Cm and y; it is cut into ceil(L_b / Q) chunks that start at its own
// first token, so no chunk mixes two sequences (the scan restarts from the
// sequence's initial state, as the chunked form of the bqwf.cn article on
// the compiler-first Mamba-2 implementation, §1.1, does per sequence).  One
// workgroup lays the chunks of all sequences out in consecutive slots: an
// exclusive scan of the chunk counts gives each sequence its first slot, and
// each wave then writes the entries of a share of the sequences, one entry
// per lane.
// For the chained single pass the same workgroup then lays out the item
// order.  An empty sequence counts as one chunk (its state is carried over).
// A counting sort orders the sequences by decreasing chunk count; they are
// dealt to the eight shares (one per XCD) in snake order, 0..7 then 7..0, so
// that the shares' totals stay close.  Within a share, round c holds chunk c
// of each of its sequences with more than c chunks; those are a prefix of the
// share's sequences, so chunk c of a sequence comes after its chunk c-1.
// The table kernel also chooses the form that runs the call (see kItemForm).
// Offsets are clamped to [0, T] and a negative length counts as empty, and
// slots never exceed the bound the workspace was sized for, so offsets that
// break the documented contract give unspecified results but every access
// stays inside the caller's buffers.  The prefill kernels that follow on the
// same stream read the table; slots after the last chunk get Qc = 0 and their
// workgroups exit at once.
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kTabThreads = 1024;

__device__ __forceinline__ long long wave_inclusive_sum_ll(long long v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

// One wave, over v in [0, n): above[v] = sum of hist[v' > v] (in place of
// hist), then R[c] = sum of above[c' < c]; returns the sum of above.  hist
// and R are in LDS or in global memory; the fence orders the first loop's
// stores before the second loop's loads by other lanes.
__device__ int above_and_rounds(int *hist, int *R, int n) {
    const int lane = threadIdx.x & 63;
    int acc = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {  // from v = n - 1 down
        const int i = i0 + lane, v = n - 1 - i;
        const int hv = i < n ? hist[v] : 0;
        const int inc = wave_inclusive_sum(hv);
        if (i < n) hist[v] = acc + inc - hv;
        acc += __shfl(inc, 63, 64);
    }
    __threadfence_block();
    acc = 0;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int c = c0 + lane;
        const int av = c < n ? hist[c] : 0;
        const int inc = wave_inclusive_sum(av);
        if (c < n) R[c] = acc + inc - av;
        acc += __shfl(inc, 63, 64);
    }
    return acc;
}

// The item-order histograms (hist, cnt, then xhist and xR of each share,
// kmax + 2 ints each for chunk counts up to kmax) live in LDS up to 40 KB
// (with the kernel's 16.5 KB of static LDS, under 64 KB per workgroup), else
// in scratch.
constexpr size_t kTableHistLds = 40 * 1024;
__host__ __device__ inline size_t table_hist_bytes(long kmax) {
    return (size_t)(2 + 2 * kChainXcds) * (kmax + 2) * sizeof(int);
}
__host__ __device__ inline bool table_hist_in_lds(long kmax) { return table_hist_bytes(kmax) <= kTableHistLds; }

// Share of the sequence at position j of the sorted order.
__device__ __forceinline__ int snake_share(int j) {
    const int q = j / kChainXcds, r = j % kChainXcds;
    return (q & 1) ? kChainXcds - 1 - r : r;
}

__global__ __launch_bounds__(kTabThreads) void chunk_table_kernel(PrefillArgs a, ChunkEntry *chunks, SeqEntry *seqs,
                                                                  unsigned *items, int *scratch) {
    __shared__ long long wsum[kTabThreads / 64];
    __shared__ long long carry;
    __shared__ int nmax;  // most chunks of one sequence
    __shared__ SeqEntry pass_seq[kTabThreads];  // this pass's sequences, for the entry writers
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long long slots = a.nchunks;
    if (tid == 0) {
        carry = 0;
        nmax = 0;
    }
    __syncthreads();
    for (int b0 = 0; b0 < a.B; b0 += kTabThreads) {
        const int b = b0 + tid;
        int start = 0, len = 0;
        long long n = 0;
        if (b < a.B) {
            start = min(max(a.cu_seqlens[b], 0), a.T);
            const int end = min(max(a.cu_seqlens[b + 1], 0), a.T);
            len = max(end - start, 0);
            n = (len + a.Q - 1) / a.Q;
        }
        const long long inc = wave_inclusive_sum_ll(n);
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        long long first = carry + inc - n;
        for (int w = 0; w < wave; ++w) first += wsum[w];
        if (b < a.B) {
            const long long f0 = min(first, slots);
            const int cnt = (int)min(n, slots - f0);
            const SeqEntry e{(int)f0, cnt, start, len};
            seqs[b] = e;
            pass_seq[tid] = e;
            atomicMax(&nmax, cnt);
        }
        __syncthreads();  // every thread has read carry; pass_seq is complete
        // the chunk entries: wave w writes those of the pass's sequences w,
        // w + 16, ..., one entry per lane at a time
        const int nb = min(kTabThreads, a.B - b0);
        for (int j = wave; j < nb; j += kTabThreads / 64) {
            const SeqEntry e = pass_seq[j];
            for (int c = lane; c < e.n; c += 64)
                chunks[(long long)e.f0 + c] = ChunkEntry{b0 + j, c, e.tok0 + c * a.Q, min(a.Q, e.len - c * a.Q)};
        }
        if (tid == kTabThreads - 1) carry = first + n;
        __syncthreads();  // carry is updated; pass_seq may be rewritten
    }
    const long long used = min(carry, slots);
    for (long long f = used + tid; f < slots; f += kTabThreads) chunks[f] = ChunkEntry{0, 0, 0, 0};
    if (!items) return;

    // ---- item order of the chained single pass.  k(b) = max(chunks of b, 1)
    // <= max(nmax, 1), so the histograms span n = max(nmax, 1) + 2 counts
    // (at most slots + 2, what scratch is sized for).  hist and cnt (the
    // sort), per share xhist and xR: in LDS when they fit (a generic pointer
    // then reaches LDS), else in scratch; pos (place of b in order of
    // decreasing k) in scratch.
    extern __shared__ int lds_hist[];
    const int n = max(nmax, 1) + 2;
    int *hist = table_hist_in_lds(n - 2) ? lds_hist : scratch;
    int *cnt = hist + n, *xhist = cnt + n, *xR = xhist + kChainXcds * n;
    int *pos = scratch + (long)(2 + 2 * kChainXcds) * n;
    for (int v = tid; v < (2 + kChainXcds) * n; v += kTabThreads) hist[v] = 0;  // hist, cnt, xhist
    __syncthreads();  // also: seqs[] as written above is visible to the workgroup
    for (int b = tid; b < a.B; b += kTabThreads) atomicAdd(&hist[max(seqs[b].n, 1)], 1);
    __syncthreads();
    if (wave == 0) above_and_rounds(hist, xR, n);  // hist -> above (xR is overwritten below)
    __syncthreads();
    for (int b = tid; b < a.B; b += kTabThreads) {
        const int k = max(seqs[b].n, 1);
        const int j = hist[k] + atomicAdd(&cnt[k], 1);  // any order among equal k
        pos[b] = j;
        atomicAdd(&xhist[snake_share(j) * n + k], 1);
    }
    __syncthreads();
    // wave x: the rounds of share x
    __shared__ int share_total[kChainXcds], share_base[kChainXcds];
    if (wave < kChainXcds) {
        const int total = above_and_rounds(xhist + wave * n, xR + wave * n, n);
        if (lane == 0) share_total[wave] = total;
    }
    __syncthreads();
    if (tid == 0) {
        // the form: chained when the effective chains H * (sum of chunks) /
        // (most chunks of one sequence) reach kChainMinChains
        const bool chained = a.packed_form >= 0 ? a.packed_form == 1
                                                : nmax > 0 && (long long)a.H * used >= kChainMinChains * nmax;
        items[kItemForm] = chained ? 1u : 0u;
    }
    if (tid < kChainXcds) {
        int base = 0;
        for (int x = 0; x < tid; ++x) base += share_total[x];
        share_base[tid] = base;
        items[tid] = (unsigned)share_total[tid];
        items[kChainXcds + tid] = (unsigned)base;
    }
    __syncthreads();
    // the records: one thread per chunk slot (its entry names the sequence
    // and the chunk), then one per empty sequence
    ItemEntry *recs = (ItemEntry *)(items + kItemHeader);
    for (long long f = tid; f < used; f += kTabThreads) {
        const ChunkEntry ch = chunks[f];
        const int b = ch.seq, c = ch.c;
        const int j = pos[b], x = snake_share(j), jl = j / kChainXcds;
        const bool last = c == seqs[b].n - 1;
        recs[share_base[x] + xR[x * n + c] + jl] =
            ItemEntry{(unsigned)f | (last ? kItemLast : 0u), (unsigned)b, ch.tok0, (c << kItemQcBits) | ch.Qc};
    }
    for (int b = tid; b < a.B; b += kTabThreads) {
        if (seqs[b].n != 0) continue;
        const int j = pos[b], x = snake_share(j), jl = j / kChainXcds;
        recs[share_base[x] + xR[x * n] + jl] = ItemEntry{kItemLast, kItemEmpty | (unsigned)b, 0, 0};
    }
}

}  // namespace

hipError_t launch_chunk_table(const PrefillArgs &a, ChunkEntry *chunks, SeqEntry *seqs, hipStream_t s,
                              unsigned *items, int *scratch, bool timed) {
    if (items && (!scratch || a.nchunks >= kItemMaxSlots || a.B > (int)kItemIndex || a.Q >= (1 << kItemQcBits)))
        return hipErrorInvalidValue;
    const size_t lds = items ? kTableHistLds : 0;  // the kernel uses it when the counts fit
    if (timed) return launch_stage("chunk_table_kernel", chunk_table_kernel, dim3(1), dim3(kTabThreads), lds, s, a, chunks,
                                   seqs, items, scratch);
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kTabThreads), lds, s, a, chunks, seqs, items, scratch);
    return hipGetLastError();
}

}  // namespace ssd
