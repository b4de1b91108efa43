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

__global__ __launch_bounds__(kTabThreads) void chunk_table_kernel(PrefillArgs a, ChunkEntry *chunks, SeqEntry *seqs) {
    __shared__ long long wsum[kTabThreads / 64];
    __shared__ long long carry;
    __shared__ SeqEntry pass_seq[kTabThreads];  // this pass's sequences, for the entry writers
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long long slots = a.nchunks;
    if (tid == 0) carry = 0;
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
}

}  // namespace

hipError_t launch_chunk_table(const PrefillArgs &a, ChunkEntry *chunks, SeqEntry *seqs, hipStream_t s) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kTabThreads), 0, s, a, chunks, seqs);
    return hipGetLastError();
}

}  // namespace ssd
