// prefill_state_pass.hip -- the sequential scan of the state across chunks.
//
// bqwf.cn article on the compiler-first Mamba-2 implementation of
// arXiv 2603.09555, §1.1: chunks are linked by a light sequential scan that
// carries the state from one chunk to the next,
//     h_{-1} = init_state (or 0),   h_c = exp(cs_last(c)) * h_{c-1} + S_c.
// ws_dec holds exp(cs_last(c)) - 1.
// The recurrence is elementwise over the P*N state entries of a (batch, head),
// so each lane owns VEC consecutive entries and walks the chunks in order;
// lanes of a wavefront cover consecutive entries, so every chunk's slice is
// read and written with fully coalesced accesses.  Chunk states are loaded a
// batch of kBatch chunks ahead of the dependent FMA chain.  The slot of chunk
// c is overwritten in place with the carried-in state h_{c-1} that the
// output stage needs; the final h goes to final_state.
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;

template <int VEC>
struct VecT;
template <> struct VecT<1> { typedef float type; };
template <> struct VecT<4> { typedef float4 type; };

__device__ __forceinline__ void vzero(float &v) { v = 0.0f; }
__device__ __forceinline__ void vzero(float4 &v) { v = make_float4(0.f, 0.f, 0.f, 0.f); }
// h + (dm1 * h + s) with dm1 = exp(chunk sum of dt*A) - 1: the state is
// rounded once per chunk, and a decay close to 1 is not quantised to the fp32
// grid below 1.
__device__ __forceinline__ float step(float dm1, float h, float s) { return h + fmaf(dm1, h, s); }
__device__ __forceinline__ float4 step(float dm1, float4 h, float4 s) {
    return make_float4(step(dm1, h.x, s.x), step(dm1, h.y, s.y), step(dm1, h.z, s.z), step(dm1, h.w, s.w));
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void state_pass_kernel(PrefillArgs a, long total) {
    typedef typename VecT<VEC>::type V;
    const long e = (long)blockIdx.x * kThreads + threadIdx.x;
    if (e >= total) return;
    const long PNv = (long)a.P * a.N / VEC;
    const long bh = e / PNv;
    const long pn = e - bh * PNv;
    const int h = (int)(bh % a.H);
    const SeqEntry sq = seq_chunks(a, bh / a.H);
    V hv;
    if (a.init_state) hv = ((const V *)a.init_state)[bh * PNv + pn];
    else vzero(hv);
    const int nch = sq.n;
    for (int c0 = 0; c0 < nch; c0 += kBatch) {
        V sv[kBatch];
        float dv[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (c0 + j < nch) {
                const long hc = ((long)sq.f0 + c0 + j) * a.H + h;
                sv[j] = ((const V *)(a.ws_S + hc * a.P * a.N))[pn];
                dv[j] = a.ws_dec[hc];
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (c0 + j < nch) {
                const long hc = ((long)sq.f0 + c0 + j) * a.H + h;
                ((V *)(a.ws_S + hc * a.P * a.N))[pn] = hv;
                hv = step(dv[j], hv, sv[j]);
            }
        }
    }
    if (a.final_state) ((V *)a.final_state)[bh * PNv + pn] = hv;
}

__global__ __launch_bounds__(kThreads) void state_copy_kernel(const float *src, float *dst, long n) {
    const long i = (long)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

}  // namespace

hipError_t launch_state_pass(const PrefillArgs &a, hipStream_t s) {
    const long PN = (long)a.P * a.N;
    const bool vec4 = (PN % 4) == 0;
    const long total = (long)a.B * a.H * (vec4 ? PN / 4 : PN);
    const long blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (blocks == 0) return hipSuccess;
    return vec4 ? launch_stage("state_pass", state_pass_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a,
                               total)
                : launch_stage("state_pass", state_pass_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a,
                               total);
}

// dst[i] = src ? src[i] : 0 (the L = 0 case of a prefill; src == dst allowed).
hipError_t launch_state_copy(const float *src, float *dst, size_t n, hipStream_t s) {
    if (n == 0 || src == dst) return hipSuccess;
    const long blocks = (long)((n + kThreads - 1) / kThreads);
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, src, dst, (long)n);
    return hipGetLastError();
}

}  // namespace ssd
