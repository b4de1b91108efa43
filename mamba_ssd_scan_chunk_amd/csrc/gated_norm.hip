// gated_norm.hip -- the normalisation that closes the layer, in the gated
// RMS form of the Mamba-2 mixer (bqwf.cn article on the compiler-first
// Mamba-2 implementation of arXiv 2603.09555: §3.2 fuses the normalisation
// with its neighbours, §4.1 computes its variance in fp32 even for bf16
// inputs).  For each row and each group of `group` consecutive channels:
//
//   g = y * silu(z)                      (g = y without a gate)
//   out = g * rsqrt(mean over the group of g^2 + eps) * w
//
// One workgroup per row (four waves, or sixteen when rows are few).  Thread
// t owns the 16-byte vectors t, t + NT, ..., so every load and store
// instruction of a wave covers 1 KiB of the row.  The sums of squares are
// fp32: a group of gv <= 64 vectors is an aligned set of gv lanes within
// one wave instruction (a butterfly over gv lanes, no LDS), and a group of a
// multiple of 64 vectors is a run of whole wave instructions (a wave sum per
// instruction, one LDS slot each, one barrier).  The gate's SiLU is Vec16's
// (hardware exp2 and reciprocal for bf16).  All loads of a row (y, z and
// the fp32 weights, which every row shares and so mostly hit L2) are issued
// before any arithmetic, so a row costs one memory round trip.  out may be
// y itself.
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

template <typename T, int NT, int VPT>
__global__ __launch_bounds__(NT) void gated_rmsnorm_kernel(NormArgs a) {
    using VT = Vec16<T>;
    constexpr int V = VT::V;
    constexpr int WV = V / 4;       // float4 weight loads per vector
    constexpr int W = NT / 64;      // waves per row
    __shared__ float slot_sum[kNormMaxVecs / 64];
    const int tid = threadIdx.x, wave = tid >> 6;
    const long row = blockIdx.x;
    const int nvec = a.D / V;
    const int gv = a.group / V;     // vectors per group
    const uint4 *yp = (const uint4 *)((const T *)a.y + row * a.D);
    const uint4 *zp = a.z ? (const uint4 *)((const T *)a.z + row * a.z_stride) : nullptr;
    const float4 *wp = (const float4 *)a.w;

    uint4 yv[VPT], zv[VPT];
    float4 wv[VPT][WV];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = tid + NT * i;
        const bool ok = v < nvec;
        yv[i] = ok ? yp[v] : make_uint4(0, 0, 0, 0);
        zv[i] = (ok && zp) ? zp[v] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = tid + NT * i;
#pragma unroll
        for (int j = 0; j < WV; ++j)
            wv[i][j] = (v < nvec && wp) ? wp[v * WV + j] : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    }

    // gated values, and their sums of squares over the aligned min(gv, 64)
    // lanes of each instruction
    float g[VPT][V], tot[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        VT::unpack(yv[i], g[i]);
        if (zp) {
            float zf[V];
            VT::unpack(zv[i], zf);
#pragma unroll
            for (int e = 0; e < V; ++e) g[i][e] *= VT::act(zf[e]);
        }
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < V; ++e) s = fmaf(g[i][e], g[i][e], s);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            if (off < gv) s += __shfl_xor(s, off, 64);
        tot[i] = s;
    }
    if (gv > 64) {
        // 64-vector slot i * W + wave holds one wave instruction; a group is a
        // run of m = gv / 64 slots
        const int m = gv >> 6;
        if ((tid & 63) == 0) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int slot = i * W + wave;
                if (slot * 64 < nvec) slot_sum[slot] = tot[i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int first = (i * W + wave) / m * m;
            float t = 0.0f;
            if (first * 64 < nvec)
                for (int k = 0; k < m; ++k) t += slot_sum[first + k];
            tot[i] = t;
        }
    }

    uint4 *op = (uint4 *)((T *)a.out + row * a.D);
    const float inv_group = 1.0f / (float)a.group;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = tid + NT * i;
        if (v >= nvec) continue;
        const float r = 1.0f / sqrtf(fmaf(tot[i], inv_group, a.eps));
        const float *wf = (const float *)&wv[i][0];
#pragma unroll
        for (int e = 0; e < V; ++e) g[i][e] = g[i][e] * r * wf[e];
        op[v] = VT::pack(g[i]);
    }
}

template <typename T, int NT, int VPT>
hipError_t launch_v(const NormArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T, NT, VPT>), dim3((unsigned)a.rows), dim3(NT), 0, s, a);
    return hipGetLastError();
}

template <typename T, int NT>
hipError_t launch_nt(const NormArgs &a, hipStream_t s) {
    static_assert(kNormMaxVecs <= 8 * 256 && kNormMaxVecs <= 2 * 1024, "vectors per thread");
    const int need = (a.D / Vec16<T>::V + NT - 1) / NT;  // vectors per thread
    if (need <= 1) return launch_v<T, NT, 1>(a, s);
    if constexpr (NT == 1024) {
        return launch_v<T, NT, 2>(a, s);
    } else {
        if (need <= 2) return launch_v<T, NT, 2>(a, s);
        if (need <= 3) return launch_v<T, NT, 3>(a, s);
        if (need <= 4) return launch_v<T, NT, 4>(a, s);
        if (need <= 6) return launch_v<T, NT, 6>(a, s);
        return launch_v<T, NT, 8>(a, s);
    }
}

// Four waves per row when there are enough rows to fill the chip twice over
// (2048 workgroups); sixteen when rows are few (a decode step's B rows), so
// that each lane holds about one vector and a row takes one round trip.
template <typename T>
hipError_t launch_t(const NormArgs &a, hipStream_t s) {
    return a.rows >= 2048 ? launch_nt<T, 256>(a, s) : launch_nt<T, 1024>(a, s);
}

}  // namespace

// Host-side checks have established: D % group == 0, group a multiple of V,
// group / V a power of two up to 64 or a multiple of 64, D / V <=
// kNormMaxVecs, 16-byte aligned rows, z_stride a multiple of V.
hipError_t launch_gated_rmsnorm(const NormArgs &a, int dtype, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    return dtype == DT_BF16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace ssd
