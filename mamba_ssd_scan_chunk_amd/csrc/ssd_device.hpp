// ssd_device.hpp -- device helpers shared by the SSD kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_internal.hpp"

namespace ssd {

typedef uint16_t bf16_t;  // raw bfloat16 bits

// ---------------------------------------------------------------- dtypes

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two floats -> packed pair of bf16 (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

template <typename T> __device__ __forceinline__ float ld(const T *p);
template <> __device__ __forceinline__ float ld<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t *p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ void st(T *p, float v);
template <> __device__ __forceinline__ void st<float>(float *p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t *p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// clamp(softplus(u), lo, hi), softplus(u) = log(1 + exp(u)) (u itself above
// 20, where the difference is below fp32 resolution).
__device__ __forceinline__ float dt_softplus_clamp(float u, float lo, float hi) {
    const float sp = u > 20.0f ? u : log1pf(expf(u));
    return fminf(fmaxf(sp, lo), hi);
}

// dt of head h from the value read: itself, or clamp(softplus(v + bias[h]),
// lo, hi).
__device__ __forceinline__ float dt_value(float v, int raw, const float *bias, int h, float lo, float hi) {
    if (!raw) return v;
    return dt_softplus_clamp(v + (bias ? bias[h] : 0.0f), lo, hi);
}

// ---------------------------------------------------------------- chunk slots
// The chunk in slot f (see PrefillArgs): from the slot table for packed
// sequences, by arithmetic for a uniform batch.
__device__ __forceinline__ ChunkEntry chunk_at(const PrefillArgs &a, long f) {
    if (a.chunks) return a.chunks[f];
    ChunkEntry e;
    e.seq = (int)(f / a.nchunks);
    e.c = (int)(f - (long)e.seq * a.nchunks);
    e.tok0 = e.seq * a.L + e.c * a.Q;
    e.Qc = min(a.Q, a.L - e.c * a.Q);
    return e;
}
// Slots of sequence b's chunks: [f0, f0 + n).
__device__ __forceinline__ SeqEntry seq_chunks(const PrefillArgs &a, long b) {
    if (a.seqs) return a.seqs[b];
    SeqEntry e;
    e.f0 = (int)(b * a.nchunks);
    e.n = a.nchunks;
    e.tok0 = (int)(b * a.L);
    e.len = a.L;
    return e;
}

// ---------------------------------------------------------------- wave ops

// Inclusive prefix sum across the 64 lanes of a wavefront, with DPP moves:
// row_shr 1, 2, 4, 8 scan each row of 16 lanes (lanes shifted in from
// outside the row read 0), then row_bcast 15 adds the last lane of rows 0
// and 2 to rows 1 and 3, and row_bcast 31 the last lane of row 1 to rows
// 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shift_add(float v) {
    const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false);
    return v + __int_as_float(moved);
}
__device__ __forceinline__ float wave_inclusive_sum(float v) {
    v = dpp_shift_add<0x111, 0xf>(v);  // row_shr:1
    v = dpp_shift_add<0x112, 0xf>(v);  // row_shr:2
    v = dpp_shift_add<0x114, 0xf>(v);  // row_shr:4
    v = dpp_shift_add<0x118, 0xf>(v);  // row_shr:8
    v = dpp_shift_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_shift_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of
// the group receives the group total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------- 16-byte vectors
// V = 16 / sizeof(T) elements per 16-byte access, widened to fp32.  act() is
// SiLU: for bf16 with the hardware exp2 and reciprocal (relative error ~1e-7,
// far below bf16 rounding), for fp32 with expf and IEEE division.
template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
    static constexpr int V = 8;
    __device__ static void unpack(const uint4 &r, float (&f)[8]) {
        const unsigned w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static uint4 pack(const float (&f)[8]) {
        unsigned w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
    __device__ static float act(float v) {
        return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * 1.44269504088896341f));
    }
};
template <> struct Vec16<float> {
    static constexpr int V = 4;
    __device__ static void unpack(const uint4 &r, float (&f)[4]) {
        f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
    __device__ static uint4 pack(const float (&f)[4]) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
    __device__ static float act(float v) { return silu(v); }
};

}  // namespace ssd
