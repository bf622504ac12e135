// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "saf_internal.h"

namespace saf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the hardware instruction (no range fix-up: results below the
// smallest normal may flush, which only affects weights < 2^-126).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Token index of the m-th key of a head's key set (see HeadWork); -1 marks a
// masked slot (a special token already on the scanning stride).
__device__ __forceinline__ int64_t key_token(const HeadWork &w, const Geom &g, int64_t m,
                                             int32_t qframe) {
    switch (w.role) {
    case POSITION: {
        const int64_t nsS = (int64_t)g.ns * g.S;
        if (m < nsS) return (m / g.ns) * g.T + (m % g.ns);
        m -= nsS;
        if (m < g.P) return (int64_t)w.anchor * g.T + g.ns + m;
        m -= g.P;
        return (int64_t)qframe * g.T + g.ns + m;
    }
    case SCANNING: {
        const int64_t s = w.budget;
        const int64_t nst = (g.N + s - 1) / s;
        if (m < nst) return m * s;
        m -= nst;
        const int64_t tok = (m / g.ns) * g.T + (m % g.ns);
        return (tok % s == 0) ? -1 : tok;
    }
    case VERTICAL:
        return w.list[m];
    default:
        return m;
    }
}

__device__ __forceinline__ int64_t key_count(const HeadWork &w, const Geom &g, int32_t qframe) {
    switch (w.role) {
    case POSITION:
        return (int64_t)g.ns * g.S + g.P + (qframe != w.anchor ? g.P : 0);
    case SCANNING:
        return (g.N + w.budget - 1) / w.budget + (int64_t)g.ns * g.S;
    case VERTICAL:
        return w.list_len;
    default:
        return g.N;
    }
}

// First key slot at which a masked slot may appear (SCANNING only).
__device__ __forceinline__ int64_t key_first_masked(const HeadWork &w, const Geom &g) {
    if (w.role == SCANNING) return (g.N + w.budget - 1) / w.budget;
    return INT64_MAX;
}

}  // namespace saf
