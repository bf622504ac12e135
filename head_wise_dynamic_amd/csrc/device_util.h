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

// Window of a broadcast head around patch position p: patches
// (y0 + j / wx) * gw + x0 + j % wx for j < n.  gw = 0 is a single row of P
// patches (a window along the patch index).
struct BcastWindow {
    int32_t y0, x0, wx, n, gw;
};
__device__ __forceinline__ BcastWindow bcast_window(const HeadWork &w, const Geom &g, int32_t p) {
    const int32_t r = w.budget, gw = w.anchor > 0 ? w.anchor : g.P, gh = g.P / gw;
    const int32_t y = p / gw, x = p % gw;
    BcastWindow b;
    b.gw = gw;
    b.y0 = max(0, y - r);
    b.x0 = max(0, x - r);
    b.wx = min(gw - 1, x + r) - b.x0 + 1;
    b.n = (min(gh - 1, y + r) - b.y0 + 1) * b.wx;
    return b;
}

// Token index of the m-th key of a head's key set (see HeadWork); -1 marks a
// masked slot (a special token already on the scanning stride).  qsel selects
// the query's set: its frame for POSITION, its patch position for BROADCAST.
__device__ __forceinline__ int64_t key_token(const HeadWork &w, const Geom &g, int64_t m,
                                             int32_t qsel) {
    switch (w.role) {
    case POSITION: {
        const int64_t nsS = (int64_t)g.ns * g.S;
        if (m < nsS) return (m / g.ns) * g.T + (m % g.ns);
        m -= nsS;
        if (m < g.P) return (int64_t)w.anchor * g.T + g.ns + m;
        m -= g.P;
        return (int64_t)qsel * g.T + g.ns + m;
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
    case BROADCAST: {
        const int64_t nsS = (int64_t)g.ns * g.S;
        if (m < nsS) return (m / g.ns) * g.T + (m % g.ns);
        m -= nsS;
        const BcastWindow b = bcast_window(w, g, qsel);
        const int32_t f = (int32_t)(m / b.n), j = (int32_t)(m % b.n);
        return (int64_t)f * g.T + g.ns + (int64_t)(b.y0 + j / b.wx) * b.gw + b.x0 + j % b.wx;
    }
    default:
        return m;
    }
}

__device__ __forceinline__ int64_t key_count(const HeadWork &w, const Geom &g, int32_t qsel) {
    switch (w.role) {
    case POSITION:
        return (int64_t)g.ns * g.S + g.P + (qsel != w.anchor ? g.P : 0);
    case SCANNING:
        return (g.N + w.budget - 1) / w.budget + (int64_t)g.ns * g.S;
    case VERTICAL:
        return w.list_len;
    case BROADCAST:
        return (int64_t)g.ns * g.S + (int64_t)g.S * bcast_window(w, g, qsel).n;
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
