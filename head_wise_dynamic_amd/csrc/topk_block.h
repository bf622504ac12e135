// Exact top-K selection helpers shared by the index builders.
//
// Ordering everywhere: score descending, then index ascending.  Scores are
// mapped to order-preserving u32 keys so ties are exact bit equality.
#pragma once

#include "device_util.h"

namespace saf {

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_to_float(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Inclusive scan of one u32 over a block of NW waves (blockDim = 64 * NW).
template <int NW>
__device__ uint32_t block_scan_incl(uint32_t x, uint32_t *sh /*[NW]*/, uint32_t *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wv] = x;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
    for (int i = 0; i < NW; ++i) {
        if (i < wv) pre += sh[i];
        tot += sh[i];
    }
    __syncthreads();
    *total = tot;
    return x + pre;
}

// Radix digits of the selection: 11 + 11 + 10 bits of the order key.
constexpr int kTopkDigit1Shift = 21;
constexpr int kTopkDigit1Bins = 2048;

// Apply f(j, key) to every j in [0, n) in a block-strided order (any order
// is fine for histograms).  Loads go out eight at a time from always-valid
// addresses so that they are in flight together; 16-byte loads when the
// scores are 16-byte aligned.
template <int NT, typename F>
__device__ __forceinline__ void for_each_key(const float *scores, int64_t n, F f) {
    const int tid = threadIdx.x;
    if (((uintptr_t)scores & 15u) == 0) {
        const int64_t n4 = n >> 2;
        const f32x4 *s4 = (const f32x4 *)scores;
        for (int64_t b = 0; b < n4; b += 8 * NT) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t i = b + u * NT + tid;
                v[u] = s4[i < n4 ? i : n4 - 1];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t i = b + u * NT + tid;
                if (i < n4) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) f(4 * i + e, order_key(v[u][e]));
                }
            }
        }
        for (int64_t j = 4 * n4 + tid; j < n; j += NT) f(j, order_key(scores[j]));
    } else {
        for (int64_t b = 0; b < n; b += 8 * NT) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t j = b + u * NT + tid;
                v[u] = scores[j < n ? j : n - 1];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t j = b + u * NT + tid;
                if (j < n) f(j, order_key(v[u]));
            }
        }
    }
}

// From a histogram hist[0..nbins) (LDS) and the rank `remaining` (1-based)
// counted from the top, find the digit d holding that rank: bins above d
// hold fewer than `remaining` keys, bins >= d at least that many.  Writes d
// and the rank inside bin d to *digit / *rem (LDS).  NT threads; nbins is a
// multiple of NT.
template <int NT>
__device__ void pick_digit(const uint32_t *hist, int nbins, uint32_t remaining, uint32_t *sh, uint32_t *digit,
                           uint32_t *rem) {
    const int tid = threadIdx.x, per = nbins / NT;
    // thread t owns bins nbins-1-per*t .. nbins-per*(t+1) (from the top)
    uint32_t c = 0;
    for (int i = 0; i < per; ++i) c += hist[nbins - 1 - per * tid - i];
    uint32_t tot;
    const uint32_t before = block_scan_incl<NT / 64>(c, sh, &tot) - c;
    if (before < remaining && remaining <= before + c) {
        uint32_t acc = before;
        for (int i = 0; i < per; ++i) {
            const uint32_t h = hist[nbins - 1 - per * tid - i];
            if (acc + h >= remaining) {
                *digit = (uint32_t)(nbins - 1 - per * tid - i);
                *rem = remaining - acc;
                break;
            }
            acc += h;
        }
    }
    __syncthreads();
}

// Block-wide exact top-K over scores[0..n) (NT = 1024 threads).  Writes the
// kept positions in ascending order through emit(pos, j).  K must be <= n.
// hist1 (optional, global memory): a complete histogram of
// order_key(score) >> kTopkDigit1Shift over all n scores, which saves the
// first pass over them.
template <typename Emit>
__device__ void block_topk_ascending(const float *scores, int64_t n, int64_t K, Emit emit,
                                     const uint32_t *hist1 = nullptr) {
    constexpr int NT = 1024;
    __shared__ uint32_t hist[kTopkDigit1Bins];
    __shared__ uint32_t sh[NT / 64];
    __shared__ uint32_t s_digit, s_rem;
    const int tid = threadIdx.x;
    if (K >= n) {
        for (int64_t j = tid; j < n; j += NT) emit(j, j);
        return;
    }
    // digit 1: bits 31..21
    for (int i = tid; i < kTopkDigit1Bins; i += NT) hist[i] = hist1 ? hist1[i] : 0u;
    __syncthreads();
    if (!hist1) {
        for_each_key<NT>(scores, n, [&](int64_t, uint32_t u) { atomicAdd(&hist[u >> kTopkDigit1Shift], 1u); });
        __syncthreads();
    }
    pick_digit<NT>(hist, kTopkDigit1Bins, (uint32_t)K, sh, &s_digit, &s_rem);
    uint32_t prefix = s_digit << 21, remaining = s_rem;
    // digit 2: bits 20..10 of the keys whose bits 31..21 match
    for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
    __syncthreads();
    for_each_key<NT>(scores, n, [&](int64_t, uint32_t u) {
        if ((u >> 21) == (prefix >> 21)) atomicAdd(&hist[(u >> 10) & 2047u], 1u);
    });
    __syncthreads();
    pick_digit<NT>(hist, 2048, remaining, sh, &s_digit, &s_rem);
    prefix |= s_digit << 10;
    remaining = s_rem;
    // digit 3: bits 9..0
    for (int i = tid; i < 1024; i += NT) hist[i] = 0u;
    __syncthreads();
    for_each_key<NT>(scores, n, [&](int64_t, uint32_t u) {
        if ((u >> 10) == (prefix >> 10)) atomicAdd(&hist[u & 1023u], 1u);
    });
    __syncthreads();
    pick_digit<NT>(hist, 1024, remaining, sh, &s_digit, &s_rem);
    const uint32_t thr = prefix | s_digit, need_eq = s_rem;

    // ordered compaction: thread t owns [t * per, (t + 1) * per), per a
    // multiple of 4 so that aligned scores are read 16 bytes at a time
    const int64_t per = ((n + NT - 1) / NT + 3) & ~(int64_t)3;
    const int64_t j0 = min<int64_t>(n, (int64_t)tid * per), j1 = min<int64_t>(n, j0 + per);
    const bool vec = ((uintptr_t)scores & 15u) == 0;
    auto walk = [&](auto f) {
        int64_t j = j0;
        if (vec) {
            for (; j + 16 <= j1; j += 16) {
                f32x4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = *(const f32x4 *)(scores + j + 4 * u);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) f(j + 4 * u + e, order_key(v[u][e]));
            }
        }
        for (; j < j1; ++j) f(j, order_key(scores[j]));
    };
    uint32_t cgt = 0, ceq = 0;
    walk([&](int64_t, uint32_t u) {
        cgt += u > thr;
        ceq += u == thr;
    });
    uint32_t tot;
    const uint32_t gt_before = block_scan_incl<NT / 64>(cgt, sh, &tot) - cgt;
    const uint32_t eq_before = block_scan_incl<NT / 64>(ceq, sh, &tot) - ceq;
    uint32_t pos = gt_before + min(eq_before, need_eq);
    uint32_t eq_rank = eq_before;
    walk([&](int64_t j, uint32_t u) {
        bool sel = u > thr;
        if (u == thr) {
            sel = eq_rank < need_eq;
            ++eq_rank;
        }
        if (sel) emit(pos++, j);
    });
}

}  // namespace saf
