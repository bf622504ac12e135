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

// Block-wide exact top-K over scores[0..n) (1024 threads).  Writes the kept
// positions in ascending order through emit(pos, j).  K must be <= n.
template <typename Emit>
__device__ void block_topk_ascending(const float *scores, int64_t n, int64_t K, Emit emit) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh[16];
    __shared__ uint32_t s_digit, s_rem;
    const int tid = threadIdx.x;
    if (K >= n) {
        for (int64_t j = tid; j < n; j += 1024) emit(j, j);
        return;
    }
    uint32_t prefix = 0, mask = 0, remaining = (uint32_t)K;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += 1024) hist[i] = 0;
        __syncthreads();
        for (int64_t j = tid; j < n; j += 1024) {
            const uint32_t u = order_key(scores[j]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t cum = 0;
            int dsel = 0;
            for (int dgt = 255; dgt >= 0; --dgt) {
                if (cum + hist[dgt] >= remaining) {
                    dsel = dgt;
                    break;
                }
                cum += hist[dgt];
            }
            s_digit = (uint32_t)dsel;
            s_rem = remaining - cum;
        }
        __syncthreads();
        prefix |= s_digit << shift;
        mask |= 255u << shift;
        remaining = s_rem;
        __syncthreads();
    }
    const uint32_t thr = prefix, need_eq = remaining;
    const int64_t per = (n + 1023) / 1024;
    const int64_t j0 = min<int64_t>(n, (int64_t)tid * per), j1 = min<int64_t>(n, j0 + per);
    uint32_t cgt = 0, ceq = 0;
    for (int64_t j = j0; j < j1; ++j) {
        const uint32_t u = order_key(scores[j]);
        cgt += u > thr;
        ceq += u == thr;
    }
    uint32_t tot;
    const uint32_t gt_before = block_scan_incl<16>(cgt, sh, &tot) - cgt;
    const uint32_t eq_before = block_scan_incl<16>(ceq, sh, &tot) - ceq;
    uint32_t pos = gt_before + min(eq_before, need_eq);
    uint32_t eq_rank = eq_before;
    for (int64_t j = j0; j < j1; ++j) {
        const uint32_t u = order_key(scores[j]);
        bool sel = u > thr;
        if (u == thr) {
            sel = eq_rank < need_eq;
            ++eq_rank;
        }
        if (sel) emit(pos++, j);
    }
}

}  // namespace saf
