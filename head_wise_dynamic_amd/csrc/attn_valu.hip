// Per-query sparse attention on the vector ALUs: one wave per query row.
//
// This is the gather-bound path of the correspondence heads (SAF3R Sec. 4.1,
// "DINO Top-K Kernel"): every query reads its own cached index row and pulls
// the selected K and V rows by token index.  A wave serves one query row for
// every head of the launch, so the index row is fetched once and shared by
// all correspondence heads of the layer.  With fp32 inputs the same kernel
// runs every role (the matrix-core path is bf16-only).
//
// Lane layout: a key row is read as 16-byte pieces, LPR lanes per row
// (8 for bf16, 16 for fp32) and RPP = 64 / LPR rows per load instruction.
// Keys are consumed in chunks of NP * RPP with an online softmax (running max
// and sum in fp32, exp2 with log2(e)/sqrt(d) folded into the logit scale).
#include "device_util.h"

namespace saf {
namespace {

template <typename T> struct Lanes;
template <> struct Lanes<uint16_t> {  // bf16 bits
    static constexpr int EPL = 8, LPR = 8, RPP = 8;
    __device__ static void load(const uint16_t *p, float *x) {
        const u32x4 r = *(const u32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_bits_to_f32(r[i] & 0xFFFFu);
            x[2 * i + 1] = bf16_bits_to_f32(r[i] >> 16);
        }
    }
    __device__ static void store(uint16_t *p, const float *x) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        *(u32x4 *)p = r;
    }
};
template <> struct Lanes<float> {
    static constexpr int EPL = 4, LPR = 16, RPP = 4;
    __device__ static void load(const float *p, float *x) {
        const f32x4 r = *(const f32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = r[i];
    }
    __device__ static void store(float *p, const float *x) {
        *(f32x4 *)p = f32x4{x[0], x[1], x[2], x[3]};
    }
};

constexpr int NP = 8;  // row loads per chunk and lane

template <typename T>
__device__ void attend_row(const ValuLaunch &L, const HeadWork &w, int64_t qtok, int32_t qframe,
                           const int32_t *idx_row, int64_t count, int lane) {
    using E = Lanes<T>;
    constexpr int EPL = E::EPL, LPR = E::LPR, RPP = E::RPP, CH = NP * RPP;
    const Geom &g = L.g;
    const int sub = lane % LPR, grp = lane / LPR;
    const int64_t hoff = (int64_t)w.head * L.head_stride, ts = L.token_stride;
    const T *Q = (const T *)L.q + hoff;
    const T *K = (const T *)L.k + hoff;
    const T *V = (const T *)L.v + hoff;

    float qv[EPL];
    E::load(Q + qtok * ts + sub * EPL, qv);
    const float sc = kLog2e * 0.125f;

    float m_run = -INFINITY, l_run = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    for (int64_t c0 = 0; c0 < count; c0 += CH) {
        int64_t tok[NP];
        float s[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int64_t m = c0 + p * RPP + grp;
            tok[p] = -1;
            if (m < count) tok[p] = idx_row ? (int64_t)idx_row[m] : key_token(w, g, m, qframe);
        }
        float kx[NP][EPL];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (tok[p] >= 0) {
                E::load(K + tok[p] * ts + sub * EPL, kx[p]);
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) kx[p][e] = 0.f;
            }
        }
        float cm = -INFINITY;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e], kx[p][e], dot);
#pragma unroll
            for (int x = 1; x < LPR; x <<= 1) dot += __shfl_xor(dot, x);
            s[p] = tok[p] >= 0 ? dot * sc : -INFINITY;
            cm = fmaxf(cm, s[p]);
        }
#pragma unroll
        for (int x = LPR; x < 64; x <<= 1) cm = fmaxf(cm, __shfl_xor(cm, x));
        if (cm == -INFINITY) continue;  // wave-uniform: every slot masked
        const float m_new = fmaxf(m_run, cm);
        const float alpha = fast_exp2(m_run - m_new);
        float lsum = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            s[p] = fast_exp2(s[p] - m_new);
            lsum += s[p];
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (tok[p] >= 0) {
                float vx[EPL];
                E::load(V + tok[p] * ts + sub * EPL, vx);
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = fmaf(s[p], vx[e], o[e]);
            }
        }
    }
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) {
        l_run += __shfl_xor(l_run, x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], x);
    }
    if (grp == 0) {
        const float inv = 1.f / l_run;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= inv;
        E::store((T *)L.o + hoff + qtok * ts + sub * EPL, o);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void valu_attn_kernel(const ValuLaunch L, int64_t nrows) {
    const Geom &g = L.g;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= nrows) return;
    int64_t tok, u = -1;
    if (L.patch_rows_only) {
        u = gw;
        tok = (u / g.P) * g.T + g.ns + (u % g.P);
    } else {
        tok = gw;
        const int64_t t = tok % g.T;
        if (t >= g.ns) u = (tok / g.T) * g.P + (t - g.ns);
    }
    const int32_t qframe = (int32_t)(tok / g.T);
    for (int i = 0; i < L.nwork; ++i) {
        const HeadWork w = L.work[i];
        const int32_t *idx_row = nullptr;
        int64_t count;
        if (w.role == CORRESPONDENCE) {
            if (u >= 0) {
                idx_row = L.corr_idx + u * L.corr_k;
                count = L.corr_k;
            } else {
                HeadWork d = w;
                d.role = DENSE;
                attend_row<T>(L, d, tok, qframe, nullptr, g.N, lane);
                continue;
            }
        } else {
            count = key_count(w, g, qframe);
        }
        attend_row<T>(L, w, tok, qframe, idx_row, count, lane);
    }
}

}  // namespace

hipError_t launch_valu_attention(const ValuLaunch &L, int64_t nrows, hipStream_t stream) {
    if (nrows <= 0 || L.nwork <= 0) return hipSuccess;
    const dim3 grid((unsigned)((nrows + 3) / 4));
    if (L.g.dtype == BF16)
        hipLaunchKernelGGL(valu_attn_kernel<uint16_t>, grid, dim3(256), 0, stream, L, nrows);
    else
        hipLaunchKernelGGL(valu_attn_kernel<float>, grid, dim3(256), 0, stream, L, nrows);
    return hipGetLastError();
}

}  // namespace saf
