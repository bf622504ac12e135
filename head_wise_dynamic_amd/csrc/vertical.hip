// Vertical-line key selection (SAF3R Sec. 4.3, "Query-Probe Top-K Kernel").
//
// The column average of S = Q K^T / sqrt(D) over all N queries equals
// qbar K^T / sqrt(D) with qbar the mean query, so the key ranking needs one
// O(N d) pass instead of the N x N score matrix:
//   1. probe_partial:  per-block channel sums of Q (fp32), fixed order;
//                      block 0 also clears the head's radix histogram
//   2. probe_scores:   qbar = (sum of the partials) / N, recomputed by every
//                      block in the same fixed order; r_j = qbar . k_j /
//                      sqrt(d) (fp32), stored, and a histogram of the top 11
//                      bits of r's order-preserving key (global atomics)
//   3. topk_select:    exact top-K of r by (r desc, j asc), written ascending:
//                      MSB-first radix select (11 + 11 + 10 bits, the first
//                      digit's histogram already built) finds the K-th largest
//                      value, then an ordered compaction keeps every larger key
//                      and the lowest-index keys equal to it.
// Passes 1 and 2 stream Q and K once with 16-byte loads, several rows in
// flight per lane; the pages call the probe's cost negligible next to
// attention, and at these rates it is (HBM-bound, two reads of N x d).
#include <algorithm>

#include "device_util.h"
#include "topk_block.h"

namespace saf {
namespace {

constexpr int kMaxVert = 16;
constexpr int kThreads = 256;
constexpr int kRowsInFlight = 8;  // 16-byte row pieces per lane and step

struct VertBatch {
    Geom g;
    const void *q, *k;
    int64_t head_stride, token_stride;
    int32_t nh;
    int32_t head[kMaxVert];
    int32_t K[kMaxVert];
    int32_t *idx_out[kMaxVert];
    char *ws[kMaxVert];
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsView {
    float *partial, *qbar, *scores;
    uint32_t *hist;  // [kTopkDigit1Bins] histogram of the first radix digit
};
__device__ inline WsView ws_view(char *base, int64_t N) {
    WsView v;
    v.partial = (float *)base;
    v.qbar = (float *)(base + align256(sizeof(float) * kProbeBlocks * 64));
    v.scores = (float *)((char *)v.qbar + align256(sizeof(float) * 64));
    v.hist = (uint32_t *)((char *)v.scores + align256(sizeof(float) * N));
    return v;
}

// One row's 64 channels as 16-byte pieces: EPL elements per lane, LPR lanes
// per row, RPW rows per wave.
template <typename T> struct Piece;
template <> struct Piece<uint16_t> {
    static constexpr int EPL = 8, LPR = 8, RPW = 8;
    __device__ static void unpack(const u32x4 &r, float *x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_bits_to_f32(r[i] & 0xFFFFu);
            x[2 * i + 1] = bf16_bits_to_f32(r[i] >> 16);
        }
    }
};
template <> struct Piece<float> {
    static constexpr int EPL = 4, LPR = 16, RPW = 4;
    __device__ static void unpack(const u32x4 &r, float *x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(r[i]);
    }
};

// grid (kProbeBlocks, nh), 256 threads.  Block b sums the channels of rows
// [b * per, (b + 1) * per): each lane keeps EPL channel sums of the rows it
// reads, then the row groups are combined in a fixed order.
template <typename T> __global__ __launch_bounds__(kThreads) void probe_partial(const VertBatch B) {
    using E = Piece<T>;
    constexpr int RPB = E::RPW * (kThreads / 64);  // rows per block step
    __shared__ float red[kThreads / 64][64];
    const int slot = blockIdx.y;
    const int64_t N = B.g.N;
    WsView v = ws_view(B.ws[slot], N);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % E::LPR, rg = wave * E::RPW + lane / E::LPR;
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < kTopkDigit1Bins; i += kThreads) v.hist[i] = 0u;
    const T *Q = (const T *)B.q + (int64_t)B.head[slot] * B.head_stride;
    const int64_t per = (N + kProbeBlocks - 1) / kProbeBlocks;
    const int64_t r0 = min<int64_t>(N, (int64_t)blockIdx.x * per), r1 = min<int64_t>(N, r0 + per);
    float acc[E::EPL];
#pragma unroll
    for (int e = 0; e < E::EPL; ++e) acc[e] = 0.f;
    for (int64_t r = r0 + rg; r < r1; r += (int64_t)RPB * kRowsInFlight) {
        u32x4 raw[kRowsInFlight];
#pragma unroll
        for (int i = 0; i < kRowsInFlight; ++i) {
            const int64_t ri = r + (int64_t)i * RPB;
            raw[i] = *(const u32x4 *)(Q + (ri < r1 ? ri : r) * B.token_stride + sub * E::EPL);
        }
#pragma unroll
        for (int i = 0; i < kRowsInFlight; ++i) {
            float x[E::EPL];
            E::unpack(raw[i], x);
            const bool ok = r + (int64_t)i * RPB < r1;
#pragma unroll
            for (int e = 0; e < E::EPL; ++e) acc[e] += ok ? x[e] : 0.f;
        }
    }
    // the row groups of a wave share a channel set: lanes l, l + LPR, ...
#pragma unroll
    for (int o = E::LPR; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < E::EPL; ++e) acc[e] += __shfl_xor(acc[e], o);
    if (lane < E::LPR)
#pragma unroll
        for (int e = 0; e < E::EPL; ++e) red[wave][sub * E::EPL + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < 64) {
        const int c = threadIdx.x;
        v.partial[blockIdx.x * 64 + c] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
    }
}

// grid (ceil(N / KPB), nh), 256 threads, KPB keys per block.
constexpr int kKeysPerBlock = 256;
template <typename T> __global__ __launch_bounds__(kThreads) void probe_scores(const VertBatch B) {
    using E = Piece<T>;
    constexpr int RPB = E::RPW * (kThreads / 64);
    constexpr int STEPS = kKeysPerBlock / RPB;
    __shared__ float qb[64];
    __shared__ float part4[kThreads / 64][64];
    __shared__ float sc[kKeysPerBlock];
    __shared__ uint32_t hist[kTopkDigit1Bins];
    const int slot = blockIdx.y;
    const int64_t N = B.g.N;
    WsView v = ws_view(B.ws[slot], N);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // qbar from the partials: quarter q of the blocks per wave, each lane a
    // channel, summed in block order; quarters combined in order
    {
        const int c = lane;
        constexpr int QB = kProbeBlocks / (kThreads / 64);
        float s = 0.f;
        float x[16];
        for (int b0 = wave * QB; b0 < (wave + 1) * QB; b0 += 16) {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = v.partial[(b0 + i) * 64 + c];
#pragma unroll
            for (int i = 0; i < 16; ++i) s += x[i];
        }
        part4[wave][c] = s;
    }
    for (int i = tid; i < kTopkDigit1Bins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    if (tid < 64) {
        const float qm = ((part4[0][tid] + part4[1][tid]) + (part4[2][tid] + part4[3][tid])) / (float)N;
        qb[tid] = qm;
        if (blockIdx.x == 0) v.qbar[tid] = qm;
    }
    __syncthreads();
    const int sub = lane % E::LPR, rg = wave * E::RPW + lane / E::LPR;
    float qv[E::EPL];
#pragma unroll
    for (int e = 0; e < E::EPL; ++e) qv[e] = qb[sub * E::EPL + e];
    const T *K = (const T *)B.k + (int64_t)B.head[slot] * B.head_stride;
    const int64_t j0 = (int64_t)blockIdx.x * kKeysPerBlock;
    u32x4 raw[STEPS];
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        const int64_t j = j0 + rg + i * RPB;
        raw[i] = *(const u32x4 *)(K + (j < N ? j : N - 1) * B.token_stride + sub * E::EPL);
    }
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        float x[E::EPL];
        E::unpack(raw[i], x);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E::EPL; ++e) dot = fmaf(qv[e], x[e], dot);
#pragma unroll
        for (int o = 1; o < E::LPR; o <<= 1) dot += __shfl_xor(dot, o);
        if (sub == 0) sc[rg + i * RPB] = dot * 0.125f;  // 1/sqrt(64)
    }
    __syncthreads();
    const int64_t j = j0 + tid;
    if (j < N) {
        const float r = sc[tid];
        v.scores[j] = r;
        atomicAdd(&hist[order_key(r) >> kTopkDigit1Shift], 1u);
    }
    __syncthreads();
    for (int i = tid; i < kTopkDigit1Bins; i += kThreads)
        if (hist[i]) atomicAdd(&v.hist[i], hist[i]);
}

// grid (1, nh), 1024 threads
__global__ __launch_bounds__(1024) void topk_select(const VertBatch B) {
    const int slot = blockIdx.y;
    const int64_t N = B.g.N;
    WsView v = ws_view(B.ws[slot], N);
    const int64_t K = min<int64_t>(B.K[slot], N);
    int32_t *out = B.idx_out[slot];
    block_topk_ascending(v.scores, N, K, [&](int64_t pos, int64_t j) { out[pos] = (int32_t)j; }, v.hist);
}

}  // namespace

size_t vertical_ws_bytes(int64_t N) {
    return align256(sizeof(float) * kProbeBlocks * 64) + align256(sizeof(float) * 64) +
           align256(sizeof(float) * N) + align256(sizeof(uint32_t) * kTopkScratch);
}

hipError_t launch_vertical_batch(const Geom &g, const void *q, const void *k, int64_t head_stride,
                                 int64_t token_stride, int nh, const int32_t *heads, const int32_t *Ks,
                                 int32_t *const *idx_out, void *const *ws, hipStream_t stream) {
    static_assert(kTopkDigit1Bins <= kTopkScratch, "histogram must fit the workspace scratch");
    static_assert(kProbeBlocks % 64 == 0, "qbar reduction reads the partials 16 at a time per wave");
    for (int h0 = 0; h0 < nh; h0 += kMaxVert) {
        VertBatch B{};
        B.g = g;
        B.q = q;
        B.k = k;
        B.head_stride = head_stride;
        B.token_stride = token_stride;
        B.nh = std::min(kMaxVert, nh - h0);
        for (int i = 0; i < B.nh; ++i) {
            B.head[i] = heads[h0 + i];
            B.K[i] = Ks[h0 + i];
            B.idx_out[i] = idx_out[h0 + i];
            B.ws[i] = (char *)ws[h0 + i];
        }
        const unsigned n = (unsigned)B.nh;
        const unsigned sb = (unsigned)((g.N + kKeysPerBlock - 1) / kKeysPerBlock);
        if (g.dtype == BF16) {
            hipLaunchKernelGGL(probe_partial<uint16_t>, dim3(kProbeBlocks, n), dim3(kThreads), 0, stream, B);
            hipLaunchKernelGGL(probe_scores<uint16_t>, dim3(sb, n), dim3(kThreads), 0, stream, B);
        } else {
            hipLaunchKernelGGL(probe_partial<float>, dim3(kProbeBlocks, n), dim3(kThreads), 0, stream, B);
            hipLaunchKernelGGL(probe_scores<float>, dim3(sb, n), dim3(kThreads), 0, stream, B);
        }
        hipLaunchKernelGGL(topk_select, dim3(1, n), dim3(1024), 0, stream, B);
    }
    return hipGetLastError();
}

hipError_t launch_vertical_index(const Geom &g, const void *q, const void *k, int64_t head_stride,
                                 int64_t token_stride, int32_t head, int32_t K, int32_t *idx_out,
                                 void *ws, hipStream_t stream) {
    return launch_vertical_batch(g, q, k, head_stride, token_stride, 1, &head, &K, &idx_out, &ws, stream);
}

}  // namespace saf
