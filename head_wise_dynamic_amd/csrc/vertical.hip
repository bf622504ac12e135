// Vertical-line key selection (SAF3R Sec. 4.3, "Query-Probe Top-K Kernel").
//
// The column average of S = Q K^T / sqrt(D) over all N queries equals
// qbar K^T / sqrt(D) with qbar the mean query, so the key ranking needs one
// O(N d) pass instead of the N x N score matrix:
//   1. probe_partial:  per-block channel sums of Q (fp32), fixed order
//   2. probe_final:    qbar = (sum of partials) / N
//   3. probe_scores:   r_j = qbar . k_j / sqrt(d) (fp32), 8 lanes per key row
//   4. topk_select:    exact top-K of r by (r desc, j asc), written ascending:
//                      MSB-first radix select on order-preserving u32 keys
//                      (four 8-bit digits) finds the K-th largest value, then
//                      an ordered compaction keeps every larger key and the
//                      lowest-index keys equal to it.
// All passes are HBM/L2 streaming; the pages call the probe's cost
// negligible next to attention.
#include <algorithm>

#include "device_util.h"
#include "topk_block.h"

namespace saf {
namespace {

constexpr int kMaxVert = 16;

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
    uint32_t *scratch;
};
__device__ inline WsView ws_view(char *base, int64_t N) {
    WsView v;
    v.partial = (float *)base;
    v.qbar = (float *)(base + align256(sizeof(float) * kProbeBlocks * 64));
    v.scores = (float *)((char *)v.qbar + align256(sizeof(float) * 64));
    v.scratch = (uint32_t *)((char *)v.scores + align256(sizeof(float) * N));
    return v;
}

template <typename T> __device__ inline float ld(const T *p);
template <> __device__ inline float ld<float>(const float *p) { return *p; }
template <> __device__ inline float ld<uint16_t>(const uint16_t *p) { return bf16_bits_to_f32(*p); }

// grid (kProbeBlocks, nh), 256 threads: thread = (channel c, row group rg)
template <typename T> __global__ __launch_bounds__(256) void probe_partial(const VertBatch B) {
    __shared__ float red[4][64];
    const int slot = blockIdx.y;
    const int64_t N = B.g.N;
    const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
    const T *Q = (const T *)B.q + (int64_t)B.head[slot] * B.head_stride;
    const int64_t per = (N + kProbeBlocks - 1) / kProbeBlocks;
    const int64_t r0 = (int64_t)blockIdx.x * per, r1 = min<int64_t>(N, r0 + per);
    float acc = 0.f;
    for (int64_t r = r0 + rg; r < r1; r += 4) acc += ld<T>(Q + r * B.token_stride + c);
    red[rg][c] = acc;
    __syncthreads();
    if (rg == 0) {
        WsView v = ws_view(B.ws[slot], N);
        v.partial[blockIdx.x * 64 + c] = ((red[0][c] + red[1][c]) + (red[2][c] + red[3][c]));
    }
}

// grid (1, nh), 64 threads
__global__ void probe_final(const VertBatch B) {
    const int slot = blockIdx.y, c = threadIdx.x;
    WsView v = ws_view(B.ws[slot], B.g.N);
    float acc = 0.f;
    for (int b = 0; b < kProbeBlocks; ++b) acc += v.partial[b * 64 + c];
    v.qbar[c] = acc / (float)B.g.N;
}

// grid (ceil(N/32), nh), 256 threads: 8 lanes per key row, 32 keys per block
template <typename T> __global__ __launch_bounds__(256) void probe_scores(const VertBatch B) {
    const int slot = blockIdx.y;
    const int64_t N = B.g.N;
    WsView v = ws_view(B.ws[slot], N);
    const int sub = threadIdx.x & 7;
    const int64_t j = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const T *K = (const T *)B.k + (int64_t)B.head[slot] * B.head_stride;
    float acc = 0.f;
    if (j < N) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(v.qbar[sub * 8 + e], ld<T>(K + j * B.token_stride + sub * 8 + e), acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (j < N && sub == 0) v.scores[j] = acc * 0.125f;  // 1/sqrt(64)
}

// grid (1, nh), 1024 threads
__global__ __launch_bounds__(1024) void topk_select(const VertBatch B) {
    const int slot = blockIdx.y;
    const int64_t N = B.g.N;
    WsView v = ws_view(B.ws[slot], N);
    const int64_t K = min<int64_t>(B.K[slot], N);
    int32_t *out = B.idx_out[slot];
    block_topk_ascending(v.scores, N, K, [&](int64_t pos, int64_t j) { out[pos] = (int32_t)j; });
}

}  // namespace

size_t vertical_ws_bytes(int64_t N) {
    return align256(sizeof(float) * kProbeBlocks * 64) + align256(sizeof(float) * 64) +
           align256(sizeof(float) * N) + align256(sizeof(uint32_t) * kTopkScratch);
}

hipError_t launch_vertical_batch(const Geom &g, const void *q, const void *k, int64_t head_stride,
                                 int64_t token_stride, int nh, const int32_t *heads, const int32_t *Ks,
                                 int32_t *const *idx_out, void *const *ws, hipStream_t stream) {
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
        if (g.dtype == BF16)
            hipLaunchKernelGGL(probe_partial<uint16_t>, dim3(kProbeBlocks, n), dim3(256), 0, stream, B);
        else
            hipLaunchKernelGGL(probe_partial<float>, dim3(kProbeBlocks, n), dim3(256), 0, stream, B);
        hipLaunchKernelGGL(probe_final, dim3(1, n), dim3(64), 0, stream, B);
        const unsigned sb = (unsigned)((g.N + 31) / 32);
        if (g.dtype == BF16)
            hipLaunchKernelGGL(probe_scores<uint16_t>, dim3(sb, n), dim3(256), 0, stream, B);
        else
            hipLaunchKernelGGL(probe_scores<float>, dim3(sb, n), dim3(256), 0, stream, B);
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
