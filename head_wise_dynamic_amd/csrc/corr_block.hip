// Block-wise correspondence index (SAF3R Sec. 4.3: the block-wise
// implementation of the DINO Top-K kernel trades retrieval accuracy for a
// cheaper build by comparing blocks of tokens instead of single tokens).
//
// A block is `b` consecutive patches of one frame (b divides P).  The
// similarity of blocks A and B is the token cosine averaged over their b x b
// patch pairs, which by bilinearity is the dot product of the blocks' mean
// unit features m_A = (1/b) sum_{u in A} f_u / |f_u| (zero features count as
// 0).  So the build is:
//   1. block_means: m_A in fp32, one work-group per block;
//   2. the block scores m_A . m_B for a chunk of query blocks at a time (a
//      tiled fp32 VALU product), then one wave per (query block, frame)
//      keeps that frame's best blocks: the per-frame index directly, or in
//      total mode the candidates of an exact selection over all frames (the
//      K best overall lie among every frame's min(K, P/b) best);
//   3. block_expand: every patch u of block A gets the patches of A's
//      selected blocks, as global tokens (ascending, since the selected
//      blocks are ascending).
// The block build costs (N_p / b)^2 Df multiply-adds instead of N_p^2 Df.
#include "device_util.h"

namespace saf {
namespace {

constexpr int kMeanThreads = 256;
constexpr int kMeanPer = 4096 / kMeanThreads;  // channels per thread (Df <= 4096)

template <typename T> __device__ inline float load_feat(const T *p, int64_t i);
template <> __device__ inline float load_feat<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ inline float load_feat<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

// one work-group per block: mean of the unit features of its b patches
template <typename T>
__global__ __launch_bounds__(kMeanThreads) void block_means(const T *F, int64_t stride, int Df, int b,
                                                          float *M) {
    __shared__ float red[kMeanThreads / 64];
    const int64_t blk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float acc[kMeanPer];
#pragma unroll
    for (int e = 0; e < kMeanPer; ++e) acc[e] = 0.f;
    for (int i = 0; i < b; ++i) {
        const int64_t u = blk * b + i;
        float x[kMeanPer];
        float ss = 0.f;
        // unconditional loads (a channel past Df reads the last one and is
        // zeroed afterwards), so that all of them are in flight together
#pragma unroll
        for (int e = 0; e < kMeanPer; ++e) x[e] = load_feat<T>(F, u * stride + min(tid + e * kMeanThreads, Df - 1));
#pragma unroll
        for (int e = 0; e < kMeanPer; ++e) {
            if (tid + e * kMeanThreads >= Df) x[e] = 0.f;
            ss = fmaf(x[e], x[e], ss);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const float tot = (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();
        const float inv = tot > 0.f ? 1.f / sqrtf(tot) : 0.f;
#pragma unroll
        for (int e = 0; e < kMeanPer; ++e) acc[e] = fmaf(x[e], inv, acc[e]);
    }
    const float ib = 1.f / (float)b;
#pragma unroll
    for (int e = 0; e < kMeanPer; ++e) {
        const int c = tid + e * kMeanThreads;
        if (c < Df) M[blk * Df + c] = acc[e] * ib;
    }
}

// out[u][j b + t] = token of patch (selected block j of u's block) * b + t
__global__ __launch_bounds__(256) void block_expand(const int32_t *bidx, int32_t kb, int32_t b, Geom g,
                                                    int32_t *out) {
    const int64_t kc = (int64_t)kb * b;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= g.Np * kc) return;
    const int64_t u = i / kc, r = i % kc;
    const int64_t sel = bidx[(u / b) * kb + r / b];
    const int64_t p = sel * b + r % b;
    out[i] = (int32_t)((p / g.P) * g.T + g.ns + p % g.P);
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

Geom corr_block_geom(const Geom &g, int32_t block) {
    Geom b = g;
    b.P = g.P / block;
    b.ns = 0;
    b.T = b.P;
    b.N = (int64_t)b.S * b.T;
    b.Np = (int64_t)b.S * b.P;
    return b;
}

// blocks in an index row of the block geometry
int32_t corr_block_row_blocks(const Geom &g, int32_t block, int32_t K, int per_frame) {
    const int64_t per = g.P / block;
    return (int32_t)(per_frame ? (int64_t)(g.S - 1) * std::min<int64_t>(K, per)
                               : std::min<int64_t>(K, (int64_t)(g.S - 1) * per));
}

static size_t inner_scratch_bytes(const Geom &gb, int32_t K, int per_frame) {
    return per_frame ? corr_frame_scratch_bytes(gb, corr_frame_chunk_rows(gb))
                     : corr_raw_total_scratch_bytes(gb, K);
}

size_t corr_block_scratch_bytes(const Geom &g, int32_t block, int32_t Df, int32_t K, int per_frame) {
    const Geom gb = corr_block_geom(g, block);
    const int32_t rb = corr_block_row_blocks(g, block, K, per_frame);
    const int32_t kk = per_frame ? std::min<int32_t>(K, gb.P) : rb;
    return a256(sizeof(float) * (size_t)gb.Np * Df) + a256(sizeof(int32_t) * (size_t)gb.Np * rb) +
           inner_scratch_bytes(gb, kk, per_frame);
}

hipError_t launch_corr_blocks(const CorrBlockBuild &B, hipStream_t stream) {
    const Geom gb = corr_block_geom(B.g, B.block);
    const int32_t rb = corr_block_row_blocks(B.g, B.block, B.K, B.per_frame);
    const int32_t kk = B.per_frame ? std::min<int32_t>(B.K, gb.P) : rb;
    char *p = (char *)B.scratch;
    float *M = (float *)p;
    p += a256(sizeof(float) * (size_t)gb.Np * B.Df);
    int32_t *bidx = (int32_t *)p;
    p += a256(sizeof(int32_t) * (size_t)gb.Np * rb);

    if (B.mark) B.mark(B.mark_user, 1, "block_means", stream);
    if (B.dino_dtype == BF16)
        hipLaunchKernelGGL(block_means<uint16_t>, dim3((unsigned)gb.Np), dim3(kMeanThreads), 0, stream,
                           (const uint16_t *)B.dino, B.row_stride, B.Df, B.block, M);
    else
        hipLaunchKernelGGL(block_means<float>, dim3((unsigned)gb.Np), dim3(kMeanThreads), 0, stream,
                           (const float *)B.dino, B.row_stride, B.Df, B.block, M);
    if (B.mark) B.mark(B.mark_user, 0, "block_means", stream);

    CorrBuild I{};
    I.g = gb;
    I.dino = M;
    I.dino_dtype = F32;
    I.Df = B.Df;
    I.row_stride = B.Df;
    I.K = kk;
    I.cap = 0;  // set by the raw-dot selection itself
    I.per_frame = B.per_frame;
    I.chunk_rows = corr_frame_chunk_rows(gb);
    I.raw_dot = 1;
    I.total_by_frames = B.per_frame ? 0 : 1;
    I.idx_out = bidx;
    I.scratch = p;
    hipError_t e = launch_corr_build(I, stream);
    if (e != hipSuccess) return e;

    const int64_t total = B.g.Np * (int64_t)rb * B.block;
    hipLaunchKernelGGL(block_expand, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, bidx, rb,
                       B.block, B.g, B.idx_out);
    return hipGetLastError();
}

}  // namespace saf
