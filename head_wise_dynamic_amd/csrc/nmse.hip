// Per-head approximation error of a sparse output against the full-attention
// output (SAF3R Sec. 4.2, Eq. 1): for every head h the sums
//   num_h = sum_{i,c} (O_full[h,i,c] - O_sparse[h,i,c])^2,   den_h = sum O_full^2
// in fp64, reduced in a fixed order (deterministic); optionally the ratio
// num_h / den_h of Eq. 1, weighted by 1 / (number of calibration samples),
// added to a per-head accumulator, so that one call per sample leaves E(c),
// the average over the calibration set, in the accumulator.
#include "device_util.h"

namespace saf {
namespace {

constexpr int kNmseThreads = 256;

// grid (kNmseBlocks, H).  Each lane loads 16 bytes (8 bf16 or 4 fp32) of a
// row; a row of d = 64 channels takes 64 / per-lane lanes, so a wave covers
// several rows per step and the block sweeps rows with stride gridDim.x x
// (rows per block step).
template <typename T>
__global__ __launch_bounds__(kNmseThreads) void nmse_partial(const T *ref, const T *test, int64_t head_stride,
                                                           int64_t token_stride, int64_t N, double *part) {
    constexpr int EPL = 16 / sizeof(T), LPR = 64 / EPL, RPW = 64 / LPR;
    constexpr int RPB = RPW * (kNmseThreads / 64);
    __shared__ double red[2][kNmseThreads / 64];
    const int h = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane / LPR, seg = lane % LPR;
    double num = 0.0, den = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * RPB + wave * RPW + sub; i < N; i += (int64_t)gridDim.x * RPB) {
        const int64_t off = h * head_stride + i * token_stride + seg * EPL;
        const u32x4 ra = *(const u32x4 *)(ref + off), rb = *(const u32x4 *)(test + off);
        float a[EPL], b[EPL];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                a[2 * w] = bf16_bits_to_f32(ra[w] & 0xFFFFu);
                a[2 * w + 1] = bf16_bits_to_f32(ra[w] >> 16);
                b[2 * w] = bf16_bits_to_f32(rb[w] & 0xFFFFu);
                b[2 * w + 1] = bf16_bits_to_f32(rb[w] >> 16);
            }
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                a[w] = __uint_as_float(ra[w]);
                b[w] = __uint_as_float(rb[w]);
            }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const double x = a[e], y = b[e];
            num += (x - y) * (x - y);
            den += x * x;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        num += __shfl_xor(num, o);
        den += __shfl_xor(den, o);
    }
    if (lane == 0) {
        red[0][wave] = num;
        red[1][wave] = den;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double *p = part + ((int64_t)h * gridDim.x + blockIdx.x) * 2;
        p[0] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        p[1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    }
}

// out (may be null): the two sums per head.  acc (may be null): acc[h *
// acc_stride] += weight * num / den (IEEE division: a head whose full output
// is all zero gets a NaN, as the definition has no value there).
__global__ void nmse_final(const double *part, int nblocks, int H, double *out, double *acc, int64_t acc_stride,
                           double weight) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    double num = 0.0, den = 0.0;
    for (int b = 0; b < nblocks; ++b) {
        num += part[((int64_t)h * nblocks + b) * 2];
        den += part[((int64_t)h * nblocks + b) * 2 + 1];
    }
    if (out) {
        out[2 * h] = num;
        out[2 * h + 1] = den;
    }
    if (acc) acc[h * acc_stride] += weight * (num / den);
}

}  // namespace

hipError_t launch_head_nmse(const Geom &g, const void *ref, const void *test, int64_t head_stride,
                            int64_t token_stride, double *part, double *out, double *acc, int64_t acc_stride,
                            double weight, hipStream_t stream) {
    const dim3 grid(kNmseBlocks, g.H);
    if (g.dtype == BF16)
        hipLaunchKernelGGL(nmse_partial<uint16_t>, grid, dim3(kNmseThreads), 0, stream, (const uint16_t *)ref,
                           (const uint16_t *)test, head_stride, token_stride, g.N, part);
    else
        hipLaunchKernelGGL(nmse_partial<float>, grid, dim3(kNmseThreads), 0, stream, (const float *)ref,
                           (const float *)test, head_stride, token_stride, g.N, part);
    hipLaunchKernelGGL(nmse_final, dim3((g.H + 63) / 64), dim3(64), 0, stream, part, kNmseBlocks, g.H, out, acc,
                       acc_stride, weight);
    return hipGetLastError();
}

}  // namespace saf
