// Declarations shared by the two parts of the correspondence index build
// (SAF3R Sec. 4.1 "DINO Top-K Kernel", Sec. 4.3): the scratch layout, the
// argument block of its kernels, the cosine-GEMM tile constants and phase
// modes, and the launcher of the cosine GEMM.  The GEMM kernel lives in
// corr_cos.hip, built once per phase mode so that its instantiations compile
// in parallel; the selection, compaction and recomputation kernels and the
// schedule live in corr_index.hip.
#pragma once

#include "device_util.h"

namespace saf {
namespace corr {


constexpr int kRowWaves = 4;  // rows per block in the per-row wave kernels
constexpr int kFallbackBlocks = 256;
constexpr int kFixBatches = 4;  // flagged rows recomputed on the matrix cores: 4 x 256

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Scratch {
    float *invn;      // [Np]
    float *theta;     // [Np]
    float *theta_g;   // [Np] filter threshold of the symmetric pass (a guess, checked at the end)
    uint32_t *cnt;    // [Np]
    uint32_t *over;   // [Np] row needs the exact per-row engine
    int32_t *row_list;    // [Np] flagged rows, for the matrix-core recomputation
    uint32_t *row_count;  // [1] entries in row_list
    float2 *cand;     // [Np * cap] (score, patch index as float bits)
    float *rowbuf;    // [kFallbackBlocks * Np] fallback scores
};

__host__ __device__ inline Scratch carve(void *base, int64_t Np, int32_t cap) {
    char *p = (char *)base;
    Scratch s;
    s.invn = (float *)p;
    p += align256(sizeof(float) * Np);
    s.theta = (float *)p;
    p += align256(sizeof(float) * Np);
    s.theta_g = (float *)p;
    p += align256(sizeof(float) * Np);
    s.cnt = (uint32_t *)p;
    p += align256(sizeof(uint32_t) * Np);
    s.over = (uint32_t *)p;
    p += align256(sizeof(uint32_t) * Np);
    s.row_list = (int32_t *)p;
    p += align256(sizeof(int32_t) * Np);
    s.row_count = (uint32_t *)p;
    p += 256;
    s.cand = (float2 *)p;
    p += align256(sizeof(float2) * (size_t)Np * cap);
    s.rowbuf = (float *)p;
    return s;
}

struct Args {
    Geom g;
    const void *F;
    int64_t stride;
    int32_t Df, K, cap;
    int32_t all_rows_fallback;
    int32_t *idx_out;
    Scratch s;
    int64_t col_lo, col_hi;  // current phase: columns
    int64_t row_lo, row_hi;  // current phase: rows
    int64_t seed_cols;       // columns of the seed phase (whole frames)
    int64_t sym_lo;          // start of the symmetric square [sym_lo, Np)^2
    float *chunk;            // STORE mode: cosines of rows [row_lo, row_hi) x all columns
    int32_t guess_k;         // compaction: also set theta_g from the guess_k-th best (0: no); bound_rows:
                             // theta_g from the guess_k-th largest lane maximum (0: no)
    int32_t guess_k_seed;    // bound_rows: that rank for rows of the two seed frames (one frame fewer seen)
    int32_t filter_guess;    // FILTER: keep scores >= theta_g (the direct pass of two operands), not theta
    int32_t raw_dot;         // scores are plain dot products (unit "norms")
    const void *Fc;          // column operand (== F for the symmetric cosine)
    int32_t tok_map;         // row u of F / Fc is token (u / P) T + ns + u % P (patches of a token layout)
    int32_t use_list;        // STORE: tile rows are positions in s.row_list (flagged rows)
    uint32_t f_bytes;        // bytes of F (and of Fc) that rows 0..Np-1 span; 0: over 0xFFFF0000
    int32_t fallback_list_from;  // >= 0: the per-row engine takes s.row_list[from, row_count); -1: every row
    int32_t lm_per_row;      // TBOUND: lane maxima stored per row (64 per column tile)
    float *pthr;             // fused per-frame mode: [S][Np] lower bound of row u's K-th best in frame f
};

// frame of patch number u: a 32-bit division (patch numbers are below
// N < 2^31, checked when the context is created; a 64-bit division takes
// several times the instructions)
__device__ __forceinline__ int32_t patch_frame(const Geom &g, int64_t u) {
    return (int32_t)((uint32_t)u / (uint32_t)g.P);
}

// element offset of patch row u in F / Fc
__device__ __forceinline__ int64_t frow(const Args &A, int64_t u) {
    if (!A.tok_map) return u * A.stride;
    const int32_t f = patch_frame(A.g, u);
    return ((int64_t)f * A.g.T + A.g.ns + (u - (int64_t)f * A.g.P)) * A.stride;
}

// ---- cosine GEMM: 256 x 256 tiles of 512 threads, channels staged 64 at a time
constexpr int CT = 256;
constexpr int CK = 64;

// Filtered phases at 64 channels: a tile's matrix work is short (one stage),
// so one work-group takes a run of this many column tiles of its row tile;
// one tile per work-group, the launches were bound by work-group dispatch.
constexpr int kFilterRun = 8;
constexpr int kCosThreads = 512;           // 8 waves: 4 (rows) x 2 (columns) of 64 x 128

// Modes:
//   SEED   rows [row_lo,row_hi) x the seed columns: every candidate is kept at
//          a fixed slot (the seed columns with the own frame removed);
//   FILTER rows [row_lo,row_hi) x columns [col_lo,col_hi): a value is kept if
//          it reaches the row's threshold;
//   SYM    the upper triangle of tiles of [sym_lo,Np) x [sym_lo,Np): cosine is
//          symmetric, so each off-diagonal tile feeds its rows (forward) and,
//          transposed, its columns' rows;
//   STORE  rows [row_lo,row_hi) x every column: the cosines are written to a
//          row-chunk buffer (per-frame selection reads them back).
//   PFSEED rows [row_lo,row_hi) x a sample of kFrameSample patches of every
//          frame (sample column c: frame c / kFrameSample): each wave's 128
//          columns are one frame's sample, and the K-th largest of its lanes'
//          maxima (each over 4 sampled patches) is a lower bound of the row's
//          K-th best cosine in that frame, written to A.pthr;
//   PFSYM  SYM with those per-(row, frame) bounds as filters (per-frame mode).
//   TBOUND rows [row_lo,row_hi) x the seed columns: per row, each lane's
//          largest cosine over its 4 columns of other frames, stored to the
//          row's candidate buffer as plain floats (bound_rows then takes
//          the row's K-th largest: a lower bound of its K-th best, reached
//          by K distinct patches).
enum CosMode { SEED = 0, FILTER = 1, SYM = 2, STORE = 3, PFSEED = 4, PFSYM = 5, TBOUND = 6 };
constexpr int kFrameSample = 128;

// One phase of the cosine GEMM over the tiles of grid, launched on stream and
// specialised for the channel count when A.f_bytes != 0 (byte offsets fit
// 32 bits).  Instantiated for every CosMode in corr_cos.hip.
template <int MODE> void launch_cos(dim3 grid, hipStream_t stream, const Args &A);

}  // namespace corr
}  // namespace saf
