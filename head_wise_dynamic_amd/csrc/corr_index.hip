// Correspondence index build (SAF3R Sec. 4.1 "DINO Top-K Kernel", Sec. 4.3):
// for every patch u, the K patches v of other frames with the largest cosine
// c_uv = f_u . f_v / (|f_u| |f_v|), ties to the lower token, stored as global
// token indices in ascending order.  Built once per sequence and cached.
//
// Total mode, bf16 features (the fast engine).  The cosine matrix is never
// stored: each phase is one MFMA GEMM over a block of the pair space (256 x
// 256 tiles, v_mfma_f32_32x32x16_bf16, fp32 accumulate, normalised after the
// dot by fp32 inverse norms) whose epilogue keeps only c >= theta_u, the
// row's current lower bound of its K-th best score, and appends survivors
// to a per-row candidate buffer (staged in LDS, one global atomic per row
// per tile).  After each phase a compaction wave per row raises theta_u to a
// lower bound of the K-th best of its buffer and drops what lies below.
//   1. seed: columns of frames 0 and 1, every candidate kept;
//   2. doubling phases [2P, 4P), [4P, 8P), ... up to W, for every row;
//   3. rows below W continue doubling over [W, Np);
//   4. the square [W, Np)^2 once per unordered pair (cosine is symmetric: a
//      tile feeds its rows and, transposed, its columns).  Its filter is a
//      guess theta_g_u of the K-th best overall (a rank of the columns seen in
//      [0, W) scaled by their share of the candidates); at the end a row's
//      exact K-th best must reach theta_g_u, else the row is recomputed;
//   5. a final wave per row selects the exact top-K, sorts it by token and
//      writes it.
//   A row whose buffer overflows or whose guess check fails is flagged and
//   recomputed exactly: up to 1,024 such rows by the cosine GEMM over a list
//   of rows (cosines stored, then an exact block selection), any further ones
//   by the per-row engine.
// fp32 features (and flagged rows): one 1024-thread block per row computes
//   every cosine with VALU FMAs into a scratch row and runs an exact block
//   top-K (radix select + ordered compaction).
// Per-frame mode (K best of every other frame): the GEMM writes fp32 row
//   chunks of the cosine matrix, then one wave per (row, frame) selects.
#include "device_util.h"
#include "topk_block.h"

namespace saf {
namespace {

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
    int32_t guess_k;         // compaction: also set theta_g from the guess_k-th best (0: no)
    int32_t raw_dot;         // scores are plain dot products (unit "norms")
    const void *Fc;          // column operand (== F for the symmetric cosine)
    int32_t tok_map;         // row u of F / Fc is token (u / P) T + ns + u % P (patches of a token layout)
    int32_t use_list;        // STORE: tile rows are positions in s.row_list (flagged rows)
    uint32_t f_bytes;        // bytes of F (and of Fc) that rows 0..Np-1 span; 0: over 0xFFFF0000
    int32_t fallback_list_from;  // >= 0: the per-row engine takes s.row_list[from, row_count); -1: every row
};

// element offset of patch row u in F / Fc
__device__ __forceinline__ int64_t frow(const Args &A, int64_t u) {
    const int64_t r = A.tok_map ? (u / A.g.P) * A.g.T + A.g.ns + u % A.g.P : u;
    return r * A.stride;
}

template <typename T> __device__ inline float ldf(const T *p, int64_t i);
template <> __device__ inline float ldf<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ inline float ldf<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

// ---- init: inverse norms, theta = -inf, counts and flags = 0 (one wave per row)
template <typename T> __global__ __launch_bounds__(256) void init_rows(const Args A) {
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (u >= A.g.Np) return;
    const T *f = (const T *)A.F + frow(A, u);
    float acc = 0.f;
    for (int c = lane; c < A.Df; c += 64) {
        const float x = ldf<T>(f, c);
        acc = fmaf(x, x, acc);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) {
        A.s.invn[u] = A.raw_dot ? 1.f : (acc > 0.f ? 1.f / sqrtf(acc) : 0.f);
        A.s.theta[u] = -INFINITY;
        A.s.theta_g[u] = -INFINITY;
        if (u == 0) *A.s.row_count = 0u;
        // the seed phase fills slots [0, seed_cols minus the own frame)
        const int64_t fr = u / A.g.P;
        A.s.cnt[u] = A.all_rows_fallback ? 0u
                                         : (uint32_t)(A.seed_cols - (fr < A.seed_cols / A.g.P ? A.g.P : 0));
        A.s.over[u] = A.all_rows_fallback ? 1u : 0u;
    }
}

// ---- one phase of the cosine GEMM with threshold filtering.
// Tile 256 x 256 per work-group of 8 waves (4 x 2); each wave owns 64 x 128
// as 2 x 4 blocks of 32 x 32 (v_mfma_f32_32x32x16_bf16, fp32 accumulators).
// Channels are staged through LDS 64 at a time, double buffered, with the
// next stage prefetched into registers while the current one is multiplied.
// Work-groups are mapped XCD by XCD (blockIdx % 8 selects the XCD): each XCD
// sweeps a contiguous, row-grouped range of tiles so that its L2 serves the
// operand panels its work-groups share.
//
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
constexpr int CT = 256;
constexpr int CK = 64;
constexpr int CROW = CK + 8;   // padded LDS row: 144 B, conflict-free 16-byte reads
constexpr int kGroupRows = 4;  // row tiles per group in the tile order

constexpr int kTileElems = CT * CROW;     // one operand tile in LDS (bf16)
constexpr int kCosThreads = 512;           // 8 waves: 4 (rows) x 2 (columns) of 64 x 128
enum CosMode { SEED = 0, FILTER = 1, SYM = 2, STORE = 3 };

// threshold of a row in units of acc * (inverse norm of the other side),
// lowered by 2^-20 relative so that the filter never drops a value the exact
// comparison would keep
__device__ __forceinline__ float scaled_threshold(float th, float inv_self) {
    if (th == -INFINITY) return -INFINITY;
    if (inv_self > 0.f) {
        const float t = th / inv_self;
        return t > 0.f ? t * (1.f - 0x1p-20f) : (t < 0.f ? t * (1.f + 0x1p-20f) : -1e-30f);
    }
    return th <= 0.f ? -INFINITY : INFINITY;  // zero-norm row: every cosine is 0
}

template <int MODE, int NK>
__global__ __launch_bounds__(kCosThreads, 1) void cos_phase(const Args A) {
    constexpr int kRowCap = MODE == SYM ? 24 : 48;  // survivors staged per row per tile
    // operand tiles: As[2], Bs[2]; after the k-loop the same memory stages the
    // surviving candidates and per-lane accumulator spills
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kTileElems];
    uint16_t (*As)[kTileElems] = (uint16_t (*)[kTileElems])smem;
    uint16_t (*Bs)[kTileElems] = (uint16_t (*)[kTileElems])(smem + 2 * kTileElems);
    __shared__ float r_thr[CT], r_iu[CT], c_thr[CT];
    __shared__ int32_t r_frame[CT];
    __shared__ uint32_t r_cnt[CT], c_cnt[CT];

    const Geom &g = A.g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;  // wave rows [64 wr, +64), columns [128 wc, +128)
    const int n = lane & 31, gq = lane >> 5;

    // ---- tile of this work-group
    int64_t row0, col0, row_hi, col_hi;
    bool diag = false;
    if (MODE == SYM) {
        const int nt = (int)((g.Np - A.sym_lo + CT - 1) / CT);
        const int total = nt * (nt + 1) / 2;
        const int per_xcd = (total + 7) / 8;
        const int tix = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
        if (tix >= total) return;
        // row i of the triangle holds tiles (i, i..nt-1) and starts at i*nt - i(i-1)/2
        const double b2 = 2.0 * nt + 1.0;
        int i = (int)((b2 - sqrt(b2 * b2 - 8.0 * tix)) * 0.5);
        i = max(0, min(i, nt - 1));
        while (i > 0 && i * nt - i * (i - 1) / 2 > tix) --i;
        while (i + 1 < nt && (i + 1) * nt - (i + 1) * i / 2 <= tix) ++i;
        const int j = i + (tix - (i * nt - i * (i - 1) / 2));
        row0 = A.sym_lo + (int64_t)i * CT;
        col0 = A.sym_lo + (int64_t)j * CT;
        row_hi = g.Np;
        col_hi = g.Np;
        diag = i == j;
    } else {
        const int nrow = (int)((A.row_hi - A.row_lo + CT - 1) / CT);
        const int ncol = (int)((A.col_hi - A.col_lo + CT - 1) / CT);
        const int total = nrow * ncol;
        const int per_xcd = (total + 7) / 8;
        const int tix = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
        if (tix >= total) return;
        const int gsize = kGroupRows * ncol;
        const int grp = tix / gsize, rem = tix % gsize;
        const int rows_in_grp = min(kGroupRows, nrow - grp * kGroupRows);
        const int rt = grp * kGroupRows + rem % rows_in_grp;
        const int ct = rem / rows_in_grp;
        row0 = A.row_lo + (int64_t)rt * CT;
        col0 = A.col_lo + (int64_t)ct * CT;
        row_hi = A.row_hi;
        col_hi = A.col_hi;
    }
    const uint16_t *F = (const uint16_t *)A.F, *Fc = (const uint16_t *)A.Fc;
    // STORE over a row list: tile rows are list positions; nothing to do past the list
    const uint32_t nlist = (MODE == STORE && A.use_list) ? *A.s.row_count : 0u;
    if (MODE == STORE && A.use_list && row0 >= (int64_t)nlist) return;
    auto actual_row = [&](int64_t pos) -> int64_t {
        if (pos >= row_hi) return -1;
        if (MODE == STORE && A.use_list) return pos < (int64_t)nlist ? (int64_t)A.s.row_list[pos] : -1;
        return pos;
    };

    if (tid < CT) {
        const int64_t u = actual_row(row0 + tid);
        float thr = INFINITY, iu = __builtin_nanf("");  // NaN: no comparison passes
        int32_t fr = -1;
        if (u >= 0) {
            iu = A.s.invn[u];
            fr = (int32_t)(u / g.P);
            thr = scaled_threshold(MODE == SYM ? A.s.theta_g[u] : A.s.theta[u], iu);
        }
        r_thr[tid] = thr;
        r_iu[tid] = iu;
        r_frame[tid] = fr;
        r_cnt[tid] = 0u;
    } else if (MODE == SYM) {
        const int t = tid - CT;
        const int64_t v = col0 + t;
        c_thr[t] = v < col_hi ? scaled_threshold(A.s.theta_g[v], A.s.invn[v]) : INFINITY;
        c_cnt[t] = 0u;
    }
    const int32_t f_row_lo = (int32_t)(row0 / g.P);
    const int32_t f_row_hi = (int32_t)((min<int64_t>(row0 + CT, row_hi) - 1) / g.P);
    const int32_t f_col_lo = (int32_t)(col0 / g.P);
    const int32_t f_col_hi = (int32_t)((min<int64_t>(col0 + CT, col_hi) - 1) / g.P);
    const bool overlap = !(f_row_hi < f_col_lo || f_col_hi < f_row_lo);

    f32x16 acc[2][4];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;
    auto mma = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < CK / 16; ++kk) {
            __builtin_amdgcn_iglp_opt(0);  // interleave LDS reads with the MFMA chain
            bf16x8 a[2], b[4];
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
                a[bi] = *(const bf16x8 *)(&As[buf][(64 * wr + 32 * bi + n) * CROW + 16 * kk + 8 * gq]);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                b[bj] = *(const bf16x8 *)(&Bs[buf][(128 * wc + 32 * bj + n) * CROW + 16 * kk + 8 * gq]);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
        }
    };
    if constexpr (NK > 0) {  // NK = Df / CK
        // Channel count known at compile time: the stage loop is unrolled
        // completely and no load sits behind a branch, so the compiler waits
        // only for the stage it stores (a run-time loop with guarded loads
        // waited for everything and ran the same tiles ~20 % slower).  Loads
        // go through buffer resources: a scalar base plus a 32-bit lane
        // offset, and an offset past the buffer reads as zero.
        const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc((void *)F, (short)0, (int)A.f_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void *)Fc, (short)0, (int)A.f_bytes, 0x00020000);
        // rows past the tile's end start at the buffer's end: with f_bytes
        // <= 0xFFFF0000 every stage offset added stays past it (no wrap)
        const uint32_t kNone = A.f_bytes;
        uint32_t aoff[4], boff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (tid + kCosThreads * i) >> 3, seg = (tid + kCosThreads * i) & 7;
            const int64_t u = actual_row(row0 + row), v = col0 + row;
            aoff[i] = u >= 0 ? 2u * ((uint32_t)frow(A, u) + 8u * seg) : kNone;
            boff[i] = v < col_hi ? 2u * ((uint32_t)frow(A, v) + 8u * seg) : kNone;
        }
        u32x4 ar[4], br[4];
        auto load = [&](int st) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ar[i] = __builtin_amdgcn_raw_buffer_load_b128(rf, aoff[i] + 2 * CK * st, 0, 0);
                br[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, boff[i] + 2 * CK * st, 0, 0);
            }
        };
        auto store = [&](int buf) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + kCosThreads * i, row = c >> 3, seg = c & 7;
                *(u32x4 *)(&As[buf][row * CROW + 8 * seg]) = ar[i];
                *(u32x4 *)(&Bs[buf][row * CROW + 8 * seg]) = br[i];
            }
        };
        load(0);
        store(0);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NK; ++t) {
            if (t + 1 < NK) load(t + 1);
            mma(t & 1);
            if (t + 1 < NK) store((t + 1) & 1);
            __syncthreads();
        }
    } else {
        // element offsets of the rows this thread loads (0xFFFFFFFF: none)
        uint32_t aoff[4], boff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (tid + kCosThreads * i) >> 3;
            const int64_t u = actual_row(row0 + row), v = col0 + row;
            aoff[i] = u >= 0 ? (uint32_t)frow(A, u) : 0xFFFFFFFFu;
            boff[i] = v < col_hi ? (uint32_t)frow(A, v) : 0xFFFFFFFFu;
        }
        u32x4 ar[4], br[4];
        auto load = [&](int k0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int seg = (tid + kCosThreads * i) & 7;
                ar[i] = aoff[i] != 0xFFFFFFFFu ? *(const u32x4 *)(F + aoff[i] + k0 + 8 * seg) : u32x4{0u, 0u, 0u, 0u};
                br[i] = boff[i] != 0xFFFFFFFFu ? *(const u32x4 *)(Fc + boff[i] + k0 + 8 * seg) : u32x4{0u, 0u, 0u, 0u};
            }
        };
        auto store = [&](int buf) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + kCosThreads * i, row = c >> 3, seg = c & 7;
                *(u32x4 *)(&As[buf][row * CROW + 8 * seg]) = ar[i];
                *(u32x4 *)(&Bs[buf][row * CROW + 8 * seg]) = br[i];
            }
        };
        const int nk = A.Df / CK;
        load(0);
        store(0);
        __syncthreads();
        for (int t = 0; t < nk; ++t) {
            const int buf = t & 1;
            if (t + 1 < nk) load((t + 1) * CK);
            mma(buf);
            if (t + 1 < nk) store(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds column n of each block, rows per register.
    // cosine = acc * (|f_u|^-1 |f_v|^-1), the same product in every mode.
    float iv[4];
    int32_t fv[4];
    const int32_t lc0 = 128 * wc + n;                   // local column of block bj: lc0 + 32 bj
    const int32_t vcol0 = (int32_t)(col0 + lc0);
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        const int64_t v = vcol0 + 32 * bj;
        const bool vok = v < col_hi;
        iv[bj] = vok ? A.s.invn[v] : __builtin_nanf("");  // NaN never passes a comparison
        fv[bj] = vok ? (int32_t)(v / g.P) : -2;
    }

    if (MODE == STORE) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 64 * wr + 32 * bi + 8 * (r >> 2) + 4 * gq + (r & 3);
                if (r_frame[lr] < 0) continue;
                const float iu = r_iu[lr];
                float *crow = A.chunk + (row0 + lr - A.row_lo) * g.Np;
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
                    if (fv[bj] >= 0) crow[vcol0 + 32 * bj] = acc[bi][bj][r] * (iu * iv[bj]);
            }
        return;
    }

    if (MODE == SEED) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 64 * wr + 32 * bi + 8 * (r >> 2) + 4 * gq + (r & 3);
                const int32_t fr = r_frame[lr];
                const float iu = r_iu[lr];
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    const int32_t v = vcol0 + 32 * bj;
                    if (fr >= 0 && fv[bj] >= 0 && fr != fv[bj]) {
                        const int32_t slot = (fv[bj] > fr) ? v - g.P : v;
                        const float c = acc[bi][bj][r] * (iu * iv[bj]);
                        A.s.cand[(row0 + lr) * A.cap + slot] = make_float2(c, __int_as_float(v));
                    }
                }
            }
        return;
    }

    // Fast path per 32 x 32 block: 16-bit masks of the lane's values that
    // reach their row's threshold (forward) and, in SYM mode, its column's
    // threshold (transposed).  Lanes with a hit spill their 16 accumulators to
    // LDS and stage each hit in the receiving row's LDS list; one global atomic
    // per row then reserves the row's buffer slots.
    __syncthreads();  // operand tiles are no longer read: reuse them
    float2 *stage = (float2 *)smem;                              // [CT][kRowCap] forward
    float2 *cstage = stage + CT * kRowCap;                       // [CT][kRowCap] transposed
    float *xl = (float *)(cstage + (MODE == SYM ? CT * kRowCap : 0)) + (wave * 64 + lane) * 16;
    const bool transposed = MODE == SYM && !diag;
    auto push = [&](uint32_t *cnt_lds, float2 *lst, int li, int64_t grow, float2 e) {
        const uint32_t slot = atomicAdd(&cnt_lds[li], 1u);
        if (slot < (uint32_t)kRowCap) {
            lst[li * kRowCap + slot] = e;
        } else {  // rare: more than kRowCap hits of one row in one tile
            const uint32_t gs = atomicAdd(&A.s.cnt[grow], 1u);
            if (gs < (uint32_t)A.cap) A.s.cand[grow * A.cap + gs] = e;
        }
    };
    const float *thr_base = r_thr + 64 * wr + 4 * gq;
    const float *iu_base = r_iu + 64 * wr + 4 * gq;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            uint32_t kf = 0, kt = 0;
            const float cth = transposed ? c_thr[lc0 + 32 * bj] : INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int o = 32 * bi + 8 * (r >> 2) + (r & 3);
                kf |= (acc[bi][bj][r] * iv[bj] >= thr_base[o]) ? (1u << r) : 0u;
                if (transposed) kt |= (acc[bi][bj][r] * iu_base[o] >= cth) ? (1u << r) : 0u;
            }
            if (kf | kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) xl[r] = acc[bi][bj][r];
                const int lc = lc0 + 32 * bj;
                const int32_t v = vcol0 + 32 * bj;
                uint32_t k = kf | kt;
                while (k) {
                    const int r = __ffs(k) - 1;
                    k &= k - 1;
                    const int lr = 64 * wr + 32 * bi + 8 * (r >> 2) + 4 * gq + (r & 3);
                    if (overlap && r_frame[lr] == fv[bj]) continue;  // own frame
                    const float c = xl[r] * (r_iu[lr] * iv[bj]);
                    if ((kf >> r) & 1u) push(r_cnt, stage, lr, row0 + lr, make_float2(c, __int_as_float(v)));
                    if ((kt >> r) & 1u)
                        push(c_cnt, cstage, lc, (int64_t)v, make_float2(c, __int_as_float((int32_t)(row0 + lr))));
                }
            }
        }
    }
    __syncthreads();
    if (tid < CT) {
        const uint32_t nloc = min(r_cnt[tid], (uint32_t)kRowCap);
        if (nloc) {
            const int64_t u = row0 + tid;
            const uint32_t base = atomicAdd(&A.s.cnt[u], nloc);
            for (uint32_t i = 0; i < nloc; ++i)
                if (base + i < (uint32_t)A.cap) A.s.cand[u * A.cap + base + i] = stage[tid * kRowCap + i];
        }
    } else if (transposed) {
        const int t = tid - CT;
        const uint32_t nloc = min(c_cnt[t], (uint32_t)kRowCap);
        if (nloc) {
            const int64_t v = col0 + t;
            const uint32_t base = atomicAdd(&A.s.cnt[v], nloc);
            for (uint32_t i = 0; i < nloc; ++i)
                if (base + i < (uint32_t)A.cap) A.s.cand[v * A.cap + base + i] = cstage[t * kRowCap + i];
        }
    }
}

// ---- per-row selection inside one wave.
// The row's n buffered candidates (n <= 64 * MAXE) are held in registers,
// lane-strided.  Counts over the row use ballot + popcount, so the search
// needs no cross-lane shuffles.
template <int MAXE> struct RowSel {
    float sc[MAXE];
    int32_t id[MAXE];
    int n, ne;         // entries, and register slots in use (ceil(n / 64))
    uint32_t thr;      // selection threshold (order key)
    int32_t ithr;      // largest index kept among keys == thr (exact mode)
    __device__ void load(const float2 *buf, int nn, int lane) {
        n = nn;
        ne = (nn + 63) / 64;
#pragma unroll
        for (int e = 0; e < MAXE; ++e) {
            sc[e] = -INFINITY;
            id[e] = INT32_MAX;
            if (e < ne) {  // wave-uniform
                // unconditional load (a lane past the end reads entry n - 1,
                // or entry 0 of an empty row, and is masked): guarded loads
                // make the compiler wait for each one on its own
                const int i = e * 64 + lane;
                const float2 x = buf[min(i, max(n - 1, 0))];
                if (i < n) {
                    sc[e] = x.x;
                    id[e] = __float_as_int(x.y);
                }
            }
        }
    }
    __device__ bool valid(int e, int lane) const { return e * 64 + lane < n; }
    __device__ uint32_t count_ge(uint32_t k, int lane) const {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < MAXE; ++e)
            if (e < ne) c += (uint32_t)__popcll(__ballot(valid(e, lane) && order_key(sc[e]) >= k));
        return c;
    }
    // Largest key prefix (the top `bits` bits resolved) with >= K entries at
    // or above it.  With bits = 32 this is the K-th largest key exactly.
    __device__ uint32_t prefix_search(int K, int lane, int bits) const {
        uint32_t prefix = 0;
        for (int bit = 31; bit >= 32 - bits; --bit) {
            const uint32_t cand = prefix | (1u << bit);
            if (count_ge(cand, lane) >= (uint32_t)K) prefix = cand;
        }
        return prefix;
    }
    // Approximate: keep every entry whose key is >= a 16-bit prefix bound of
    // the K-th largest key (at least K entries, a few more near the bound).
    __device__ void select_bound(int K, int lane) {
        thr = prefix_search(K, lane, 16);
        ithr = INT32_MAX;
    }
    // Exact: the K entries first by (score desc, index asc).
    __device__ void select_exact(int K, int lane) {
        thr = prefix_search(K, lane, 32);
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < MAXE; ++e) {
            if (e < ne) {
                const uint32_t key = order_key(sc[e]);
                gt += (uint32_t)__popcll(__ballot(valid(e, lane) && key > thr));
                eq += (uint32_t)__popcll(__ballot(valid(e, lane) && key == thr));
            }
        }
        const uint32_t need = (uint32_t)K - gt;
        if (eq == need) {
            ithr = INT32_MAX;
            return;
        }
        // largest x with #(key == thr && id < x) < need  ->  the need-th smallest id
        uint32_t lo = 0;
        for (int bit = 30; bit >= 0; --bit) {
            const uint32_t cand = lo | (1u << bit);
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < MAXE; ++e)
                if (e < ne)
                    c += (uint32_t)__popcll(
                        __ballot(valid(e, lane) && order_key(sc[e]) == thr && (uint32_t)id[e] < cand));
            if (c < need) lo = cand;
        }
        ithr = (int32_t)lo;
    }
    __device__ bool kept(int e, int lane) const {
        const uint32_t key = order_key(sc[e]);
        return e < ne && valid(e, lane) && (key > thr || (key == thr && id[e] <= ithr));
    }
};

// Between phases: raise theta_u to a lower bound of the row's K-th best score
// and drop the entries below it.  The bound comes from the first 64 * MAXE
// entries (the K-th best of a subset never exceeds the K-th best of the row);
// a longer row is then filtered by streaming over all its entries.
template <int MAXE>
__global__ __launch_bounds__(256) void compact_rows(const Args A) {
    // only rows [row_lo, row_hi) received candidates in the last phase
    const int64_t u = A.row_lo + (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (u >= A.row_hi) return;
    const uint32_t c = A.s.cnt[u];
    const uint32_t nn = min(c, (uint32_t)A.cap);
    if (c > (uint32_t)A.cap && lane == 0) A.s.over[u] = 1u;
    if ((int)nn <= A.K) {
        if (A.guess_k && lane == 0) A.s.theta_g[u] = A.s.theta[u];
        return;
    }
    float2 *buf = A.s.cand + u * A.cap;
    uint32_t total = nn, thr = 0, gkey = 0;
    for (int pass = 0; pass < 4 && (int)total > A.K; ++pass) {
        const int nreg = (int)min<uint32_t>(total, 64u * MAXE);
        RowSel<MAXE> R;
        R.load(buf, nreg, lane);
        R.select_bound(A.K, lane);
        thr = R.thr;
        if (A.guess_k) gkey = R.prefix_search(A.guess_k, lane, 16);
        if ((int)total == nreg) {
            uint32_t mine = 0;
#pragma unroll
            for (int e = 0; e < MAXE; ++e) mine += R.kept(e, lane) ? 1u : 0u;
            uint32_t incl = mine;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            total = __shfl(incl, 63);
            uint32_t pos = incl - mine;
#pragma unroll
            for (int e = 0; e < MAXE; ++e)
                if (R.kept(e, lane)) buf[pos++] = make_float2(R.sc[e], __int_as_float(R.id[e]));
            break;
        }
        // in-place ordered filter: the write position never passes the read
        // one.  Four 64-entry chunks are loaded before any is written back (all
        // four are then held in registers, and writes land below the next
        // group), so four loads are in flight instead of one.
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        uint32_t pos = 0;
        constexpr int kChunks = 4;
        for (uint32_t i0 = 0; i0 < total; i0 += 64 * kChunks) {
            float2 x[kChunks];
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const uint32_t i = i0 + 64 * c + lane;
                x[c] = buf[min(i, total - 1)];  // unconditional, masked below
                if (i >= total) x[c] = make_float2(-INFINITY, 0.f);
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const uint32_t i = i0 + 64 * c + lane;
                const bool keep = i < total && order_key(x[c].x) >= thr;
                const uint64_t m = __ballot(keep);
                if (keep) buf[pos + (uint32_t)__popcll(m & below)] = x[c];
                pos += (uint32_t)__popcll(m);
            }
        }
        total = pos;
    }
    if (lane == 0) {
        A.s.cnt[u] = total;
        A.s.theta[u] = order_key_to_float(thr);
        if (A.guess_k) A.s.theta_g[u] = order_key_to_float(max(gkey, thr));
    }
}

template <int MAXE>
__global__ __launch_bounds__(256) void finalize_rows(const Args A, uint32_t lo_cnt, uint32_t hi_cnt) {
    __shared__ int32_t sel[kRowWaves][1024];
    const int wv = threadIdx.x >> 6;
    const int64_t u = (int64_t)blockIdx.x * kRowWaves + wv;
    const int lane = threadIdx.x & 63;
    if (u >= A.g.Np) return;
    const uint32_t c = A.s.cnt[u];
    if (c <= lo_cnt || c > hi_cnt) return;
    if (A.s.over[u] || c > (uint32_t)A.cap) return;  // exact per-row engine
    if (c > 64u * MAXE) {  // more than fits the registers: exact per-row engine
        if (lane == 0) A.s.over[u] = 1u;
        return;
    }
    const int nn = (int)c;
    if (nn < A.K) {  // cannot happen without an overflow; recompute exactly
        if (lane == 0) A.s.over[u] = 1u;
        return;
    }
    const float2 *buf = A.s.cand + u * A.cap;
    RowSel<MAXE> R;
    R.load(buf, nn, lane);
    R.select_exact(A.K, lane);
    // A row of the symmetric pass kept only columns >= theta_g there; its
    // K-th best is exact when it reaches theta_g, else recompute the row.
    if (u >= A.sym_lo && R.thr < order_key(A.s.theta_g[u])) {
        if (lane == 0) A.s.over[u] = 1u;
        return;
    }
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) mine += R.kept(e, lane) ? 1u : 0u;
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    uint32_t pos = incl - mine;
    int32_t *s = sel[wv];
#pragma unroll
    for (int e = 0; e < MAXE; ++e)
        if (R.kept(e, lane)) s[pos++] = R.id[e];
    // ascending order: bitonic sort of the K ids padded to a power of two
    // (K <= 1024) with a sentinel above every id, in the wave's LDS slice
    int n = 1;
    while (n < A.K) n <<= 1;
    for (int i = A.K + lane; i < n; i += 64) s[i] = INT32_MAX;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    for (int k = 2; k <= n; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = lane; i < n; i += 64) {
                const int l = i ^ j;
                if (l > i) {
                    const int32_t a = s[i], b = s[l];
                    if ((a > b) == ((i & k) == 0)) {
                        s[i] = b;
                        s[l] = a;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        }
    int32_t *out = A.idx_out + u * A.K;
    const Geom &g = A.g;
    for (int i = lane; i < A.K; i += 64) {
        const int32_t v = s[i];
        out[i] = (int32_t)((v / g.P) * g.T + g.ns + (v % g.P));
    }
}

// ---- cosines of a row chunk on the VALU (fp32 features, or a channel count
// the matrix-core tiles do not cover): 64 x 64 output tiles per work-group,
// 16-channel slices of both operands staged in LDS, 4 x 4 outputs per thread.
constexpr int kStoreTile = 64, kStoreK = 16;
template <typename T> __global__ __launch_bounds__(256) void cos_store_tiled(const Args A) {
    __shared__ float As[kStoreK][kStoreTile + 4], Bs[kStoreK][kStoreTile + 4];
    const Geom &g = A.g;
    const T *F = (const T *)A.F, *Fc = (const T *)A.Fc;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t r0 = A.row_lo + (int64_t)blockIdx.y * kStoreTile, c0 = (int64_t)blockIdx.x * kStoreTile;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int k0 = 0; k0 < A.Df; k0 += kStoreK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i, r = e / kStoreK, k = e % kStoreK;
            const int64_t u = r0 + r, v = c0 + r;
            const bool kin = k0 + k < A.Df;
            As[k][r] = (u < A.row_hi && kin) ? ldf<T>(F, frow(A, u) + k0 + k) : 0.f;
            Bs[k][r] = (v < g.Np && kin) ? ldf<T>(Fc, frow(A, v) + k0 + k) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kStoreK; ++k) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = As[k][ty + 16 * i];
                b[i] = Bs[k][tx + 16 * i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t u = r0 + ty + 16 * i;
        if (u >= A.row_hi) continue;
        const float iu = A.s.invn[u];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t v = c0 + tx + 16 * j;
            if (v < g.Np) A.chunk[(u - A.row_lo) * g.Np + v] = acc[i][j] * (iu * A.s.invn[v]);
        }
    }
}

// ---- per-frame mode: one wave per (row, other frame) selects the frame's K
// best patches by (cosine desc, index asc) and writes their tokens ascending.
// Patch i of the frame sits in register slot i / 64 of lane i % 64, so an
// ordered ballot compaction over (slot, lane) emits the kept set in index
// order.  Small K: K rounds of a wave-wide argmax; otherwise a bitwise search
// for the K-th key and the index cut among its ties.
constexpr int kFrameRoundsMaxK = 8;

template <int MAXE, bool CAND>
__global__ __launch_bounds__(256) void frame_topk(const Args A) {
    const Geom &g = A.g;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    const int64_t rows = A.row_hi - A.row_lo;
    if (item >= rows * g.S) return;
    const int64_t u = A.row_lo + item / g.S;
    const int32_t gf = (int32_t)(item % g.S), fu = (int32_t)(u / g.P);
    if (gf == fu) return;
    const float *src = A.chunk + (u - A.row_lo) * g.Np + (int64_t)gf * g.P;
    const int ne = (g.P + 63) / 64;
    uint32_t key[MAXE];  // order_key of the cosine; 0 marks an empty slot
    // unconditional loads (a slot past the frame reads its last patch and is
    // emptied afterwards), so that all of them are in flight together
    float x[MAXE];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) x[e] = src[min(e * 64 + lane, g.P - 1)];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int i = e * 64 + lane;
        key[e] = (e < ne && i < g.P) ? max(order_key(x[e]), 1u) : 0u;
    }
    const uint32_t K = (uint32_t)A.K;
    uint64_t keep = 0;  // bit e: slot e is selected
    if (K <= kFrameRoundsMaxK) {
        for (uint32_t k = 0; k < K; ++k) {
            // best of this lane among unselected slots: largest key, then lowest slot
            uint32_t bk = 0;
            int be = -1;
#pragma unroll
            for (int e = 0; e < MAXE; ++e)
                if (e < ne && !((keep >> e) & 1ull) && key[e] > bk) {
                    bk = key[e];
                    be = e;
                }
            // wave argmax of (key desc, patch index asc)
            uint64_t w = ((uint64_t)bk << 32) | (uint32_t)(0x7FFFFFFF - (be < 0 ? 0x7FFFFFFF : be * 64 + lane));
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const uint64_t x = __shfl_xor(w, o);
                w = x > w ? x : w;
            }
            const uint32_t wi = 0x7FFFFFFFu - (uint32_t)(w & 0xFFFFFFFFu);
            if ((w >> 32) != 0 && (int)(wi & 63) == lane) keep |= 1ull << (wi >> 6);
        }
    } else {
        auto count = [&](auto pred) {
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < MAXE; ++e)
                if (e < ne) c += (uint32_t)__popcll(__ballot(key[e] != 0u && pred(e)));
            return c;
        };
        uint32_t thr = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            if (count([&](int e) { return key[e] >= cand; }) >= K) thr = cand;
        }
        const uint32_t need = K - count([&](int e) { return key[e] > thr; });
        int32_t ithr = INT32_MAX;
        if (count([&](int e) { return key[e] == thr; }) != need) {
            uint32_t lo = 0;  // largest index cut with fewer than need tied entries below it
            for (int bit = 30; bit >= 0; --bit) {
                const uint32_t cand = lo | (1u << bit);
                if (count([&](int e) { return key[e] == thr && (uint32_t)(e * 64 + lane) < cand; }) < need)
                    lo = cand;
            }
            ithr = (int32_t)lo;
        }
#pragma unroll
        for (int e = 0; e < MAXE; ++e)
            if (e < ne && key[e] != 0u && (key[e] > thr || (key[e] == thr && e * 64 + lane <= ithr)))
                keep |= 1ull << e;
    }
    const int32_t slot = gf - (gf > fu ? 1 : 0);
    if (CAND) {
        // candidates (score, patch) for an exact selection over all frames
        float2 *cand = A.s.cand + u * A.cap + (int64_t)slot * A.K;
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        uint32_t pos = 0;
#pragma unroll
        for (int e = 0; e < MAXE; ++e) {
            if (e < ne) {
                const bool kp = (keep >> e) & 1ull;
                const uint64_t m = __ballot(kp);
                if (kp)
                    cand[pos + (uint32_t)__popcll(m & below)] =
                        make_float2(order_key_to_float(key[e]), __int_as_float(gf * g.P + e * 64 + lane));
                pos += (uint32_t)__popcll(m);
            }
        }
        if (slot == 0 && lane == 0) {
            A.s.cnt[u] = (uint32_t)((g.S - 1) * A.K);
            A.s.over[u] = 0u;
        }
        return;
    }
    int32_t *out = A.idx_out + u * ((int64_t)(g.S - 1) * A.K) + (int64_t)slot * A.K;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t tok0 = gf * g.T + g.ns;
    uint32_t pos = 0;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        if (e < ne) {
            const bool kp = (keep >> e) & 1ull;
            const uint64_t m = __ballot(kp);
            if (kp) out[pos + (uint32_t)__popcll(m & below)] = tok0 + e * 64 + lane;
            pos += (uint32_t)__popcll(m);
        }
    }
}

// ---- flagged rows (overflow or a failed guess check) into a list
__global__ __launch_bounds__(256) void list_flagged(const Args A) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= A.g.Np || !A.s.over[u]) return;
    const uint32_t pos = atomicAdd(A.s.row_count, 1u);
    A.s.row_list[pos] = (int32_t)u;
}

// ---- exact selection of listed rows [batch0, batch0 + gridDim.x) whose
// cosines a row-list STORE pass wrote to A.chunk; clears their flag
__global__ __launch_bounds__(1024) void select_listed(const Args A, int64_t batch0) {
    const Geom &g = A.g;
    const int64_t pos = batch0 + blockIdx.x;
    if (pos >= (int64_t)*A.s.row_count) return;
    const int64_t u = A.s.row_list[pos];
    float *row = A.chunk + (int64_t)blockIdx.x * g.Np;
    const int64_t f0 = (u / g.P) * g.P;  // own-frame patches can never be selected
    for (int64_t j = threadIdx.x; j < g.P; j += 1024) row[f0 + j] = -INFINITY;
    __syncthreads();
    int32_t *out = A.idx_out + u * A.K;
    block_topk_ascending(row, g.Np, A.K, [&](int64_t p, int64_t v) {
        out[p] = (int32_t)((v / g.P) * g.T + g.ns + (v % g.P));
    });
    if (threadIdx.x == 0) A.s.over[u] = 0u;
}

// ---- exact per-row engine: one 1024-thread block per flagged row
template <typename T> __global__ __launch_bounds__(1024) void fallback_rows(const Args A) {
    __shared__ float fu[4096];
    const Geom &g = A.g;
    float *row = A.s.rowbuf + (int64_t)blockIdx.x * g.Np;
    const T *F = (const T *)A.F, *Fc = (const T *)A.Fc;
    // after the matrix-core recomputation only listed rows past its batches
    // can still be flagged: walk that part of the list, not every row
    const bool listed = A.fallback_list_from >= 0;
    const int64_t n = listed ? (int64_t)*A.s.row_count : g.Np;
    for (int64_t p = (listed ? A.fallback_list_from : 0) + blockIdx.x; p < n; p += gridDim.x) {
        const int64_t u = listed ? (int64_t)A.s.row_list[p] : p;
        if (!A.s.over[u]) continue;
        __syncthreads();
        for (int c = threadIdx.x; c < A.Df; c += 1024) fu[c] = ldf<T>(F + frow(A, u), c);
        __syncthreads();
        const float iu = A.s.invn[u];
        const int64_t fr = u / g.P;
        for (int64_t v = threadIdx.x; v < g.Np; v += 1024) {
            float acc = 0.f;
            const T *fv = Fc + frow(A, v);
            for (int c = 0; c < A.Df; ++c) acc = fmaf(fu[c], ldf<T>(fv, c), acc);
            // own-frame patches can never be selected: the candidate count
            // (S-1)P is >= K, so they are given the lowest possible score
            row[v] = (v / g.P == fr) ? -INFINITY : acc * iu * A.s.invn[v];
        }
        __syncthreads();
        int32_t *out = A.idx_out + u * A.K;
        block_topk_ascending(row, g.Np, A.K, [&](int64_t pos, int64_t v) {
            out[pos] = (int32_t)((v / g.P) * g.T + g.ns + (v % g.P));
        });
        __syncthreads();
    }
}

}  // namespace

// Start of the symmetric square: the first doubling boundary W (2P, 4P, ...)
// with Np - W <= 24 W, so that every row's guess of its K-th best comes from
// at least a twenty-fifth of the columns before the square is visited once.
int64_t corr_sym_start(const Geom &g) {
    int64_t b = std::min<int64_t>(g.Np, 2 * (int64_t)g.P);
    while (b < g.Np && g.Np - b > 24 * b) b *= 2;
    return std::min<int64_t>(b, g.Np);
}

int32_t corr_capacity(const Geom &g, int32_t K) {
    // the seed phase stores two frames' candidates; a doubling phase adds
    // ~K; the symmetric pass, filtering with a guess near 2.5 x the K-th
    // best's rank, adds ~2.5 K per direction.  A row that still overflows is
    // flagged and recomputed exactly.
    int64_t cap = std::max<int64_t>(2 * (int64_t)g.P, 8 * (int64_t)K);
    cap = std::max<int64_t>(cap, 6 * (int64_t)K + 256);
    cap = (cap + 63) / 64 * 64;
    return (int32_t)cap;
}

// bytes carve() lays out before rowbuf
static size_t carve_head_bytes(int64_t Np, int32_t cap) {
    return align256(sizeof(float) * Np) * 3 + align256(sizeof(uint32_t) * Np) * 2 +
           align256(sizeof(int32_t) * Np) + 256 + align256(sizeof(float2) * (size_t)Np * cap);
}

size_t corr_scratch_bytes(const Geom &g, int32_t K, int32_t cap) {
    (void)K;
    return carve_head_bytes(g.Np, cap) + align256(sizeof(float) * (size_t)kFallbackBlocks * g.Np);
}

// Rank whose value guesses the K-th best over all candidates from the W seen
// columns: with the seen columns a fraction f of the candidates, the K-th best
// overall sits near rank K f among them; 2.5x that rank keeps the chance that
// fewer than K candidates reach the guess small (such rows are recomputed).
static int32_t corr_guess_rank(const Geom &g, int32_t K, int64_t W) {
    const double f = (double)W / ((double)(g.S - 1) * g.P);
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(K, (int64_t)std::ceil(2.5 * K * f)));
}

// rows per chunk of the per-frame mode: a multiple of the tile height whose
// fp32 cosine block stays near kFrameChunkBytes
constexpr size_t kFrameChunkBytes = (size_t)512 << 20;
int32_t corr_frame_chunk_rows(const Geom &g) {
    const int64_t want = (int64_t)(kFrameChunkBytes / (sizeof(float) * (size_t)g.Np)) / CT * CT;
    const int64_t all = (g.Np + CT - 1) / CT * CT;
    return (int32_t)std::max<int64_t>(CT, std::min<int64_t>(want, all));
}

size_t corr_frame_scratch_bytes(const Geom &g, int32_t chunk_rows) {
    return carve_head_bytes(g.Np, 0) + align256(sizeof(float) * (size_t)chunk_rows * g.Np);
}

size_t corr_raw_total_scratch_bytes(const Geom &g, int32_t K) {
    const int32_t cap = (g.S - 1) * std::min<int32_t>(K, g.P);
    const int64_t rows = std::max<int64_t>(corr_frame_chunk_rows(g), kFallbackBlocks);
    return carve_head_bytes(g.Np, cap) + align256(sizeof(float) * (size_t)rows * g.Np);
}

// elements of F (and Fc) that rows 0..Np-1 span; the matrix-core kernels
// address them with 32-bit offsets
static int64_t feature_span(const CorrBuild &B) {
    const int64_t last = B.tok_map ? (int64_t)(B.g.S - 1) * B.g.T + B.g.ns + B.g.P - 1 : B.g.Np - 1;
    return last * B.row_stride + B.Df;
}

// cos_phase launch with the stage count fixed at compile time for the usual
// feature widths (ViT-S/B/L: 384, 768, 1024 channels)
template <int MODE> static void launch_cos(dim3 grid, hipStream_t stream, const Args &A) {
    const bool fixed = A.f_bytes != 0;  // byte offsets fit 32 bits
    if (fixed && A.Df == 1024)
        hipLaunchKernelGGL((cos_phase<MODE, 16>), grid, dim3(kCosThreads), 0, stream, A);
    else if (fixed && A.Df == 768)
        hipLaunchKernelGGL((cos_phase<MODE, 12>), grid, dim3(kCosThreads), 0, stream, A);
    else if (fixed && A.Df == 384)
        hipLaunchKernelGGL((cos_phase<MODE, 6>), grid, dim3(kCosThreads), 0, stream, A);
    else
        hipLaunchKernelGGL((cos_phase<MODE, 0>), grid, dim3(kCosThreads), 0, stream, A);
}

// cand = false: per-frame index into A.idx_out.  cand = true: every row's
// per-frame top-A.K as (score, patch) candidates in A.s.cand (A.cap =
// (S-1) A.K per row), for an exact selection over all frames afterwards.
static hipError_t launch_corr_frames(Args &A, const CorrBuild &B, bool cand, hipStream_t stream) {
    const Geom &g = B.g;
    const int64_t Np = g.Np;
    if (B.chunk_rows < 1) return hipErrorInvalidValue;
    A.chunk = A.s.rowbuf;  // the chunk follows the per-row arrays and candidates
    const bool gemm = B.dino_dtype == BF16 && (B.Df % CK) == 0 && feature_span(B) < 0xFFFFFFFFll;
    for (int64_t r0 = 0; r0 < Np; r0 += B.chunk_rows) {
        A.row_lo = r0;
        A.row_hi = std::min<int64_t>(Np, r0 + B.chunk_rows);
        A.col_lo = 0;
        A.col_hi = Np;
        const int64_t rows = A.row_hi - A.row_lo;
        if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
        if (gemm) {
            const int64_t tiles = ((rows + CT - 1) / CT) * ((Np + CT - 1) / CT);
            launch_cos<STORE>(dim3((unsigned)(8 * ((tiles + 7) / 8))), stream, A);
        } else {
            const dim3 grid((unsigned)((Np + kStoreTile - 1) / kStoreTile),
                            (unsigned)((rows + kStoreTile - 1) / kStoreTile));
            if (B.dino_dtype == BF16)
                hipLaunchKernelGGL(cos_store_tiled<uint16_t>, grid, dim3(256), 0, stream, A);
            else
                hipLaunchKernelGGL(cos_store_tiled<float>, grid, dim3(256), 0, stream, A);
        }
        if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
        const unsigned fb = (unsigned)((rows * g.S + kRowWaves - 1) / kRowWaves);
        if (cand) {
            if (g.P <= 24 * 64)
                hipLaunchKernelGGL((frame_topk<24, true>), dim3(fb), dim3(256), 0, stream, A);
            else
                hipLaunchKernelGGL((frame_topk<64, true>), dim3(fb), dim3(256), 0, stream, A);
        } else {
            if (g.P <= 24 * 64)
                hipLaunchKernelGGL((frame_topk<24, false>), dim3(fb), dim3(256), 0, stream, A);
            else
                hipLaunchKernelGGL((frame_topk<64, false>), dim3(fb), dim3(256), 0, stream, A);
        }
    }
    return hipGetLastError();
}

hipError_t launch_corr_build(const CorrBuild &B, hipStream_t stream) {
    Args A{};
    A.g = B.g;
    A.F = B.dino;
    A.Fc = B.dino_cols ? B.dino_cols : B.dino;
    A.tok_map = B.tok_map;
    A.stride = B.row_stride;
    A.Df = B.Df;
    A.K = B.K;
    A.cap = B.cap;
    A.idx_out = B.idx_out;
    A.raw_dot = B.raw_dot;
    A.fallback_list_from = -1;
    const int64_t span = feature_span(B);
    A.f_bytes = 2 * span <= 0xFFFF0000ll ? (uint32_t)(2 * span) : 0u;
    const bool gemm = B.dino_dtype == BF16 && (B.Df % CK) == 0 && B.K <= 1024 && span < 0xFFFFFFFFll;
    A.all_rows_fallback = gemm ? 0 : 1;
    A.s = carve(B.scratch, B.g.Np, B.per_frame ? 0 : B.cap);
    const int64_t Np = B.g.Np;
    if (B.per_frame) {
        if (B.g.P > kFrameMaxP) return hipErrorInvalidValue;
        A.all_rows_fallback = 1;  // init_rows: norms only
        const unsigned rb = (unsigned)((Np + 3) / 4);
        if (B.dino_dtype == BF16)
            hipLaunchKernelGGL(init_rows<uint16_t>, dim3(rb), dim3(256), 0, stream, A);
        else
            hipLaunchKernelGGL(init_rows<float>, dim3(rb), dim3(256), 0, stream, A);
        return launch_corr_frames(A, B, false, stream);
    }
    if (B.total_by_frames) {
        // Total mode by way of frames: the K best overall lie among the
        // min(K, P) best of each frame, so every row's per-frame top lists
        // become its candidates and finalize selects exactly among them.
        if (B.g.P > kFrameMaxP) return hipErrorInvalidValue;
        const int32_t kf = std::min<int32_t>(B.K, B.g.P);
        A.cap = (B.g.S - 1) * kf;
        A.s = carve(B.scratch, Np, A.cap);
        A.seed_cols = 0;
        A.sym_lo = Np;
        A.all_rows_fallback = 0;
        const unsigned rb = (unsigned)((Np + 3) / 4);
        if (B.dino_dtype == BF16)
            hipLaunchKernelGGL(init_rows<uint16_t>, dim3(rb), dim3(256), 0, stream, A);
        else
            hipLaunchKernelGGL(init_rows<float>, dim3(rb), dim3(256), 0, stream, A);
        Args F = A;
        F.K = kf;
        hipError_t e = launch_corr_frames(F, B, true, stream);
        if (e != hipSuccess) return e;
        const unsigned cb = (unsigned)((Np + kRowWaves - 1) / kRowWaves);
        hipLaunchKernelGGL(finalize_rows<16>, dim3(cb), dim3(256), 0, stream, A, 0u, 16u * 64u);
        hipLaunchKernelGGL(finalize_rows<64>, dim3(cb), dim3(256), 0, stream, A, 16u * 64u, 0xFFFFFFFFu);
        const unsigned fb = (unsigned)std::min<int64_t>(kFallbackBlocks, Np);
        if (B.dino_dtype == BF16)
            hipLaunchKernelGGL(fallback_rows<uint16_t>, dim3(fb), dim3(1024), 0, stream, A);
        else
            hipLaunchKernelGGL(fallback_rows<float>, dim3(fb), dim3(1024), 0, stream, A);
        return hipGetLastError();
    }
    A.seed_cols = std::min<int64_t>(Np, 2 * (int64_t)B.g.P);
    // the symmetric square needs one operand for rows and columns
    A.sym_lo = (A.Fc == A.F) ? corr_sym_start(B.g) : Np;
    const unsigned rb = (unsigned)((Np + 3) / 4);
    if (B.dino_dtype == BF16)
        hipLaunchKernelGGL(init_rows<uint16_t>, dim3(rb), dim3(256), 0, stream, A);
    else
        hipLaunchKernelGGL(init_rows<float>, dim3(rb), dim3(256), 0, stream, A);
    if (gemm) {
        const unsigned cb = (unsigned)((Np + kRowWaves - 1) / kRowWaves);
        const uint32_t small = 16 * 64;
        auto compact = [&]() {
            const unsigned nb = (unsigned)((A.row_hi - A.row_lo + kRowWaves - 1) / kRowWaves);
            hipLaunchKernelGGL(compact_rows<16>, dim3(nb), dim3(256), 0, stream, A);
        };
        const int64_t W = A.sym_lo;
        const int32_t guess = corr_guess_rank(B.g, B.K, W);
        auto rect = [&](int mode, int64_t r_lo, int64_t r_hi, int64_t c_lo, int64_t c_hi) {
            A.row_lo = r_lo;
            A.row_hi = r_hi;
            A.col_lo = c_lo;
            A.col_hi = c_hi;
            const int64_t tiles = ((r_hi - r_lo + CT - 1) / CT) * ((c_hi - c_lo + CT - 1) / CT);
            const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)));
            if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
            if (mode == SEED)
                launch_cos<SEED>(grid, stream, A);
            else
                launch_cos<FILTER>(grid, stream, A);
            if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
            // the compaction after every row has seen [0, W) sets the
            // symmetric pass's thresholds
            A.guess_k = (W < Np && r_lo == 0 && r_hi == Np && c_hi == W) ? guess : 0;
            compact();
            A.guess_k = 0;
        };
        // 1. seed: frames 0 and 1 for every row, every candidate kept
        rect(SEED, 0, Np, 0, A.seed_cols);
        // 2. doubling filtered phases for every row up to W
        for (int64_t lo = A.seed_cols; lo < W; lo = std::min<int64_t>(2 * lo, W))
            rect(FILTER, 0, Np, lo, std::min<int64_t>(2 * lo, W));
        if (W < Np) {
            // 3. rows below W keep doubling over the remaining columns
            for (int64_t lo = W; lo < Np; lo = std::min<int64_t>(2 * lo, Np))
                rect(FILTER, 0, W, lo, std::min<int64_t>(2 * lo, Np));
            // 4. the square [W, Np)^2 once per unordered pair
            const int64_t nt = (Np - W + CT - 1) / CT;
            const int64_t tiles = nt * (nt + 1) / 2;
            A.row_lo = W;
            A.row_hi = Np;
            if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
            launch_cos<SYM>(dim3((unsigned)(8 * ((tiles + 7) / 8))), stream, A);
            if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
            compact();
        }
        hipLaunchKernelGGL(finalize_rows<16>, dim3(cb), dim3(256), 0, stream, A, 0u, small);
        hipLaunchKernelGGL(finalize_rows<64>, dim3(cb), dim3(256), 0, stream, A, small, 0xFFFFFFFFu);
        // rows flagged for an exact recomputation: the first kFixBatches x
        // kFallbackBlocks on the matrix cores (cosines of a batch of listed
        // rows into the fallback rows, then an exact block selection), the
        // rest, if any, on the per-row engine below
        hipLaunchKernelGGL(list_flagged, dim3((unsigned)((Np + 255) / 256)), dim3(256), 0, stream, A);
        Args L = A;
        L.use_list = 1;
        L.col_lo = 0;
        L.col_hi = Np;
        L.chunk = A.s.rowbuf;
        const int64_t ct = (Np + CT - 1) / CT;
        for (int b = 0; b < kFixBatches; ++b) {
            L.row_lo = (int64_t)b * kFallbackBlocks;
            L.row_hi = L.row_lo + kFallbackBlocks;
            launch_cos<STORE>(dim3((unsigned)(8 * ((ct + 7) / 8))), stream, L);
            hipLaunchKernelGGL(select_listed, dim3(kFallbackBlocks), dim3(1024), 0, stream, L, L.row_lo);
        }
        A.fallback_list_from = kFixBatches * kFallbackBlocks;
    }
    const unsigned fb = (unsigned)std::min<int64_t>(kFallbackBlocks, Np);
    if (B.dino_dtype == BF16)
        hipLaunchKernelGGL(fallback_rows<uint16_t>, dim3(fb), dim3(1024), 0, stream, A);
    else
        hipLaunchKernelGGL(fallback_rows<float>, dim3(fb), dim3(1024), 0, stream, A);
    return hipGetLastError();
}

}  // namespace saf
