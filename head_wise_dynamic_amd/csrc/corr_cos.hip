// Cosine GEMM of the correspondence index build (SAF3R Sec. 4.1 "DINO Top-K
// Kernel"): one phase over a block of the patch-pair space, on the matrix
// cores, with the filtering epilogue of its mode.  Building with
// -DSAF_COS_MODE=m instantiates the launcher for mode m only (the library
// build compiles this file once per mode, in parallel); without it every
// mode is instantiated.
#include "corr_common.h"

namespace saf {
namespace corr {
namespace {

// ---- one phase of the cosine GEMM with threshold filtering.
// Tile 256 x 256 per work-group of 8 waves (4 x 2); each wave owns 64 x 128
// as 2 x 4 blocks of 32 x 32 (v_mfma_f32_32x32x16_bf16, fp32 accumulators).
// Channels are staged through LDS 64 at a time, double buffered, with the
// next stage prefetched into registers while the current one is multiplied.
// Work-groups are mapped XCD by XCD (blockIdx % 8 selects the XCD): each XCD
// sweeps a contiguous, row-grouped range of tiles so that its L2 serves the
// operand panels its work-groups share.
// The phase modes are listed with CosMode.
constexpr int CROW = CK + 8;   // padded LDS row: 144 B, conflict-free 16-byte reads
constexpr int kGroupRows = 4;  // row tiles per group in the tile order
constexpr int kTileElems = CT * CROW;     // one operand tile in LDS (bf16)

// a compile-time bool as a value (for generic lambdas)
template <bool B> struct BoolTag {
    static constexpr bool value = B;
};

// value of lane (lane ^ j) within each group of 32 lanes (ds_swizzle in its
// and/or/xor mode: and 0x1F, or 0, xor j)
__device__ __forceinline__ float xor_lanes32(float x, int j) {
    const int b = __float_as_int(x);
    switch (j) {
    case 1: return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x1F | (1 << 10)));
    case 2: return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x1F | (2 << 10)));
    case 4: return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x1F | (4 << 10)));
    case 8: return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x1F | (8 << 10)));
    default: return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x1F | (16 << 10)));
    }
}

// patch of sample column c (-1 past the last frame); P >= 2 kFrameSample
// keeps the sampled patches of a frame distinct and evenly spread
__device__ __forceinline__ int64_t sample_patch(const Geom &g, int64_t c) {
    const int64_t f = c / kFrameSample, j = c % kFrameSample;
    return f < g.S ? f * g.P + (j * g.P) / kFrameSample : -1;
}

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
    constexpr bool kSym = MODE == SYM || MODE == PFSYM;
    constexpr int kRowCap = kSym ? 24 : 48;  // survivors staged per row per tile
    // operand tiles: As[2], Bs[2]; after the k-loop the same memory stages the
    // surviving candidates and per-lane accumulator spills
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kTileElems];
    uint16_t (*As)[kTileElems] = (uint16_t (*)[kTileElems])smem;
    uint16_t (*Bs)[kTileElems] = (uint16_t (*)[kTileElems])(smem + 2 * kTileElems);
    // thresholds per row (and per column in the symmetric modes); PFSYM holds
    // two per row, one for each frame the tile's columns (rows) span
    __shared__ float r_thr[2 * CT], r_iu[CT], c_thr[2 * CT];
    __shared__ float c_iv[CT];  // inverse norms of the tile's columns (NaN past the end)
    __shared__ int32_t r_frame[CT];
    __shared__ uint32_t r_cnt[CT], c_cnt[CT];

    const Geom &g = A.g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;  // wave rows [64 wr, +64), columns [128 wc, +128)
    const int n = lane & 31, gq = lane >> 5;

    // ---- tile of this work-group (a run of `run` column tiles from col0)
    constexpr int kRun = (MODE == FILTER && NK == 1) ? kFilterRun : 1;
    int64_t row0, col0, row_hi, col_hi;
    int run = 1;
    bool diag = false;
    if (kSym) {
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
        const int ncol_tiles = (int)((A.col_hi - A.col_lo + CT - 1) / CT);
        const int ncol = (ncol_tiles + kRun - 1) / kRun;  // column runs
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
        col0 = A.col_lo + (int64_t)ct * kRun * CT;
        run = min(kRun, ncol_tiles - ct * kRun);
        row_hi = A.row_hi;
        col_hi = A.col_hi;
    }
    const int64_t col_first = col0;
    for (int ci = 0; ci < run; ++ci) {
        const int64_t col0 = col_first + (int64_t)ci * CT;
        if (ci > 0) __syncthreads();  // the previous tile's flush is done with the LDS
        const uint16_t *F = (const uint16_t *)A.F, *Fc = (const uint16_t *)A.Fc;
        // STORE over a row list: tile rows are list positions; nothing to do past the list
        const uint32_t nlist = (MODE == STORE && A.use_list) ? *A.s.row_count : 0u;
        if (MODE == STORE && A.use_list && row0 >= (int64_t)nlist) return;
        auto actual_row = [&](int64_t pos) -> int64_t {
            if (pos >= row_hi) return -1;
            if (MODE == STORE && A.use_list) return pos < (int64_t)nlist ? (int64_t)A.s.row_list[pos] : -1;
            return pos;
        };
        // patch of column c (-1: none)
        auto col_operand = [&](int64_t c) -> int64_t {
            if (MODE == PFSEED) return c < col_hi ? sample_patch(g, c) : -1;
            return c < col_hi ? c : -1;
        };

        const int32_t f_row_lo = patch_frame(g, row0);
        const int32_t f_row_hi = patch_frame(g, min<int64_t>(row0 + CT, row_hi) - 1);
        const int32_t f_col_lo = patch_frame(g, col0);
        const int32_t f_col_hi = patch_frame(g, min<int64_t>(col0 + CT, col_hi) - 1);
        // Per-tile set-up: rows' inverse norms, thresholds and frames, and the
        // columns' (thresholds in the symmetric modes).  It runs after the first
        // operand stage's loads are issued, and every load here is unconditional
        // from a valid index (selected afterwards): a load under a per-lane
        // condition is waited for on its own, which serialised these loads.
        auto prologue = [&]() {
            if (tid < CT) {
                const int64_t u = actual_row(row0 + tid);
                const int64_t uc = u >= 0 ? u : 0;
                const float iu_l = A.s.invn[uc];
                float t0 = 0.f, t1 = 0.f;
                if (MODE == PFSYM) {
                    t0 = A.pthr[(int64_t)f_col_lo * g.Np + uc];
                    t1 = A.pthr[(int64_t)f_col_hi * g.Np + uc];
                } else {
                    t0 = (MODE == SYM || (MODE == FILTER && A.filter_guess)) ? A.s.theta_g[uc] : A.s.theta[uc];
                }
                float th0 = INFINITY, th1 = INFINITY, iu = __builtin_nanf("");  // NaN: no comparison passes
                int32_t fr = -1;
                if (u >= 0) {
                    iu = iu_l;
                    fr = patch_frame(g, u);
                    if (MODE == PFSYM) {
                        // a tile's columns span at most two frames (P >= CT); the
                        // own frame is never a candidate
                        if (f_col_lo != fr) th0 = scaled_threshold(t0, iu);
                        if (f_col_hi != f_col_lo && f_col_hi != fr) th1 = scaled_threshold(t1, iu);
                    } else {
                        th0 = scaled_threshold(t0, iu);
                    }
                }
                r_thr[tid] = th0;
                if (MODE == PFSYM) r_thr[CT + tid] = th1;
                r_iu[tid] = iu;
                r_frame[tid] = fr;
                r_cnt[tid] = 0u;
            } else {
                const int t = tid - CT;
                const int64_t v = col_operand(col0 + t);
                const int64_t vc = v >= 0 ? v : 0;
                const float iv_l = A.s.invn[vc];
                float t0 = 0.f, t1 = 0.f;
                if (MODE == PFSYM) {
                    t0 = A.pthr[(int64_t)f_row_lo * g.Np + vc];
                    t1 = A.pthr[(int64_t)f_row_hi * g.Np + vc];
                } else if (kSym) {
                    t0 = A.s.theta_g[vc];
                }
                c_iv[t] = v >= 0 ? iv_l : __builtin_nanf("");
                if (kSym) {
                    float th0 = INFINITY, th1 = INFINITY;
                    if (v >= 0) {
                        if (MODE == PFSYM) {
                            const int32_t fv = patch_frame(g, v);
                            if (f_row_lo != fv) th0 = scaled_threshold(t0, iv_l);
                            if (f_row_hi != f_row_lo && f_row_hi != fv) th1 = scaled_threshold(t1, iv_l);
                        } else {
                            th0 = scaled_threshold(t0, iv_l);
                        }
                    }
                    c_thr[t] = th0;
                    if (MODE == PFSYM) c_thr[CT + t] = th1;
                    c_cnt[t] = 0u;
                }
            }
        };
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
                const int64_t u = actual_row(row0 + row), v = col_operand(col0 + row);
                aoff[i] = u >= 0 ? 2u * ((uint32_t)frow(A, u) + 8u * seg) : kNone;
                boff[i] = v >= 0 ? 2u * ((uint32_t)frow(A, v) + 8u * seg) : kNone;
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
            prologue();
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
                const int64_t u = actual_row(row0 + row), v = col_operand(col0 + row);
                aoff[i] = u >= 0 ? (uint32_t)frow(A, u) : 0xFFFFFFFFu;
                boff[i] = v >= 0 ? (uint32_t)frow(A, v) : 0xFFFFFFFFu;
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
            prologue();
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
            const int64_t v = col_operand(vcol0 + 32 * bj);
            iv[bj] = c_iv[lc0 + 32 * bj];  // NaN never passes a comparison
            fv[bj] = v >= 0 ? patch_frame(g, v) : -2;
        }

        if (MODE == PFSEED) {
            // the wave's 128 columns are the sample of frame fs
            const int64_t fs = col0 / kFrameSample + wc;
            if (fs >= g.S) return;
            // per row, the largest of the lane's 4 sampled cosines
            float m[2][16];
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lr = 64 * wr + 32 * bi + 8 * (r >> 2) + 4 * gq + (r & 3);
                    const float iu = r_iu[lr];
                    float x = -INFINITY;
#pragma unroll
                    for (int bj = 0; bj < 4; ++bj) {
                        const float c = acc[bi][bj][r] * (iu * iv[bj]);
                        x = c > x ? c : x;
                    }
                    m[bi][r] = x;
                }
            // bitonic sort of the 32 lanes of each half-wave, descending: lane n
            // then holds the (n+1)-th largest lane maximum of every row.  The K
            // lanes with the largest maxima hold K distinct sampled patches at or
            // above lane K-1's value, so it never exceeds the frame's K-th best.
#pragma unroll
            for (int k = 2; k <= 32; k <<= 1)
#pragma unroll
                for (int j = k >> 1; j > 0; j >>= 1) {
                    const bool want_max = ((n & j) == 0) == ((n & k) == 0);
#pragma unroll
                    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float y = xor_lanes32(m[bi][r], j);
                            m[bi][r] = want_max ? fmaxf(m[bi][r], y) : fminf(m[bi][r], y);
                        }
                }
            if (n == A.K - 1) {
                float *dst = A.pthr + fs * g.Np + row0;
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int lr = 64 * wr + 32 * bi + 8 * (r >> 2) + 4 * gq + (r & 3);
                        if (r_frame[lr] >= 0) dst[lr] = m[bi][r];
                    }
            }
            return;
        }

        if (MODE == TBOUND) {
            // per row, the lane's largest cosine over its columns of other
            // frames (own frame and columns past the seed excluded); one slot
            // per (column tile, wave column half, lane)
            float *lm = (float *)A.s.cand;
            const int64_t slot = (col0 - A.col_lo) / CT * 64 + 32 * wc + n;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lr = 64 * wr + 32 * bi + 8 * (r >> 2) + 4 * gq + (r & 3);
                    const int32_t fr = r_frame[lr];
                    if (fr < 0) continue;
                    const float iu = r_iu[lr];
                    float x = -INFINITY;
#pragma unroll
                    for (int bj = 0; bj < 4; ++bj) {
                        const float c = acc[bi][bj][r] * (iu * iv[bj]);
                        if (fv[bj] >= 0 && fv[bj] != fr && c > x) x = c;
                    }
                    lm[(row0 + lr) * 2 * (int64_t)A.cap + slot] = x;
                }
            return;
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
        float *xl = (float *)(cstage + (kSym ? CT * kRowCap : 0)) + (wave * 64 + lane) * 16;
        const bool transposed = kSym && !diag;
        // a hit's slot in its row's LDS list, or (rare: more than kRowCap hits
        // of one row in one tile) straight into the row's global buffer
        auto place = [&](uint32_t slot, float2 *lst, int li, int64_t grow, float2 e) {
            if (slot < (uint32_t)kRowCap) {
                lst[li * kRowCap + slot] = e;
            } else {
                // one 64-bit store: a float2 store here was merged with the LDS
                // one into a flat (generic address) store on the common path
                const uint32_t gs = atomicAdd(&A.s.cnt[grow], 1u);
                if (gs < (uint32_t)A.cap)
                    ((unsigned long long *)A.s.cand)[grow * A.cap + gs] =
                        ((unsigned long long)__float_as_uint(e.y) << 32) | __float_as_uint(e.x);
            }
        };
        const float *thr_base = r_thr + 64 * wr + 4 * gq;
        const float *iu_base = r_iu + 64 * wr + 4 * gq;
        // PFSYM: columns from col_split on (rows from row_split on) lie in the
        // second frame the tile spans and use the second threshold
        const int64_t col_split = (int64_t)(f_col_lo + 1) * g.P, row_split = (int64_t)(f_row_lo + 1) * g.P;
        float cth[4], cth1[4];
        bool csec[4];
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            cth[bj] = transposed ? c_thr[lc0 + 32 * bj] : INFINITY;
            cth1[bj] = (MODE == PFSYM && transposed) ? c_thr[CT + lc0 + 32 * bj] : INFINITY;
            csec[bj] = MODE == PFSYM && vcol0 + 32 * bj >= col_split;
        }
        // keep masks of the lane's 16 values of each block of row block bi,
        // built from the last row down so that row r lands on bit r; a row's
        // thresholds are read once for the four blocks.  TR (transposed
        // comparisons too) is a compile-time flag: a run-time test inside the
        // loop became a branch per comparison.
        auto keep_masks = [&](auto tr, int bi, uint32_t (&kfa)[4], uint32_t (&kta)[4]) {
            constexpr bool TR = decltype(tr)::value;
#pragma unroll
            for (int r = 15; r >= 0; --r) {
                const int o = 32 * bi + 8 * (r >> 2) + (r & 3);
                const float t0 = thr_base[o];
                const float t1 = MODE == PFSYM ? thr_base[CT + o] : t0;
                const float iu = iu_base[o];
                const bool rsec = MODE == PFSYM && row0 + 64 * wr + 4 * gq + o >= row_split;
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    const float a = acc[bi][bj][r];
                    kfa[bj] = kfa[bj] + kfa[bj] + (uint32_t)(a * iv[bj] >= (csec[bj] ? t1 : t0));
                    if (TR) kta[bj] = kta[bj] + kta[bj] + (uint32_t)(a * iu >= (rsec ? cth1[bj] : cth[bj]));
                }
            }
        };
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            uint32_t kfa[4] = {0u, 0u, 0u, 0u}, kta[4] = {0u, 0u, 0u, 0u};
            if (transposed)
                keep_masks(BoolTag<true>{}, bi, kfa, kta);
            else
                keep_masks(BoolTag<false>{}, bi, kfa, kta);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const uint32_t kf = kfa[bj], kt = kta[bj];
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
                        const bool hf = (kf >> r) & 1u, ht = (kt >> r) & 1u;
                        // both slot reservations issued before either result is waited for
                        uint32_t sf = 0u, st = 0u;
                        if (hf) sf = atomicAdd(&r_cnt[lr], 1u);
                        if (ht) st = atomicAdd(&c_cnt[lc], 1u);
                        if (hf) place(sf, stage, lr, row0 + lr, make_float2(c, __int_as_float(v)));
                        if (ht) place(st, cstage, lc, (int64_t)v, make_float2(c, __int_as_float((int32_t)(row0 + lr))));
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
}

}  // namespace

template <int MODE> void launch_cos(dim3 grid, hipStream_t stream, const Args &A) {
    const bool fixed = A.f_bytes != 0;  // byte offsets fit 32 bits
    if (fixed && A.Df == 1024)
        hipLaunchKernelGGL((cos_phase<MODE, 16>), grid, dim3(kCosThreads), 0, stream, A);
    else if (fixed && A.Df == 768)
        hipLaunchKernelGGL((cos_phase<MODE, 12>), grid, dim3(kCosThreads), 0, stream, A);
    else if (fixed && A.Df == 384)
        hipLaunchKernelGGL((cos_phase<MODE, 6>), grid, dim3(kCosThreads), 0, stream, A);
    else if (fixed && A.Df == 64) {
        dim3 gr = grid;
        if (MODE == FILTER) {  // a work-group per run of kFilterRun column tiles
            const int64_t nrow = (A.row_hi - A.row_lo + CT - 1) / CT;
            const int64_t runs = ((A.col_hi - A.col_lo + CT - 1) / CT + kFilterRun - 1) / kFilterRun;
            gr = dim3((unsigned)(8 * ((nrow * runs + 7) / 8)));
        }
        hipLaunchKernelGGL((cos_phase<MODE, 1>), gr, dim3(kCosThreads), 0, stream, A);
    }
    else
        hipLaunchKernelGGL((cos_phase<MODE, 0>), grid, dim3(kCosThreads), 0, stream, A);
}

#ifdef SAF_COS_MODE
template void launch_cos<SAF_COS_MODE>(dim3, hipStream_t, const Args &);
#else
template void launch_cos<SEED>(dim3, hipStream_t, const Args &);
template void launch_cos<FILTER>(dim3, hipStream_t, const Args &);
template void launch_cos<SYM>(dim3, hipStream_t, const Args &);
template void launch_cos<STORE>(dim3, hipStream_t, const Args &);
template void launch_cos<PFSEED>(dim3, hipStream_t, const Args &);
template void launch_cos<PFSYM>(dim3, hipStream_t, const Args &);
template void launch_cos<TBOUND>(dim3, hipStream_t, const Args &);
#endif

}  // namespace corr
}  // namespace saf
