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
// Direct square (4 K + 128 <= P, one operand for rows and columns, and the
// two seed frames holding on average at least 5 of a row's K best:
// 2 K >= 5 (S - 1)): the seed phase's lane maxima (as in 1. below) give
// every row a guess theta_g_u of its K-th best, their r-th largest with r
// the guess rank over the seed columns of other frames; the whole square
// [0, Np)^2 is then filtered by it once per unordered pair, compacted, and
// finalized with the guess check of 4./5.  With two operands (a head's
// logits q_u . k_v: no symmetry), the same guess filters one pass over every
// (row, column) pair instead.  Otherwise:
//   1. seed: columns of frames 0 and 1.  When 4 K + 128 <= P, only each
//      lane's largest cosine over its 4 seed columns of other frames is
//      kept, and a row's K-th largest such value (reached by K distinct
//      patches) becomes its first theta_u; the first filtered phase then
//      covers [0, 4P).  Otherwise every seed candidate is kept;
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
// Per-frame mode (K best of every other frame), fused (bf16, P >= 256,
//   K <= 8): the cosine matrix is never stored either.
//   1. bounds: every row against a 128-patch sample of every frame; the K-th
//      largest of the 32 lane maxima (each over 4 sampled patches) of a
//      (row, frame) is attained by K distinct patches of that frame, so it is
//      a lower bound of the row's K-th best there;
//   2. the symmetric square once, keeping c >= the bound of (row, frame of
//      the column) in both directions, into per-row candidate buffers;
//   3. per row: counting sort of the candidates by frame in LDS, then a few
//      lanes per frame keep the K best in sorted register lists, merged;
//   4. a row whose buffer overflowed (or a frame short of K) is recomputed
//      exactly, as in total mode but selected per frame.
// Per-frame mode otherwise (and on request): the GEMM writes fp32 row chunks
//   of the cosine matrix, then one wave per (row, frame) selects.
#include "corr_common.h"
#include "topk_block.h"

namespace saf {

using namespace corr;

namespace {

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

// ---- bound seed: each row's K-th largest stored lane maximum (TBOUND) as
// its first threshold; a row with fewer than K of them gets none (-inf).
// With a guess rank (A.guess_k), also theta_g from the guess_k-th largest:
// the direct square's filter, checked when the row is finalized.
template <int MAXE> __global__ __launch_bounds__(256) void bound_rows(const Args A) {
    const int64_t u = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (u >= A.g.Np) return;
    const float *lm = (const float *)A.s.cand + u * 2 * (int64_t)A.cap;
    const int n = A.lm_per_row;
    uint32_t key[MAXE];  // order key; 0: no value
    float x[MAXE];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) x[e] = lm[min(e * 64 + lane, n - 1)];  // unconditional, masked below
#pragma unroll
    for (int e = 0; e < MAXE; ++e) key[e] = (e * 64 + lane < n && x[e] > -INFINITY) ? order_key(x[e]) : 0u;
    // largest order key reached by at least `rank` stored values (0: fewer values)
    auto kth_key = [&](uint32_t rank) {
        uint32_t thr = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < MAXE; ++e) c += (uint32_t)__popcll(__ballot(key[e] >= cand));
            if (c >= rank) thr = cand;
        }
        return thr;
    };
    const uint32_t thr = kth_key((uint32_t)A.K);
    if (lane == 0) A.s.theta[u] = thr ? order_key_to_float(thr) : -INFINITY;
    if (A.guess_k) {
        const uint32_t rank = (uint32_t)(u < 2 * (int64_t)A.g.P ? A.guess_k_seed : A.guess_k);
        const uint32_t gthr = kth_key(rank);
        if (lane == 0) A.s.theta_g[u] = gthr ? order_key_to_float(gthr) : -INFINITY;
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

// Selection of one frame's K best among its P cosines at src (one wave):
// key[e] receives the order key of patch e * 64 + lane (0: no patch), and
// bit e of the result is set when that patch is kept.
template <int MAXE>
__device__ uint64_t frame_keep(const float *src, int32_t P, uint32_t K, int lane, uint32_t (&key)[MAXE]) {
    const int ne = (P + 63) / 64;
    // unconditional loads (a slot past the frame reads its last patch and is
    // emptied afterwards), so that all of them are in flight together
    float x[MAXE];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) x[e] = src[min(e * 64 + lane, P - 1)];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int i = e * 64 + lane;
        key[e] = (e < ne && i < P) ? max(order_key(x[e]), 1u) : 0u;
    }
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
                const uint64_t y = __shfl_xor(w, o);
                w = y > w ? y : w;
            }
            const uint32_t wi = 0x7FFFFFFFu - (uint32_t)(w & 0xFFFFFFFFu);
            if ((w >> 32) != 0 && (int)(wi & 63) == lane) keep |= 1ull << (wi >> 6);
        }
        return keep;
    }
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
    return keep;
}

// tokens of the kept patches of frame gf, ascending, to out[0, K)
template <int MAXE>
__device__ void frame_emit(const Geom &g, int32_t gf, uint64_t keep, int lane, int32_t *out) {
    const int ne = (g.P + 63) / 64;
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

// Items are (row, frame) pairs of rows [row_lo, row_hi), whose cosines lie in
// A.chunk; with A.use_list the rows are positions of s.row_list (flagged
// rows of the fused mode) and the chunk holds them in list order.
template <int MAXE, bool CAND>
__global__ __launch_bounds__(256) void frame_topk(const Args A) {
    const Geom &g = A.g;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    const int64_t rows = A.row_hi - A.row_lo;
    if (item >= rows * g.S) return;
    const int64_t pos = A.row_lo + item / g.S;
    int64_t u = pos;
    if (A.use_list) {
        if (pos >= (int64_t)*A.s.row_count) return;
        u = A.s.row_list[pos];
    }
    const int32_t gf = (int32_t)(item % g.S), fu = (int32_t)(u / g.P);
    if (gf == fu) return;
    const float *src = A.chunk + (pos - A.row_lo) * g.Np + (int64_t)gf * g.P;
    uint32_t key[MAXE];  // order_key of the cosine; 0 marks an empty slot
    const uint64_t keep = frame_keep<MAXE>(src, g.P, (uint32_t)A.K, lane, key);
    const int32_t slot = gf - (gf > fu ? 1 : 0);
    if (CAND) {
        // candidates (score, patch) for an exact selection over all frames
        const int ne = (g.P + 63) / 64;
        float2 *cand = A.s.cand + u * A.cap + (int64_t)slot * A.K;
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        uint32_t p = 0;
#pragma unroll
        for (int e = 0; e < MAXE; ++e) {
            if (e < ne) {
                const bool kp = (keep >> e) & 1ull;
                const uint64_t m = __ballot(kp);
                if (kp)
                    cand[p + (uint32_t)__popcll(m & below)] =
                        make_float2(order_key_to_float(key[e]), __int_as_float(gf * g.P + e * 64 + lane));
                p += (uint32_t)__popcll(m);
            }
        }
        if (slot == 0 && lane == 0) {
            A.s.cnt[u] = (uint32_t)((g.S - 1) * A.K);
            A.s.over[u] = 0u;
        }
        return;
    }
    frame_emit<MAXE>(g, gf, keep, lane, A.idx_out + u * ((int64_t)(g.S - 1) * A.K) + (int64_t)slot * A.K);
}

// ---- fused per-frame mode: a row's candidates from the filtered symmetric
// pass are bucketed by frame in LDS (counting sort), then a group of lanes
// per frame keeps the K best by (cosine desc, patch asc) and writes their
// tokens ascending.  Every frame must hold at least K
// candidates (the filter bounds never exceed the K-th best); a row that
// overflowed its buffer, or a frame short of K, flags the row for an exact
// recomputation.
constexpr int kFinThreads = 512;
constexpr int kFinPer = 24;  // candidates per thread: capacity <= 12288
template <int KMAX>
__global__ __launch_bounds__(kFinThreads) void frame_finalize(const Args A) {
    extern __shared__ __attribute__((aligned(16))) unsigned char fin_lds[];
    __shared__ int bad;
    const Geom &g = A.g;
    const int64_t u = blockIdx.x;
    const int tid = threadIdx.x;
    uint32_t *hist = (uint32_t *)fin_lds;                          // [S] entries per frame
    uint32_t *base = hist + g.S;                                   // [S] bucket starts
    float2 *ent = (float2 *)(fin_lds + align256(8 * (size_t)g.S));  // [cap] bucketed entries
    const uint32_t n = A.s.cnt[u];
    if (A.s.over[u] || n > (uint32_t)A.cap || n == 0u) {
        if (tid == 0) A.s.over[u] = 1u;
        return;
    }
    for (int f = tid; f < g.S; f += kFinThreads) hist[f] = 0u;
    if (tid == 0) bad = 0;
    __syncthreads();
    const float2 *cand = A.s.cand + u * A.cap;
    float2 e[kFinPer];
    uint32_t fp[kFinPer];  // frame << 16 | position in the frame's bucket
#pragma unroll
    for (int i = 0; i < kFinPer; ++i) e[i] = cand[min((uint32_t)(tid + i * kFinThreads), n - 1)];
#pragma unroll
    for (int i = 0; i < kFinPer; ++i) {
        if ((uint32_t)(tid + i * kFinThreads) < n) {
            const uint32_t f = (uint32_t)__float_as_int(e[i].y) / (uint32_t)g.P;
            fp[i] = (f << 16) | atomicAdd(&hist[f], 1u);
        }
    }
    __syncthreads();
    if (tid < 64) {  // exclusive scan of the bucket sizes, one wave
        const int per = (g.S + 63) / 64, f0 = tid * per, f1 = min(f0 + per, g.S);
        uint32_t sum = 0;
        for (int f = f0; f < f1; ++f) sum += hist[f];
        uint32_t incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(incl, o);
            if (tid >= o) incl += y;
        }
        uint32_t run = incl - sum;
        for (int f = f0; f < f1; ++f) {
            base[f] = run;
            run += hist[f];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kFinPer; ++i)
        if ((uint32_t)(tid + i * kFinThreads) < n) ent[base[fp[i] >> 16] + (fp[i] & 0xFFFFu)] = e[i];
    __syncthreads();
    const int32_t fu = (int32_t)(u / g.P);
    const int K = A.K;
    // G lanes per frame (8 when the frames fit the block that way): lane gl
    // of a group keeps the KMAX best of the bucket entries gl, gl + G, ... in a
    // sorted register list of keys (cosine order key above, complemented patch
    // below, so ties go to the lower patch); the group's lists are then merged
    // by a butterfly of bitonic merges
    const int G = g.S * 8 <= kFinThreads ? 8 : g.S * 4 <= kFinThreads ? 4 : g.S * 2 <= kFinThreads ? 2 : 1;
    const int gl = tid & (G - 1);
    for (int fb = 0; fb < g.S; fb += kFinThreads / G) {
        const int f = fb + tid / G;
        const bool active = f < g.S && f != fu;
        const uint32_t c = active ? hist[f] : 0u, b0 = active ? base[f] : 0u;
        if (active && c < (uint32_t)K) bad = 1;
        uint64_t L[KMAX];
#pragma unroll
        for (int s = 0; s < KMAX; ++s) L[s] = 0ull;
        for (uint32_t i = gl; i < c; i += G) {
            const float2 x = ent[b0 + i];
            uint64_t key = ((uint64_t)max(order_key(x.x), 1u) << 32) | (0xFFFFFFFFu - (uint32_t)__float_as_int(x.y));
            if (key > L[KMAX - 1]) {
#pragma unroll
                for (int s = 0; s < KMAX; ++s) {
                    const uint64_t hi = key > L[s] ? key : L[s];
                    key = key > L[s] ? L[s] : key;
                    L[s] = hi;
                }
            }
        }
        for (int o = 1; o < G; o <<= 1) {
            // the KMAX best of two descending lists: the elementwise max of one
            // and the other reversed is bitonic; a half-cleaner cascade sorts it
            uint64_t M[KMAX];
#pragma unroll
            for (int s = 0; s < KMAX; ++s) {
                const uint64_t r = __shfl_xor(L[KMAX - 1 - s], o);
                M[s] = L[s] > r ? L[s] : r;
            }
#pragma unroll
            for (int j = KMAX / 2; j > 0; j >>= 1)
#pragma unroll
                for (int s = 0; s < KMAX; ++s)
                    if ((s & j) == 0) {
                        const uint64_t hi = M[s] > M[s + j] ? M[s] : M[s + j];
                        const uint64_t lo = M[s] > M[s + j] ? M[s + j] : M[s];
                        M[s] = hi;
                        M[s + j] = lo;
                    }
#pragma unroll
            for (int s = 0; s < KMAX; ++s) L[s] = M[s];
        }
        if (!active || gl != 0 || c < (uint32_t)K) continue;
        // the K best patches in ascending order (odd-even transposition sort)
        int32_t p[KMAX];
#pragma unroll
        for (int s = 0; s < KMAX; ++s) p[s] = s < K ? (int32_t)(0xFFFFFFFFu - (uint32_t)L[s]) : INT32_MAX;
#pragma unroll
        for (int pass = 0; pass < KMAX; ++pass)
#pragma unroll
            for (int s = pass & 1; s + 1 < KMAX; s += 2) {
                const int32_t lo = min(p[s], p[s + 1]), hi = max(p[s], p[s + 1]);
                p[s] = lo;
                p[s + 1] = hi;
            }
        int32_t *out = A.idx_out + u * ((int64_t)(g.S - 1) * K) + (int64_t)(f - (f > fu ? 1 : 0)) * K;
        const int32_t tok0 = f * g.T + g.ns - f * g.P;
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
            if (s < K) out[s] = tok0 + p[s];
    }
    __syncthreads();
    if (tid == 0 && bad) A.s.over[u] = 1u;
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
template <typename T, bool PER_FRAME = false> __global__ __launch_bounds__(1024) void fallback_rows(const Args A) {
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
        if constexpr (PER_FRAME) {
            // the K best of every other frame, one wave per frame
            const int lane = threadIdx.x & 63;
            for (int32_t f = (int32_t)(threadIdx.x >> 6); f < g.S; f += 16) {
                if (f == fr) continue;
                int32_t *out = A.idx_out + u * ((int64_t)(g.S - 1) * A.K) + (int64_t)(f - (f > fr ? 1 : 0)) * A.K;
                const float *src = row + (int64_t)f * g.P;
                if (g.P <= 24 * 64) {
                    uint32_t key[24];
                    frame_emit<24>(g, f, frame_keep<24>(src, g.P, (uint32_t)A.K, lane, key), lane, out);
                } else {
                    uint32_t key[64];
                    frame_emit<64>(g, f, frame_keep<64>(src, g.P, (uint32_t)A.K, lane, key), lane, out);
                }
            }
        } else {
            int32_t *out = A.idx_out + u * A.K;
            block_topk_ascending(row, g.Np, A.K, [&](int64_t pos, int64_t v) {
                out[pos] = (int32_t)((v / g.P) * g.T + g.ns + (v % g.P));
            });
        }
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

constexpr size_t kFrameFusedMaxBytes = (size_t)32 << 30;
constexpr int32_t kFrameFusedMaxK = 8;

size_t corr_frame_fused_scratch_bytes(const Geom &g, int32_t cap) {
    return carve_head_bytes(g.Np, cap) + align256(sizeof(float) * (size_t)kFallbackBlocks * g.Np) +
           align256(sizeof(float) * (size_t)g.S * g.Np);
}

static int64_t feature_span(const CorrBuild &B);

int32_t corr_frame_fused_cap(const CorrBuild &B) {
    const Geom &g = B.g;
    if (!B.per_frame || B.frames_stored || B.dino_dtype != BF16 || (B.Df % CK) != 0) return 0;
    if ((B.dino_cols && B.dino_cols != B.dino) || feature_span(B) >= 0xFFFFFFFFll) return 0;
    if (g.P < CT || g.P > kFrameMaxP || B.K < 1 || B.K > kFrameFusedMaxK || g.S < 2 || g.S > 4096) return 0;
    // candidates per (row, frame) passing a bound at the K-th largest of 32
    // lane maxima of a 128-patch sample: about K (P+1)/129 (1 + K/64) for
    // ranks in random order; the capacity allows 20 % more plus 512
    const double per = (double)(g.P + 1) / (kFrameSample + 1) * B.K * (1.0 + B.K / 64.0);
    int64_t cap = (int64_t)std::ceil((g.S - 1) * per * 1.2) + 512;
    cap = (cap + 63) / 64 * 64;
    if (cap > (int64_t)kFinThreads * kFinPer) return 0;
    if (corr_frame_fused_scratch_bytes(g, (int32_t)cap) > kFrameFusedMaxBytes) return 0;
    return (int32_t)cap;
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
// feature widths (ViT-S/B/L: 384, 768, 1024 channels) and for 64 (an
// attention head's q and k, the index taken from a head's logits)

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

// Fused per-frame mode: per-(row, frame) bounds from a sampled pass, the
// symmetric square once filtered by them, per-row frame buckets, then any
// flagged rows exactly (a cosine row batch on the matrix cores, else the
// per-row engine).
static hipError_t launch_corr_frames_fused(Args &A, const CorrBuild &B, hipStream_t stream) {
    const Geom &g = B.g;
    const int64_t Np = g.Np;
    A.cap = B.cap;
    A.s = carve(B.scratch, Np, A.cap);
    A.pthr = (float *)((char *)A.s.rowbuf + align256(sizeof(float) * (size_t)kFallbackBlocks * Np));
    A.seed_cols = 0;
    A.sym_lo = 0;
    A.all_rows_fallback = 0;
    hipLaunchKernelGGL(init_rows<uint16_t>, dim3((unsigned)((Np + 3) / 4)), dim3(256), 0, stream, A);
    // 1. bounds: every row against kFrameSample patches of every frame
    A.row_lo = 0;
    A.row_hi = Np;
    A.col_lo = 0;
    A.col_hi = (int64_t)g.S * kFrameSample;
    {
        const int64_t tiles = ((Np + CT - 1) / CT) * ((A.col_hi + CT - 1) / CT);
        if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
        launch_cos<PFSEED>(dim3((unsigned)(8 * ((tiles + 7) / 8))), stream, A);
        if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
    }
    // 2. the square once per unordered pair, filtered by the bounds
    {
        const int64_t nt = (Np + CT - 1) / CT;
        const int64_t tiles = nt * (nt + 1) / 2;
        A.col_lo = 0;
        A.col_hi = Np;
        if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
        launch_cos<PFSYM>(dim3((unsigned)(8 * ((tiles + 7) / 8))), stream, A);
        if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
    }
    // 3. every row: candidates bucketed by frame, the K best of each
    const size_t lds = align256(8 * (size_t)g.S) + sizeof(float2) * (size_t)A.cap;
    hipError_t e;
    if (A.K <= 4) {
        e = hipFuncSetAttribute((const void *)frame_finalize<4>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(frame_finalize<4>, dim3((unsigned)Np), dim3(kFinThreads), lds, stream, A);
    } else {
        e = hipFuncSetAttribute((const void *)frame_finalize<8>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(frame_finalize<8>, dim3((unsigned)Np), dim3(kFinThreads), lds, stream, A);
    }
    // 4. flagged rows: kFixBatches x kFallbackBlocks of them as cosine rows on
    // the matrix cores, selected per frame; the rest on the per-row engine
    hipLaunchKernelGGL(list_flagged, dim3((unsigned)((Np + 255) / 256)), dim3(256), 0, stream, A);
    Args L = A;
    L.use_list = 1;
    L.col_lo = 0;
    L.col_hi = Np;
    L.chunk = A.s.rowbuf;
    const int64_t ct = (Np + CT - 1) / CT;
    const unsigned fb_items = (unsigned)(((int64_t)kFallbackBlocks * g.S + kRowWaves - 1) / kRowWaves);
    for (int b = 0; b < kFixBatches; ++b) {
        L.row_lo = (int64_t)b * kFallbackBlocks;
        L.row_hi = L.row_lo + kFallbackBlocks;
        launch_cos<STORE>(dim3((unsigned)(8 * ((ct + 7) / 8))), stream, L);
        if (g.P <= 24 * 64)
            hipLaunchKernelGGL((frame_topk<24, false>), dim3(fb_items), dim3(256), 0, stream, L);
        else
            hipLaunchKernelGGL((frame_topk<64, false>), dim3(fb_items), dim3(256), 0, stream, L);
    }
    A.fallback_list_from = kFixBatches * kFallbackBlocks;
    const unsigned fb = (unsigned)std::min<int64_t>(kFallbackBlocks, Np);
    hipLaunchKernelGGL((fallback_rows<uint16_t, true>), dim3(fb), dim3(1024), 0, stream, A);
    return hipGetLastError();
}

static bool corr_uses_engine(const CorrBuild &B) {
    return B.dino_dtype == BF16 && (B.Df % CK) == 0 && B.K <= 1024 && feature_span(B) < 0xFFFFFFFFll;
}

bool corr_build_lists_rows(const CorrBuild &B) {
    if (B.per_frame) return B.cap > 0;
    return !B.total_by_frames && corr_uses_engine(B);
}

void corr_recomputed_list(void *scratch, int64_t Np, int32_t cap, int32_t **rows, uint32_t **count) {
    const Scratch s = carve(scratch, Np, cap);
    *rows = s.row_list;
    *count = s.row_count;
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
    const bool gemm = corr_uses_engine(B);
    A.all_rows_fallback = gemm ? 0 : 1;
    A.s = carve(B.scratch, B.g.Np, B.per_frame ? 0 : B.cap);
    const int64_t Np = B.g.Np;
    if (B.per_frame) {
        if (B.g.P > kFrameMaxP) return hipErrorInvalidValue;
        if (B.cap > 0) {
            if (B.cap != corr_frame_fused_cap(B)) return hipErrorInvalidValue;
            return launch_corr_frames_fused(A, B, stream);
        }
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
    const int64_t seed_cols = std::min<int64_t>(Np, 2 * (int64_t)B.g.P);
    // Bound seed: instead of storing every cosine of the seed frames (then
    // compacting them), their lane maxima give each row a lower bound of its
    // K-th best, and the first filtered phase starts at column 0.  Needs K
    // lane maxima of other frames in every row (4 K + 128 <= P) and the lane
    // maxima within the candidate buffer's row.
    const bool bound_seed = gemm && seed_cols == 2 * (int64_t)B.g.P && B.g.P <= 4096 &&
                            4 * (int64_t)B.K + 128 <= B.g.P;
    A.seed_cols = bound_seed ? 0 : seed_cols;
    // Direct square (bound seed, one operand for rows and columns): every
    // row's guess of its K-th best comes from the seed frames' lane maxima,
    // and the whole square [0, Np)^2 is filtered by it once per unordered pair
    // (no filtered column phases, no compaction between them).  The seed
    // frames hold on average K 2P / ((S-1) P) of a row's K best; below 5 the
    // guess fails too often (each failure is a recomputed row).
    const bool guess_ok = bound_seed && (int64_t)B.K * seed_cols >= 5ll * (B.g.S - 1) * B.g.P;
    const bool direct = guess_ok && A.Fc == A.F;
    // two operands: one filtered pass over [0, Np) x [0, Np) with the guess
    const bool direct_rect = guess_ok && A.Fc != A.F;
    // the symmetric square needs one operand for rows and columns; with a
    // direct pass every row's guess is checked when it is finalized
    A.sym_lo = (direct || direct_rect) ? 0 : (A.Fc == A.F) ? corr_sym_start(B.g) : Np;
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
        int64_t lo0 = seed_cols;
        auto bound_and_guess = [&]() {
            // the seed frames' lane maxima: a lower bound (theta) and a guess
            // (theta_g) of every row's K-th best; the guess rank is
            // corr_guess_rank's over the seed columns of other frames
            A.row_lo = 0;
            A.row_hi = Np;
            A.col_lo = 0;
            A.col_hi = seed_cols;
            A.lm_per_row = (int32_t)((seed_cols + CT - 1) / CT * 64);
            const int64_t tiles = ((Np + CT - 1) / CT) * ((seed_cols + CT - 1) / CT);
            if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
            launch_cos<TBOUND>(dim3((unsigned)(8 * ((tiles + 7) / 8))), stream, A);
            if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
            A.guess_k = corr_guess_rank(B.g, B.K, seed_cols);
            A.guess_k_seed = corr_guess_rank(B.g, B.K, seed_cols - B.g.P);
            if (A.lm_per_row <= 16 * 64)
                hipLaunchKernelGGL(bound_rows<16>, dim3(cb), dim3(256), 0, stream, A);
            else
                hipLaunchKernelGGL(bound_rows<32>, dim3(cb), dim3(256), 0, stream, A);
            A.guess_k = A.guess_k_seed = 0;
        };
        if (direct_rect) {
            // 1. bound and guess from the seed frames; 2. every pair once,
            // filtered by the guess; then compaction, finalize and its check
            bound_and_guess();
            A.filter_guess = 1;
            rect(FILTER, 0, Np, 0, Np);
            A.filter_guess = 0;
            lo0 = Np;
        } else if (direct) {
            // 1. the seed frames' lane maxima: a lower bound (theta) and a
            // guess (theta_g) of every row's K-th best; the guess rank is
            // corr_guess_rank's over the seed columns of other frames
            A.row_lo = 0;
            A.row_hi = Np;
            A.col_lo = 0;
            A.col_hi = seed_cols;
            A.lm_per_row = (int32_t)((seed_cols + CT - 1) / CT * 64);
            const int64_t tiles = ((Np + CT - 1) / CT) * ((seed_cols + CT - 1) / CT);
            if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
            launch_cos<TBOUND>(dim3((unsigned)(8 * ((tiles + 7) / 8))), stream, A);
            if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
            A.guess_k = corr_guess_rank(B.g, B.K, seed_cols);
            A.guess_k_seed = corr_guess_rank(B.g, B.K, seed_cols - B.g.P);
            if (A.lm_per_row <= 16 * 64)
                hipLaunchKernelGGL(bound_rows<16>, dim3(cb), dim3(256), 0, stream, A);
            else
                hipLaunchKernelGGL(bound_rows<32>, dim3(cb), dim3(256), 0, stream, A);
            A.guess_k = A.guess_k_seed = 0;
            // 2. the square [0, Np)^2 once per unordered pair
            const int64_t nt = (Np + CT - 1) / CT;
            const int64_t sq = nt * (nt + 1) / 2;
            A.row_lo = 0;
            A.row_hi = Np;
            A.col_lo = 0;
            A.col_hi = Np;
            if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
            launch_cos<SYM>(dim3((unsigned)(8 * ((sq + 7) / 8))), stream, A);
            if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
            compact();
        } else if (bound_seed) {
            // 1. bounds from the seed frames' lane maxima, then the first
            // filtered phase over [0, 2 seed)
            A.row_lo = 0;
            A.row_hi = Np;
            A.col_lo = 0;
            A.col_hi = seed_cols;
            A.lm_per_row = (int32_t)((seed_cols + CT - 1) / CT * 64);
            const int64_t tiles = ((Np + CT - 1) / CT) * ((seed_cols + CT - 1) / CT);
            if (B.mark) B.mark(B.mark_user, 1, "cosine_gemm", stream);
            launch_cos<TBOUND>(dim3((unsigned)(8 * ((tiles + 7) / 8))), stream, A);
            if (B.mark) B.mark(B.mark_user, 0, "cosine_gemm", stream);
            if (A.lm_per_row <= 16 * 64)
                hipLaunchKernelGGL(bound_rows<16>, dim3(cb), dim3(256), 0, stream, A);
            else
                hipLaunchKernelGGL(bound_rows<32>, dim3(cb), dim3(256), 0, stream, A);
            lo0 = std::min<int64_t>(2 * seed_cols, W);
            rect(FILTER, 0, Np, 0, lo0);
        } else {
            // 1. seed: frames 0 and 1 for every row, every candidate kept
            rect(SEED, 0, Np, 0, seed_cols);
        }
        // 2. doubling filtered phases for every row up to W
        for (int64_t lo = lo0; !direct && lo < W; lo = std::min<int64_t>(2 * lo, W))
            rect(FILTER, 0, Np, lo, std::min<int64_t>(2 * lo, W));
        if (!direct && !direct_rect && W < Np) {
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
