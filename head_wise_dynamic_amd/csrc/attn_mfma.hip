// Shared-key sparse attention on MFMA (bf16 in, fp32 accumulate).
//
// Used for the heads whose queries share one key set inside a query tile:
// position heads (tile = part of one frame), vertical-line and scanning heads
// (one set for every query), dense heads, and the special-token rows of
// correspondence heads (which attend to every key).  This is the pages'
// "Static", "Query-Probe Top-K" and "Uniform Sampling" kernels (SAF3R,
// Sec. 4.1) on CDNA4 matrix cores: the selected keys are gathered by token
// index straight into LDS tiles, so no packed copy of K/V is ever written.
//
// Work-group = 4 waves = 256 query rows (64 per wave, as two 32-row blocks
// that share every K and V fragment read from LDS); key tiles of 64.
// Per wave and tile, S^T = K Q^T is formed with v_mfma_f32_32x32x16_bf16 so
// that a lane owns one query column: the online softmax (running max m, sum l)
// needs one cross-lane exchange (lane ^ 32) per tile.  The key rows of the
// S^T A-operand are read in a permuted order (bits 2 and 3 of the row index
// swapped) so that the accumulator registers a lane feeds to the P.V product
// cover 8 consecutive keys.  V stays row-major in LDS and the V^T operand
// of O^T = V^T P^T is read with the transposing LDS loads of gfx950
// (ds_read_b64_tr_b16).  O^T accumulates in fp32 and is normalised at the
// end; the softmax denominator is summed from the same bf16-rounded weights
// that enter P.V (v_dot2c_f32_bf16), so the output is an exact convex
// combination of the V rows under those weights.
// exp is computed as exp2 with log2(e)/sqrt(d) folded into one FMA.
//
// Softmax shift.  Softmax is unchanged by subtracting any per-query constant
// from the logits; the running maximum is only one choice.  With the head's
// largest key norm known (key_norm_kernel), every logit of query q is at most
// B_q = |q| max_j |k_j| (Cauchy-Schwarz; scaled to log2 units).  A wave whose
// queries all have B_q <= kShiftBoundMax subtracts the fixed shift
// m_q = max(B_q - kShiftHeadroom, 0): every weight is at most 2^kShiftHeadroom,
// and the largest weight (its logit is >= -B_q) is at least
// 2^-(2 kShiftBoundMax - kShiftHeadroom) = 2^-80, far above the smallest
// normal float, so no per-tile maximum, cross-lane exchange or rescale of O
// is needed.  Other waves keep the online running maximum.
#include "device_util.h"

namespace saf {
namespace {

constexpr int QT = kQueryTile;
constexpr int KT = 64;
constexpr int KROW = 72;   // K tile row in LDS: 64 bf16 + 8 pad
constexpr int VROWS = 72;  // V tile row in LDS (keys row-major): 64 bf16 + 8 pad

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Four consecutive keys of one channel from a row-major V tile in LDS
// (ds_read_b64_tr_b16): within each 16-lane group, lane j receives element
// j % 4 of the 8-byte pieces that lanes j / 4, j / 4 + 4, j / 4 + 8 and
// j / 4 + 12 address; lane t addresses key row base + t / 4 at channel
// c0 + 4 (t % 4), so lane j gets keys base .. base + 3 of channel c0 + j.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
}

// sum of the two bf16 halves of w, added to acc (v_dot2c_f32_bf16 with 1.0)
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                           acc, false);
}
constexpr int PSTRIDE = kRecStride;  // split partial record: m, l, o[64]
constexpr float kShiftBoundMax = 56.f;  // log2 units
constexpr float kShiftHeadroom = 32.f;

template <int M>
struct IntTag {
    static constexpr int value = M;
};

__device__ __forceinline__ int kswz(int row) { return 4 * ((row >> 3) & 1); }

__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

struct RowMap {
    int32_t valid;     // rows in this tile
    int32_t qsel;      // key-set selector: query frame (position), patch position (broadcast)
    int64_t row0;      // first row (FRAME/ALL)
    int32_t specials;  // row index m -> (m/ns)*T + m%ns
    int32_t by_pos;    // row index m -> m*T + ns + qsel (frames of one patch position)
    int32_t m0;
};

__device__ __forceinline__ int64_t tile_row(const RowMap &rm, const Geom &g, int r) {
    if (rm.specials) {
        const int m = rm.m0 + r;
        return (int64_t)(m / g.ns) * g.T + (m % g.ns);
    }
    if (rm.by_pos) return (int64_t)(rm.m0 + r) * g.T + g.ns + rm.qsel;
    return rm.row0 + r;
}

__device__ __forceinline__ RowMap make_rowmap(const HeadWork &w, const Geom &g, int tile) {
    RowMap rm{};
    if (w.rows == ROWS_FRAME) {
        const int tpf = (g.T + QT - 1) / QT;
        const int f = tile / tpf, t0 = (tile % tpf) * QT;
        rm.qsel = f;
        rm.row0 = (int64_t)f * g.T + t0;
        rm.valid = min(QT, g.T - t0);
    } else if (w.rows == ROWS_BY_POSITION) {
        const int tps = (g.S + QT - 1) / QT;
        rm.by_pos = 1;
        rm.qsel = tile / tps;
        rm.m0 = (tile % tps) * QT;
        rm.valid = min(QT, g.S - rm.m0);
    } else if (w.rows == ROWS_ALL) {
        rm.row0 = (int64_t)tile * QT;
        rm.valid = (int)min<int64_t>(QT, g.N - rm.row0);
    } else {
        rm.specials = 1;
        rm.m0 = tile * QT;
        rm.valid = min(QT, g.ns * g.S - rm.m0);
    }
    return rm;
}

constexpr int kAttnThreads = 256;  // 4 waves x 64 query rows
constexpr int kSpecTable = 4096;   // special tokens an LDS table holds (ns S <= this)

// Work-groups are dealt to the 8 XCDs in turn (block b runs on XCD b % 8).
// Runs of kXcdRun consecutive logical blocks (neighbouring query tiles of one
// head) are kept on one XCD, in dispatch order, so they share its L2.  A
// bijection on [0, nb): the last nb mod (8 kXcdRun) blocks keep their number.
constexpr int kXcdRun = 16;
__device__ __forceinline__ int xcd_grouped(int bid, int nb) {
    const int full = nb / (8 * kXcdRun) * (8 * kXcdRun);
    if (bid >= full) return bid;
    const int xcd = bid & 7, slot = bid >> 3;
    return ((slot / kXcdRun) * 8 + xcd) * kXcdRun + slot % kXcdRun;
}

// DENSE = true is the dense flash-attention kernel: every head attends to all
// N keys, so key tiles are contiguous token ranges [kt, kt + 64): no key-set
// enumeration, no per-key validity tests except on the ragged last tile.
template <bool DENSE>
__global__ __launch_bounds__(kAttnThreads, 2) void mfma_attn_kernel(const MfmaLaunch L) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][KT * VROWS];
    __shared__ float kbias[2][KT];
    // token of the m-th special token (m < ns S) for position and scanning
    // heads; -1 for a scanning head's special already on its stride
    __shared__ int32_t spec_tok[kSpecTable];

    const Geom &g = L.g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, gq = lane >> 5;
    // LDS swizzle (bank-conflict-free stores and reads): K rows r >= 8 of
    // each group of 16 hold their 16-byte channel chunks XOR 4
    const int kx = 4 * ((n >> 2) & 1);  // K rows are read as swap_bits23(n): bit 3 of the row = bit 2 of n

    // ---- locate this work-group's head, query tile and key split
    const int b = (DENSE ? (int)blockIdx.x : xcd_grouped((int)blockIdx.x, (int)gridDim.x)) + L.block_base;
    int wi = 0;
    for (int i = 1; i < L.nwork; ++i)
        if (L.work[i].block0 <= b) wi = i;
    const HeadWork w = L.work[wi];
    const int local = b - w.block0;
    const int split = local % w.nsplit;
    const int tile = local / w.nsplit;
    const RowMap rm = make_rowmap(w, g, tile);

    const int64_t hoff = (int64_t)w.head * L.head_stride;
    const int64_t ts = L.token_stride;
    const uint16_t *Q = (const uint16_t *)L.q + hoff;
    // a packed key set: contiguous rows, key slot = row, no masked slot
    const bool packed = !DENSE && w.pk != nullptr;
    const uint16_t *K = packed ? w.pk : (const uint16_t *)L.k + hoff;
    const uint16_t *V = packed ? w.pv : (const uint16_t *)L.v + hoff;
    const int64_t kts = packed ? 64 : ts;  // key row stride

    // key slots in 32 bits: a key set holds at most N + ns S < 2^31 slots
    const int32_t count = (int32_t)(DENSE ? g.N : packed ? w.pcount : key_count(w, g, rm.qsel));
    const int32_t per = ((count + w.nsplit - 1) / w.nsplit + KT - 1) / KT * KT;
    const int32_t kbeg = split * per;
    const int32_t kend = min(count, kbeg + per);
    const int32_t first_masked =
        (DENSE || packed) ? INT32_MAX : (int32_t)min<int64_t>(key_first_masked(w, g), INT32_MAX);

    // Key enumeration without 64-bit divisions (N < 2^31): position and
    // scanning sets are the special tokens (from an LDS table built once per
    // work-group) and affine token ranges; vertical sets come from their
    // list; broadcast sets keep the general enumeration.
    const int32_t nsS = g.ns * g.S;
    const bool table = !DENSE && !packed && (w.role == POSITION || w.role == SCANNING) && nsS <= kSpecTable;
    if (table) {
        for (int i = tid; i < nsS; i += kAttnThreads) {
            const int32_t tok = (i / g.ns) * g.T + i % g.ns;
            spec_tok[i] = (w.role == SCANNING && tok % w.budget == 0) ? -1 : tok;
        }
        __syncthreads();
    }
    // a vertical head's list in the same LDS table (read from memory per tile,
    // a list entry is one more round trip before the tile's gathers)
    const bool vtable = !DENSE && w.role == VERTICAL && w.list_len <= kSpecTable;
    if (vtable) {
        constexpr int kPer = kSpecTable / kAttnThreads;
        int32_t e[kPer];  // every entry requested before any is stored (clamped indices)
#pragma unroll
        for (int j = 0; j < kPer; ++j) e[j] = w.list[min(tid + kAttnThreads * j, w.list_len - 1)];
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (tid + kAttnThreads * j < w.list_len) spec_tok[tid + kAttnThreads * j] = e[j];
        __syncthreads();
    }
    const int32_t anchor_base = w.anchor * g.T + g.ns, own_base = rm.qsel * g.T + g.ns;
    const int32_t nst = w.role == SCANNING ? (int32_t)((g.N + w.budget - 1) / w.budget) : 0;
    auto token_of = [&](int64_t m64) -> int64_t {
        if (DENSE || packed) return m64;
        if (vtable) return spec_tok[(int32_t)m64];
        if (!table) return key_token(w, g, m64, rm.qsel);
        const int32_t m = (int32_t)m64;
        if (w.role == POSITION) {
            if (m < nsS) return spec_tok[m];
            return m < nsS + g.P ? anchor_base + (m - nsS) : own_base + (m - nsS - g.P);
        }
        return m < nst ? m * w.budget : spec_tok[m - nst];  // scanning
    };

    // ---- this wave's 64 query rows as two 32-row B operands (4 k-steps each)
    bool qvalid[2];
    int32_t qtok[2];  // N < 2^30
    bf16x8 qreg[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qr = wave * 64 + 32 * qb + n;
        qvalid[qb] = qr < rm.valid;
        qtok[qb] = qvalid[qb] ? (int32_t)tile_row(rm, g, qr) : 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (qvalid[qb]) raw = *(const u32x4 *)(Q + (int64_t)qtok[qb] * ts + 16 * c + 8 * gq);
            qreg[qb][c] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    const float sc = kLog2e * 0.125f;  // log2(e) / sqrt(64)
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    // fixed softmax shift from the Cauchy-Schwarz bound (see the top of the
    // file); lanes n and n + 32 hold the two channel halves of a query
    bool fixed = false;
    if (L.knorm) {
        static_assert(kNormParts % 64 == 0, "whole partials per lane");
        float k2 = 0.f;
#pragma unroll
        for (int i = 0; i < kNormParts / 64; ++i) k2 = fmaxf(k2, L.knorm[wi * kNormParts + 64 * i + lane]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) k2 = fmaxf(k2, __shfl_xor(k2, off));
        float bmax = 0.f, bq[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float q2 = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 u = __builtin_bit_cast(u32x4, qreg[qb][c]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(u[e] << 16), hi = __uint_as_float(u[e] & 0xFFFF0000u);
                    q2 = fmaf(lo, lo, fmaf(hi, hi, q2));
                }
            }
            q2 += __shfl_xor(q2, 32);
            bq[qb] = sqrtf(q2 * k2) * sc;
            bmax = fmaxf(bmax, bq[qb]);
        }
        fixed = !__any(!(bmax <= kShiftBoundMax));  // a NaN bound takes the running maximum
        if (fixed) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) m_run[qb] = fmaxf(bq[qb] - kShiftHeadroom, 0.f);
        }
    }
    f32x16 oacc[2][2];  // [query block][channel block]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;

    // ---- tile loader: unit = (key pair p, channel segment seg), one unit
    // per thread; K and V rows are stored as loaded (16 bytes per key row)
    constexpr int kUnits = (KT / 2) * 8 / kAttnThreads;
    u32x4 kreg[kUnits][2], vreg[kUnits][2];
    bool kval[kUnits][2];
    auto load_tile = [&](int32_t kt) {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int unit = tid + kAttnThreads * j, lp = unit >> 3, lseg = unit & 7;
            // both keys' tokens first (a vertical head reads them from its
            // list), then every gather unconditionally: a slot without a key
            // reads token 0 and is zeroed when the tile is stored.  Guarded
            // loads would make the compiler wait for them before the current
            // tile's first MFMA, which defeats the prefetch.
            int32_t tk[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int32_t m = kt + 2 * lp + i;
                tk[i] = (m < kend) ? (int32_t)token_of(m) : -1;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                kval[j][i] = tk[i] >= 0;
                const int64_t tc = kval[j][i] ? tk[i] : 0;
                kreg[j][i] = *(const u32x4 *)(K + tc * kts + 8 * lseg);
                vreg[j][i] = *(const u32x4 *)(V + tc * kts + 8 * lseg);
            }
        }
    };
    // full = every slot of the tile holds a key (dense tiles but the last):
    // no zeroing of empty slots, no bias entries (wave-uniform)
    auto store_tile = [&](int buf, bool full) {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int unit = tid + kAttnThreads * j, lp = unit >> 3, lseg = unit & 7;
            u32x4 kz[2], vz[2];
            if (DENSE && full) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    kz[i] = kreg[j][i];
                    vz[i] = vreg[j][i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kz[i][e] = kval[j][i] ? kreg[j][i][e] : 0u;
                        vz[i][e] = kval[j][i] ? vreg[j][i][e] : 0u;
                    }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) *(u32x4 *)(&Ks[buf][(2 * lp + i) * KROW + 8 * (lseg ^ kswz(2 * lp + i))]) = kz[i];
#pragma unroll
            for (int i = 0; i < 2; ++i) *(u32x4 *)(&Vs[buf][(2 * lp + i) * VROWS + 8 * lseg]) = vz[i];
            if (!(DENSE && full) && lseg == 0) {
                kbias[buf][2 * lp] = kval[j][0] ? 0.f : -INFINITY;
                kbias[buf][2 * lp + 1] = kval[j][1] ? 0.f : -INFINITY;
            }
        }
    };

    const int32_t ntiles = (kend - kbeg + KT - 1) / KT;
    if (ntiles > 0) {
        load_tile(kbeg);
        store_tile(0, kbeg + KT <= kend);
    }
    // every load so far (Q, the first tile) complete on every path: the
    // compiler's wait analysis is not path-sensitive, and a Q load it
    // believes pending at the loop head makes it wait for all loads in
    // flight, the next tile's prefetch included, before each tile's MFMAs
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt at their maxima
    __syncthreads();

    // One key tile.  MODE 0: fixed shift, every slot a key (pipelined);
    // 1: fixed shift, masked slots; 2: running maximum.
    auto tile_step = [&](int32_t t, auto mode_tag) {
        constexpr int MODE = decltype(mode_tag)::value;
        constexpr bool FIXED = MODE != 2;
        const int buf = t & 1;
        const int32_t kt = kbeg + t * KT;
        if (t + 1 < ntiles) load_tile(kt + KT);

        // S^T = K Q^T for one 32-key block (bb) and both 32-query blocks;
        // each K fragment feeds both query blocks
        f32x16 s[2][2];
        auto s_block = [&](int bb) {
            const uint16_t *krow = &Ks[buf][(32 * bb + swap_bits23(n)) * KROW];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 a = *(const bf16x8 *)(krow + 8 * ((2 * c + gq) ^ kx));
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    s[bb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][c], c ? s[bb][qb] : f32x16{}, 0,
                                                                        0, 0);
            }
        };
        // weights of one key block with the fixed shift
        auto weights = [&](int bb) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[bb][qb][r] = fast_exp2(fmaf(s[bb][qb][r], sc, -m_run[qb]));
        };
        // O^T += V^T P^T for the 16 keys 16 e ..; each V^T fragment feeds
        // both query blocks
        auto pv = [&](int e) {
            const int bb = e >> 1, h8 = (e & 1) * 8;
            bf16x8 pb[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                u32x4 pk;
                pk[0] = pack_bf16x2(s[bb][qb][h8 + 0], s[bb][qb][h8 + 1]);
                pk[1] = pack_bf16x2(s[bb][qb][h8 + 2], s[bb][qb][h8 + 3]);
                pk[2] = pack_bf16x2(s[bb][qb][h8 + 4], s[bb][qb][h8 + 5]);
                pk[3] = pack_bf16x2(s[bb][qb][h8 + 6], s[bb][qb][h8 + 7]);
                pb[qb] = __builtin_bit_cast(bf16x8, pk);
                // the row sum from the same rounded weights the P.V product uses
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) l_run[qb] = add_bf16_pair(pk[w2], l_run[qb]);
            }
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                // keys 16 e + 8 gq .. + 7 of channel 32 db + n, as two
                // transposing reads of four keys each (see lds_read_tr)
                const int t16 = lane & 15;
                const uint16_t *vp = &Vs[buf][(16 * e + 8 * gq + (t16 >> 2)) * VROWS + 32 * db + 16 * ((lane >> 4) & 1) +
                                              4 * (t16 & 3)];
                const s16x4 lo = lds_read_tr(vp), hi = lds_read_tr(vp + 4 * VROWS);
                const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb], oacc[qb][db], 0, 0, 0);
            }
        };
        if (MODE == 0) {
            // Fixed shift, every slot a key: the weights of one key block need
            // only that block's logits, so each wave issues the matrix-core
            // work of one block beside the vector work of the other:
            //   S(keys 0-31) | S(keys 32-63) + weights(0-31)
            //   | P.V(0-31) + weights(32-63) | P.V(32-63)
            s_block(0);
            __builtin_amdgcn_sched_barrier(0);
            s_block(1);
            weights(0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);  // the block's K fragments
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            pv(0);
            pv(1);
            weights(1);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 2);  // V^T fragments of keys 0-31
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 2);  // packed weights of keys 0-15
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
                __builtin_amdgcn_sched_group_barrier(0x002, 11, 2);
            }
            __builtin_amdgcn_sched_barrier(0);
            pv(2);
            pv(3);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 3);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 3);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 3);
            }
            __builtin_amdgcn_sched_barrier(0);
        } else {
            s_block(0);
            s_block(1);
            // masked slots: ragged tail, or specials already on the scanning stride
            if (kt + KT > kend || kt + KT > first_masked) {
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float bias = kbias[buf][32 * bb + 16 * (r >> 3) + 8 * gq + (r & 7)];
#pragma unroll
                        for (int qb = 0; qb < 2; ++qb) s[bb][qb][r] += bias;
                    }
            }
            if (FIXED) {
                weights(0);
                weights(1);
            } else {
                // online running max per query block (log2 domain), only
                // raised when a logit exceeds it by more than 8 (weights stay
                // <= 2^8), so the O rescale is skipped on most tiles
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    float mx = s[0][qb][0];
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[bb][qb][r]);
                    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sc;
                    if (__any(mx > m_run[qb] + 8.f)) {
                        const float m_new = fmaxf(m_run[qb], mx);
                        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[qb] - m_new);
                        l_run[qb] *= alpha;
#pragma unroll
                        for (int db = 0; db < 2; ++db)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
                        m_run[qb] = m_new;
                    }
                    const float m_use = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) s[bb][qb][r] = fast_exp2(fmaf(s[bb][qb][r], sc, -m_use));
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) pv(e);
        }

        if (t + 1 < ntiles) store_tile(buf ^ 1, kt + 2 * KT <= kend);
        __syncthreads();
    };
    if (fixed) {
        // tiles [0, t_full) hold no masked slot
        const int32_t t_full = max(0, min(ntiles, (min(kend, first_masked) - kbeg) / KT));
        for (int32_t t = 0; t < t_full; ++t) tile_step(t, IntTag<0>{});
        for (int32_t t = t_full; t < ntiles; ++t) tile_step(t, IntTag<1>{});
    } else {
        for (int32_t t = 0; t < ntiles; ++t) tile_step(t, IntTag<2>{});
    }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
        if (!qvalid[qb]) continue;
        const int qr = wave * 64 + 32 * qb + n;
        if (w.nsplit == 1 && !w.rec_out) {
            const float inv = 1.f / l_tot;
            uint16_t *O = (uint16_t *)L.o + hoff + (int64_t)qtok[qb] * ts;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d0 = 32 * db + 8 * q4 + 4 * gq;
                    u32x2 pk;
                    pk[0] = pack_bf16x2(oacc[qb][db][4 * q4 + 0] * inv, oacc[qb][db][4 * q4 + 1] * inv);
                    pk[1] = pack_bf16x2(oacc[qb][db][4 * q4 + 2] * inv, oacc[qb][db][4 * q4 + 3] * inv);
                    *(u32x2 *)(O + d0) = pk;
                }
        } else {
            float *rec = w.part + ((int64_t)(tile * QT + qr) * w.nsplit + split) * PSTRIDE;
            if (gq == 0) {
                rec[0] = m_run[qb];
                rec[1] = l_tot;
            }
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d0 = 32 * db + 8 * q4 + 4 * gq;
                    *(f32x4 *)(rec + 2 + d0) = f32x4{oacc[qb][db][4 * q4], oacc[qb][db][4 * q4 + 1],
                                                     oacc[qb][db][4 * q4 + 2], oacc[qb][db][4 * q4 + 3]};
                }
        }
    }
}

// parts[wi * kNormParts + p]: largest |k|^2 over token range p of work wi's
// head.  8 lanes per key row (16 bytes each), 32 rows per pass of a block,
// four passes' loads in flight (rows past the range re-read its last row).
__global__ __launch_bounds__(256) void key_norm_kernel(const MfmaLaunch L, float *parts) {
    __shared__ float red[4];
    const int wi = blockIdx.y, p = blockIdx.x, tid = threadIdx.x, seg = tid & 7;
    const int64_t N = L.g.N, per = (N + kNormParts - 1) / kNormParts;
    const int64_t r0 = (int64_t)p * per, r1 = min<int64_t>(N, r0 + per);
    const uint16_t *K = (const uint16_t *)L.k + (int64_t)L.work[wi].head * L.head_stride + 8 * seg;
    float mx = 0.f;
    for (int64_t r = r0 + (tid >> 3); r < r1; r += 4 * 32) {
        u32x4 raw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = *(const u32x4 *)(K + min<int64_t>(r + 32 * i, r1 - 1) * L.token_stride);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float q2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = __uint_as_float(raw[i][e] << 16), hi = __uint_as_float(raw[i][e] & 0xFFFF0000u);
                q2 = fmaf(lo, lo, fmaf(hi, hi, q2));
            }
            q2 += __shfl_xor(q2, 1);
            q2 += __shfl_xor(q2, 2);
            q2 += __shfl_xor(q2, 4);
            mx = fmaxf(mx, q2);
        }
    }
#pragma unroll
    for (int off = 32; off >= 8; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) parts[wi * kNormParts + p] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Packed scanning sets: rows [0, nst) are the stride tokens m * s, then the
// specials not on the stride, in token order.  pack_specials_kernel (one
// block per work) lists those specials' tokens in order (per-thread keep
// masks and a block-wide scan of their counts); pack_rows_kernel then copies
// every row, 8 lanes per 128-byte K or V row, all rows in parallel.
__global__ __launch_bounds__(256) void pack_specials_kernel(const MfmaLaunch L) {
    __shared__ uint32_t wsum[4];
    const HeadWork &w = L.work[blockIdx.y];
    const Geom &g = L.g;
    if (!w.pk || g.ns == 0) return;
    constexpr int kPer = kPackSpecials / 256;  // thread t owns specials [kPer t, kPer t + kPer)
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int32_t s = w.budget, nsS = g.ns * g.S;
    uint32_t keep = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int32_t m = kPer * tid + i;
        const int64_t tok = (int64_t)(m / g.ns) * g.T + m % g.ns;
        if (m < nsS && tok % s != 0) keep |= 1u << i;
    }
    const uint32_t c = __popc(keep);
    uint32_t incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    uint32_t pos = incl - c;
    for (int i = 0; i < wv; ++i) pos += wsum[i];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if ((keep >> i) & 1u) {
            const int32_t m = kPer * tid + i;
            w.pspec[pos++] = (m / g.ns) * g.T + m % g.ns;
        }
}

__global__ __launch_bounds__(256) void pack_rows_kernel(const MfmaLaunch L) {
    const HeadWork &w = L.work[blockIdx.y];
    if (!w.pk) return;
    const Geom &g = L.g;
    const int seg = threadIdx.x & 7;
    const int64_t hoff = (int64_t)w.head * L.head_stride, ts = L.token_stride;
    const uint16_t *K = (const uint16_t *)L.k + hoff, *V = (const uint16_t *)L.v + hoff;
    const int32_t s = w.budget, nst = (int32_t)((g.N + s - 1) / s);
    for (int64_t r = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3); r < w.pcount; r += (int64_t)gridDim.x * 32) {
        const int64_t tok = r < nst ? r * s : (int64_t)w.pspec[r - nst];
        const u32x4 kx = *(const u32x4 *)(K + tok * ts + 8 * seg), vx = *(const u32x4 *)(V + tok * ts + 8 * seg);
        *(u32x4 *)(w.pk + r * 64 + 8 * seg) = kx;
        *(u32x4 *)(w.pv + r * 64 + 8 * seg) = vx;
    }
}

// Combine key splits: one wave per query row, lane = channel.
__global__ __launch_bounds__(256) void split_combine_kernel(const MfmaLaunch L) {
    const Geom &g = L.g;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    // walk the split works in order; rows of a work are tiles*QT slots
    int64_t base = 0;
    for (int i = 0; i < L.nwork; ++i) {
        const HeadWork &w = L.work[i];
        if (w.nsplit <= 1) continue;
        const int64_t tiles = (w.rows == ROWS_SPECIALS) ? ((int64_t)g.ns * g.S + QT - 1) / QT
                              : (w.rows == ROWS_ALL)    ? (g.N + QT - 1) / QT
                                                        : (int64_t)g.S * ((g.T + QT - 1) / QT);
        const int64_t slots = tiles * QT;
        if (gw < base + slots) {
            const int64_t slot = gw - base;
            const int tile = (int)(slot / QT), r = (int)(slot % QT);
            const RowMap rm = make_rowmap(w, g, tile);
            if (r >= rm.valid) return;
            const float *rec = w.part + slot * w.nsplit * PSTRIDE;
            float M = -INFINITY;
            for (int s = 0; s < w.nsplit; ++s) M = fmaxf(M, rec[s * PSTRIDE]);
            const float Mu = (M == -INFINITY) ? 0.f : M;
            float l = 0.f, o = 0.f;
            for (int s = 0; s < w.nsplit; ++s) {
                const float f = fast_exp2(rec[s * PSTRIDE] - Mu);
                l += rec[s * PSTRIDE + 1] * f;
                o += rec[s * PSTRIDE + 2 + lane] * f;
            }
            const int64_t tok = tile_row(rm, g, r);
            uint16_t *O = (uint16_t *)L.o + (int64_t)w.head * L.head_stride + tok * L.token_stride;
            O[lane] = (uint16_t)f32_to_bf16_bits(o / l);
            return;
        }
        base += slots;
    }
}

}  // namespace

// Dynamic LDS that holds the key-set kernel to one work-group per compute
// unit: more than half of the CU's LDS per work-group (0: not possible).
// A failed query leaves no error behind: the launch then runs unshared.
static int share_cu_lds() {
    int dev = 0, lds_cu = 0;
    hipFuncAttributes fa{};
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipFuncGetAttributes(&fa, (const void *)mfma_attn_kernel<false>) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int dyn = lds_cu / 2 + 256 - (int)fa.sharedSizeBytes;
    if (dyn <= 0 || (int)fa.sharedSizeBytes + dyn > lds_cu) return 0;
    if (hipFuncSetAttribute((const void *)mfma_attn_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            dyn) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return dyn;
}

hipError_t launch_mfma_attention(const MfmaLaunch &L, int32_t nblocks, bool share_cu, hipStream_t stream) {
    if (nblocks <= 0) return hipSuccess;
    // every piece of work a dense head over all rows: the contiguous-key kernel
    bool dense = true;
    for (int i = 0; i < L.nwork; ++i)
        dense = dense && L.work[i].role == DENSE && L.work[i].rows == ROWS_ALL && L.work[i].nsplit == 1 &&
                !L.work[i].rec_out;
    if (dense) {
        hipLaunchKernelGGL(mfma_attn_kernel<true>, dim3(nblocks), dim3(kAttnThreads), 0, stream, L);
    } else {
        const int dyn = share_cu ? share_cu_lds() : 0;
        hipLaunchKernelGGL(mfma_attn_kernel<false>, dim3(nblocks), dim3(kAttnThreads), (unsigned)dyn, stream, L);
    }
    return hipGetLastError();
}

hipError_t launch_key_norms(const MfmaLaunch &L, float *parts, hipStream_t stream) {
    if (L.nwork <= 0) return hipSuccess;
    hipLaunchKernelGGL(key_norm_kernel, dim3(kNormParts, L.nwork), dim3(256), 0, stream, L, parts);
    return hipGetLastError();
}

hipError_t launch_pack_keys(const MfmaLaunch &L, hipStream_t stream) {
    bool any = false;
    for (int i = 0; i < L.nwork; ++i) any = any || L.work[i].pk != nullptr;
    if (!any) return hipSuccess;
    int32_t rows = 0;
    for (int i = 0; i < L.nwork; ++i) rows = max(rows, L.work[i].pk ? L.work[i].pcount : 0);
    hipLaunchKernelGGL(pack_specials_kernel, dim3(1, L.nwork), dim3(256), 0, stream, L);
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)((rows + 31) / 32), L.nwork), dim3(256), 0, stream, L);
    return hipGetLastError();
}

hipError_t launch_split_combine(const MfmaLaunch &L, hipStream_t stream) {
    int64_t slots = 0;
    for (int i = 0; i < L.nwork; ++i) {
        const HeadWork &w = L.work[i];
        if (w.nsplit <= 1) continue;
        const int64_t tiles = (w.rows == ROWS_SPECIALS) ? ((int64_t)L.g.ns * L.g.S + QT - 1) / QT
                              : (w.rows == ROWS_ALL)    ? (L.g.N + QT - 1) / QT
                                                        : (int64_t)L.g.S * ((L.g.T + QT - 1) / QT);
        slots += tiles * QT;
    }
    if (slots == 0) return hipSuccess;
    hipLaunchKernelGGL(split_combine_kernel, dim3((unsigned)((slots + 3) / 4)), dim3(256), 0, stream, L);
    return hipGetLastError();
}

}  // namespace saf
