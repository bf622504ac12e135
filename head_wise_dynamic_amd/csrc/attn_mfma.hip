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
// cover 8 consecutive keys; V^T is then read from LDS as 16-byte rows.
// O^T = V^T P^T accumulates in fp32 and is normalised at the end.
// exp is computed as exp2 with log2(e)/sqrt(d) folded into one FMA.
#include "device_util.h"

namespace saf {
namespace {

constexpr int QT = kQueryTile;
constexpr int KT = 64;
constexpr int KROW = 72;   // K tile row in LDS: 64 bf16 + 8 pad
constexpr int VROW = 72;   // V^T tile row in LDS: 64 keys + 8 pad
constexpr int PSTRIDE = kRecStride;  // split partial record: m, l, o[64]

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

__global__ __launch_bounds__(kAttnThreads, 2) void mfma_attn_kernel(const MfmaLaunch L) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][64 * VROW];
    __shared__ float kbias[2][KT];

    const Geom &g = L.g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, gq = lane >> 5;
    // LDS swizzles (bank-conflict-free stores and reads): K rows r >= 8 of
    // each group of 16 hold their 16-byte channel chunks XOR 4; the key-pair
    // words of V^T row c are XOR 4 * ((c >> 3) & 7)
    const int kx = 4 * ((n >> 2) & 1);  // K rows are read as swap_bits23(n): bit 3 of the row = bit 2 of n
    const int vx = 4 * (n >> 3);

    // ---- locate this work-group's head, query tile and key split
    const int b = blockIdx.x;
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
    const uint16_t *K = (const uint16_t *)L.k + hoff;
    const uint16_t *V = (const uint16_t *)L.v + hoff;

    const int64_t count = key_count(w, g, rm.qsel);
    const int64_t per = ((count + w.nsplit - 1) / w.nsplit + KT - 1) / KT * KT;
    const int64_t kbeg = (int64_t)split * per;
    const int64_t kend = min<int64_t>(count, kbeg + per);
    const int64_t first_masked = key_first_masked(w, g);

    // ---- this wave's 64 query rows as two 32-row B operands (4 k-steps each)
    bool qvalid[2];
    int64_t qtok[2];
    bf16x8 qreg[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qr = wave * 64 + 32 * qb + n;
        qvalid[qb] = qr < rm.valid;
        qtok[qb] = qvalid[qb] ? tile_row(rm, g, qr) : 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (qvalid[qb]) raw = *(const u32x4 *)(Q + qtok[qb] * ts + 16 * c + 8 * gq);
            qreg[qb][c] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    const float sc = kLog2e * 0.125f;  // log2(e) / sqrt(64)
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    f32x16 oacc[2][2];  // [query block][channel block]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;

    // ---- tile loader: unit = (key pair p, channel segment seg), one unit
    // per thread; V^T is written two keys per 32-bit LDS store
    constexpr int kUnits = (KT / 2) * 8 / kAttnThreads;
    u32x4 kreg[kUnits][2], vreg[kUnits][2];
    bool kval[kUnits][2];
    auto load_tile = [&](int64_t kt) {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int unit = tid + kAttnThreads * j, lp = unit >> 3, lseg = unit & 7;
            // both keys' tokens first (a vertical head reads them from its
            // list), then every gather unconditionally: a slot without a key
            // reads token 0 and is zeroed when the tile is stored.  Guarded
            // loads would make the compiler wait for them before the current
            // tile's first MFMA, which defeats the prefetch.
            int64_t tk[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int64_t m = kt + 2 * lp + i;
                tk[i] = (m < kend) ? key_token(w, g, m, rm.qsel) : -1;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                kval[j][i] = tk[i] >= 0;
                const int64_t tc = kval[j][i] ? tk[i] : 0;
                kreg[j][i] = *(const u32x4 *)(K + tc * ts + 8 * lseg);
                vreg[j][i] = *(const u32x4 *)(V + tc * ts + 8 * lseg);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int unit = tid + kAttnThreads * j, lp = unit >> 3, lseg = unit & 7;
            u32x4 kz[2], vz[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kz[i][e] = kval[j][i] ? kreg[j][i][e] : 0u;
                    vz[i][e] = kval[j][i] ? vreg[j][i][e] : 0u;
                }
#pragma unroll
            for (int i = 0; i < 2; ++i) *(u32x4 *)(&Ks[buf][(2 * lp + i) * KROW + 8 * (lseg ^ kswz(2 * lp + i))]) = kz[i];
            uint32_t *vt = (uint32_t *)&Vt[buf][(8 * lseg) * VROW] + (lp ^ (4 * lseg));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // channels 2e and 2e+1 of the two keys
                vt[(2 * e) * (VROW / 2)] = __builtin_amdgcn_perm(vz[1][e], vz[0][e], 0x05040100u);
                vt[(2 * e + 1) * (VROW / 2)] = __builtin_amdgcn_perm(vz[1][e], vz[0][e], 0x07060302u);
            }
            if (lseg == 0) {
                kbias[buf][2 * lp] = kval[j][0] ? 0.f : -INFINITY;
                kbias[buf][2 * lp + 1] = kval[j][1] ? 0.f : -INFINITY;
            }
        }
    };

    const int64_t ntiles = (kend - kbeg + KT - 1) / KT;
    if (ntiles > 0) {
        load_tile(kbeg);
        store_tile(0);
    }
    // every load so far (Q, the first tile) complete on every path: the
    // compiler's wait analysis is not path-sensitive, and a Q load it
    // believes pending at the loop head makes it wait for all loads in
    // flight, the next tile's prefetch included, before each tile's MFMAs
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt at their maxima
    __syncthreads();

    for (int64_t t = 0; t < ntiles; ++t) {
        const int buf = (int)(t & 1);
        const int64_t kt = kbeg + t * KT;
        if (t + 1 < ntiles) load_tile(kt + KT);

        // S^T = K Q^T: two 32-key blocks x two 32-query blocks; each K
        // fragment feeds both query blocks
        f32x16 s[2][2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[bb][qb][r] = 0.f;
            const uint16_t *krow = &Ks[buf][(32 * bb + swap_bits23(n)) * KROW];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 a = *(const bf16x8 *)(krow + 8 * ((2 * c + gq) ^ kx));
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    s[bb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][c], s[bb][qb], 0, 0, 0);
            }
        }
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
        // online softmax per query block (log2 domain).  The running max is
        // only raised when a logit exceeds it by more than 8 (weights stay
        // <= 2^8), so the O rescale is skipped on most tiles.
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
            float lsum = 0.f;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(s[bb][qb][r], sc, -m_use));
                    s[bb][qb][r] = p;
                    lsum += p;
                }
            l_run[qb] += lsum;
        }

        // O^T += V^T P^T, four k-steps of 16 keys; each V^T fragment feeds
        // both query blocks
#pragma unroll
        for (int e = 0; e < 4; ++e) {
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
            }
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const bf16x8 a = *(const bf16x8 *)(&Vt[buf][(32 * db + n) * VROW + 2 * ((8 * e + 4 * gq) ^ (16 * db + vx))]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb], oacc[qb][db], 0, 0, 0);
            }
        }

        if (t + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
        if (!qvalid[qb]) continue;
        const int qr = wave * 64 + 32 * qb + n;
        if (w.nsplit == 1 && !w.rec_out) {
            const float inv = 1.f / l_tot;
            uint16_t *O = (uint16_t *)L.o + hoff + qtok[qb] * ts;
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

hipError_t launch_mfma_attention(const MfmaLaunch &L, hipStream_t stream) {
    if (L.total_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(mfma_attn_kernel, dim3(L.total_blocks), dim3(kAttnThreads), 0, stream, L);
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
