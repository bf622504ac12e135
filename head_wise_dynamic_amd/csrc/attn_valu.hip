// Per-query sparse attention on the vector ALUs: one wave per query row.
//
// This is the gather-bound path of the correspondence heads (SAF3R Sec. 4.1,
// "DINO Top-K Kernel"): every query reads its own cached index row and pulls
// the selected K and V rows by token index.  Two kernels:
//   gather_attn_kernel (bf16 correspondence rows): a wave serves one patch
//   row for a group of up to three heads, reading each chunk's index
//   entries once for the group and the K and V rows of all its heads
//   together;
//   valu_attn_kernel (fp32 inputs, where it runs every role: the matrix-core
//   path is bf16-only): a wave serves one query row for every head of the
//   launch, one head after the other, each head's pass reading the row's
//   index entries again (only the first pass finds them outside the caches).
//
// Lane layout: a key row is read as 16-byte pieces, LPR lanes per row
// (8 for bf16, 16 for fp32) and RPP = 64 / LPR rows per load instruction.
// Keys are consumed in chunks of NP * RPP with an online softmax (running max
// and sum in fp32, exp2 with log2(e)/sqrt(d) folded into the logit scale).
#include "device_util.h"

namespace saf {
namespace {

template <typename T> struct Lanes;
template <> struct Lanes<uint16_t> {  // bf16 bits
    static constexpr int EPL = 8, LPR = 8, RPP = 8;
    __device__ static void unpack_raw(const u32x4 &r, float *x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_bits_to_f32(r[i] & 0xFFFFu);
            x[2 * i + 1] = bf16_bits_to_f32(r[i] >> 16);
        }
    }
    __device__ static void load(const uint16_t *p, float *x) { unpack_raw(*(const u32x4 *)p, x); }
    __device__ static void store(uint16_t *p, const float *x) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        *(u32x4 *)p = r;
    }
};
template <> struct Lanes<float> {
    static constexpr int EPL = 4, LPR = 16, RPP = 4;
    __device__ static void load(const float *p, float *x) {
        const f32x4 r = *(const f32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = r[i];
    }
    __device__ static void store(float *p, const float *x) {
        *(f32x4 *)p = f32x4{x[0], x[1], x[2], x[3]};
    }
};

constexpr int NP = 8;  // row loads per chunk and lane

// Running softmax state of one query row: m is wave-uniform; l and o are
// per lane group (each group of LPR lanes takes different keys) until finish.
template <typename T> struct RowAcc {
    float qv[Lanes<T>::EPL];
    float m, l, o[Lanes<T>::EPL];
};

template <typename T>
__device__ void row_init(const ValuLaunch &L, const HeadWork &w, int64_t qtok, int lane, RowAcc<T> &a) {
    using E = Lanes<T>;
    const int sub = lane % E::LPR;
    const T *Q = (const T *)L.q + (int64_t)w.head * L.head_stride;
    E::load(Q + qtok * L.token_stride + sub * E::EPL, a.qv);
    a.m = -INFINITY;
    a.l = 0.f;
#pragma unroll
    for (int e = 0; e < E::EPL; ++e) a.o[e] = 0.f;
}

// Continue the row's online softmax over `count` keys: idx_row[m] when given,
// else the m-th key of w's key set.  skip > 0 drops listed keys on that
// stride (they are counted by another key list of the same row).
template <typename T>
__device__ void row_accumulate(const ValuLaunch &L, const HeadWork &w, int32_t qsel, const int32_t *idx_row,
                               int64_t count, int64_t skip, int lane, RowAcc<T> &a) {
    using E = Lanes<T>;
    constexpr int EPL = E::EPL, LPR = E::LPR, RPP = E::RPP, CH = NP * RPP;
    const Geom &g = L.g;
    const int sub = lane % LPR, grp = lane / LPR;
    const int64_t hoff = (int64_t)w.head * L.head_stride, ts = L.token_stride;
    const T *K = (const T *)L.k + hoff;
    const T *V = (const T *)L.v + hoff;
    const float sc = kLog2e * 0.125f;

    for (int64_t c0 = 0; c0 < count; c0 += CH) {
        int64_t tok[NP];
        float s[NP];
        // Every load of a chunk is unconditional (a slot past the end reads
        // the last key, a slot without a key token 0; both are masked
        // afterwards by select), so that all of them are in flight together:
        // guarded loads make the compiler wait for each one on its own.
        // (the list reads go out together before any test on their values)
        if (idx_row) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int64_t m = c0 + p * RPP + grp;
                tok[p] = (int64_t)idx_row[m < count ? m : count - 1];
            }
        } else {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int64_t m = c0 + p * RPP + grp, mc = m < count ? m : count - 1;
                if constexpr (sizeof(T) == 4)
                    tok[p] = key_token(w, g, mc, qsel);
                else
                    tok[p] = mc;  // bf16 rows gather listed keys only (checked at launch)
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p)
            if (c0 + p * RPP + grp >= count) tok[p] = -1;
        if (skip > 0) {
#pragma unroll
            for (int p = 0; p < NP; ++p)
                if (tok[p] >= 0 && tok[p] % skip == 0) tok[p] = -1;
        }
        float kx[NP][EPL];
#pragma unroll
        for (int p = 0; p < NP; ++p) E::load(K + (tok[p] >= 0 ? tok[p] : 0) * ts + sub * EPL, kx[p]);
        float cm = -INFINITY;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dot = fmaf(a.qv[e], kx[p][e], dot);
#pragma unroll
            for (int x = 1; x < LPR; x <<= 1) dot += __shfl_xor(dot, x);
            s[p] = tok[p] >= 0 ? dot * sc : -INFINITY;
            cm = fmaxf(cm, s[p]);
        }
#pragma unroll
        for (int x = LPR; x < 64; x <<= 1) cm = fmaxf(cm, __shfl_xor(cm, x));
        if (cm == -INFINITY) continue;  // wave-uniform: every slot masked
        const float m_new = fmaxf(a.m, cm);
        const float alpha = fast_exp2(a.m - m_new);
        float lsum = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            s[p] = fast_exp2(s[p] - m_new);
            lsum += s[p];
        }
        a.l = a.l * alpha + lsum;
        a.m = m_new;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a.o[e] *= alpha;
        float vx[NP][EPL];
#pragma unroll
        for (int p = 0; p < NP; ++p) E::load(V + (tok[p] >= 0 ? tok[p] : 0) * ts + sub * EPL, vx[p]);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const bool ok = tok[p] >= 0;
#pragma unroll
            for (int e = 0; e < EPL; ++e) a.o[e] = ok ? fmaf(s[p], vx[p][e], a.o[e]) : a.o[e];
        }
    }
}

template <typename T> __device__ void row_reduce(int lane, RowAcc<T> &a) {
#pragma unroll
    for (int x = Lanes<T>::LPR; x < 64; x <<= 1) {
        a.l += __shfl_xor(a.l, x);
#pragma unroll
        for (int e = 0; e < Lanes<T>::EPL; ++e) a.o[e] += __shfl_xor(a.o[e], x);
    }
}

template <typename T>
__device__ void row_store(const ValuLaunch &L, const HeadWork &w, int64_t qtok, int lane, RowAcc<T> &a) {
    using E = Lanes<T>;
    row_reduce<T>(lane, a);
    if (lane / E::LPR == 0) {
        const float inv = 1.f / a.l;
#pragma unroll
        for (int e = 0; e < E::EPL; ++e) a.o[e] *= inv;
        E::store((T *)L.o + (int64_t)w.head * L.head_stride + qtok * L.token_stride + (lane % E::LPR) * E::EPL,
                 a.o);
    }
}

// unnormalised record (m, l, o[64]) for a later merge
template <typename T> __device__ void row_record(float *rec, int lane, RowAcc<T> &a) {
    using E = Lanes<T>;
    row_reduce<T>(lane, a);
    if (lane / E::LPR == 0) {
#pragma unroll
        for (int e = 0; e < E::EPL; ++e) rec[2 + (lane % E::LPR) * E::EPL + e] = a.o[e];
        if (lane == 0) {
            rec[0] = a.m;
            rec[1] = a.l;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void valu_attn_kernel(const ValuLaunch L, int64_t nrows) {
    const Geom &g = L.g;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= nrows) return;
    int64_t tok, u = -1;
    if (L.patch_rows_only) {
        u = gw;
        tok = (u / g.P) * g.T + g.ns + (u % g.P);
    } else {
        tok = gw;
        const int64_t t = tok % g.T;
        if (t >= g.ns) u = (tok / g.T) * g.P + (t - g.ns);
    }
    const int32_t qframe = (int32_t)(tok / g.T);
    for (int i = 0; i < L.nwork; ++i) {
        const HeadWork w = L.work[i];
        RowAcc<T> acc;
        row_init<T>(L, w, tok, lane, acc);
        // up to two key lists continue one online softmax (a single call
        // site keeps the register budget of the plain roles)
        HeadWork kw = w;
        const int32_t *idx_row = nullptr, *second = nullptr;
        int64_t count = 0, skip = 0;
        int32_t qsel = qframe;
        bool record = false;
        if (w.role == CORRESPONDENCE || w.role == CORR_STRIDE) {
            if (u < 0) {  // special-token query: every key
                kw.role = DENSE;
                count = g.N;
            } else if (w.role == CORRESPONDENCE) {
                idx_row = L.corr_idx + u * L.corr_k;
                count = L.corr_k;
            } else if (w.rec_out) {
                // gathered keys off the stride; the stride set comes from the matrix cores
                idx_row = L.corr_idx + u * L.corr_k;
                count = L.corr_k;
                skip = w.budget;
                record = true;
            } else {  // stride set, then the gathered keys off the stride
                kw.role = SCANNING;
                count = key_count(kw, g, qframe);
                second = L.corr_idx + u * L.corr_k;
            }
        } else if (w.role == BROADCAST) {
            if (u < 0) {  // special-token query: every key
                kw.role = DENSE;
                count = g.N;
            } else {
                qsel = (int32_t)(tok % g.T) - g.ns;  // the query's patch position
                count = key_count(w, g, qsel);
            }
        } else {
            count = key_count(w, g, qframe);
        }
        for (int ph = 0; ph < 2; ++ph) {
            row_accumulate<T>(L, kw, qsel, idx_row, count, skip, lane, acc);
            if (!second) break;
            kw = w;
            idx_row = second;
            count = L.corr_k;
            skip = w.budget;
            second = nullptr;
        }
        if (record)
            row_record<T>(w.part + u * kRecStride, lane, acc);
        else
            row_store<T>(L, w, tok, lane, acc);
    }
}

// Cross-lane steps on the DPP path (no LDS round trip): the sum over the 8
// lanes of a key row (quad swaps 1 and 2, then the half-row mirror pairs
// lane i with 7 - i), and the wave-wide maximum of a value that is uniform
// within each 8-lane group (row rotate by 8, then the four rows' lane 0).
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum8(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp<0x141>(x);  // row_half_mirror
    return x;
}
__device__ __forceinline__ float max_groups(float x) {
    x = fmaxf(x, dpp<0x128>(x));  // row_ror 8: groups 2r and 2r + 1 of each row
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// ---- bf16 correspondence rows: every head of a group in one pass over the
// row's index.  One wave per patch row; per chunk of NP * 8 keys the index
// entries are read once for the group, then the K and the V rows of every
// head of the group are requested together (unconditional loads from the
// listed, always valid tokens; slots past the row's end are masked by select
// afterwards), so a chunk costs one memory round trip for all NH heads.  The
// softmax of each head runs online over the chunks; lanes of one 8-lane
// group hold one key row, 16 bytes each.
constexpr int kIdxRun = 256;  // index entries staged in LDS per wave at a time

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// q . k over a lane's 8 channels: four v_dot2 on the packed bf16 pairs (the
// products are exact in fp32), one call per 32-bit word
__device__ __forceinline__ float dot2_word(uint32_t q, uint32_t k, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q), __builtin_bit_cast(bf16x2, k), acc, false);
}
__device__ __forceinline__ float dot8_bf16(u32x4 q, u32x4 k) {
    const uint32_t q0 = q.x, q1 = q.y, q2 = q.z, q3 = q.w;
    const uint32_t k0 = k.x, k1 = k.y, k2 = k.z, k3 = k.w;
    return dot2_word(q3, k3, dot2_word(q2, k2, dot2_word(q1, k1, dot2_word(q0, k0, 0.f))));
}

template <int NH, int NP>
__device__ void gather_group(const ValuLaunch &L, const HeadWork *hw, int64_t u, int64_t tok, int lane,
                             int32_t *sidx) {
    constexpr int RPP = 8, CH = NP * RPP;
    static_assert(kIdxRun % CH == 0 && kIdxRun % 64 == 0, "chunks within one staged run");
    const int sub = lane & 7, grp = lane >> 3;
    const int64_t ts = L.token_stride;
    const float sc = kLog2e * 0.125f;
    const uint16_t *Kh[NH], *Vh[NH];
    u32x4 q[NH];
    float o[NH][8], m[NH], l[NH];
    int32_t skip[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int64_t hoff = (int64_t)hw[h].head * L.head_stride + sub * 8;
        Kh[h] = (const uint16_t *)L.k + hoff;
        Vh[h] = (const uint16_t *)L.v + hoff;
        q[h] = *(const u32x4 *)((const uint16_t *)L.q + hoff + tok * ts);
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
        skip[h] = hw[h].rec_out ? hw[h].budget : 0;
    }
    const int32_t *idx = L.corr_idx + u * L.corr_k;
    const int32_t count = L.corr_k;
    for (int32_t c0 = 0; c0 < count; c0 += CH) {
        // the row's index entries reach LDS kIdxRun at a time, read by the
        // whole wave at once (coalesced), so that each chunk waits for one
        // memory round trip (its K and V rows), not two; a wave reads back
        // only what it wrote itself (in order: no barrier)
        const int32_t run0 = c0 / kIdxRun * kIdxRun;
        if (c0 == run0) {
            int32_t e[kIdxRun / 64];
#pragma unroll
            for (int j = 0; j < kIdxRun / 64; ++j) e[j] = idx[min(run0 + lane + 64 * j, count - 1)];
#pragma unroll
            for (int j = 0; j < kIdxRun / 64; ++j) sidx[lane + 64 * j] = e[j];
        }
        int32_t t[NP];
        bool in[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int32_t mi = c0 + p * RPP + grp;
            in[p] = mi < count;
            t[p] = sidx[(in[p] ? mi : count - 1) - run0];
        }
        u32x4 kr[NH][NP], vr[NH][NP];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int p = 0; p < NP; ++p) kr[h][p] = *(const u32x4 *)(Kh[h] + (int64_t)t[p] * ts);
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int p = 0; p < NP; ++p) vr[h][p] = *(const u32x4 *)(Vh[h] + (int64_t)t[p] * ts);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float s[NP], cm = -INFINITY;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float dot = sum8(dot8_bf16(q[h], kr[h][p]));
                const bool ok = in[p] && !(skip[h] > 0 && t[p] % skip[h] == 0);
                s[p] = ok ? dot * sc : -INFINITY;
                cm = fmaxf(cm, s[p]);
            }
            cm = max_groups(cm);
            if (cm == -INFINITY) continue;  // wave-uniform: every slot masked
            const float m_new = fmaxf(m[h], cm);
            const float alpha = fast_exp2(m[h] - m_new);
            // weights rounded to bf16 once; the sum and P.V take the same
            // rounded values (an exact convex combination of V rows under
            // them), P.V as two dot2 per channel pair against (p, 0) and
            // (0, p).  Masked slots weigh 0 and read a listed (finite) row.
            uint32_t pw[NP];
            float lsum = 0.f;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                pw[p] = pack_bf16x2(fast_exp2(s[p] - m_new), 0.f);
                lsum += __uint_as_float(pw[p] << 16);
            }
            l[h] = l[h] * alpha + lsum;
            m[h] = m_new;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const uint32_t plo = pw[p], phi = pw[p] << 16;
                const u32x4 vv = vr[h][p];
                const uint32_t v0 = vv.x, v1 = vv.y, v2 = vv.z, v3 = vv.w;
                o[h][0] = dot2_word(v0, plo, o[h][0]);
                o[h][1] = dot2_word(v0, phi, o[h][1]);
                o[h][2] = dot2_word(v1, plo, o[h][2]);
                o[h][3] = dot2_word(v1, phi, o[h][3]);
                o[h][4] = dot2_word(v2, plo, o[h][4]);
                o[h][5] = dot2_word(v2, phi, o[h][5]);
                o[h][6] = dot2_word(v3, plo, o[h][6]);
                o[h][7] = dot2_word(v3, phi, o[h][7]);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int x = 8; x < 64; x <<= 1) {
            l[h] += __shfl_xor(l[h], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] += __shfl_xor(o[h][e], x);
        }
        if (grp != 0) continue;
        if (hw[h].rec_out) {
            float *rec = hw[h].part + u * kRecStride;
#pragma unroll
            for (int e = 0; e < 8; ++e) rec[2 + sub * 8 + e] = o[h][e];
            if (sub == 0) {
                rec[0] = m[h];
                rec[1] = l[h];
            }
        } else {
            const float inv = 1.f / l[h];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= inv;
            Lanes<uint16_t>::store((uint16_t *)L.o + (int64_t)hw[h].head * L.head_stride + tok * ts + sub * 8, o[h]);
        }
    }
}

constexpr int kGatherGroup = 3;  // heads per pass over a row's index
constexpr int kGatherNP = 4;     // key rows per lane and chunk (32 keys per chunk)

__global__ __launch_bounds__(256) void gather_attn_kernel(const ValuLaunch L) {
    const Geom &g = L.g;
    const int lane = threadIdx.x & 63;
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= g.Np) return;
    const int64_t tok = (u / g.P) * g.T + g.ns + (u % g.P);
    __shared__ int32_t sidx[4][kIdxRun];
    int32_t *my = sidx[threadIdx.x >> 6];
    for (int i0 = 0; i0 < L.nwork; i0 += kGatherGroup) {
        const int nh = min(kGatherGroup, L.nwork - i0);
        if (nh == 3)
            gather_group<3, kGatherNP>(L, L.work + i0, u, tok, lane, my);
        else if (nh == 2)
            gather_group<2, kGatherNP>(L, L.work + i0, u, tok, lane, my);
        else
            gather_group<1, kGatherNP>(L, L.work + i0, u, tok, lane, my);
    }
}

// one wave per (patch row, head), lane = channel
__global__ __launch_bounds__(256) void union_merge_kernel(const UnionMerge U) {
    const Geom &g = U.g;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= g.Np * U.nhead) return;
    const int hi = (int)(gw / g.Np);
    const int64_t u = gw % g.Np;
    const int64_t tok = (u / g.P) * g.T + g.ns + (u % g.P);
    const float *ra = U.rec_tok[hi] + tok * kRecStride;
    const float *rb = U.rec_patch[hi] + u * kRecStride;
    const float ma = ra[0], mb = rb[0];
    const float M = fmaxf(ma, mb);
    const float fa = ma == -INFINITY ? 0.f : fast_exp2(ma - M);
    const float fb = mb == -INFINITY ? 0.f : fast_exp2(mb - M);
    const float l = ra[1] * fa + rb[1] * fb;
    const float o = ra[2 + lane] * fa + rb[2 + lane] * fb;
    uint16_t *O = (uint16_t *)U.o + (int64_t)U.head[hi] * U.head_stride + tok * U.token_stride;
    O[lane] = (uint16_t)f32_to_bf16_bits(o / l);
}

}  // namespace

hipError_t launch_valu_attention(const ValuLaunch &L, int64_t nrows, hipStream_t stream) {
    if (nrows <= 0 || L.nwork <= 0) return hipSuccess;
    // bf16: the row kernel gathers the correspondence keys of patch rows; the
    // static key sets of the other roles run on the matrix cores
    if (L.g.dtype == BF16) {
        if (!L.patch_rows_only) return hipErrorInvalidValue;
        for (int i = 0; i < L.nwork; ++i)
            if (!(L.work[i].role == CORRESPONDENCE || (L.work[i].role == CORR_STRIDE && L.work[i].rec_out)))
                return hipErrorInvalidValue;
    }
    const dim3 grid((unsigned)((nrows + 3) / 4));
    if (L.g.dtype == BF16)
        hipLaunchKernelGGL(gather_attn_kernel, grid, dim3(256), 0, stream, L);
    else
        hipLaunchKernelGGL(valu_attn_kernel<float>, grid, dim3(256), 0, stream, L, nrows);
    return hipGetLastError();
}

hipError_t launch_union_merge(const UnionMerge &U, hipStream_t stream) {
    if (U.nhead <= 0) return hipSuccess;
    const int64_t waves = U.g.Np * U.nhead;
    hipLaunchKernelGGL(union_merge_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, U);
    return hipGetLastError();
}

}  // namespace saf
