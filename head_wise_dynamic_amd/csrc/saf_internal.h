// Internal declarations shared by the host API (api.cpp) and the HIP kernels.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saf {

enum Role : int32_t {
    POSITION = 0, VERTICAL = 1, CORRESPONDENCE = 2, SCANNING = 3, DENSE = 4, CORR_STRIDE = 5, BROADCAST = 6
};
enum Dtype : int32_t { F32 = 0, BF16 = 1 };

// Geometry with derived sizes.  Token j = f * T + t; special iff t < ns.
struct Geom {
    int32_t S, ns, P, T, H, d;
    int64_t N, Np;
    int32_t dtype;
};

// Query rows a piece of work covers:
//   FRAME    -- rows f*T .. f*T+T-1 for every frame f (position heads: the key
//               set depends on the query frame, so tiles never cross frames)
//   ALL      -- rows 0 .. N-1
//   SPECIALS -- the ns*S special-token rows, m -> (m / ns) * T + m % ns
//   BY_POSITION -- patch rows grouped by patch position: ceil(S / 256) tiles
//               per position p, tile rows = frames, row f -> f*T + ns + p
//               (broadcast heads: the key set depends on p only)
enum RowSpace : int32_t { ROWS_FRAME = 0, ROWS_ALL = 1, ROWS_SPECIALS = 2, ROWS_BY_POSITION = 3 };

// One head's key-set description as the attention kernels see it.
//   POSITION: specials (ns*S) ++ anchor-frame patches (P) ++ own-frame
//             patches (P, only when the query frame is not the anchor)
//   SCANNING: tokens m*stride for m < ceil(N/stride) ++ specials, where a
//             special that already lies on the stride is a masked slot
//   VERTICAL: list[0 .. list_len)
//   DENSE:    every token (also the special rows of correspondence and
//             broadcast heads)
//   BROADCAST: specials (ns*S) ++ for every frame, the patches of the window
//             of radius budget around the query's patch position, row-major
//             over a grid anchor patches wide (anchor = 0: one row of P)
struct HeadWork {
    int32_t head;       // head index (pointer offsets)
    int32_t role;       // key-set rule, see above
    int32_t budget;     // stride for SCANNING
    int32_t anchor;     // anchor frame for POSITION
    int32_t rows;       // RowSpace
    int32_t list_len;   // VERTICAL
    int32_t nsplit;     // key splits per query tile (1 = no split)
    int32_t block0;     // first work-group of this head in the launch
    const int32_t *list;// VERTICAL key list (device, ascending)
    float *part;        // split partials (nsplit > 1 or rec_out): [tiles*QT rows][nsplit] x (m, l, o[64])
    int32_t rec_out;    // write the (m, l, o) record even with nsplit == 1 (merged later)
    // SCANNING, bf16: the key set gathered once into contiguous rows (the
    // stride tokens, then the specials off the stride), 64 bf16 per row;
    // null: keys enumerated and gathered per tile
    uint16_t *pk, *pv;
    int32_t *pspec;     // the specials off the stride, in order (filled with pk, pv)
    int32_t pcount;     // rows of the packed set
};

// Softmax partial record of one query row: running max m (log2 units of the
// scaled logit), l = sum 2^(s - m), o[64] = sum 2^(s - m) v.
constexpr int kRecStride = 66;

constexpr int kMaxWork = 24;
constexpr int kQueryTile = 256;  // query rows per work-group of the matrix-core kernel

// Partial maxima of |k|^2 per piece of work of a matrix-core launch (each
// over a contiguous range of the head's tokens); the attention kernel
// reduces them to the head's largest key norm in its prologue.
constexpr int kNormParts = 256;

struct MfmaLaunch {
    Geom g;
    const void *q, *k, *v;
    void *o;
    int64_t head_stride, token_stride;
    // [kMaxWork][kNormParts] squared-norm maxima (launch_key_norms), or null:
    // then every wave keeps a running maximum of its logits
    const float *knorm;
    int32_t nwork;
    int32_t total_blocks;
    int32_t block_base;  // a launch runs blocks [block_base, block_base + grid) of the work list
    HeadWork work[kMaxWork];
};

// VALU row kernel: one wave per query row, looping over every listed head.
//   rows = ROWS_ALL: every token row; rows = patch rows only when
//   patch_rows_only (correspondence heads of the bf16 path).
struct ValuLaunch {
    Geom g;
    const void *q, *k, *v;
    void *o;
    int64_t head_stride, token_stride;
    const int32_t *corr_idx;   // [Np, corr_k] global token ids
    int32_t corr_k;
    int32_t patch_rows_only;
    int32_t nwork;
    HeadWork work[kMaxWork];
};

// ---------------------------------------------------------------- launchers
// Each returns the hipError_t of its launch.
// Blocks [L.block_base, L.block_base + nblocks).  share_cu: at most one
// work-group per compute unit (a larger LDS allocation), so that a kernel on
// another stream finds registers beside it on every SIMD.
hipError_t launch_mfma_attention(const MfmaLaunch &L, int32_t nblocks, bool share_cu, hipStream_t stream);
// parts[wi * kNormParts + p] = largest |k|^2 over the p-th token range of
// work wi's head (bf16 K; parts holds kMaxWork * kNormParts floats)
hipError_t launch_key_norms(const MfmaLaunch &L, float *parts, hipStream_t stream);
hipError_t launch_split_combine(const MfmaLaunch &L, hipStream_t stream);
// Fill the packed key sets (pk, pv) of every work of L that has them.
hipError_t launch_pack_keys(const MfmaLaunch &L, hipStream_t stream);
// Specials a packed scanning set can hold (ns S at most this).
constexpr int kPackSpecials = 4096;
hipError_t launch_valu_attention(const ValuLaunch &L, int64_t nrows, hipStream_t stream);
// CORR_STRIDE heads (bf16): merge, for every patch row, the stride set's
// record from the matrix-core kernel (rows = tokens) with the gathered
// keys' record (rows = patches) and write O.
struct UnionMerge {
    Geom g;
    void *o;
    int64_t head_stride, token_stride;
    int32_t nhead;
    int32_t head[kMaxWork];
    const float *rec_tok[kMaxWork];    // [N rows (tiles*QT)] x kRecStride
    const float *rec_patch[kMaxWork];  // [Np] x kRecStride
};
hipError_t launch_union_merge(const UnionMerge &U, hipStream_t stream);

// Vertical probe: qbar (fp32) of one head, probe scores, exact top-K.
//   ws layout per head: partial sums [kProbeBlocks][64] f32, qbar [64] f32,
//   scores [N] f32, histogram/scratch [kTopkScratch] u32.
constexpr int kProbeBlocks = 256;
constexpr int kTopkScratch = 4096;
size_t vertical_ws_bytes(int64_t N);
hipError_t launch_vertical_index(const Geom &g, const void *q, const void *k, int64_t head_stride,
                                 int64_t token_stride, int32_t head, int32_t K, int32_t *idx_out,
                                 void *ws, hipStream_t stream);
// nh heads in one set of launches (grid.y = head)
hipError_t launch_vertical_batch(const Geom &g, const void *q, const void *k, int64_t head_stride,
                                 int64_t token_stride, int nh, const int32_t *heads, const int32_t *Ks,
                                 int32_t *const *idx_out, void *const *ws, hipStream_t stream);

// Correspondence index build (cosine top-K over other frames).
struct CorrBuild {
    Geom g;
    const void *dino;
    int32_t dino_dtype;
    int32_t Df;
    int64_t row_stride;
    int32_t K;      // kept per row (total mode) or per other frame (per-frame mode), clamped
    int32_t cap;    // candidate capacity per row (total mode; fused per-frame mode, 0: stored cosines)
    int32_t per_frame;  // 1: the K best of every other frame, [Np, (S-1) K]
    int32_t frames_stored;  // per-frame mode: always materialise the cosine rows (no filtered pass)
    int32_t chunk_rows; // per-frame mode: rows whose cosines are materialised at once
    int32_t raw_dot;    // 1: rank by the plain dot product f_u . f_v (no normalisation)
    const void *dino_cols;  // column operand (nullptr: the rows' own features, symmetric)
    int32_t tok_map;    // 1: patch row u lives at token (u / P) T + ns + u % P of a token layout
    int32_t total_by_frames;  // total mode as per-frame candidates + exact selection (short rows)
    int32_t *idx_out;   // [Np, K] or [Np, (S-1) K]
    void *scratch;      // corr_scratch_bytes() / corr_frame_scratch_bytes() / corr_frame_fused_scratch_bytes()
    // optional tracing hook: called with begin = 1 / 0 around every cosine
    // GEMM launch (the caller records events on the stream)
    void (*mark)(void *user, int begin, const char *name, hipStream_t stream);
    void *mark_user;
};
size_t corr_scratch_bytes(const Geom &g, int32_t K, int32_t cap);
int32_t corr_capacity(const Geom &g, int32_t K);
constexpr int32_t kFrameMaxP = 4096;  // per-frame mode: patches per frame the selection holds
int32_t corr_frame_chunk_rows(const Geom &g);
size_t corr_frame_scratch_bytes(const Geom &g, int32_t chunk_rows);
// Fused per-frame mode (a filtered symmetric pass, no stored cosines): the
// candidate capacity per row, or 0 when B takes the stored-cosine path
// (fp32 or non-symmetric operands, P < 256, K > 8, a long index row, or
// scratch beyond the mode's limit).
int32_t corr_frame_fused_cap(const CorrBuild &B);
size_t corr_frame_fused_scratch_bytes(const Geom &g, int32_t cap);
// total_by_frames total mode (per-frame candidates, then an exact selection)
size_t corr_raw_total_scratch_bytes(const Geom &g, int32_t K);
hipError_t launch_corr_build(const CorrBuild &B, hipStream_t stream);
// Total-mode builds on the matrix-core engine and fused per-frame builds list,
// in their scratch, the rows they recomputed exactly (buffer overflow, an
// unconfirmed threshold guess, a frame short of candidates).
bool corr_build_lists_rows(const CorrBuild &B);
void corr_recomputed_list(void *scratch, int64_t Np, int32_t cap, int32_t **rows, uint32_t **count);

// Block-wise index: blocks of `block` consecutive patches of a frame; block
// similarity = dot of the blocks' mean unit features (the token cosine
// averaged over the block pairs); each patch gets the patches of its block's
// selected blocks.
struct CorrBlockBuild {
    Geom g;                 // token geometry (P % block == 0)
    const void *dino;
    int32_t dino_dtype, Df;
    int64_t row_stride;
    int32_t block;          // patches per block
    int32_t K;              // blocks kept per query block (total) or per other frame (clamped)
    int32_t per_frame;
    int32_t *idx_out;       // [Np, Kc] tokens, Kc = kept blocks * block
    void *scratch;          // corr_block_scratch_bytes()
    void (*mark)(void *user, int begin, const char *name, hipStream_t stream);
    void *mark_user;
};
Geom corr_block_geom(const Geom &g, int32_t block);
int32_t corr_block_row_blocks(const Geom &g, int32_t block, int32_t K, int per_frame);
size_t corr_block_scratch_bytes(const Geom &g, int32_t block, int32_t Df, int32_t K, int per_frame);
hipError_t launch_corr_blocks(const CorrBlockBuild &B, hipStream_t stream);

// Per-head error sums of Eq. 1 (fp64): out[2h] = sum (ref - test)^2,
// out[2h + 1] = sum ref^2 (out may be null); acc (may be null):
// acc[h * acc_stride] += weight * out[2h] / out[2h + 1].  part: 2 * H *
// kNmseBlocks doubles.  d = 64, rows 16-byte aligned.
constexpr int kNmseBlocks = 256;
hipError_t launch_head_nmse(const Geom &g, const void *ref, const void *test, int64_t head_stride,
                            int64_t token_stride, double *part, double *out, double *acc, int64_t acc_stride,
                            double weight, hipStream_t stream);

}  // namespace saf
