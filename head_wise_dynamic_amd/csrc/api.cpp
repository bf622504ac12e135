// C ABI of libsaf3r.so: argument validation, the context (correspondence
// index cache), workspace layout and kernel dispatch.  The declarations and
// their contracts are in include/saf3r.h.
//
// Every argument check runs before the first HIP call, so errors come back
// synchronously and a context can be created and validated without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/saf3r.h"
#include "saf_internal.h"
#include "api_internal.h"

struct saf_ctx {
    saf::Geom g{};
    std::string err;
    int32_t *corr_idx = nullptr;  // [Np, corr_k]
    int32_t corr_k = 0;
    int32_t corr_build_k = 0;  // K requested for the index (per frame or per block set), before clamping
    size_t corr_bytes = 0;
    void *corr_scratch = nullptr;
    size_t corr_scratch_bytes = 0;
    // the last build's list of exactly recomputed rows lives in corr_scratch
    // (carved with this candidate capacity); false when it kept none
    bool corr_listed = false;
    int32_t corr_list_cap = 0;
    double *nmse_part = nullptr;  // [H][kNmseBlocks][2] partial sums of the error kernel
    // side stream for the gather path (default priority), fork/join events
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    // per-launch timing
    bool timing = false;
    struct Rec {
        const char *name;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
};

namespace {

// Brackets one launch group with events when the context records timings.
struct Timed {
    saf_ctx *c;
    hipStream_t s;
    const char *name;
    hipEvent_t a = nullptr, b = nullptr;
    Timed(saf_ctx *c_, hipStream_t s_, const char *n) : c(c_), s(s_), name(n) {
        if (!c->timing) return;
        a = take();
        b = take();
        if (a && b) (void)hipEventRecord(a, s);
    }
    hipEvent_t take() {
        hipEvent_t e = nullptr;
        if (!c->pool.empty()) {
            e = c->pool.back();
            c->pool.pop_back();
        } else if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
        }
        return e;
    }
    ~Timed() {
        if (!c->timing || !a || !b) return;
        (void)hipEventRecord(b, s);
        c->recs.push_back({name, a, b});
    }
};

// Tracing hook for launch groups that live inside one launcher (the cosine
// GEMM phases of the index build): begin opens a Timed record, end closes it.
void mark_launch(void *user, int begin, const char *name, hipStream_t s) {
    saf_ctx *c = (saf_ctx *)user;
    static thread_local Timed *open = nullptr;
    if (!c->timing) return;
    if (begin) {
        open = new (std::nothrow) Timed(c, s, name);
    } else if (open) {
        delete open;
        open = nullptr;
    }
}

}  // namespace

namespace {

std::string g_create_error;

saf_status_t fail(saf_ctx_t *c, saf_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (c)
        c->err = buf;
    else
        g_create_error = buf;
    return st;
}

saf_status_t hip_fail(saf_ctx_t *c, hipError_t e, const char *what) {
    return fail(c, SAF_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Testing hook (saf_debug_fail_alloc): the number of device allocations
// still allowed to succeed before the next one reports out-of-memory;
// negative = no limit.
std::atomic<int64_t> g_alloc_allowance{-1};

// Every device allocation of the library goes through here.
hipError_t dev_alloc(void **p, size_t bytes) {
    *p = nullptr;
    int64_t a = g_alloc_allowance.load();
    while (a >= 0) {
        if (a == 0) return hipErrorOutOfMemory;
        if (g_alloc_allowance.compare_exchange_weak(a, a - 1)) break;
    }
    const hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
    }
    return e;
}

constexpr int QT = saf::kQueryTile;  // query tile of the matrix-core kernel
constexpr int kSplitKeys = 8192;  // keys per split for dense special rows

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

saf_status_t check_layout(saf_ctx_t *c, const saf_layout_t &lay) {
    const saf::Geom &g = c->g;
    const int64_t q = g.dtype == saf::BF16 ? 8 : 4;  // elements per 16 bytes
    if (lay.token_stride < g.d || lay.head_stride < 0)
        return fail(c, SAF_EINVAL, "layout: token_stride %lld < head_dim or negative head_stride",
                    (long long)lay.token_stride);
    if (lay.token_stride % q || lay.head_stride % q)
        return fail(c, SAF_EINVAL, "layout: strides must be multiples of 16 bytes");
    // heads and tokens must not overlap: either [H,N,d] or [N,H,d] style
    const bool hnd = lay.head_stride >= (int64_t)g.N * lay.token_stride;
    const bool nhd = lay.token_stride >= (int64_t)g.H * lay.head_stride && lay.head_stride >= g.d;
    if (g.H > 1 && !hnd && !nhd)
        return fail(c, SAF_EINVAL, "layout: head and token strides overlap");
    return SAF_OK;
}

saf_status_t check_tensors(saf_ctx_t *c, const void *q, const void *k, const void *v, void *o) {
    if (!q || !k || !v || !o) return fail(c, SAF_EINVAL, "null q/k/v/o pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(c, SAF_EINVAL, "q/k/v/o must be 16-byte aligned");
    return SAF_OK;
}

struct PlanInfo {
    int nvert = 0, ncorr = 0, nunion = 0, nbcast = 0;
    int64_t vert_ws = 0;      // bytes for in-call vertical index builds
    int64_t split_ws = 0;     // bytes for dense-row split partials
    int64_t union_ws = 0;     // bytes for the records of correspondence + stride heads
    int64_t norm_ws = 0;      // bytes for the key-norm maxima of the matrix-core launches
    int64_t pack_ws = 0;      // bytes for the packed key sets of the scanning heads
    int corr_splits = 1;
};

// Rows of a scanning head's packed key set: the stride tokens, then the
// specials off the stride; 0 when the set is not packed (fp32, or more
// specials than the packing kernel holds).
int64_t scan_pack_rows(const saf::Geom &g, int32_t stride) {
    if (g.dtype != saf::BF16 || stride < 1 || (int64_t)g.ns * g.S > saf::kPackSpecials) return 0;
    int64_t on = 0;
    for (int64_t f = 0; f < g.S; ++f)
        for (int64_t t = 0; t < g.ns; ++t) on += ((f * g.T + t) % stride == 0);
    return (g.N + stride - 1) / stride + (int64_t)g.ns * g.S - on;
}
int64_t scan_pack_bytes(const saf::Geom &g, int32_t stride) {
    const int64_t rows = scan_pack_rows(g, stride);
    if (rows == 0) return 0;
    return 2 * (int64_t)align256(sizeof(uint16_t) * 64 * (size_t)rows) +
           (int64_t)align256(sizeof(int32_t) * (size_t)g.ns * g.S + 4);
}

// key-norm maxima of one matrix-core launch group (bf16 contexts)
int64_t norm_bytes(const saf::Geom &g) {
    return g.dtype == saf::BF16 ? (int64_t)align256(sizeof(float) * saf::kMaxWork * saf::kNormParts) : 0;
}

int corr_special_splits(const saf::Geom &g) {
    const int64_t s = (g.N + kSplitKeys - 1) / kSplitKeys;
    return (int)std::max<int64_t>(1, std::min<int64_t>(s, 64));
}

// records of one correspondence + stride head: the stride set's (one per
// token row of the matrix-core tiles) and the gathered keys' (one per patch)
int64_t union_tok_rec_bytes(const saf::Geom &g) {
    return (int64_t)align256(sizeof(float) * saf::kRecStride * (size_t)((g.N + QT - 1) / QT * QT));
}
int64_t union_rec_bytes(const saf::Geom &g) {
    return union_tok_rec_bytes(g) + (int64_t)align256(sizeof(float) * saf::kRecStride * (size_t)g.Np);
}

int64_t split_part_bytes(const saf::Geom &g, int nsplit) {
    const int64_t rows = ((int64_t)g.ns * g.S + QT - 1) / QT * QT;
    return (int64_t)align256(sizeof(float) * 66 * rows * nsplit);
}

saf_status_t check_plan(saf_ctx_t *c, const saf_head_plan_t *plan, PlanInfo *pi) {
    const saf::Geom &g = c->g;
    if (!plan) return fail(c, SAF_EINVAL, "null plan");
    *pi = PlanInfo{};
    for (int h = 0; h < g.H; ++h) {
        const saf_head_plan_t &p = plan[h];
        if (p.flags != 0) return fail(c, SAF_EUNSUPPORTED, "head %d: flags must be 0", h);
        switch (p.role) {
        case SAF_POSITION:
            if (p.anchor_frame < 0 || p.anchor_frame >= g.S)
                return fail(c, SAF_EINVAL, "head %d: anchor frame %d outside [0, %d)", h, p.anchor_frame, g.S);
            break;
        case SAF_VERTICAL:
            if (p.budget < 1) return fail(c, SAF_EINVAL, "head %d: vertical budget %d < 1", h, p.budget);
            ++pi->nvert;
            break;
        case SAF_CORRESPONDENCE:
            if (g.S < 2) return fail(c, SAF_EINVAL, "head %d: correspondence needs S >= 2", h);
            if (p.budget < 0) return fail(c, SAF_EINVAL, "head %d: negative budget", h);
            ++pi->ncorr;
            break;
        case SAF_CORR_STRIDE:
            if (g.S < 2) return fail(c, SAF_EINVAL, "head %d: correspondence needs S >= 2", h);
            if (p.budget < 1) return fail(c, SAF_EINVAL, "head %d: stride %d < 1", h, p.budget);
            ++pi->ncorr;
            ++pi->nunion;
            break;
        case SAF_SCANNING:
            if (p.budget < 1) return fail(c, SAF_EINVAL, "head %d: scanning stride %d < 1", h, p.budget);
            if (g.ns == 0 && p.budget > g.N) {
                // stride set is {0}: still non-empty
            }
            break;
        case SAF_DENSE:
            break;
        case SAF_BROADCAST:
            if (p.budget < 0) return fail(c, SAF_EINVAL, "head %d: broadcast radius %d < 0", h, p.budget);
            if (p.anchor_frame < 0 || (p.anchor_frame > 0 && g.P % p.anchor_frame != 0))
                return fail(c, SAF_EINVAL, "head %d: grid width %d does not divide P = %d", h, p.anchor_frame, g.P);
            ++pi->nbcast;
            break;
        default:
            return fail(c, SAF_EINVAL, "head %d: unknown role %d", h, p.role);
        }
    }
    pi->vert_ws = (int64_t)pi->nvert * (int64_t)(align256(saf::vertical_ws_bytes(g.N)) +
                                                 align256(sizeof(int32_t) * g.N));
    // heads whose special-token rows attend to every key on the matrix cores
    const int ndense_specials = pi->ncorr + pi->nbcast;
    if (ndense_specials && g.dtype == saf::BF16) {
        pi->corr_splits = corr_special_splits(g);
        if (pi->corr_splits > 1) pi->split_ws = (int64_t)ndense_specials * split_part_bytes(g, pi->corr_splits);
        pi->union_ws = (int64_t)pi->nunion * union_rec_bytes(g);
    }
    pi->norm_ws = norm_bytes(g);
    for (int h = 0; h < g.H; ++h)
        if (plan[h].role == SAF_SCANNING) pi->pack_ws += scan_pack_bytes(g, plan[h].budget);
    return SAF_OK;
}

hipStream_t as_stream(void *s) { return (hipStream_t)s; }

}  // namespace

extern "C" {

saf_status_t saf_create(const saf_geometry_t *geom, saf_ctx_t **out) {
    if (!out) return fail(nullptr, SAF_EINVAL, "null output pointer");
    *out = nullptr;
    if (!geom) return fail(nullptr, SAF_EINVAL, "null geometry");
    const saf_geometry_t &G = *geom;
    if (G.num_frames < 1 || G.specials_per_frame < 0 || G.patches_per_frame < 1 || G.num_heads < 1 ||
        G.num_heads > 64)
        return fail(nullptr, SAF_EINVAL, "geometry: need S >= 1, ns >= 0, P >= 1, 1 <= H <= 64");
    if (G.dtype != SAF_F32 && G.dtype != SAF_BF16) return fail(nullptr, SAF_EINVAL, "geometry: bad dtype");
    if (G.head_dim != 64) return fail(nullptr, SAF_EUNSUPPORTED, "geometry: head_dim must be 64");
    const int64_t T = (int64_t)G.specials_per_frame + G.patches_per_frame;
    const int64_t N = T * G.num_frames;
    // key-set sizes (at most N + ns S) stay below 2^31; a larger N would not
    // fit one GPU's memory anyway (Q alone: H x 2^30 x 64 x 2 bytes)
    if (N >= (int64_t)1 << 30) return fail(nullptr, SAF_EINVAL, "geometry: N must be < 2^30");
    saf_ctx_t *c = new (std::nothrow) saf_ctx_t();
    if (!c) return fail(nullptr, SAF_ENOMEM, "out of host memory");
    c->g.S = G.num_frames;
    c->g.ns = G.specials_per_frame;
    c->g.P = G.patches_per_frame;
    c->g.T = (int32_t)T;
    c->g.H = G.num_heads;
    c->g.d = G.head_dim;
    c->g.N = N;
    c->g.Np = (int64_t)G.num_frames * G.patches_per_frame;
    c->g.dtype = G.dtype;
    *out = c;
    return SAF_OK;
}

void saf_destroy(saf_ctx_t *c) {
    if (!c) return;
    for (auto &r : c->recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (hipEvent_t e : c->pool) (void)hipEventDestroy(e);
    if (c->side) {
        (void)hipStreamSynchronize(c->side);
        (void)hipStreamDestroy(c->side);
    }
    if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
    if (c->ev_join) (void)hipEventDestroy(c->ev_join);
    if (c->corr_idx || c->corr_scratch || c->nmse_part) {
        (void)hipDeviceSynchronize();
        if (c->corr_idx) (void)hipFree(c->corr_idx);
        if (c->corr_scratch) (void)hipFree(c->corr_scratch);
        if (c->nmse_part) (void)hipFree(c->nmse_part);
    }
    delete c;
}

const char *saf_last_error(const saf_ctx_t *c) { return c ? c->err.c_str() : g_create_error.c_str(); }

saf_status_t saf_workspace_size(const saf_ctx_t *cc, const saf_head_plan_t *plan, size_t *bytes) {
    saf_ctx_t *c = const_cast<saf_ctx_t *>(cc);
    if (!c) return SAF_EINVAL;
    if (!bytes) return fail(c, SAF_EINVAL, "null bytes pointer");
    *bytes = 0;
    if (!plan) {  // dense attention: the key-norm maxima (bf16)
        const int64_t nb = norm_bytes(c->g);
        *bytes = nb ? (size_t)nb + 256 : 0;
        return SAF_OK;
    }
    PlanInfo pi;
    const saf_status_t st = check_plan(c, plan, &pi);
    if (st != SAF_OK) return st;
    *bytes = (size_t)(pi.vert_ws + pi.split_ws + pi.union_ws + pi.norm_ws + pi.pack_ws) + 256;
    return SAF_OK;
}

// Forget the cached index: a build or copy that failed after writing into it
// leaves nothing usable, and later calls needing an index return SAF_ESTATE.
static void drop_corr_index(saf_ctx_t *c) {
    if (c->corr_idx) (void)hipFree(c->corr_idx);
    c->corr_idx = nullptr;
    c->corr_bytes = 0;
    c->corr_k = 0;
    c->corr_build_k = 0;
    c->corr_listed = false;
}

// Index storage for rows of K entries.  A new buffer is allocated before the
// old one is released, so an allocation failure leaves the cached index as
// it was.  Once a new buffer is in place the index counts as absent
// (corr_k = 0) until the caller's build or copy has been enqueued.
static saf_status_t ensure_corr_storage(saf_ctx_t *c, int32_t K) {
    const size_t need = sizeof(int32_t) * (size_t)c->g.Np * (size_t)K;
    if (c->corr_idx && c->corr_bytes == need) return SAF_OK;
    void *p = nullptr;
    if (dev_alloc(&p, need) != hipSuccess)
        return fail(c, SAF_ENOMEM, "hipMalloc(%zu) for the correspondence index failed", need);
    if (c->corr_idx) {
        const hipError_t e = hipFree(c->corr_idx);
        c->corr_idx = nullptr;
        if (e != hipSuccess) {
            (void)hipFree(p);
            drop_corr_index(c);
            return hip_fail(c, e, "hipFree(corr index)");
        }
    }
    c->corr_idx = (int32_t *)p;
    c->corr_bytes = need;
    c->corr_k = 0;
    c->corr_build_k = 0;
    c->corr_listed = false;
    return SAF_OK;
}

// grow the context-owned build scratch to at least sb bytes (the scratch
// holds no state the cached index depends on, except the list of recomputed
// rows, which a regrown scratch no longer has)
static saf_status_t ensure_corr_scratch(saf_ctx_t *c, size_t sb) {
    if (c->corr_scratch_bytes >= sb) return SAF_OK;
    c->corr_listed = false;
    if (c->corr_scratch) {
        hipError_t e = hipFree(c->corr_scratch);
        c->corr_scratch = nullptr;
        c->corr_scratch_bytes = 0;
        if (e != hipSuccess) return hip_fail(c, e, "hipFree(corr scratch)");
    }
    if (dev_alloc(&c->corr_scratch, sb) != hipSuccess)
        return fail(c, SAF_ENOMEM, "hipMalloc(%zu) for index scratch failed", sb);
    c->corr_scratch_bytes = sb;
    return SAF_OK;
}

saf_status_t saf_build_corr_index(saf_ctx_t *c, const void *dino, int32_t dino_dtype, int32_t Df,
                                  int64_t row_stride, int32_t K, int32_t mode, void *stream) {
    if (!c) return SAF_EINVAL;
    const saf::Geom &g = c->g;
    if (!dino) return fail(c, SAF_EINVAL, "null dino pointer");
    if (dino_dtype != SAF_F32 && dino_dtype != SAF_BF16) return fail(c, SAF_EINVAL, "bad dino dtype");
    if (g.S < 2) return fail(c, SAF_EINVAL, "correspondence index needs S >= 2");
    if (K < 1) return fail(c, SAF_EINVAL, "K %d < 1", K);
    if (Df < 1) return fail(c, SAF_EINVAL, "Df %d < 1", Df);
    if (row_stride < Df) return fail(c, SAF_EINVAL, "dino row stride %lld < Df", (long long)row_stride);
    if (mode != SAF_CORR_TOTAL && mode != SAF_CORR_PER_FRAME && mode != SAF_CORR_PER_FRAME_STORED)
        return fail(c, SAF_EINVAL, "bad mode %d", mode);
    const bool per_frame = mode != SAF_CORR_TOTAL;
    if (Df > 4096) return fail(c, SAF_EUNSUPPORTED, "Df %d > 4096", Df);
    const int64_t q = dino_dtype == SAF_BF16 ? 8 : 4;
    if (row_stride % q || !aligned16(dino))
        return fail(c, SAF_EINVAL, "dino rows must be 16-byte aligned");
    // K kept per row (total) or per other frame (per-frame); Kc = index row length
    int32_t Kk, Kc;
    if (per_frame) {
        if (g.P > saf::kFrameMaxP) return fail(c, SAF_EUNSUPPORTED, "per-frame mode: P %d > %d", g.P, saf::kFrameMaxP);
        Kk = std::min(K, g.P);
        const int64_t row = (int64_t)(g.S - 1) * Kk;
        if (row > INT32_MAX / 2) return fail(c, SAF_EUNSUPPORTED, "index row of %lld entries", (long long)row);
        Kc = (int32_t)row;
    } else {
        const int64_t ncand = (int64_t)(g.S - 1) * g.P;
        Kk = Kc = (int32_t)std::min<int64_t>(K, ncand);
        if (Kc > 1024) return fail(c, SAF_EUNSUPPORTED, "K %d > 1024", Kc);
    }

    saf::CorrBuild B{};
    B.g = g;
    B.dino = dino;
    B.dino_dtype = dino_dtype;
    B.Df = Df;
    B.row_stride = row_stride;
    B.K = Kk;
    B.per_frame = per_frame ? 1 : 0;
    B.frames_stored = mode == SAF_CORR_PER_FRAME_STORED ? 1 : 0;
    const int32_t cap = per_frame ? saf::corr_frame_fused_cap(B) : saf::corr_capacity(g, Kc);
    const int32_t chunk_rows = per_frame && cap == 0 ? saf::corr_frame_chunk_rows(g) : 0;
    const size_t sb = !per_frame ? saf::corr_scratch_bytes(g, Kc, cap)
                      : cap > 0  ? saf::corr_frame_fused_scratch_bytes(g, cap)
                                 : saf::corr_frame_scratch_bytes(g, chunk_rows);
    saf_status_t st = ensure_corr_scratch(c, sb);
    if (st != SAF_OK) return st;
    if ((st = ensure_corr_storage(c, Kc)) != SAF_OK) return st;
    B.cap = cap;
    B.chunk_rows = chunk_rows;
    B.idx_out = c->corr_idx;
    B.scratch = c->corr_scratch;
    B.mark = mark_launch;
    B.mark_user = c;
    hipError_t e;
    {
        Timed tm(c, as_stream(stream), "corr_index");
        e = saf::launch_corr_build(B, as_stream(stream));
    }
    if (e != hipSuccess) {
        drop_corr_index(c);
        return hip_fail(c, e, "correspondence index kernels");
    }
    c->corr_k = Kc;
    c->corr_build_k = K;
    c->corr_listed = saf::corr_build_lists_rows(B);
    c->corr_list_cap = cap;
    return SAF_OK;
}

saf_status_t saf_build_corr_index_qk(saf_ctx_t *c, const void *q, const void *k, saf_layout_t lay, int32_t head,
                                     int32_t K, int32_t mode, void *stream) {
    if (!c) return SAF_EINVAL;
    const saf::Geom &g = c->g;
    if (!q || !k) return fail(c, SAF_EINVAL, "null q/k pointer");
    if (g.S < 2) return fail(c, SAF_EINVAL, "correspondence index needs S >= 2");
    if (head < 0 || head >= g.H) return fail(c, SAF_EINVAL, "head %d outside [0, %d)", head, g.H);
    if (K < 1) return fail(c, SAF_EINVAL, "K %d < 1", K);
    if (mode != SAF_CORR_TOTAL && mode != SAF_CORR_PER_FRAME && mode != SAF_CORR_PER_FRAME_STORED)
        return fail(c, SAF_EINVAL, "bad mode %d", mode);
    saf_status_t st = check_layout(c, lay);
    if (st != SAF_OK) return st;
    if (!aligned16(q) || !aligned16(k)) return fail(c, SAF_EINVAL, "q/k must be 16-byte aligned");
    const bool per_frame = mode != SAF_CORR_TOTAL;
    int32_t Kk, Kc;
    if (per_frame) {
        if (g.P > saf::kFrameMaxP) return fail(c, SAF_EUNSUPPORTED, "per-frame mode: P %d > %d", g.P, saf::kFrameMaxP);
        Kk = std::min(K, g.P);
        const int64_t row = (int64_t)(g.S - 1) * Kk;
        if (row > INT32_MAX / 2) return fail(c, SAF_EUNSUPPORTED, "index row of %lld entries", (long long)row);
        Kc = (int32_t)row;
    } else {
        Kk = Kc = (int32_t)std::min<int64_t>(K, (int64_t)(g.S - 1) * g.P);
        if (Kc > 1024) return fail(c, SAF_EUNSUPPORTED, "K %d > 1024", Kc);
    }
    const int32_t cap = per_frame ? 0 : saf::corr_capacity(g, Kc);
    const int32_t chunk_rows = per_frame ? saf::corr_frame_chunk_rows(g) : 0;
    const size_t sb = per_frame ? saf::corr_frame_scratch_bytes(g, chunk_rows) : saf::corr_scratch_bytes(g, Kc, cap);
    if ((st = ensure_corr_scratch(c, sb)) != SAF_OK) return st;
    if ((st = ensure_corr_storage(c, Kc)) != SAF_OK) return st;
    const size_t es = g.dtype == saf::BF16 ? 2 : 4;
    saf::CorrBuild B{};
    B.g = g;
    B.dino = (const char *)q + (size_t)head * lay.head_stride * es;
    B.dino_cols = (const char *)k + (size_t)head * lay.head_stride * es;
    B.tok_map = 1;
    B.raw_dot = 1;
    B.dino_dtype = g.dtype;
    B.Df = g.d;
    B.row_stride = lay.token_stride;
    B.K = Kk;
    B.cap = cap;
    B.per_frame = per_frame ? 1 : 0;
    B.frames_stored = per_frame ? 1 : 0;  // q and k differ: no symmetric filtered pass
    B.chunk_rows = chunk_rows;
    B.idx_out = c->corr_idx;
    B.scratch = c->corr_scratch;
    B.mark = mark_launch;
    B.mark_user = c;
    hipError_t e;
    {
        Timed tm(c, as_stream(stream), "corr_index_qk");
        e = saf::launch_corr_build(B, as_stream(stream));
    }
    if (e != hipSuccess) {
        drop_corr_index(c);
        return hip_fail(c, e, "logit index kernels");
    }
    c->corr_k = Kc;
    c->corr_build_k = K;
    c->corr_listed = saf::corr_build_lists_rows(B);
    c->corr_list_cap = cap;
    return SAF_OK;
}

saf_status_t saf_build_corr_index_blocks(saf_ctx_t *c, const void *dino, int32_t dino_dtype, int32_t Df,
                                         int64_t row_stride, int32_t block, int32_t K, int32_t mode,
                                         void *stream) {
    if (!c) return SAF_EINVAL;
    const saf::Geom &g = c->g;
    if (!dino) return fail(c, SAF_EINVAL, "null dino pointer");
    if (dino_dtype != SAF_F32 && dino_dtype != SAF_BF16) return fail(c, SAF_EINVAL, "bad dino dtype");
    if (g.S < 2) return fail(c, SAF_EINVAL, "correspondence index needs S >= 2");
    if (K < 1) return fail(c, SAF_EINVAL, "K %d < 1", K);
    if (Df < 1) return fail(c, SAF_EINVAL, "Df %d < 1", Df);
    if (row_stride < Df) return fail(c, SAF_EINVAL, "dino row stride %lld < Df", (long long)row_stride);
    if (block < 1 || g.P % block) return fail(c, SAF_EINVAL, "block %d does not divide P = %d", block, g.P);
    if (mode != SAF_CORR_TOTAL && mode != SAF_CORR_PER_FRAME) return fail(c, SAF_EINVAL, "bad mode %d", mode);
    if (Df > 4096) return fail(c, SAF_EUNSUPPORTED, "Df %d > 4096", Df);
    const bool per_frame = mode == SAF_CORR_PER_FRAME;
    const int32_t per = g.P / block;
    if (per_frame && per > saf::kFrameMaxP)
        return fail(c, SAF_EUNSUPPORTED, "per-frame mode: %d blocks per frame > %d", per, saf::kFrameMaxP);
    const int32_t rb = saf::corr_block_row_blocks(g, block, K, per_frame ? 1 : 0);
    if (!per_frame && rb > 1024) return fail(c, SAF_EUNSUPPORTED, "%d blocks per row > 1024", rb);
    const int64_t kc64 = (int64_t)rb * block;
    if (kc64 > INT32_MAX / 2) return fail(c, SAF_EUNSUPPORTED, "index row of %lld entries", (long long)kc64);
    const int32_t Kc = (int32_t)kc64;
    saf_status_t st = ensure_corr_scratch(c, saf::corr_block_scratch_bytes(g, block, Df, K, per_frame ? 1 : 0));
    if (st != SAF_OK) return st;
    if ((st = ensure_corr_storage(c, Kc)) != SAF_OK) return st;
    saf::CorrBlockBuild B{};
    B.g = g;
    B.dino = dino;
    B.dino_dtype = dino_dtype;
    B.Df = Df;
    B.row_stride = row_stride;
    B.block = block;
    B.K = per_frame ? std::min(K, per) : rb;
    B.per_frame = per_frame ? 1 : 0;
    B.idx_out = c->corr_idx;
    B.scratch = c->corr_scratch;
    B.mark = mark_launch;
    B.mark_user = c;
    hipError_t e;
    {
        Timed tm(c, as_stream(stream), "corr_index_blocks");
        e = saf::launch_corr_blocks(B, as_stream(stream));
    }
    if (e != hipSuccess) {
        drop_corr_index(c);
        return hip_fail(c, e, "block correspondence index kernels");
    }
    c->corr_k = Kc;
    c->corr_build_k = K;
    c->corr_listed = false;
    return SAF_OK;
}

saf_status_t saf_set_corr_index(saf_ctx_t *c, const int32_t *dev_idx, int32_t Kc, void *stream) {
    if (!c) return SAF_EINVAL;
    if (!dev_idx) return fail(c, SAF_EINVAL, "null index pointer");
    if (c->g.S < 2) return fail(c, SAF_EINVAL, "correspondence index needs S >= 2");
    if (Kc < 1 || (int64_t)Kc > (int64_t)(c->g.S - 1) * c->g.P)
        return fail(c, SAF_EINVAL, "Kc %d outside [1, (S-1)P]", Kc);
    saf_status_t st = ensure_corr_storage(c, Kc);
    if (st != SAF_OK) return st;
    hipError_t e = hipMemcpyAsync(c->corr_idx, dev_idx, c->corr_bytes, hipMemcpyDeviceToDevice, as_stream(stream));
    if (e != hipSuccess) {
        drop_corr_index(c);
        return hip_fail(c, e, "hipMemcpyAsync(index)");
    }
    c->corr_k = Kc;
    c->corr_build_k = Kc;
    c->corr_listed = false;
    return SAF_OK;
}

saf_status_t saf_corr_recomputed_rows(saf_ctx_t *c, int32_t *host_rows, int32_t max_rows, int32_t *count,
                                      void *stream) {
    if (!c) return SAF_EINVAL;
    if (!count) return fail(c, SAF_EINVAL, "null count pointer");
    if (max_rows < 0 || (max_rows > 0 && !host_rows)) return fail(c, SAF_EINVAL, "bad host_rows / max_rows");
    *count = 0;
    if (!c->corr_idx || c->corr_k < 1 || !c->corr_listed || !c->corr_scratch)
        return fail(c, SAF_ESTATE, "the last index build kept no list of recomputed rows");
    int32_t *rows = nullptr;
    uint32_t *cnt = nullptr;
    saf::corr_recomputed_list(c->corr_scratch, c->g.Np, c->corr_list_cap, &rows, &cnt);
    const hipStream_t s = as_stream(stream);
    uint32_t n = 0;
    hipError_t e = hipMemcpyAsync(&n, cnt, sizeof n, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(c, e, "reading the recomputed-row count");
    if ((int64_t)n > c->g.Np) return fail(c, SAF_ESTATE, "recomputed-row count %u exceeds S*P", n);
    const int32_t take = std::min<int32_t>((int32_t)n, max_rows);
    if (take > 0) {
        e = hipMemcpyAsync(host_rows, rows, sizeof(int32_t) * (size_t)take, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(c, e, "reading the recomputed rows");
    }
    *count = (int32_t)n;
    return SAF_OK;
}

saf_status_t saf_get_corr_index(const saf_ctx_t *cc, int32_t *dev_out, int32_t *Kc, void *stream) {
    saf_ctx_t *c = const_cast<saf_ctx_t *>(cc);
    if (!c) return SAF_EINVAL;
    if (!c->corr_idx || c->corr_k < 1) return fail(c, SAF_ESTATE, "no correspondence index has been built");
    if (Kc) *Kc = c->corr_k;
    if (!dev_out) return SAF_OK;
    hipError_t e = hipMemcpyAsync(dev_out, c->corr_idx, c->corr_bytes, hipMemcpyDeviceToDevice, as_stream(stream));
    if (e != hipSuccess) return hip_fail(c, e, "hipMemcpyAsync(index)");
    return SAF_OK;
}

saf_status_t saf_build_vertical_index(saf_ctx_t *c, const void *q, const void *k, saf_layout_t lay,
                                      int32_t head, int32_t K, int32_t *dev_idx_out, void *ws,
                                      size_t ws_bytes, void *stream) {
    if (!c) return SAF_EINVAL;
    if (!q || !k || !dev_idx_out || !ws) return fail(c, SAF_EINVAL, "null pointer");
    if (head < 0 || head >= c->g.H) return fail(c, SAF_EINVAL, "head %d outside [0, %d)", head, c->g.H);
    if (K < 1) return fail(c, SAF_EINVAL, "K %d < 1", K);
    saf_status_t st = check_layout(c, lay);
    if (st != SAF_OK) return st;
    if (!aligned16(q) || !aligned16(k)) return fail(c, SAF_EINVAL, "q/k must be 16-byte aligned");
    const size_t need = saf::vertical_ws_bytes(c->g.N);
    if (ws_bytes < need) return fail(c, SAF_EINVAL, "workspace %zu < %zu bytes", ws_bytes, need);
    hipError_t e;
    {
        Timed tm(c, as_stream(stream), "vertical_index");
        e = saf::launch_vertical_index(c->g, q, k, lay.head_stride, lay.token_stride, head, K, dev_idx_out, ws,
                                       as_stream(stream));
    }
    if (e != hipSuccess) return hip_fail(c, e, "vertical index kernels");
    return SAF_OK;
}

}  // extern "C"

// One layer (saf_sparse_attention).  one_stream: every launch on the caller's
// stream (no side stream, no stream or event creation).
static saf_status_t sparse_attention(saf_ctx_t *c, const saf_head_plan_t *plan, const void *q, const void *k,
                                     const void *v, void *o, saf_layout_t lay, const int32_t *vert_idx,
                                     int64_t vert_ld, void *ws, size_t ws_bytes, void *stream, bool one_stream) {
    if (!c) return SAF_EINVAL;
    const saf::Geom &g = c->g;
    PlanInfo pi;
    saf_status_t st = check_plan(c, plan, &pi);
    if (st != SAF_OK) return st;
    if ((st = check_tensors(c, q, k, v, o)) != SAF_OK) return st;
    if ((st = check_layout(c, lay)) != SAF_OK) return st;
    if (vert_idx && pi.nvert && vert_ld < 1) return fail(c, SAF_EINVAL, "vert_ld must be >= 1");
    for (int h = 0; h < g.H && vert_idx; ++h)
        if (plan[h].role == SAF_VERTICAL && vert_ld < std::min<int64_t>(plan[h].budget, g.N))
            return fail(c, SAF_EINVAL, "vert_ld %lld < head %d's key count", (long long)vert_ld, h);
    if (pi.ncorr) {
        if (!c->corr_idx || c->corr_k < 1) return fail(c, SAF_ESTATE, "a correspondence head needs a built index");
        for (int h = 0; h < g.H; ++h)
            if (plan[h].role == SAF_CORRESPONDENCE && plan[h].budget != 0 && plan[h].budget != c->corr_k &&
                plan[h].budget != c->corr_build_k)
                return fail(c, SAF_ESTATE, "head %d budget %d differs from the index's K %d (row length %d)", h,
                            plan[h].budget, c->corr_build_k, c->corr_k);
    }
    size_t need = (size_t)((vert_idx ? 0 : pi.vert_ws) + pi.split_ws + pi.union_ws + pi.norm_ws + pi.pack_ws);
    if (need > 0) need += 256;  // room to align the start to 256 bytes
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(c, SAF_EINVAL, "workspace %zu < %zu bytes", ws_bytes, need);
    if (ws && !aligned16(ws)) return fail(c, SAF_EINVAL, "workspace must be 16-byte aligned");

    hipStream_t s = as_stream(stream);
    char *wp = (char *)ws;
    if (wp) wp = (char *)(((uintptr_t)wp + 255) & ~(uintptr_t)255);

    // 1. vertical key sets: given by the caller, or built here (one batch)
    std::vector<const int32_t *> vlist(g.H, nullptr);
    std::vector<int32_t> vheads, vK;
    std::vector<int32_t *> vout;
    std::vector<void *> vws;
    for (int h = 0; h < g.H; ++h) {
        if (plan[h].role != SAF_VERTICAL) continue;
        if (vert_idx) {
            vlist[h] = vert_idx + (int64_t)h * vert_ld;
            continue;
        }
        int32_t *idx = (int32_t *)wp;
        wp += align256(sizeof(int32_t) * g.N);
        vws.push_back(wp);
        wp += align256(saf::vertical_ws_bytes(g.N));
        vheads.push_back(h);
        vK.push_back(plan[h].budget);
        vout.push_back(idx);
        vlist[h] = idx;
    }
    auto build_vertical = [&](hipStream_t st) -> hipError_t {
        if (vheads.empty()) return hipSuccess;
        Timed tm(c, st, "vertical_index");
        return saf::launch_vertical_batch(g, q, k, lay.head_stride, lay.token_stride, (int)vheads.size(),
                                          vheads.data(), vK.data(), vout.data(), vws.data(), st);
    };

    if (g.dtype == saf::F32) {
        // fp32: every head on the VALU row kernel, in stream order
        hipError_t e = build_vertical(s);
        if (e != hipSuccess) return hip_fail(c, e, "vertical index kernels");
        saf::ValuLaunch L{};
        L.g = g;
        L.q = q;
        L.k = k;
        L.v = v;
        L.o = o;
        L.head_stride = lay.head_stride;
        L.token_stride = lay.token_stride;
        L.corr_idx = c->corr_idx;
        L.corr_k = c->corr_k;
        L.patch_rows_only = 0;
        for (int h0 = 0; h0 < g.H; h0 += saf::kMaxWork) {
            L.nwork = 0;
            for (int h = h0; h < std::min(g.H, h0 + saf::kMaxWork); ++h) {
                saf::HeadWork &w = L.work[L.nwork++];
                w = saf::HeadWork{};
                w.head = h;
                w.role = plan[h].role;
                w.budget = plan[h].role == SAF_BROADCAST ? std::min(plan[h].budget, g.P) : plan[h].budget;
                w.anchor = plan[h].anchor_frame;
                w.list = vlist[h];
                w.list_len = plan[h].role == SAF_VERTICAL ? (int32_t)std::min<int64_t>(plan[h].budget, g.N) : 0;
                w.nsplit = 1;
            }
            {
                Timed tm(c, s, "valu_attention");
                e = saf::launch_valu_attention(L, g.N, s);
            }
            if (e != hipSuccess) return hip_fail(c, e, "attention kernel (fp32)");
        }
        return SAF_OK;
    }

    // records of the correspondence + stride heads (bf16): the stride set's
    // from the matrix-core kernel, the gathered keys' from the row kernel
    std::vector<float *> union_tok(g.H, nullptr), union_patch(g.H, nullptr);
    for (int h = 0; h < g.H; ++h)
        if (plan[h].role == SAF_CORR_STRIDE) {
            union_tok[h] = (float *)wp;
            union_patch[h] = (float *)(wp + union_tok_rec_bytes(g));
            wp += union_rec_bytes(g);
        }

    // 2. bf16.  The vertical sets are built first, on the caller's stream
    // (a few tens of microseconds on an idle GPU: its small work-groups
    // would otherwise wait for free compute units behind the attention
    // kernels).  Then a side stream (default priority) runs the gathered
    // correspondence rows (HBM-bound) while the caller's stream runs one
    // matrix-core launch group for every shared-key head; the caller's
    // stream joins the side stream at the end of the call.
    // Scanning heads' key sets packed into contiguous rows first, while the
    // GPU is idle (beside the gather their small copies wait for free slots)
    std::vector<saf::HeadWork> packed(g.H);
    {
        saf::MfmaLaunch P{};
        P.g = g;
        P.k = k;
        P.v = v;
        P.head_stride = lay.head_stride;
        P.token_stride = lay.token_stride;
        hipError_t pe = hipSuccess;
        for (int h = 0; h < g.H && pe == hipSuccess; ++h) {
            if (plan[h].role != SAF_SCANNING) continue;
            const int64_t rows = scan_pack_rows(g, plan[h].budget);
            if (rows == 0) continue;
            const int64_t half = (int64_t)align256(sizeof(uint16_t) * 64 * (size_t)rows);
            saf::HeadWork &w = packed[h];
            w.head = h;
            w.role = saf::SCANNING;
            w.budget = plan[h].budget;
            w.pk = (uint16_t *)wp;
            w.pv = (uint16_t *)(wp + half);
            w.pspec = (int32_t *)(wp + 2 * half);
            w.pcount = (int32_t)rows;
            wp += scan_pack_bytes(g, plan[h].budget);
            P.work[P.nwork++] = w;
            if (P.nwork == saf::kMaxWork) {
                Timed tm(c, s, "pack_keys");
                pe = saf::launch_pack_keys(P, s);
                P.nwork = 0;
            }
        }
        if (pe == hipSuccess && P.nwork) {
            Timed tm(c, s, "pack_keys");
            pe = saf::launch_pack_keys(P, s);
        }
        if (pe != hipSuccess) return hip_fail(c, pe, "key packing kernels");
    }
    hipError_t e = build_vertical(s);
    if (e != hipSuccess) return hip_fail(c, e, "vertical index kernels");
    bool forked = false;
    if (pi.ncorr && !one_stream) {
        if (!c->side) {
            if (hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess ||
                hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess ||
                hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess) {
                (void)hipGetLastError();
                if (c->side) (void)hipStreamDestroy(c->side);
                c->side = nullptr;
            }
        }
        if (c->side && hipEventRecord(c->ev_fork, s) == hipSuccess &&
            hipStreamWaitEvent(c->side, c->ev_fork, 0) == hipSuccess)
            forked = true;
    }
    const hipStream_t ss = forked ? c->side : s;
    // every return from here on first joins the side stream
    struct Join {
        saf_ctx *c;
        hipStream_t s;
        bool armed;
        ~Join() {
            if (armed) {
                (void)hipEventRecord(c->ev_join, c->side);
                (void)hipStreamWaitEvent(s, c->ev_join, 0);
            }
        }
    } join{c, s, forked};

    if (pi.ncorr) {
        saf::ValuLaunch L{};
        L.g = g;
        L.q = q;
        L.k = k;
        L.v = v;
        L.o = o;
        L.head_stride = lay.head_stride;
        L.token_stride = lay.token_stride;
        L.corr_idx = c->corr_idx;
        L.corr_k = c->corr_k;
        L.patch_rows_only = 1;
        L.nwork = 0;
        for (int h = 0; h < g.H && e == hipSuccess; ++h) {
            if (plan[h].role != SAF_CORRESPONDENCE && plan[h].role != SAF_CORR_STRIDE) continue;
            if (L.nwork == saf::kMaxWork) {
                Timed tm(c, ss, "gather_attention");
                e = saf::launch_valu_attention(L, g.Np, ss);
                L.nwork = 0;
            }
            saf::HeadWork &w = L.work[L.nwork++];
            w = saf::HeadWork{};
            w.head = h;
            w.role = plan[h].role;
            w.nsplit = 1;
            if (plan[h].role == SAF_CORR_STRIDE) {
                w.budget = plan[h].budget;
                w.rec_out = 1;
                w.part = union_patch[h];
            }
        }
        if (e == hipSuccess && L.nwork) {
            Timed tm(c, ss, "gather_attention");
            e = saf::launch_valu_attention(L, g.Np, ss);
        }
        if (e != hipSuccess) return hip_fail(c, e, "gather attention kernel");
    }

    // shared-key heads on the matrix cores, longest key sets first
    struct Item {
        saf::HeadWork w;
        int64_t tiles;
        double cost;
    };
    std::vector<Item> items;
    const int64_t tpf = (g.T + QT - 1) / QT;
    const int64_t all_tiles = (g.N + QT - 1) / QT;
    for (int h = 0; h < g.H; ++h) {
        saf::HeadWork w{};
        w.head = h;
        w.role = plan[h].role;
        w.budget = plan[h].budget;
        w.anchor = plan[h].anchor_frame;
        w.nsplit = 1;
        Item it{};
        if (plan[h].role == SAF_CORR_STRIDE) {
            // the stride set for every row, as records merged with the gathered keys'
            saf::HeadWork sw = w;
            sw.role = saf::SCANNING;
            sw.rows = saf::ROWS_ALL;
            sw.rec_out = 1;
            sw.part = union_tok[h];
            Item si{};
            si.w = sw;
            si.tiles = all_tiles;
            si.cost = (double)((g.N + sw.budget - 1) / sw.budget) + (double)g.ns * g.S;
            items.push_back(si);
        }
        switch (plan[h].role) {
        case SAF_POSITION:
            w.rows = saf::ROWS_FRAME;
            it.tiles = (int64_t)g.S * tpf;
            it.cost = (double)g.ns * g.S + 2.0 * g.P;
            break;
        case SAF_VERTICAL:
            w.rows = saf::ROWS_ALL;
            w.list = vlist[h];
            w.list_len = (int32_t)std::min<int64_t>(plan[h].budget, g.N);
            it.tiles = all_tiles;
            it.cost = w.list_len;
            break;
        case SAF_SCANNING: {
            w.rows = saf::ROWS_ALL;
            it.tiles = all_tiles;
            it.cost = (double)((g.N + w.budget - 1) / w.budget) + (double)g.ns * g.S;
            // one key set for every query, packed above
            w.pk = packed[h].pk;
            w.pv = packed[h].pv;
            w.pspec = packed[h].pspec;
            w.pcount = packed[h].pcount;
            break;
        }
        case SAF_DENSE:
            w.rows = saf::ROWS_ALL;
            it.tiles = all_tiles;
            it.cost = (double)g.N;
            break;
        case SAF_CORRESPONDENCE:
        case SAF_CORR_STRIDE:
            if (g.ns == 0) continue;
            w.role = saf::DENSE;  // special-token rows attend to every key
            w.rows = saf::ROWS_SPECIALS;
            w.nsplit = pi.corr_splits;
            it.tiles = ((int64_t)g.ns * g.S + QT - 1) / QT;
            it.cost = (double)g.N / w.nsplit;
            break;
        case SAF_BROADCAST: {
            // patch rows grouped by patch position: one key set per position
            w.budget = std::min(plan[h].budget, g.P);
            w.rows = saf::ROWS_BY_POSITION;
            it.tiles = (int64_t)g.P * ((g.S + QT - 1) / QT);
            const int64_t gw = plan[h].anchor_frame > 0 ? plan[h].anchor_frame : g.P, gh = g.P / gw;
            const int64_t side = 2 * (int64_t)w.budget + 1;
            it.cost = (double)g.ns * g.S + (double)g.S * std::min(side, gw) * std::min(side, gh);
            if (g.ns > 0) {  // special-token rows attend to every key
                saf::HeadWork sw = w;
                sw.role = saf::DENSE;
                sw.rows = saf::ROWS_SPECIALS;
                sw.nsplit = pi.corr_splits;
                Item si{};
                si.w = sw;
                si.tiles = ((int64_t)g.ns * g.S + QT - 1) / QT;
                si.cost = (double)g.N / sw.nsplit;
                items.push_back(si);
            }
            break;
        }
        }
        it.w = w;
        items.push_back(it);
    }
    std::stable_sort(items.begin(), items.end(), [](const Item &a, const Item &b) { return a.cost > b.cost; });
    // While the side stream's gather runs, the first (longest) matrix-core
    // blocks run at one work-group per compute unit: two take all of a
    // SIMD's registers, and the gather's waves would wait for them to
    // finish.  About as many blocks as finish while the gather runs: its
    // K/V row bytes and the blocks' logit FLOP at the rates the two kernels
    // reach side by side on MI355X (~5 TB/s and ~0.72 PFLOP/s, the values
    // that time best: at S = 100 every block shares and the layer is flat
    // from half to all of them; at S = 500, 0.8x this many blocks is 2 %
    // faster than 1.25x and 4 % faster than 0.5x, where the gather is left
    // to finish behind full-occupancy blocks).
    constexpr double kShareGatherBytesPerMs = 5.0e9, kShareMfmaFlopPerMs = 0.72e12;
    double share_ms = 0.0;
    if (forked) {
        double gather_bytes = 0.0;
        for (int h = 0; h < g.H; ++h)
            if (plan[h].role == SAF_CORRESPONDENCE || plan[h].role == SAF_CORR_STRIDE)
                gather_bytes += (double)g.Np * c->corr_k * 4.0 * g.d;  // a K and a V bf16 row per key
        share_ms = gather_bytes / kShareGatherBytesPerMs;
    }
    saf::MfmaLaunch M{};
    M.g = g;
    M.q = q;
    M.k = k;
    M.v = v;
    M.o = o;
    M.head_stride = lay.head_stride;
    M.token_stride = lay.token_stride;
    // key-norm maxima: one buffer, reused by the launch groups in stream order
    float *knorm = (float *)wp;
    wp += pi.norm_ws;
    M.knorm = knorm;
    for (size_t i0 = 0; i0 < items.size(); i0 += saf::kMaxWork) {
        M.nwork = 0;
        int64_t blocks = 0;
        for (size_t i = i0; i < std::min(items.size(), i0 + saf::kMaxWork); ++i) {
            saf::HeadWork w = items[i].w;
            if (w.nsplit > 1) {
                w.part = (float *)wp;
                wp += split_part_bytes(g, w.nsplit);
            }
            w.block0 = (int32_t)blocks;
            blocks += items[i].tiles * w.nsplit;
            M.work[M.nwork++] = w;
        }
        if (blocks >= ((int64_t)1 << 31)) return fail(c, SAF_EINVAL, "launch too large");
        M.total_blocks = (int32_t)blocks;
        int64_t shared_blocks = 0;  // blocks [0, shared_blocks) share the CUs with the gather
        for (size_t i = i0; i < std::min(items.size(), i0 + saf::kMaxWork) && share_ms > 0.0; ++i) {
            const int64_t nb = items[i].tiles * items[i].w.nsplit;
            const double ms_per_block = 4.0 * g.d * QT * items[i].cost / kShareMfmaFlopPerMs;
            const int64_t take = std::min<int64_t>(nb, (int64_t)std::ceil(share_ms / ms_per_block));
            shared_blocks += take;
            share_ms = take < nb ? 0.0 : share_ms - (double)take * ms_per_block;
        }
        {
            Timed tm(c, s, "key_norms");
            e = saf::launch_key_norms(M, knorm, s);
        }
        if (e != hipSuccess) return hip_fail(c, e, "key norm kernel");
        {
            Timed tm(c, s, "shared_attention");
            M.block_base = 0;
            e = saf::launch_mfma_attention(M, (int32_t)shared_blocks, true, s);
            if (e == hipSuccess) {
                M.block_base = (int32_t)shared_blocks;
                e = saf::launch_mfma_attention(M, (int32_t)(blocks - shared_blocks), false, s);
            }
        }
        if (e != hipSuccess) return hip_fail(c, e, "matrix-core attention kernel");
        {
            Timed tm(c, s, "split_combine");
            e = saf::launch_split_combine(M, s);
        }
        if (e != hipSuccess) return hip_fail(c, e, "split combine kernel");
    }
    if (pi.nunion) {
        // both records exist once the side stream's gather is done
        if (forked) {
            e = hipEventRecord(c->ev_join, ss);
            if (e == hipSuccess) e = hipStreamWaitEvent(s, c->ev_join, 0);
            if (e != hipSuccess) return hip_fail(c, e, "joining the gather stream");
        }
        saf::UnionMerge U{};
        U.g = g;
        U.o = o;
        U.head_stride = lay.head_stride;
        U.token_stride = lay.token_stride;
        for (int h = 0; h < g.H; ++h) {
            if (plan[h].role != SAF_CORR_STRIDE) continue;
            U.head[U.nhead] = h;
            U.rec_tok[U.nhead] = union_tok[h];
            U.rec_patch[U.nhead] = union_patch[h];
            if (++U.nhead == saf::kMaxWork || h == g.H - 1) {
                Timed tm(c, s, "union_merge");
                e = saf::launch_union_merge(U, s);
                if (e != hipSuccess) return hip_fail(c, e, "union merge kernel");
                U.nhead = 0;
            }
        }
        if (U.nhead) {
            Timed tm(c, s, "union_merge");
            e = saf::launch_union_merge(U, s);
            if (e != hipSuccess) return hip_fail(c, e, "union merge kernel");
        }
    }
    return SAF_OK;
}

extern "C" {

saf_status_t saf_sparse_attention(saf_ctx_t *c, const saf_head_plan_t *plan, const void *q, const void *k,
                                  const void *v, void *o, saf_layout_t lay, const int32_t *vert_idx,
                                  int64_t vert_ld, void *ws, size_t ws_bytes, void *stream) {
    return sparse_attention(c, plan, q, k, v, o, lay, vert_idx, vert_ld, ws, ws_bytes, stream, false);
}

saf_status_t saf_dense_attention(saf_ctx_t *c, const void *q, const void *k, const void *v, void *o,
                                 saf_layout_t lay, void *ws, size_t ws_bytes, void *stream) {
    if (!c) return SAF_EINVAL;
    const saf::Geom &g = c->g;
    saf_status_t st;
    if ((st = check_tensors(c, q, k, v, o)) != SAF_OK) return st;
    if ((st = check_layout(c, lay)) != SAF_OK) return st;
    const int64_t nb = norm_bytes(g);
    const size_t need = nb ? (size_t)nb + 256 : 0;
    if (need > 0 && (!ws || ws_bytes < need)) return fail(c, SAF_EINVAL, "workspace %zu < %zu bytes", ws_bytes, need);
    if (ws && !aligned16(ws)) return fail(c, SAF_EINVAL, "workspace must be 16-byte aligned");
    float *knorm = nb ? (float *)(((uintptr_t)ws + 255) & ~(uintptr_t)255) : nullptr;
    hipStream_t s = as_stream(stream);
    if (g.dtype == saf::F32) {
        saf::ValuLaunch L{};
        L.g = g;
        L.q = q;
        L.k = k;
        L.v = v;
        L.o = o;
        L.head_stride = lay.head_stride;
        L.token_stride = lay.token_stride;
        for (int h0 = 0; h0 < g.H; h0 += saf::kMaxWork) {
            L.nwork = 0;
            for (int h = h0; h < std::min(g.H, h0 + saf::kMaxWork); ++h) {
                saf::HeadWork &w = L.work[L.nwork++];
                w = saf::HeadWork{};
                w.head = h;
                w.role = saf::DENSE;
                w.nsplit = 1;
            }
            hipError_t e;
            {
                Timed tm(c, s, "dense_attention");
                e = saf::launch_valu_attention(L, g.N, s);
            }
            if (e != hipSuccess) return hip_fail(c, e, "dense attention kernel (fp32)");
        }
        return SAF_OK;
    }
    saf::MfmaLaunch M{};
    M.g = g;
    M.q = q;
    M.k = k;
    M.v = v;
    M.o = o;
    M.head_stride = lay.head_stride;
    M.token_stride = lay.token_stride;
    M.knorm = knorm;
    const int64_t all_tiles = (g.N + QT - 1) / QT;
    for (int h0 = 0; h0 < g.H; h0 += saf::kMaxWork) {
        M.nwork = 0;
        int64_t blocks = 0;
        for (int h = h0; h < std::min(g.H, h0 + saf::kMaxWork); ++h) {
            saf::HeadWork w{};
            w.head = h;
            w.role = saf::DENSE;
            w.rows = saf::ROWS_ALL;
            w.nsplit = 1;
            w.block0 = (int32_t)blocks;
            blocks += all_tiles;
            M.work[M.nwork++] = w;
        }
        M.total_blocks = (int32_t)blocks;
        M.block_base = 0;
        hipError_t e;
        {
            Timed tm(c, s, "dense_attention");
            e = saf::launch_key_norms(M, knorm, s);
            if (e == hipSuccess) e = saf::launch_mfma_attention(M, M.total_blocks, false, s);
        }
        if (e != hipSuccess) return hip_fail(c, e, "dense attention kernel");
    }
    return SAF_OK;
}

saf_status_t saf_debug_fail_alloc(int32_t allowed) {
    g_alloc_allowance.store(allowed < 0 ? -1 : (int64_t)allowed);
    return SAF_OK;
}

saf_status_t saf_set_kernel_timing(saf_ctx_t *c, int32_t enable) {
    if (!c) return SAF_EINVAL;
    c->timing = enable != 0;
    return SAF_OK;
}

saf_status_t saf_read_kernel_timing(saf_ctx_t *c, int32_t max, const char **names, float *ms, int32_t *count) {
    if (!c || !count) return SAF_EINVAL;
    if (max > 0 && (!names || !ms)) return fail(c, SAF_EINVAL, "null names/ms with max > 0");
    saf_status_t st = SAF_OK;
    int32_t i = 0;
    for (auto &r : c->recs) {
        if (i < max) {
            float t = 0.f;
            hipError_t e = hipEventElapsedTime(&t, r.a, r.b);
            if (e != hipSuccess && st == SAF_OK) st = hip_fail(c, e, "hipEventElapsedTime");
            names[i] = r.name;
            ms[i] = t;
        }
        ++i;
        c->pool.push_back(r.a);
        c->pool.push_back(r.b);
    }
    c->recs.clear();
    *count = i;
    return st;
}

}  // extern "C"

// ------------------------------------------------ entry points in other files
saf_status_t saf_layer_internal(saf_ctx_t *c, const saf_head_plan_t *plan, const void *q, const void *k,
                                const void *v, void *o, saf_layout_t lay, const int32_t *vert_idx, int64_t vert_ld,
                                void *ws, size_t ws_bytes, void *stream, size_t ws_cap, size_t *ws_need) {
    if (!c) return SAF_EINVAL;
    PlanInfo pi;
    saf_status_t st = check_plan(c, plan, &pi);
    if (st != SAF_OK) return st;
    *ws_need = (size_t)((vert_idx ? 0 : pi.vert_ws) + pi.split_ws + pi.union_ws + pi.norm_ws + pi.pack_ws) + 256;
    if (*ws_need > ws_cap)
        return fail(c, SAF_EUNSUPPORTED, "this plan needs %zu bytes of workspace; the static scratch holds %zu",
                    *ws_need, ws_cap);
    if (!ws) return SAF_OK;  // size query
    // one stream and no timing events: the call creates nothing
    const bool timing = c->timing;
    c->timing = false;
    st = sparse_attention(c, plan, q, k, v, o, lay, vert_idx, vert_ld, ws, ws_bytes, stream, true);
    c->timing = timing;
    return st;
}

saf_status_t saf_fail_internal(saf_ctx_t *c, int32_t status, const char *msg) {
    return fail(c, (saf_status_t)status, "%s", msg);
}

// ------------------------------------------------------------ offline profiling
static saf_status_t head_nmse(saf_ctx_t *c, const void *o_full, const void *o_sparse, saf_layout_t lay,
                              double *sums, double *acc, int64_t acc_stride, double weight, void *stream) {
    saf_status_t st = check_layout(c, lay);
    if (st != SAF_OK) return st;
    if (!aligned16(o_full) || !aligned16(o_sparse)) return fail(c, SAF_EINVAL, "outputs must be 16-byte aligned");
    if (!c->nmse_part) {
        const size_t bytes = sizeof(double) * 2 * (size_t)c->g.H * saf::kNmseBlocks;
        if (dev_alloc((void **)&c->nmse_part, bytes) != hipSuccess)
            return fail(c, SAF_ENOMEM, "hipMalloc(%zu) for error partials failed", bytes);
    }
    hipError_t e;
    {
        Timed tm(c, as_stream(stream), "head_nmse");
        e = saf::launch_head_nmse(c->g, o_full, o_sparse, lay.head_stride, lay.token_stride, c->nmse_part, sums,
                                  acc, acc_stride, weight, as_stream(stream));
    }
    if (e != hipSuccess) return hip_fail(c, e, "error kernels");
    return SAF_OK;
}

saf_status_t saf_head_nmse(saf_ctx_t *c, const void *o_full, const void *o_sparse, saf_layout_t lay,
                           double *dev_out, void *stream) {
    if (!c) return SAF_EINVAL;
    if (!o_full || !o_sparse || !dev_out) return fail(c, SAF_EINVAL, "null pointer");
    return head_nmse(c, o_full, o_sparse, lay, dev_out, nullptr, 0, 0.0, stream);
}

saf_status_t saf_head_nmse_accumulate(saf_ctx_t *c, const void *o_full, const void *o_sparse, saf_layout_t lay,
                                      double weight, double *dev_err, int64_t err_stride, void *stream) {
    if (!c) return SAF_EINVAL;
    if (!o_full || !o_sparse || !dev_err) return fail(c, SAF_EINVAL, "null pointer");
    if (err_stride < 1) return fail(c, SAF_EINVAL, "err_stride %lld < 1", (long long)err_stride);
    if (!(weight >= 0.0) || weight > 1e300) return fail(c, SAF_EINVAL, "weight must be finite and >= 0");
    if (((uintptr_t)dev_err & 7u) != 0) return fail(c, SAF_EINVAL, "dev_err must be 8-byte aligned");
    return head_nmse(c, o_full, o_sparse, lay, nullptr, dev_err, err_stride, weight, stream);
}

saf_status_t saf_head_pairs(const saf_ctx_t *cc, const saf_head_plan_t *head, int32_t corr_kc, int64_t *pairs) {
    saf_ctx_t *c = const_cast<saf_ctx_t *>(cc);
    if (!c) return SAF_EINVAL;
    if (!head || !pairs) return fail(c, SAF_EINVAL, "null pointer");
    const saf::Geom &g = c->g;
    const int64_t N = g.N, S = g.S, ns = g.ns, P = g.P, T = g.T;
    switch (head->role) {
    case SAF_DENSE:
        *pairs = N * N;
        return SAF_OK;
    case SAF_POSITION: {
        if (head->anchor_frame < 0 || head->anchor_frame >= g.S)
            return fail(c, SAF_EINVAL, "anchor frame %d outside [0, S)", head->anchor_frame);
        // the anchor frame's rows see specials + their own frame; the others also the anchor
        *pairs = T * (ns * S + P) + (S - 1) * T * (ns * S + 2 * P);
        return SAF_OK;
    }
    case SAF_SCANNING: {
        const int64_t s = head->budget;
        if (s < 1) return fail(c, SAF_EINVAL, "stride %lld < 1", (long long)s);
        int64_t keys = (N + s - 1) / s;
        for (int64_t f = 0; f < S; ++f)
            for (int64_t t = 0; t < ns; ++t) keys += ((f * T + t) % s) ? 1 : 0;
        *pairs = N * keys;
        return SAF_OK;
    }
    case SAF_VERTICAL:
        if (head->budget < 1) return fail(c, SAF_EINVAL, "K %d < 1", head->budget);
        *pairs = N * std::min<int64_t>(head->budget, N);
        return SAF_OK;
    case SAF_BROADCAST: {
        const int64_t r = head->budget, gw = head->anchor_frame > 0 ? head->anchor_frame : P;
        if (r < 0) return fail(c, SAF_EINVAL, "radius %lld < 0", (long long)r);
        if (head->anchor_frame < 0 || P % gw != 0)
            return fail(c, SAF_EINVAL, "grid width %d does not divide P", head->anchor_frame);
        // a patch row sees the specials and, in every frame, its window;
        // special rows attend to every key
        const int64_t gh = P / gw;
        int64_t win = 0;
        for (int64_t p = 0; p < P; ++p) {
            const int64_t y = p / gw, x = p % gw;
            win += (std::min(gh - 1, y + r) - std::max<int64_t>(0, y - r) + 1) *
                   (std::min(gw - 1, x + r) - std::max<int64_t>(0, x - r) + 1);
        }
        *pairs = S * (P * ns * S + S * win) + ns * S * N;
        return SAF_OK;
    }
    case SAF_CORRESPONDENCE: {
        const int64_t kc = corr_kc > 0 ? corr_kc : c->corr_k;
        if (kc < 1) return fail(c, SAF_ESTATE, "no index row length given and no cached index");
        // patch rows gather kc keys; special rows attend to every key
        *pairs = S * P * std::min<int64_t>(kc, (S - 1) * P) + ns * S * N;
        return SAF_OK;
    }
    default:
        return fail(c, SAF_EINVAL, "bad role %d", head->role);
    }
}

saf_status_t saf_head_cost(const saf_ctx_t *cc, const saf_head_plan_t *head, int32_t corr_kc, double *flops) {
    if (!cc) return SAF_EINVAL;
    if (!flops) return fail(const_cast<saf_ctx_t *>(cc), SAF_EINVAL, "null pointer");
    int64_t pairs = 0;
    const saf_status_t st = saf_head_pairs(cc, head, corr_kc, &pairs);
    if (st != SAF_OK) return st;
    *flops = 4.0 * (double)cc->g.d * (double)pairs;
    return SAF_OK;
}

int32_t saf_profile_select(const double *errors, const double *costs, int32_t n) {
    if (!errors || !costs || n < 1) return -1;
    int32_t best = 0;
    for (int32_t i = 1; i < n; ++i)
        if (costs[i] <= costs[0] && errors[i] < errors[best]) best = i;
    return best;
}

int32_t saf_baseline_stride(double sigma) {
    if (!(sigma >= 0.0 && sigma < 1.0)) return -1;
    int32_t s = 1;
    while ((1.0 / s) > (1.0 - sigma) + 1e-12) ++s;  // smallest stride keeping <= 1 - sigma of the keys
    return s;
}
