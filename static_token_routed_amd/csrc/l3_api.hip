// Host side of the C ABI declared in include/l3.h: plan validation, workspace
// layout, launch sequencing, the decode-time prefetch, and stage timing.
#include <algorithm>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>
#include <vector>

#include "l3_internal.h"

using namespace l3;

// A second stream for work that depends only on the weights (the factored W_mix's
// F and G): forked from the caller's stream at the start of a forward and joined
// before the first kernel that reads it, so it runs beside the route.  The mutex
// keeps one forward's record / wait sequence whole when several host threads share
// a plan.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex mu;
    ~SideStream() {
        if (join) (void)hipEventDestroy(join);
        if (fork) (void)hipEventDestroy(fork);
        if (s) (void)hipStreamDestroy(s);
    }
};

struct l3_plan_s {
    int64_t vocab = 0, v = 0;
    int32_t k = 0, max_d = 0;
    Dims dims{};
    int64_t *d_off = nullptr;   // device CSR offsets (vocab + 1)
    std::vector<int64_t> h_off; // host copy, used by the prefetch path
    bool owns_off = true;
    SideStream *side = nullptr; // bf16 plans (owned unless owns_off is false: a view)
};

struct l3_staging_s {
    l3_plan_t plan = nullptr;
    int64_t max_rows = 0, max_tokens = 0;
    void *d_K = nullptr, *d_V = nullptr;
    // one step's index arrays, packed as [coff (m+1) | src (m) | ids (n)]: the compact
    // CSR over the step's distinct IDs, each ID's first table row, and the step's IDs
    // remapped to [0, m); built on the host in h_meta (pinned), copied to d_meta
    char *d_meta = nullptr, *h_meta = nullptr;
    int64_t *d_off = nullptr;  // into d_meta, for the current step
    int32_t *d_ids = nullptr;
    hipEvent_t small_done = nullptr;  // last copy out of h_meta
    bool small_pending = false;
    // recorded after each l3_forward_staged on its stream: the next prefetch's side
    // stream waits for it before it overwrites the staged rows and index block
    hipEvent_t consumed = nullptr;
    bool consumed_pending = false;
    int64_t n = 0, m = 0, rows = 0, max_d = 0;
    // device-resident cache of hot IDs' rows (l3_staging_set_cache)
    void *c_K = nullptr, *c_V = nullptr;
    std::vector<int64_t> cache_row;  // per ID: first cache row, or -1
    int64_t cached_rows = 0;         // rows of the last prefetch served by the cache
};

namespace {

size_t esize(int dtype) { return dtype == L3_BF16 ? 2 : 4; }

// ---- stage timing (benchmark aid)
// forward: 0 route, 1 gather (matrix cores), 2 gather (wavefront), 3 W_up, 4 W_mix
// preparation, 5 W_mix; backward: 6 forward recompute of h and its statistics,
// 7 dense products and LayerNorm backward, 8 attention backward, 9 key / value gradients
constexpr int kProfStages = 10;
struct Prof {
    bool on = false;
    struct Pair { hipEvent_t a, b; int stage; };
    std::vector<Pair> pending;
    std::vector<hipEvent_t> pool;
    double ms[kProfStages] = {};
    int64_t launches[kProfStages] = {};
} g_prof;

hipEvent_t prof_event() {
    if (!g_prof.pool.empty()) {
        hipEvent_t e = g_prof.pool.back();
        g_prof.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

struct StageTimer {
    hipStream_t s;
    hipEvent_t a = nullptr;
    int stage;
    StageTimer(int st, hipStream_t str) : s(str), stage(st) {
        if (g_prof.on && (a = prof_event())) (void)hipEventRecord(a, s);
    }
    ~StageTimer() {
        if (!a) return;
        hipEvent_t b = prof_event();
        if (!b) return;
        (void)hipEventRecord(b, s);
        g_prof.pending.push_back({a, b, stage});
    }
};

int validate_dims(const l3_dims_t *d) {
    if (!d) return L3_ERR_INVALID_ARG;
    if (d->d_in <= 0 || d->d_emb <= 0 || d->d_up <= 0 || d->d_out <= 0) return L3_ERR_INVALID_ARG;
    if (d->dtype != L3_F32 && d->dtype != L3_BF16) return L3_ERR_INVALID_ARG;
    if (!(d->ln_eps >= 0.f)) return L3_ERR_INVALID_ARG;
    if (d->dtype == L3_BF16) {
        if (d->d_in % 64 || d->d_up % 64 || d->d_out % 64) return L3_ERR_UNSUPPORTED;
        if (d->d_in > 4096) return L3_ERR_UNSUPPORTED;
        // d_emb 1024 and 2048 for tied tables only (d_in = d_emb; the forward then
        // requires W_V to be the W_K buffer)
        const bool tied_wide = (d->d_emb == 1024 || d->d_emb == 2048) && d->d_in == d->d_emb;
        if (d->d_emb != 64 && d->d_emb != 128 && d->d_emb != 256 && d->d_emb != 512 && !tied_wide)
            return L3_ERR_UNSUPPORTED;
    }
    return L3_OK;
}

// Device arrays are read and written with 16-byte vector accesses.
bool aligned16(std::initializer_list<const void *> ps) {
    for (const void *q : ps)
        if (reinterpret_cast<uintptr_t>(q) & 15) return false;
    return true;
}

int check_offsets(const int64_t *off, int64_t vocab, int64_t v, int32_t k, int32_t *max_d) {
    if (off[0] != 0) return L3_ERR_BAD_OFFSETS;
    int64_t mx = 0;
    for (int64_t t = 0; t < vocab; ++t) {
        const int64_t d = off[t + 1] - off[t];
        if (d < 1 || d > k) return L3_ERR_BAD_OFFSETS;
        mx = std::max(mx, d);
    }
    if (off[vocab] != v) return L3_ERR_BAD_OFFSETS;
    *max_d = (int32_t)mx;
    return L3_OK;
}

// Route and gather-attention over any CSR/table view: fills the route buffers, the
// work lists and o (L.o) in the workspace.
int route_attend(const l3_plan_s &P, const void *x, const int32_t *ids, int64_t n, const void *WK,
                 const void *WV, void *ws, const WsLayout &L, RouteBufs &b, hipStream_t s) {
    const Dims &D = P.dims;
    b.hdr = ws_ptr<int32_t>(ws, L.hdr);
    b.keys_a = ws_ptr<int32_t>(ws, L.keys_a);
    b.vals_a = ws_ptr<int32_t>(ws, L.vals_a);
    b.keys_b = ws_ptr<int32_t>(ws, L.keys_b);
    b.vals_b = ws_ptr<int32_t>(ws, L.vals_b);
    b.rank = ws_ptr<int32_t>(ws, L.rank);
    b.hist = ws_ptr<int32_t>(ws, L.hist);
    b.tile_cnt = ws_ptr<int32_t>(ws, L.tile_cnt);
    b.inv_perm = ws_ptr<int32_t>(ws, L.inv_perm);
    b.uniq = ws_ptr<int32_t>(ws, L.uniq);
    b.counts = ws_ptr<int32_t>(ws, L.counts);
    b.seg_start = ws_ptr<int32_t>(ws, L.seg_start);
    int4 *light = ws_ptr<int4>(ws, L.light);
    int4 *light_long = ws_ptr<int4>(ws, L.light_long);
    int2 *heavy = ws_ptr<int2>(ws, L.heavy);
    int2 *dense = ws_ptr<int2>(ws, L.dense);
    void *o = ws_ptr<char>(ws, L.o);

    if (L.slots > 0) {
        // small batch: split-row gather-attention (no light / heavy / dense lists)
        const SplitLists sl{ws_ptr<int4>(ws, L.sitems), ws_ptr<int4>(ws, L.blkinfo),
                            ws_ptr<int32_t>(ws, L.blk_of)};
        {
            StageTimer tm(0, s);
            L3_HIP_TRY(launch_route_small_split(ids, n, P.vocab, P.d_off, split_rows(D.d_in),
                                                split_tokens(D.d_in), b, sl, s));
        }
        SplitArgs sa{};
        sa.x = x; sa.WK = WK; sa.WV = WV; sa.off = P.d_off;
        sa.uniq = b.uniq; sa.perm = b.perm; sa.hdr = b.hdr; sa.blk_of = sl.blk_of;
        sa.items = sl.items; sa.blkinfo = sl.blkinfo;
        sa.n = n; sa.d_in = D.d_in; sa.d_emb = D.d_emb;
        sa.pml = ws_ptr<float2>(ws, L.pml); sa.po = ws_ptr<float>(ws, L.po); sa.o = o;
        StageTimer tm(2, s);
        L3_HIP_TRY(launch_attn_split(sa, s));
        return L3_OK;
    }
    const int light_tok = attn_light_tokens(D.d_in, D.d_emb, D.dtype);
    const int heavy_min = attn_heavy_min_tokens(D.d_in, D.d_emb, D.dtype, P.max_d);
    const int dense_min = attn_dense_min_tokens(D.d_in, D.d_emb, D.dtype);
    {
        StageTimer tm(0, s);
        if (n <= kRouteSmallMax) {
            L3_HIP_TRY(launch_route_small(ids, n, P.vocab, P.d_off, heavy_min, dense_min, light_tok, b,
                                          light, heavy, dense, s));
        } else {
            // (clears the header too)
            L3_HIP_TRY(launch_route(ids, n, P.vocab, b, L.ntiles, P.d_off, heavy_min, dense_min, light_tok,
                                    light, heavy, dense, D.dtype == L3_BF16 ? light_long : nullptr, s));
        }
    }
    {
        AttnArgs a{};
        a.x = x; a.WK = WK; a.WV = WV; a.off = P.d_off;
        a.uniq = b.uniq; a.seg_start = b.seg_start; a.perm = b.perm; a.hdr = b.hdr;
        a.queue = b.hdr + HDR_QUEUE;
        a.light = light; a.light_long = light_long; a.heavy = heavy; a.dense = dense;
        a.n = n; a.d_in = D.d_in; a.d_emb = D.d_emb; a.vocab = P.vocab;
        a.o = o; a.scores = ws_ptr<float>(ws, L.scores); a.max_d = P.max_d;
        if (heavy_min != INT32_MAX) {
            StageTimer tm(1, s);
            L3_HIP_TRY(launch_attn_heavy(a, s));
        }
        {
            StageTimer tm(2, s);
            L3_HIP_TRY(launch_attn_light(a, D.dtype, s));
        }
    }
    return L3_OK;
}

// One forward over any CSR/table view (the full tables, or a staging's compact copy).
int forward_impl(const l3_plan_s &P, const void *x, const int32_t *ids, int64_t n, const void *WK,
                 const void *WV, const void *W_up, const float *gamma, const float *beta,
                 const void *W_mix, void *out, void *ws, size_t ws_bytes, hipStream_t s) {
    const Dims &D = P.dims;
    if (tied_only(D) && WV != WK) return L3_ERR_UNSUPPORTED;
    const WsLayout L = ws_layout(D, n, P.max_d);
    if (ws_bytes < L.total) return L3_ERR_CAPACITY;
    const bool factored = D.dtype == L3_BF16 && n > kSkinnyMaxM;
    void *fold = ws_ptr<char>(ws, L.fold);
    void *factor = ws_ptr<char>(ws, L.factor);
    // F and G (weights only) on the side stream, beside the route and gather-attention
    // (their workspace regions are not touched by those); the caller's stream waits for
    // them before the first kernel that reads them, or before returning on an error
    struct Join {
        SideStream *side = nullptr;
        hipStream_t s = nullptr;
        std::unique_lock<std::mutex> lock;
        hipError_t now() {
            if (!side) return hipSuccess;
            SideStream *t = side;
            side = nullptr;
            hipError_t e = hipEventRecord(t->join, t->s);
            if (e == hipSuccess) e = hipStreamWaitEvent(s, t->join, 0);
            lock.unlock();
            return e;
        }
        ~Join() { (void)now(); }
    } join;
    if (factored) {
        hipStream_t ps = s;
        if (P.side) {
            join.lock = std::unique_lock<std::mutex>(P.side->mu);
            L3_HIP_TRY(hipEventRecord(P.side->fork, s));
            L3_HIP_TRY(hipStreamWaitEvent(P.side->s, P.side->fork, 0));
            join.side = P.side;
            join.s = s;
            ps = P.side->s;
        }
        StageTimer tm(4, ps);
        L3_HIP_TRY(launch_mix_factor((const uint16_t *)W_up, (const uint16_t *)W_mix, gamma, beta, fold, factor,
                                     D.d_emb, D.d_up, D.d_in, D.d_out, ps));
    }
    RouteBufs b{};
    const int rc = route_attend(P, x, ids, n, WK, WV, ws, L, b, s);
    if (rc != L3_OK) return rc;
    L3_HIP_TRY(join.now());
    void *o = ws_ptr<char>(ws, L.o);
    void *h = ws_ptr<char>(ws, L.h);
    float *lnp = ws_ptr<float>(ws, L.lnp);

    if (D.dtype == L3_BF16 && n <= kSkinnyMaxM) {
        float *part = ws_ptr<float>(ws, L.part);
        {
            StageTimer tm(3, s);
            L3_HIP_TRY(launch_gemm_skinny_bf16((const uint16_t *)o, (const uint16_t *)W_up, (uint16_t *)h,
                                               n, D.d_up, D.d_emb, lnp, part, s));
        }
        {
            StageTimer tm(5, s);
            L3_HIP_TRY(launch_gemm_mix_skinny_bf16((const uint16_t *)h, (const uint16_t *)x, lnp, gamma,
                                                   beta, D.eps, (const uint16_t *)W_mix, (uint16_t *)out,
                                                   n, D.d_up, D.d_in, D.d_out, part, s));
        }
    } else if (D.dtype == L3_BF16) {
        // W_mix factored through W_up (gemm.hip): h is never formed; LayerNorm's variance
        // comes from o^T G o (its per-row shares in lnp, turned into rstd by the W_mix GEMM)
        {
            StageTimer tm(3, s);
            L3_HIP_TRY(launch_ln_quad_stats_bf16((const uint16_t *)o, factor, n, D.d_emb, D.d_up, D.d_out,
                                                 lnp, s));
        }
        {
            StageTimer tm(5, s);
            L3_HIP_TRY(launch_gemm_mix_factored_bf16((const uint16_t *)o, (const uint16_t *)x, lnp, D.eps,
                                                     (const uint16_t *)W_mix, (uint16_t *)out, fold, factor,
                                                     n, D.d_emb, D.d_up, D.d_in, D.d_out, s));
        }
    } else {
        {
            StageTimer tm(3, s);
            L3_HIP_TRY(launch_gemm_f32((const float *)o, (const float *)W_up, (float *)h, n, D.d_up,
                                       D.d_emb, s));
        }
        {
            StageTimer tm(5, s);
            L3_HIP_TRY(launch_gemm_mix_f32((const float *)h, (const float *)x, lnp, gamma, beta, D.eps,
                                           (const float *)W_mix, (float *)out, n, D.d_up, D.d_in,
                                           D.d_out, s));
        }
    }
    return L3_OK;
}


// Backward workspace: the forward's regions, then those of the backward pass.
struct BwdLayout {
    WsLayout f;
    size_t wmt, dy, dh, y, doutT, zT, dhT, oT, wupT, dov, dob, tstat, P, dS, part, kv, splitk, total;
    int kv_cap;
    int64_t n_pad;
};

BwdLayout bwd_layout(const Dims &d, int64_t n_max, int32_t max_d) {
    BwdLayout B{};
    B.f = ws_layout(d, n_max, max_d);
    const int64_t n = std::max<int64_t>(n_max, 1);
    B.n_pad = (n + 63) / 64 * 64;
    const size_t es = esize(d.dtype);
    const int64_t Z = d.d_up + d.d_in;
    size_t off = B.f.total;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) & ~(size_t)255;
        return o;
    };
    B.wmt = take((size_t)Z * d.d_out * es);
    B.dy = take((size_t)n * d.d_up * 4);
    B.dh = take((size_t)n * d.d_up * es);
    B.y = take((size_t)n * d.d_up * es);
    B.doutT = take((size_t)d.d_out * B.n_pad * es);
    B.zT = take((size_t)Z * B.n_pad * es);
    B.dhT = take((size_t)d.d_up * B.n_pad * es);
    B.oT = take((size_t)d.d_emb * B.n_pad * es);
    B.wupT = take((size_t)d.d_emb * d.d_up * es);
    B.dov = take((size_t)n * d.d_emb * 4);
    B.dob = take(d.dtype == L3_BF16 ? (size_t)n * d.d_emb * 2 : 0);
    B.tstat = take(d.dtype == L3_BF16 ? (size_t)n * 16 : 0);
    B.P = take((size_t)n * std::max(max_d, 1) * 4);
    B.dS = take((size_t)n * std::max(max_d, 1) * 4);
    B.part = take((size_t)ln_param_chunks(n) * d.d_up * 8);
    // distinct rows of a batch: at most n tokens' worth of max_d rows
    B.kv_cap = kv_item_capacity(n, (int64_t)n * std::max(max_d, 1), d.d_in, d.d_emb, d.dtype);
    B.kv = take((size_t)B.kv_cap * 8);
    // split-K slabs of the two parameter-gradient products (K = tokens), bf16 plans
    B.splitk = take(d.dtype == L3_BF16 ? std::max(gemm_f32_split_bytes(d.d_out, Z, B.n_pad),
                                                   gemm_f32_split_bytes(d.d_up, d.d_emb, B.n_pad))
                                       : 0);
    B.total = off;
    return B;
}

// C = A B^T (A: M x K, B: N x K), fp32 output written or added, by dtype.
hipError_t gemm_f32out(int dtype, const void *A, const void *B, float *C, int64_t M, int64_t N,
                       int64_t K, bool acc, hipStream_t s) {
    if (dtype == L3_BF16)
        return launch_gemm_bf16_f32out((const uint16_t *)A, (const uint16_t *)B, C, M, N, K, acc, s);
    return launch_gemm_f32_acc((const float *)A, (const float *)B, C, M, N, K, acc, s);
}

int backward_impl(const l3_plan_s &P, const void *x, const int32_t *ids, int64_t n, const void *WK,
                  const void *WV, const void *W_up, const float *gamma, const float *beta,
                  const void *W_mix, const void *dout, float *dx, float *dWK, float *dWV, float *dWup,
                  float *dgamma, float *dbeta, float *dWmix, void *ws, size_t ws_bytes,
                  hipStream_t s) {
    const Dims &D = P.dims;
    const BwdLayout B = bwd_layout(D, n, P.max_d);
    if (ws_bytes < B.total) return L3_ERR_CAPACITY;
    const WsLayout &L = B.f;
    const int dt = D.dtype;
    const size_t es = esize(dt);
    const int64_t Z = D.d_up + D.d_in, np = B.n_pad;
    // forward again up to LayerNorm's statistics: o, h, (mean, rstd)
    RouteBufs b{};
    int rc = route_attend(P, x, ids, n, WK, WV, ws, L, b, s);
    if (rc != L3_OK) return rc;
    void *o = ws_ptr<char>(ws, L.o), *h = ws_ptr<char>(ws, L.h);
    float *lnp = ws_ptr<float>(ws, L.lnp), *stats = ws_ptr<float>(ws, L.stats);
    {
    StageTimer tm(6, s);
    if (dt == L3_BF16) {
        if (n <= kSkinnyMaxM)
            L3_HIP_TRY(launch_gemm_skinny_bf16((const uint16_t *)o, (const uint16_t *)W_up, (uint16_t *)h,
                                               n, D.d_up, D.d_emb, lnp, ws_ptr<float>(ws, L.part), s));
        else
            L3_HIP_TRY(launch_gemm_bf16((const uint16_t *)o, (const uint16_t *)W_up, (uint16_t *)h, n,
                                        D.d_up, D.d_emb, lnp, s));
        L3_HIP_TRY(launch_ln_finalize(lnp, n, D.d_up, D.eps, stats, s));
    } else {
        L3_HIP_TRY(launch_gemm_f32((const float *)o, (const float *)W_up, (float *)h, n, D.d_up, D.d_emb,
                                   s));
        L3_HIP_TRY(launch_ln_stats_f32((const float *)h, n, D.d_up, D.eps, stats, s));
    }
    }
    char *wmt = ws_ptr<char>(ws, B.wmt);
    float *dy = ws_ptr<float>(ws, B.dy), *dov = ws_ptr<float>(ws, B.dov);
    void *dh = ws_ptr<char>(ws, B.dh), *y = ws_ptr<char>(ws, B.y);
    char *doutT = ws_ptr<char>(ws, B.doutT), *zT = ws_ptr<char>(ws, B.zT);
    void *dhT = ws_ptr<char>(ws, B.dhT), *oT = ws_ptr<char>(ws, B.oT), *wupT = ws_ptr<char>(ws, B.wupT);
    {
    StageTimer tm(7, s);
    // dy = W1^T dout, dx = W2^T dout  (W_mix^T rows [0, d_up) and [d_up, Z))
    L3_HIP_TRY(launch_transpose(W_mix, Z, D.d_out, Z, wmt, D.d_out, D.d_out, dt, s));
    L3_HIP_TRY(gemm_f32out(dt, dout, wmt, dy, n, D.d_up, D.d_out, false, s));
    L3_HIP_TRY(gemm_f32out(dt, dout, wmt + (size_t)D.d_up * D.d_out * es, dx, n, D.d_in, D.d_out, false,
                           s));
    // LayerNorm: dh, y, dgamma, dbeta
    L3_HIP_TRY(launch_ln_bwd(h, stats, gamma, beta, dy, n, D.d_up, dh, y, ws_ptr<float2>(ws, B.part),
                             dgamma, dbeta, dt, s));
    // dW_mix += dout^T [y ; x]   (K = tokens, zero-padded to a multiple of 64)
    L3_HIP_TRY(launch_transpose(dout, D.d_out, n, D.d_out, doutT, np, np, dt, s));
    L3_HIP_TRY(launch_transpose(y, D.d_up, n, D.d_up, zT, np, np, dt, s));
    L3_HIP_TRY(launch_transpose(x, D.d_in, n, D.d_in, zT + (size_t)D.d_up * np * es, np, np, dt, s));
    float *splitk = ws_ptr<float>(ws, B.splitk);
    if (dt == L3_BF16)
        L3_HIP_TRY(launch_gemm_bf16_f32acc_split((const uint16_t *)doutT, (const uint16_t *)zT, dWmix,
                                                 D.d_out, Z, np, splitk, s));
    else
        L3_HIP_TRY(gemm_f32out(dt, doutT, zT, dWmix, D.d_out, Z, np, true, s));
    // dW_up += dh o^T, do = W_up^T dh
    L3_HIP_TRY(launch_transpose(dh, D.d_up, n, D.d_up, dhT, np, np, dt, s));
    L3_HIP_TRY(launch_transpose(o, D.d_emb, n, D.d_emb, oT, np, np, dt, s));
    if (dt == L3_BF16)
        L3_HIP_TRY(launch_gemm_bf16_f32acc_split((const uint16_t *)dhT, (const uint16_t *)oT, dWup, D.d_up,
                                                 D.d_emb, np, splitk, s));
    else
        L3_HIP_TRY(gemm_f32out(dt, dhT, oT, dWup, D.d_up, D.d_emb, np, true, s));
    L3_HIP_TRY(launch_transpose(W_up, D.d_emb, D.d_up, D.d_emb, wupT, D.d_up, D.d_up, dt, s));
    L3_HIP_TRY(gemm_f32out(dt, dh, wupT, dov, n, D.d_emb, D.d_up, false, s));
    }
    // attention: items of one or two tokens over every block, then the key / value gradients
    int4 *items = ws_ptr<int4>(ws, L.light);
    L3_HIP_TRY(launch_zero_i32(b.hdr + HDR_NLIGHT, 4, s));  // NLIGHT, NHEAVY, NDENSE, NKV
    L3_HIP_TRY(launch_worklist(b, n, P.d_off, P.vocab, INT32_MAX, INT32_MAX,
                               attn_bwd_tokens(D.d_in, D.d_emb, dt), items,
                               ws_ptr<int2>(ws, L.heavy), ws_ptr<int2>(ws, L.dense), s));
    BwdArgs a{};
    a.x = x; a.WK = WK; a.WV = WV; a.off = P.d_off;
    a.uniq = b.uniq; a.seg_start = b.seg_start; a.perm = b.perm; a.hdr = b.hdr;
    a.items = items; a.dov = dov; a.o = o;
    a.d_in = D.d_in; a.d_emb = D.d_emb; a.vocab = P.vocab; a.max_d = P.max_d;
    a.dx = dx; a.P = ws_ptr<float>(ws, B.P); a.dS = ws_ptr<float>(ws, B.dS);
    a.dWK = dWK; a.dWV = dWV;
    a.kv_items = ws_ptr<int2>(ws, B.kv); a.kv_cap = B.kv_cap;
    a.n = n; a.dob = dt == L3_BF16 ? ws_ptr<uint16_t>(ws, B.dob) : nullptr;
    a.tstat = dt == L3_BF16 ? ws_ptr<float4>(ws, B.tstat) : nullptr;
    {
        StageTimer tm(8, s);
        L3_HIP_TRY(launch_attn_bwd(a, dt, 0, s));
    }
    {
        StageTimer tm(9, s);
        L3_HIP_TRY(launch_attn_bwd(a, dt, 1, s));
    }
    return L3_OK;
}

// The largest layout over every batch size 1 .. n_max.  Every region grows with n,
// except the split-row partials of small bf16 batches: they exist only while
// n * ceil(max_d / split_rows) stays within kSplitMaxSlots (and n <= kSplitMaxN),
// so the layout grows with n up to the last size that has them, drops when they
// switch off, and grows again.  The maximum is therefore at n_max or at that last
// size.
template <class Total>
size_t max_layout_bytes(const Dims &d, int64_t n_max, int32_t max_d, Total total) {
    size_t need = total(d, n_max, max_d);
    const int64_t per = (std::max<int32_t>(max_d, 1) + split_rows(d.d_in) - 1) / split_rows(d.d_in);
    const int64_t n_split = std::min<int64_t>({n_max, kSplitMaxN, kSplitMaxSlots / per});
    if (n_split >= 1) need = std::max(need, total(d, n_split, max_d));
    return need;
}

size_t ws_total(const Dims &d, int64_t n, int32_t max_d) { return ws_layout(d, n, max_d).total; }
size_t bwd_total(const Dims &d, int64_t n, int32_t max_d) { return bwd_layout(d, n, max_d).total; }

}  // namespace

namespace l3 {

WsLayout ws_layout(const Dims &d, int64_t n_max, int32_t max_d) {
    WsLayout L{};
    const int64_t n = std::max<int64_t>(n_max, 1);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) & ~(size_t)255;
        return o;
    };
    L.ntiles = (n + kSortTile - 1) / kSortTile;
    L.hdr = take(HDR_WORDS * 4);
    L.keys_a = take(n * 4);
    L.vals_a = take(n * 4);
    L.keys_b = take(n * 4);
    L.vals_b = take(n * 4);
    L.rank = take(n * 4);
    L.hist = take((size_t)kRadix * (L.ntiles + 1) * 4);  // + the digit totals (k_hist_scan)
    L.tile_cnt = take(L.ntiles * 2 * 4);  // head counts, then first head positions
    L.inv_perm = take(n * 4);
    L.uniq = take(n * 4);
    L.counts = take(n * 4);
    L.seg_start = take((n + 1) * 4);
    L.light = take(n * 16);
    L.light_long = take(d.dtype == L3_BF16 ? n * 16 : 0);
    L.heavy = take(n * 8);
    L.dense = take(n * 8);
    L.scores = take(d.dtype == L3_F32 ? (size_t)n * std::max(max_d, 1) * 4 : 0);
    const size_t es = esize(d.dtype);
    L.o = take((size_t)n * d.d_emb * es);
    L.h = take((size_t)n * d.d_up * es);
    const int64_t np = (d.d_up + kLnPart - 1) / kLnPart;
    L.lnp = take((size_t)n * std::max<int64_t>(std::max<int64_t>(np, 1) * 2, ln_quad_parts(d.d_emb)) * 4);
    L.stats = take((size_t)n * 2 * 4);
    L.fold = take(d.dtype == L3_BF16 ? mix_fold_bytes(d.d_up, d.d_out) : 0);
    L.factor = take(d.dtype == L3_BF16 && n > kSkinnyMaxM ? mix_factor_bytes(d.d_emb, d.d_up, d.d_out) : 0);
    const int64_t ns = std::min<int64_t>(n, kSkinnyMaxM);
    // (sized at min(n, kSkinnyMaxM) above kSkinnyMaxM tokens too, so the size never falls
    // as n grows)
    const size_t skinny = std::max(skinny_part_bytes(ns, d.d_up, d.d_emb),
                                   skinny_part_bytes(ns, d.d_out, d.d_up + d.d_in));
    L.part = take(d.dtype != L3_BF16 ? 0 : skinny);
    L.slots = split_slots(d, n, max_d);
    L.sitems = take((size_t)L.slots * 16);
    L.blkinfo = take(L.slots ? (size_t)n * 16 : 0);
    L.blk_of = take(L.slots ? (size_t)n * 4 : 0);
    L.pml = take((size_t)L.slots * 8);
    L.po = take((size_t)L.slots * d.d_emb * 4);
    L.total = off;
    return L;
}

}  // namespace l3

extern "C" {

const char *l3_strerror(int status) {
    switch (status) {
        case L3_OK: return "ok";
        case L3_ERR_INVALID_ARG: return "invalid argument";
        case L3_ERR_BAD_OFFSETS: return "bad offsets: need off[0]=0, 1<=d_t<=k, off[vocab]=v";
        case L3_ERR_TOKEN_RANGE: return "token id outside [0, vocab)";
        case L3_ERR_UNSUPPORTED: return "unsupported dimensions";
        case L3_ERR_CAPACITY: return "capacity exceeded (workspace or staging too small)";
        case L3_ERR_NOMEM: return "out of memory";
        case L3_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int l3_plan(const int64_t *offsets, int64_t vocab, int64_t v, int32_t k, const l3_dims_t *dims,
            l3_plan_t *plan) {
    if (!plan) return L3_ERR_INVALID_ARG;
    *plan = nullptr;
    if (!offsets || vocab <= 0 || v <= 0 || k < 1) return L3_ERR_INVALID_ARG;
    if (v >= (1ll << 31) || vocab >= (1ll << 31) - 1) return L3_ERR_UNSUPPORTED;  // 32-bit row and ID indices
    if (vocab >= (1ll << 30) || v >= (1ll << 31)) return L3_ERR_UNSUPPORTED;
    int rc = validate_dims(dims);
    if (rc) return rc;
    int32_t max_d = 0;
    rc = check_offsets(offsets, vocab, v, k, &max_d);
    if (rc) return rc;
    l3_plan_s *p = new (std::nothrow) l3_plan_s();
    if (!p) return L3_ERR_NOMEM;
    p->vocab = vocab;
    p->v = v;
    p->k = k;
    p->max_d = max_d;
    p->dims = Dims{dims->d_in, dims->d_emb, dims->d_up, dims->d_out, dims->dtype, dims->ln_eps};
    try {
        p->h_off.assign(offsets, offsets + vocab + 1);
    } catch (...) {
        delete p;
        return L3_ERR_NOMEM;
    }
    const size_t bytes = (size_t)(vocab + 1) * sizeof(int64_t);
    if (hipMalloc(&p->d_off, bytes) != hipSuccess) {
        delete p;
        return L3_ERR_HIP;
    }
    if (hipMemcpy(p->d_off, offsets, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(p->d_off);
        delete p;
        return L3_ERR_HIP;
    }
    if (p->dims.dtype == L3_BF16) {
        // the side stream of the factored W_mix (default priority, not blocking on the
        // legacy null stream: every dependency is an explicit event wait)
        p->side = new (std::nothrow) SideStream();
        if (!p->side || hipStreamCreateWithFlags(&p->side->s, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&p->side->fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&p->side->join, hipEventDisableTiming) != hipSuccess) {
            delete p->side;
            (void)hipFree(p->d_off);
            delete p;
            return L3_ERR_HIP;
        }
    }
    *plan = p;
    return L3_OK;
}

int l3_plan_destroy(l3_plan_t p) {
    if (!p) return L3_OK;
    if (p->owns_off && p->d_off) (void)hipFree(p->d_off);
    if (p->owns_off) delete p->side;
    delete p;
    return L3_OK;
}

int l3_plan_info(l3_plan_t p, int64_t *vocab, int64_t *v, int32_t *k, int32_t *max_d) {
    if (!p) return L3_ERR_INVALID_ARG;
    if (vocab) *vocab = p->vocab;
    if (v) *v = p->v;
    if (k) *k = p->k;
    if (max_d) *max_d = p->max_d;
    return L3_OK;
}

int l3_worklist_rule(l3_plan_t p, int32_t *min_tokens, int32_t *min_rows) {
    if (!p) return L3_ERR_INVALID_ARG;
    const int hm = attn_heavy_min_tokens(p->dims.d_in, p->dims.d_emb, p->dims.dtype, p->max_d);
    if (min_tokens) *min_tokens = hm;
    if (min_rows) *min_rows = hm == INT32_MAX ? INT32_MAX : kHeavyMinRows;
    return L3_OK;
}

size_t l3_workspace_size(l3_plan_t p, int64_t n_max) {
    if (!p || n_max < 0) return 0;
    return max_layout_bytes(p->dims, n_max, p->max_d, ws_total);
}

size_t l3_workspace_size_dims(const l3_dims_t *dims, int32_t max_d, int64_t n_max) {
    if (validate_dims(dims) != L3_OK || max_d < 1 || n_max < 0) return 0;
    const Dims d{dims->d_in, dims->d_emb, dims->d_up, dims->d_out, dims->dtype, dims->ln_eps};
    return max_layout_bytes(d, n_max, max_d, ws_total);
}

int l3_forward(l3_plan_t p, const void *x, const int32_t *ids, int64_t n, const void *WK,
               const void *WV, const void *W_up, const float *gamma, const float *beta,
               const void *W_mix, void *out, void *ws, size_t ws_bytes, void *stream) {
    if (!p || n < 0) return L3_ERR_INVALID_ARG;
    if (n == 0) return L3_OK;
    if (n >= (1ll << 30)) return L3_ERR_UNSUPPORTED;
    if (!x || !ids || !WK || !WV || !W_up || !gamma || !beta || !W_mix || !out || !ws)
        return L3_ERR_INVALID_ARG;
    if (!aligned16({x, WK, WV, W_up, gamma, beta, W_mix, out, ws})) return L3_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(ids) & 3) return L3_ERR_INVALID_ARG;
    return forward_impl(*p, x, ids, n, WK, WV, W_up, gamma, beta, W_mix, out, ws, ws_bytes,
                        (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free forward
//
// l3_forward_noalloc runs l3_forward with its workspace in this file-scope device
// array instead of caller memory, for callers that cannot allocate.  Every GPU the
// library runs on holds its own copy until the process ends.  Host code must not
// pass the array's name to a kernel or a copy (on the host it is only a stand-in):
// its device address is taken once per device with hipGetSymbolAddress, with that
// device current, and only that address is used.
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kScratchDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The current device's address of `scratch` (looked up on the first call on that device).
int scratch_address(void **out) {
    int dev = -1;
    L3_HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kScratchDevices) return L3_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return L3_ERR_HIP;
        }
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return L3_OK;
}

}  // namespace

extern "C" {

int l3_forward_noalloc(l3_plan_t p, const void *x, const int32_t *ids, int64_t n, const void *WK,
                       const void *WV, const void *W_up, const float *gamma, const float *beta,
                       const void *W_mix, void *out, void *stream) {
    if (!p || n < 0) return L3_ERR_INVALID_ARG;
    if (n == 0) return L3_OK;
    if (n >= (1ll << 30)) return L3_ERR_UNSUPPORTED;
    if (!x || !ids || !WK || !WV || !W_up || !gamma || !beta || !W_mix || !out)
        return L3_ERR_INVALID_ARG;
    if (!aligned16({x, WK, WV, W_up, gamma, beta, W_mix, out})) return L3_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(ids) & 3) return L3_ERR_INVALID_ARG;
    // the layout this batch uses must fit the array (checked before anything is enqueued)
    if (ws_layout(p->dims, n, p->max_d).total > kScratchBytes) return L3_ERR_CAPACITY;
    void *ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != L3_OK) return rc;
    return forward_impl(*p, x, ids, n, WK, WV, W_up, gamma, beta, W_mix, out, ws, kScratchBytes,
                        (hipStream_t)stream);
}

size_t l3_backward_workspace_size(l3_plan_t p, int64_t n_max) {
    if (!p || n_max < 0) return 0;
    return max_layout_bytes(p->dims, n_max, p->max_d, bwd_total);
}

int l3_backward(l3_plan_t p, const void *x, const int32_t *ids, int64_t n, const void *WK,
                const void *WV, const void *W_up, const float *gamma, const float *beta,
                const void *W_mix, const void *dout, float *dx, float *dWK, float *dWV, float *dWup,
                float *dgamma, float *dbeta, float *dWmix, void *ws, size_t ws_bytes, void *stream) {
    if (!p || n < 0) return L3_ERR_INVALID_ARG;
    if (n == 0) return L3_OK;
    if (n >= (1ll << 30) || tied_only(p->dims)) return L3_ERR_UNSUPPORTED;
    if (!x || !ids || !WK || !WV || !W_up || !gamma || !beta || !W_mix || !dout || !dx || !dWK ||
        !dWV || !dWup || !dgamma || !dbeta || !dWmix || !ws)
        return L3_ERR_INVALID_ARG;
    if (!aligned16({x, WK, WV, W_up, gamma, beta, W_mix, dout, dx, dWK, dWV, dWup, dgamma, dbeta,
                    dWmix, ws}))
        return L3_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(ids) & 3) return L3_ERR_INVALID_ARG;
    if (p->dims.d_in > 4096 || p->dims.d_emb > 1024) return L3_ERR_UNSUPPORTED;
    return backward_impl(*p, x, ids, n, WK, WV, W_up, gamma, beta, W_mix, dout, dx, dWK, dWV, dWup,
                         dgamma, dbeta, dWmix, ws, ws_bytes, (hipStream_t)stream);
}

int l3_route(l3_plan_t p, const int32_t *ids, int64_t n, void *ws, size_t ws_bytes, void *stream,
             int32_t *perm, int32_t *sorted_ids, int32_t *inv_perm, int32_t *uniq, int32_t *counts,
             int32_t *seg_start, int32_t *num_segments) {
    if (!p || n < 0 || !ws) return L3_ERR_INVALID_ARG;
    if (n == 0) return L3_OK;
    if (!ids) return L3_ERR_INVALID_ARG;
    if (n >= (1ll << 30)) return L3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const WsLayout L = ws_layout(p->dims, n, p->max_d);
    if (ws_bytes < L.total) return L3_ERR_CAPACITY;
    RouteBufs b{};
    b.hdr = ws_ptr<int32_t>(ws, L.hdr);
    b.keys_a = ws_ptr<int32_t>(ws, L.keys_a);
    b.vals_a = ws_ptr<int32_t>(ws, L.vals_a);
    b.keys_b = ws_ptr<int32_t>(ws, L.keys_b);
    b.vals_b = ws_ptr<int32_t>(ws, L.vals_b);
    b.rank = ws_ptr<int32_t>(ws, L.rank);
    b.hist = ws_ptr<int32_t>(ws, L.hist);
    b.tile_cnt = ws_ptr<int32_t>(ws, L.tile_cnt);
    b.inv_perm = ws_ptr<int32_t>(ws, L.inv_perm);
    b.uniq = ws_ptr<int32_t>(ws, L.uniq);
    b.counts = ws_ptr<int32_t>(ws, L.counts);
    b.seg_start = ws_ptr<int32_t>(ws, L.seg_start);
    if (n <= kRouteSmallMax) {
        L3_HIP_TRY(launch_route_small(ids, n, p->vocab, p->d_off, INT32_MAX, INT32_MAX, 1, b,
                                      ws_ptr<int4>(ws, L.light), ws_ptr<int2>(ws, L.heavy),
                                      ws_ptr<int2>(ws, L.dense), s));
    } else {
        L3_HIP_TRY(launch_route(ids, n, p->vocab, b, L.ntiles, p->d_off, INT32_MAX, INT32_MAX, 1,
                                ws_ptr<int4>(ws, L.light), ws_ptr<int2>(ws, L.heavy),
                                ws_ptr<int2>(ws, L.dense), nullptr, s));  // clears the header too
    }
    const size_t nb = (size_t)n * 4;
    auto cp = [&](int32_t *dst, const int32_t *src, size_t bytes) -> hipError_t {
        return dst ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s) : hipSuccess;
    };
    L3_HIP_TRY(cp(perm, b.perm, nb));
    L3_HIP_TRY(cp(sorted_ids, b.sorted_ids, nb));
    L3_HIP_TRY(cp(inv_perm, b.inv_perm, nb));
    L3_HIP_TRY(cp(uniq, b.uniq, nb));
    L3_HIP_TRY(cp(counts, b.counts, nb));
    L3_HIP_TRY(cp(seg_start, b.seg_start, nb + 4));
    L3_HIP_TRY(cp(num_segments, b.hdr + HDR_NSEG, 4));
    return L3_OK;
}

int l3_status(void *ws, void *stream) {
    if (!ws) return L3_ERR_INVALID_ARG;
    L3_HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
    int32_t flag = 0;
    L3_HIP_TRY(hipMemcpy(&flag, ws_ptr<int32_t>(ws, 0) + HDR_ERR, 4, hipMemcpyDeviceToHost));
    return flag ? L3_ERR_TOKEN_RANGE : L3_OK;
}

size_t l3_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || M > kSkinnyMaxM) return 0;
    return skinny_part_bytes(M, N, K);
}

int l3_gemm_bf16(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, void *ws,
                 size_t ws_bytes, void *stream) {
    if (!A || !B || !C || M < 0 || N < 0 || K <= 0) return L3_ERR_INVALID_ARG;
    if (K % 64 || N % 64) return L3_ERR_UNSUPPORTED;
    if (!aligned16({A, B, C, ws})) return L3_ERR_INVALID_ARG;
    const size_t need = l3_gemm_workspace_size(M, N, K);
    if (need > 0 && (!ws || ws_bytes < need)) return L3_ERR_CAPACITY;
    if (need > 0)
        L3_HIP_TRY(launch_gemm_skinny_bf16((const uint16_t *)A, (const uint16_t *)B, (uint16_t *)C, M,
                                           N, K, nullptr, (float *)ws, (hipStream_t)stream));
    else
        L3_HIP_TRY(launch_gemm_bf16((const uint16_t *)A, (const uint16_t *)B, (uint16_t *)C, M, N, K,
                                    nullptr, (hipStream_t)stream));
    return L3_OK;
}

// ---------------------------------------------------------------- decode staging

static size_t staging_meta_bytes(int64_t max_tokens) {
    return (size_t)(2 * max_tokens + 1) * sizeof(int64_t) + (size_t)max_tokens * sizeof(int32_t);
}

int l3_staging_create(l3_plan_t p, int64_t max_rows, int64_t max_tokens, l3_staging_t *out) {
    if (!p || !out || max_rows <= 0 || max_tokens <= 0) return L3_ERR_INVALID_ARG;
    *out = nullptr;
    if (tied_only(p->dims)) return L3_ERR_UNSUPPORTED;  // stagings hold K and V rows apart
    l3_staging_s *st = new (std::nothrow) l3_staging_s();
    if (!st) return L3_ERR_NOMEM;
    st->plan = p;
    st->max_rows = max_rows;
    st->max_tokens = max_tokens;
    const size_t es = esize(p->dims.dtype);
    const size_t meta = staging_meta_bytes(max_tokens);
    bool ok = hipMalloc(&st->d_K, max_rows * p->dims.d_in * es) == hipSuccess &&
              hipMalloc(&st->d_V, max_rows * p->dims.d_emb * es) == hipSuccess &&
              hipMalloc(&st->d_meta, meta) == hipSuccess &&
              hipHostMalloc(&st->h_meta, meta, 0) == hipSuccess &&
              hipEventCreateWithFlags(&st->small_done, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&st->consumed, hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        l3_staging_destroy(st);
        return L3_ERR_HIP;
    }
    *out = st;
    return L3_OK;
}

int l3_staging_destroy(l3_staging_t st) {
    if (!st) return L3_OK;
    if (st->small_pending && st->small_done) (void)hipEventSynchronize(st->small_done);
    if (st->d_K) (void)hipFree(st->d_K);
    if (st->d_V) (void)hipFree(st->d_V);
    if (st->d_meta) (void)hipFree(st->d_meta);
    if (st->c_K) (void)hipFree(st->c_K);
    if (st->c_V) (void)hipFree(st->c_V);
    if (st->h_meta) (void)hipHostFree(st->h_meta);
    if (st->small_done) (void)hipEventDestroy(st->small_done);
    if (st->consumed) (void)hipEventDestroy(st->consumed);
    delete st;
    return L3_OK;
}

int l3_prefetch(l3_plan_t p, const int32_t *ids, int64_t n, const void *WK_host,
                const void *WV_host, l3_staging_t st, void *side_stream, void *ready_event) {
    if (!p || !st || st->plan != p || n < 0 || !WK_host || !WV_host) return L3_ERR_INVALID_ARG;
    if (n > 0 && !ids) return L3_ERR_INVALID_ARG;
    if (n > st->max_tokens) return L3_ERR_CAPACITY;
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= p->vocab) return L3_ERR_TOKEN_RANGE;
    // the kernel reads the tables through their device mapping: they must be
    // pinned host memory (hipHostMalloc), 16-byte aligned
    void *WK_dev = nullptr, *WV_dev = nullptr;
    if (hipHostGetDevicePointer(&WK_dev, const_cast<void *>(WK_host), 0) != hipSuccess ||
        hipHostGetDevicePointer(&WV_dev, const_cast<void *>(WV_host), 0) != hipSuccess) {
        (void)hipGetLastError();
        return L3_ERR_INVALID_ARG;
    }
    if (!aligned16({WK_host, WV_host, WK_dev, WV_dev})) return L3_ERR_INVALID_ARG;
    std::vector<int32_t> u(ids, ids + n);
    std::sort(u.begin(), u.end());
    u.erase(std::unique(u.begin(), u.end()), u.end());
    const int64_t m = (int64_t)u.size();
    int64_t rows = 0, max_d = 0;
    for (int32_t t : u) {
        const int64_t d = p->h_off[t + 1] - p->h_off[t];
        rows += d;
        max_d = std::max(max_d, d);
    }
    if (rows > st->max_rows) return L3_ERR_CAPACITY;
    hipStream_t s = (hipStream_t)side_stream;
    // the pinned mirror may still feed the previous step's copy
    if (st->small_pending) L3_HIP_TRY(hipEventSynchronize(st->small_done));
    st->small_pending = false;
    int64_t *h_coff = reinterpret_cast<int64_t *>(st->h_meta);
    int64_t *h_src = h_coff + (m + 1);
    int32_t *h_ids = reinterpret_cast<int32_t *>(h_src + m);
    h_coff[0] = 0;
    int64_t cached = 0;
    for (int64_t i = 0; i < m; ++i) {
        const int64_t d = p->h_off[u[i] + 1] - p->h_off[u[i]];
        h_coff[i + 1] = h_coff[i] + d;
        const int64_t cr = st->cache_row.empty() ? -1 : st->cache_row[u[i]];
        h_src[i] = cr >= 0 ? -1 - cr : p->h_off[u[i]];
        if (cr >= 0) cached += d;
    }
    st->cached_rows = cached;
    for (int64_t i = 0; i < n; ++i)
        h_ids[i] = (int32_t)(std::lower_bound(u.begin(), u.end(), ids[i]) - u.begin());
    int64_t *d_coff = reinterpret_cast<int64_t *>(st->d_meta);
    st->d_off = d_coff;
    st->d_ids = reinterpret_cast<int32_t *>(d_coff + (2 * m + 1));
    if (n > 0) {
        // the previous staged forward may still read the rows and index block
        if (st->consumed_pending) L3_HIP_TRY(hipStreamWaitEvent(s, st->consumed, 0));
        const size_t bytes = (size_t)(2 * m + 1) * sizeof(int64_t) + (size_t)n * sizeof(int32_t);
        L3_HIP_TRY(hipMemcpyAsync(st->d_meta, st->h_meta, bytes, hipMemcpyHostToDevice, s));
        L3_HIP_TRY(hipEventRecord(st->small_done, s));
        st->small_pending = true;
        const size_t es = esize(p->dims.dtype);
        L3_HIP_TRY(launch_stage_rows(d_coff, d_coff + (m + 1), m, rows, WK_dev, WV_dev, st->c_K,
                                     st->c_V, st->d_K, st->d_V, p->dims.d_in * es, p->dims.d_emb * es,
                                     s));
    }
    if (ready_event) L3_HIP_TRY(hipEventRecord((hipEvent_t)ready_event, s));
    st->n = n;
    st->m = m;
    st->rows = rows;
    st->max_d = max_d;
    return L3_OK;
}

int l3_staging_set_cache(l3_staging_t st, const int32_t *hot_ids, int64_t n_hot, const void *WK_host,
                         const void *WV_host, void *stream) {
    if (!st || n_hot < 0 || (n_hot > 0 && (!hot_ids || !WK_host || !WV_host))) return L3_ERR_INVALID_ARG;
    l3_plan_s *p = st->plan;
    hipStream_t s = (hipStream_t)stream;
    // drop the previous cache (work enqueued earlier, on any stream, may still read it)
    if (st->c_K || st->c_V) L3_HIP_TRY(hipDeviceSynchronize());
    if (st->small_pending) L3_HIP_TRY(hipEventSynchronize(st->small_done));
    st->small_pending = false;
    if (st->c_K) (void)hipFree(st->c_K);
    if (st->c_V) (void)hipFree(st->c_V);
    st->c_K = st->c_V = nullptr;
    st->cache_row.clear();
    if (n_hot == 0) return L3_OK;
    void *WK_dev = nullptr, *WV_dev = nullptr;
    if (hipHostGetDevicePointer(&WK_dev, const_cast<void *>(WK_host), 0) != hipSuccess ||
        hipHostGetDevicePointer(&WV_dev, const_cast<void *>(WV_host), 0) != hipSuccess) {
        (void)hipGetLastError();
        return L3_ERR_INVALID_ARG;
    }
    if (!aligned16({WK_host, WV_host, WK_dev, WV_dev})) return L3_ERR_INVALID_ARG;
    std::vector<int32_t> u(hot_ids, hot_ids + n_hot);
    for (int32_t t : u)
        if (t < 0 || t >= p->vocab) return L3_ERR_TOKEN_RANGE;
    std::sort(u.begin(), u.end());
    u.erase(std::unique(u.begin(), u.end()), u.end());
    const int64_t m = (int64_t)u.size();
    std::vector<int64_t> meta(2 * m + 1);
    meta[0] = 0;
    std::vector<int64_t> row(p->vocab, -1);
    for (int64_t i = 0; i < m; ++i) {
        row[u[i]] = meta[i];
        meta[i + 1] = meta[i] + (p->h_off[u[i] + 1] - p->h_off[u[i]]);
        meta[m + 1 + i] = p->h_off[u[i]];
    }
    const int64_t rows = meta[m];
    const size_t es = esize(p->dims.dtype);
    int64_t *d_meta = nullptr;
    bool ok = hipMalloc(&st->c_K, rows * p->dims.d_in * es) == hipSuccess &&
              hipMalloc(&st->c_V, rows * p->dims.d_emb * es) == hipSuccess &&
              hipMalloc(&d_meta, meta.size() * sizeof(int64_t)) == hipSuccess;
    ok = ok && hipMemcpyAsync(d_meta, meta.data(), meta.size() * sizeof(int64_t), hipMemcpyHostToDevice,
                              s) == hipSuccess;
    // the same gather kernel, from the host tables into the cache
    ok = ok && launch_stage_rows(d_meta, d_meta + m + 1, m, rows, WK_dev, WV_dev, nullptr, nullptr,
                                 st->c_K, st->c_V, p->dims.d_in * es, p->dims.d_emb * es, s) == hipSuccess;
    ok = ok && hipStreamSynchronize(s) == hipSuccess;
    if (d_meta) (void)hipFree(d_meta);
    if (!ok) {
        if (st->c_K) (void)hipFree(st->c_K);
        if (st->c_V) (void)hipFree(st->c_V);
        st->c_K = st->c_V = nullptr;
        return L3_ERR_HIP;
    }
    st->cache_row.swap(row);
    return L3_OK;
}

int l3_staging_stats(l3_staging_t st, int64_t *rows, int64_t *cached_rows) {
    if (!st) return L3_ERR_INVALID_ARG;
    if (rows) *rows = st->rows;
    if (cached_rows) *cached_rows = st->cached_rows;
    return L3_OK;
}

int l3_forward_staged(l3_staging_t st, const void *x, int64_t n, const void *W_up,
                      const float *gamma, const float *beta, const void *W_mix, void *out, void *ws,
                      size_t ws_bytes, void *stream) {
    if (!st || n < 0) return L3_ERR_INVALID_ARG;
    if (n != st->n) return L3_ERR_INVALID_ARG;
    if (n == 0) return L3_OK;
    if (!x || !W_up || !gamma || !beta || !W_mix || !out || !ws) return L3_ERR_INVALID_ARG;
    if (!aligned16({x, W_up, gamma, beta, W_mix, out, ws})) return L3_ERR_INVALID_ARG;
    // a plan view over the compact CSR; workspace sizing uses the full plan's max_d
    l3_plan_s view;
    view.vocab = st->m;
    view.v = st->rows;
    view.k = st->plan->k;
    view.max_d = st->plan->max_d;
    view.dims = st->plan->dims;
    view.d_off = st->d_off;
    view.side = st->plan->side;
    view.owns_off = false;
    const int rc = forward_impl(view, x, st->d_ids, n, st->d_K, st->d_V, W_up, gamma, beta, W_mix,
                                out, ws, ws_bytes, (hipStream_t)stream);
    if (rc != L3_OK) return rc;
    L3_HIP_TRY(hipEventRecord(st->consumed, (hipStream_t)stream));
    st->consumed_pending = true;
    return L3_OK;
}

// ---------------------------------------------------------------- stage timing

int l3_profile_enable(int enable) {
    g_prof.on = enable != 0;
    if (g_prof.on) {
        std::memset(g_prof.ms, 0, sizeof(g_prof.ms));
        std::memset(g_prof.launches, 0, sizeof(g_prof.launches));
    }
    return L3_OK;
}

int l3_profile_read(double *ms_total, int64_t *launches, int max_stages) {
    for (auto &pr : g_prof.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(pr.b) != hipSuccess) return L3_ERR_HIP;
        if (hipEventElapsedTime(&ms, pr.a, pr.b) != hipSuccess) return L3_ERR_HIP;
        g_prof.ms[pr.stage] += ms;
        g_prof.launches[pr.stage] += 1;
        g_prof.pool.push_back(pr.a);
        g_prof.pool.push_back(pr.b);
    }
    g_prof.pending.clear();
    for (int i = 0; i < max_stages && i < kProfStages; ++i) {
        if (ms_total) ms_total[i] = g_prof.ms[i];
        if (launches) launches[i] = g_prof.launches[i];
    }
    return L3_OK;
}

}  // extern "C"
