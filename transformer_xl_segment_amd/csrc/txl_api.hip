// txl_api.hip -- the C ABI declared in include/txl.h: argument checks,
// workspace layout and the launch sequence of each entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/txl.h"
#include "txl_internal.hpp"

using namespace txl;

namespace {

thread_local std::string g_last_error;

txl_status fail(txl_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

txl_status hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return TXL_OK;
    return fail(TXL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define TXL_TRY(expr)                          \
    do {                                       \
        txl_status st_ = (expr);               \
        if (st_ != TXL_OK) return st_;         \
    } while (0)

size_t es_of(txl_dtype dt) { return dt == TXL_BF16 ? 2 : 4; }
long long round_up(long long x, long long a) { return (x + a - 1) / a * a; }
bool al4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// ---------------------------------------------------------------------------
// Workspace layout. Every buffer starts on a 256-byte boundary.
// ---------------------------------------------------------------------------
struct Layout {
    size_t qu, qv, ke, vt, rk, o;      // attention operands and output
    size_t lse;                        // encoding variants: per-query log-sum-exp
    size_t part_o, part_ml;            // key-split parts of the attention output
    int nsplit;                        // most key splits any launch of this layout uses
    size_t z, z2, h1, f;               // block: fp32 pre-LN sums (z2: second half of a split FFN2), LN1 output,
                                       // FFN hidden
    size_t hb0, hb1;                   // stack: inter-layer activations
    // block with rows that are not 16-byte aligned: activations at the padded
    // pitches Dp and Fp (pad columns zero), the input rows copied to that pitch
    // (hx) and W_o, W1 repacked to Dp (wo, w1) and W2 to Fp (w2), so that the
    // block's own GEMMs take the direct-to-LDS kernel
    bool pad;
    int Dp, Fp;
    size_t hx, wo, w1, w2;
    size_t total;
    int Wp, Kp, dp;
};

Layout plan(txl_op op, txl_dtype dt, int B, int W, int Kmax, int D, int H, int F) {
    Layout L;
    memset(&L, 0, sizeof(L));
    const size_t es = es_of(dt);
    const int dh = D / H;
    L.dp = attn_dp(dh);
    // query rows per (b, h) of the projected q: whole waves of 32 (a
    // workgroup's last wave past W reads clamped rows and writes nothing)
    L.Wp = (int)round_up(W, 32);
    L.Kp = (int)round_up(Kmax, ATTN_KBLOCK);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = (size_t)round_up((long long)(off + bytes), 256);
        return at;
    };
    L.Dp = D;
    L.Fp = F;
    if (op == TXL_OP_LAYER || op == TXL_OP_STACK) {
        const int epr = 16 / (int)es;                 // elements per 16 bytes
        L.Dp = (int)round_up(D, epr);
        L.Fp = (int)round_up(F, epr);
        L.pad = L.Dp != D || L.Fp != F;
    }
    const size_t q_bytes = (size_t)B * H * L.Wp * L.dp * es;
    const size_t k_bytes = (size_t)B * H * L.Kp * L.dp * es;
    L.qu = take(q_bytes);
    L.qv = take(q_bytes);
    if (op != TXL_OP_REL_ATTN_CACHED) {
        L.ke = take(k_bytes);
        L.vt = take(k_bytes);
    }
    L.rk = take((size_t)H * rk_table_rows(L.Kp) * L.dp * es);
    L.o = take((size_t)B * W * L.Dp * es);
    if (op == TXL_OP_ATTN_VARIANT) L.lse = take((size_t)B * H * L.Wp * 4);
    L.nsplit = attn_splits(B, H, W, Kmax);
    if (L.nsplit > 1) {
        L.part_o = take((size_t)L.nsplit * B * H * L.Wp * L.dp * 4);
        L.part_ml = take((size_t)L.nsplit * B * H * L.Wp * 2 * 4);
    }
    if (op == TXL_OP_LAYER || op == TXL_OP_STACK) {
        L.z = take((size_t)B * W * L.Dp * 4);
        L.z2 = take((size_t)B * W * L.Dp * 4);
        L.h1 = take((size_t)B * W * L.Dp * es);
        L.f = take((size_t)B * W * L.Fp * es);
        if (L.pad) {
            L.hx = take((size_t)B * W * L.Dp * es);
            L.wo = take((size_t)D * L.Dp * es);
            L.w1 = take((size_t)F * L.Dp * es);
            L.w2 = take((size_t)D * L.Fp * es);
        }
    }
    if (op == TXL_OP_STACK) {
        L.hb0 = take((size_t)B * W * L.Dp * es);
        L.hb1 = take((size_t)B * W * L.Dp * es);
    }
    L.total = off;
    return L;
}

// ---------------------------------------------------------------------------
// Attention-kernel timing (txl_profile_begin / txl_profile_end).
// ---------------------------------------------------------------------------
struct Profiler {
    bool on = false;
    int used = 0;
    std::vector<hipEvent_t> start, stop;
    std::vector<double> times;      // per-launch milliseconds of the last finished window
} g_prof;

hipError_t attn_launch(bool bf16, const AttnArgs &a, hipStream_t s) {
    if (g_prof.on && g_prof.used < (int)g_prof.start.size()) {
        const int i = g_prof.used++;
        return launch_rel_attn(bf16, a, s, g_prof.start[i], g_prof.stop[i]);
    }
    return launch_rel_attn(bf16, a, s);
}

// ---------------------------------------------------------------------------
// Argument checks shared by the entry points.
// ---------------------------------------------------------------------------
txl_status check_shape(txl_dtype dt, int B, int W, int D, int H) {
    if (dt != TXL_FP32 && dt != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
    if (B < 1 || W < 1 || D < 2 || H < 1) return fail(TXL_ERR_ARG, "sizes must be positive (B=%d W=%d D=%d H=%d)", B, W, D, H);
    if (D % H) return fail(TXL_ERR_ARG, "D=%d is not a multiple of H=%d", D, H);
    if (D % 2) return fail(TXL_ERR_ARG, "D=%d must be even", D);
    if (!rel_attn_supported(D / H)) return fail(TXL_ERR_UNSUPPORTED, "head width %d > 64 is not supported", D / H);
    if ((long long)B * W > (1LL << 22) / 2) return fail(TXL_ERR_UNSUPPORTED, "B*W=%lld too large", (long long)B * W);
    return TXL_OK;
}

txl_status check_mem(const txl_mem *mem, int W) {
    if (!mem) return TXL_OK;
    if (mem->M < 1) return fail(TXL_ERR_ARG, "memory capacity M=%d must be >= 1", mem->M);
    if (mem->len < 0 || mem->len > mem->M) return fail(TXL_ERR_ARG, "memory len=%d outside [0, M=%d]", mem->len, mem->M);
    if (mem->head < 0 || mem->head >= mem->M) return fail(TXL_ERR_ARG, "memory head=%d outside [0, M=%d)", mem->head, mem->M);
    if (!mem->data) return fail(TXL_ERR_ARG, "memory data is NULL");
    if (!al4(mem->data)) return fail(TXL_ERR_ARG, "memory data must be 4-byte aligned");
    if ((long long)mem->M + W > (1LL << 20)) return fail(TXL_ERR_UNSUPPORTED, "M + W too large");
    return TXL_OK;
}

int kv_capacity(int M, int W) { return (int)round_up((long long)M + W, ATTN_KBLOCK); }

// A key/value cache that takes n more rows in one call and has at least
// `cap` slots: an attention call keeps the window and the n new rows at once
// (cap = M + n); an append only overwrites slots of rows that leave the window
// (cap = M + 8).
txl_status check_kv_cache(txl_dtype dt, const txl_kv_cache *c, int n, long long cap, int B, int D, int H) {
    if (!c) return fail(TXL_ERR_ARG, "cache is NULL");
    if (c->M < 8 || c->M % 8) return fail(TXL_ERR_UNSUPPORTED, "cache M=%d must be a positive multiple of 8", c->M);
    if (n % 8) return fail(TXL_ERR_UNSUPPORTED, "rows added to a cache per call (%d) must be a multiple of 8", n);
    if (c->C % ATTN_KBLOCK || c->C < cap)
        return fail(TXL_ERR_ARG, "cache capacity C=%d must be a multiple of %d and >= %lld "
                    "(txl_kv_cache_capacity)", c->C, ATTN_KBLOCK, cap);
    if (c->len < 0 || c->len > c->M || c->len % 8)
        return fail(TXL_ERR_ARG, "cache len=%d must be a multiple of 8 in [0, M=%d]", c->len, c->M);
    if (c->head < 0 || c->head >= c->C || c->head % 8)
        return fail(TXL_ERR_ARG, "cache head=%d must be a multiple of 8 in [0, C=%d)", c->head, c->C);
    if (!c->k || !c->vt) return fail(TXL_ERR_ARG, "cache k and vt must not be NULL");
    if (((uintptr_t)c->k | (uintptr_t)c->vt) % 16) return fail(TXL_ERR_ARG, "cache k and vt must be 16-byte aligned");
    if ((long long)B * H * c->C * attn_dp(D / H) * (long long)es_of(dt) >= (1LL << 40))
        return fail(TXL_ERR_UNSUPPORTED, "cache too large");
    return TXL_OK;
}

// The GEMM epilogue splits row indices with a float reciprocal, exact below 2^22.
txl_status check_rows_budget(int B, int W, int M) {
    const long long kp = round_up((long long)M + W, ATTN_KBLOCK);
    if ((long long)B * kp >= (1LL << 22) || (long long)B * round_up(W, ATTN_QBLOCK) >= (1LL << 22))
        return fail(TXL_ERR_UNSUPPORTED, "B * (M + W) = %lld rows exceeds 2^22", (long long)B * kp);
    return TXL_OK;
}

txl_status check_attn_params(const txl_layer_params *p) {
    if (!p) return fail(TXL_ERR_ARG, "params is NULL");
    const void *ptrs[] = {p->Wq, p->WkE, p->WkR, p->Wv, p->Wo, p->u, p->v};
    const char *names[] = {"Wq", "WkE", "WkR", "Wv", "Wo", "u", "v"};
    for (int i = 0; i < 7; ++i) {
        if (!ptrs[i]) return fail(TXL_ERR_ARG, "parameter %s is NULL", names[i]);
        if (!al4(ptrs[i])) return fail(TXL_ERR_ARG, "parameter %s must be 4-byte aligned", names[i]);
    }
    return TXL_OK;
}

txl_status check_block_params(const txl_layer_params *p, int F) {
    TXL_TRY(check_attn_params(p));
    if (F < 2 || F % 2) return fail(TXL_ERR_ARG, "F=%d must be even and >= 2", F);
    const void *ptrs[] = {p->ln1_g, p->ln1_b, p->W1, p->b1, p->W2, p->b2, p->ln2_g, p->ln2_b};
    const char *names[] = {"ln1_g", "ln1_b", "W1", "b1", "W2", "b2", "ln2_g", "ln2_b"};
    for (int i = 0; i < 8; ++i) {
        if (!ptrs[i]) return fail(TXL_ERR_ARG, "parameter %s is NULL", names[i]);
        if (!al4(ptrs[i])) return fail(TXL_ERR_ARG, "parameter %s must be 4-byte aligned", names[i]);
    }
    return TXL_OK;
}

txl_status check_rows(const void *p, long long bstride, int W, int D, txl_dtype dt, const char *name) {
    if (!p) return fail(TXL_ERR_ARG, "%s is NULL", name);
    if (!al4(p)) return fail(TXL_ERR_ARG, "%s must be 4-byte aligned", name);
    if (bstride < (long long)W * D) return fail(TXL_ERR_ARG, "%s batch stride %lld < W*D", name, bstride);
    if ((bstride * (long long)es_of(dt)) % 4) return fail(TXL_ERR_ARG, "%s batch stride must keep rows 4-byte aligned", name);
    return TXL_OK;
}

// ---------------------------------------------------------------------------
// Enqueue projections + fused attention; the attention output lands in ws+L.o
// as [B][W][D] rows.
// ---------------------------------------------------------------------------
// Projection of rows into a key/value cache (EPI_KV into ring slots
// (head + len + t) mod C): rows x[b][t] for t < n.
GemmProblem kv_cache_problem(int B, int n, int D, int H, int dp, const void *x, long long x_bstride,
                             const txl_layer_params *p, const txl_kv_cache *c) {
    GemmProblem kv;
    memset(&kv, 0, sizeof(kv));
    kv.rows = B * n; kv.cols = 2 * H * dp; kv.kdim = D;
    kv.seg_rows = n; kv.valid_rows = n;
    kv.a_mode = A_ROWS; kv.a = x; kv.a_ld = D; kv.a_bstride = x_bstride;
    kv.b_mode = B_HEADS; kv.b0 = p->WkE; kv.b1 = p->Wv; kv.b_split = H * dp; kv.b_ld = D;
    kv.dh = D / H; kv.dhp = dp; kv.heads = H;
    kv.epi = EPI_KV; kv.c0 = c->k; kv.c1 = c->vt;
    kv.kv_slots = c->C; kv.kv_base = (int)(((long long)c->head + c->len) % c->C);
    return kv;
}

// Window of a key/value cache after n rows were appended.
void kv_cache_advance(txl_kv_cache *c, int n) {
    const int len = c->len + n < c->M ? c->len + n : c->M;
    c->head = (int)(((long long)c->head + c->len + n - len) % c->C);
    c->len = len;
}

// An encoding other than Transformer-XL's: Shaw et al.'s clipped embeddings
// (aK, aV, clip) or absolute positions (no distance term).
struct Variant {
    txl_pos_variant kind;
    const void *aK, *aV;
    int clip;
};

// h rows are h_ld elements apart (0: D), the attention output o is written at
// row pitch o_ld (0: D); `extra` copies ride along the projection launch.
txl_status enqueue_attention(txl_dtype dt, int B, int W, int D, int H, const void *h, long long h_bstride,
                             const txl_mem *mem, const txl_kv_cache *cache, const txl_layer_params *p,
                             const void *R, char *ws, const Layout &L, hipStream_t s,
                             const Variant *var = nullptr, long long h_ld = 0, long long o_ld = 0,
                             const PitchCopy *extra = nullptr, int n_extra = 0) {
    if (h_ld <= 0) h_ld = D;
    if (o_ld <= 0) o_ld = D;
    const bool bf = dt == TXL_BF16;
    const int dh = D / H, dp = L.dp;
    const int m = cache ? cache->len : mem ? mem->len : 0;
    const int K = m + W;
    const int Kp = (int)round_up(K, ATTN_KBLOCK);

    GemmProblem q, kv, r;
    memset(&q, 0, sizeof(q));
    memset(&kv, 0, sizeof(kv));
    memset(&r, 0, sizeof(r));
    // Q: (h Wq^T + u, + v) * log2(e)/sqrt(dh), head-major

    q.rows = B * L.Wp; q.cols = H * dp; q.kdim = D;
    q.seg_rows = L.Wp; q.valid_rows = W;
    q.a_mode = A_ROWS; q.a = h; q.a_ld = h_ld; q.a_bstride = h_bstride;
    q.b_mode = B_HEADS; q.b0 = p->Wq; q.b_split = q.cols; q.b_ld = D;
    q.dh = dh; q.dhp = dp; q.heads = H;
    q.epi = EPI_QUV; q.c0 = ws + L.qu; q.c1 = ws + L.qv;
    q.u = var ? nullptr : p->u; q.v = var ? nullptr : p->v;        // the variants have no u, v
    q.qscale = (float)(1.4426950408889634 / sqrt((double)dh));
    // K_E and V: of the context [mem; h], or of the segment rows into the cache
    if (cache) {
        kv = kv_cache_problem(B, W, D, H, dp, h, h_bstride, p, cache);
    } else {
    kv.rows = B * Kp; kv.cols = 2 * H * dp; kv.kdim = D;
    kv.seg_rows = Kp; kv.valid_rows = W;
    kv.a_mode = A_CONTEXT; kv.a = h; kv.a_ld = h_ld; kv.a_bstride = h_bstride;
    kv.ring = m > 0 ? mem->data : h; kv.ring_bstride = m > 0 ? (long long)mem->M * D : 0; kv.ring_ld = D;
    kv.ring_M = m > 0 ? mem->M : 1; kv.ring_head = m > 0 ? mem->head : 0; kv.mem_len = m;
    kv.b_mode = B_HEADS; kv.b0 = p->WkE; kv.b1 = p->Wv; kv.b_split = H * dp; kv.b_ld = D;
    kv.dh = dh; kv.dhp = dp; kv.heads = H;
    kv.epi = EPI_KV; kv.c0 = ws + L.ke; kv.c1 = ws + L.vt;
    kv.kv_slots = Kp; kv.kv_base = 0;
    }
    // r = R[0:K] WkR^T, shared by the batch
    r.rows = Kp + 2 * ATTN_RPAD; r.cols = H * dp; r.kdim = D;
    r.seg_rows = Kp + 2 * ATTN_RPAD; r.valid_rows = K; r.a_first = ATTN_RPAD;
    r.a_mode = A_ROWS; r.a = R; r.a_ld = D; r.a_bstride = 0;
    r.b_mode = B_HEADS; r.b0 = p->WkR; r.b_split = r.cols; r.b_ld = D;
    r.dh = dh; r.dhp = dp; r.heads = H;
    r.epi = EPI_RFRAG; r.c0 = ws + L.rk;
    r.frag_off = rk_frag_off(m); r.frag_hstride = (long long)rk_table_rows(Kp) * dp;
    // Q and r first: their tiles end with the slower epilogues (two outputs;
    // the fragment-major table), so they are dealt out ahead of the key/value
    // tiles and all start in the launch's first round, which then leaves only
    // key/value tiles for the partly filled second round
    GemmLaunch g;
    memset(&g, 0, sizeof(g));
    g.p[0] = q;
    if (var) {                                                       // the variants need no R W_kR^T
        g.p[1] = kv;
        g.count = 2;
        g.lead = 1;
    } else {
        g.p[1] = r;
        g.p[2] = kv;
        g.count = 3;
        g.lead = 2;
    }
    int t = 0;
    for (int i = 0; i < g.count; ++i) {
        GemmProblem &P = g.p[i];
        P.tiles_n = (P.cols + 127) / 128;
        P.tile_begin = t;
        P.tile_count = ((P.rows + 127) / 128) * P.tiles_n;
        t += P.tile_count;
    }
    g.total_tiles = t;
    for (int i = 0; i < n_extra; ++i) g.pc[i] = extra[i];
    g.pc_count = n_extra;
    TXL_TRY(hip_check(launch_gemm(bf, g, s), "projection GEMM launch"));
    if (var && var->kind == TXL_POS_SHAW)
        TXL_TRY(hip_check(launch_shaw_rows(bf, ws + L.rk, var->aK, var->clip, K, Kp, dh, dp, rk_frag_off(m), s),
                          "distance table launch"));

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.qu = ws + L.qu; a.qv = ws + L.qv; a.rk = ws + L.rk;
    a.rk_hstride = var ? 0 : (long long)rk_table_rows(Kp) * dp;      // Shaw: one table for all heads
    a.dist = !(var && var->kind == TXL_POS_ABSOLUTE);
    a.lse = var && var->kind == TXL_POS_SHAW ? (float *)(ws + L.lse) : nullptr;
    a.ke = cache ? cache->k : (const void *)(ws + L.ke);
    a.vt = cache ? cache->vt : (const void *)(ws + L.vt);
    a.o = ws + L.o; a.o_bstride = (long long)W * o_ld; a.o_ld = o_ld;
    a.B = B; a.H = H; a.W = W; a.Wp = L.Wp; a.m = m; a.K = K; a.Kp = Kp; a.dh = dh; a.dp = dp; a.D = D;
    a.C = cache ? cache->C : Kp;
    a.khead = cache ? cache->head : 0;
    // key split (non-decreasing in K, so never more parts than the layout holds)
    a.nsplit = std::min(attn_splits(B, H, W, K), L.nsplit);
    if (a.nsplit > 1) {
        a.part_o = (float *)(ws + L.part_o);
        a.part_ml = (float *)(ws + L.part_ml);
    } else {
        a.nsplit = 1;
    }
    TXL_TRY(hip_check(attn_launch(bf, a, s), "attention launch"));
    if (a.lse) TXL_TRY(hip_check(launch_shaw_values(bf, a, var->aV, var->clip, s), "value-term launch"));
    return TXL_OK;
}

GemmLaunch single(const GemmProblem &p) {
    GemmLaunch g;
    memset(&g, 0, sizeof(g));
    g.p[0] = p;
    g.p[0].tiles_n = (p.cols + 127) / 128;
    g.p[0].tile_begin = 0;
    g.p[0].tile_count = ((p.rows + 127) / 128) * g.p[0].tiles_n;
    g.count = 1;
    g.total_tiles = g.p[0].tile_count;
    return g;
}

GemmLaunch grouped(std::initializer_list<GemmProblem> ps) {
    GemmLaunch g;
    memset(&g, 0, sizeof(g));
    int t = 0;
    for (const GemmProblem &p0 : ps) {
        GemmProblem &P = g.p[g.count++];
        P = p0;
        P.tiles_n = (P.cols + 127) / 128;
        P.tile_begin = t;
        P.tile_count = ((P.rows + 127) / 128) * P.tiles_n;
        t += P.tile_count;
    }
    g.total_tiles = t;
    return g;
}

// Dense rows GEMM: C(b, t) = A(b, t) W^T (+bias, relu, +res), A/C [B][W][*].
GemmProblem rows_problem(int B, int W, int kdim, int cols, const void *a, long long a_ld, long long a_bstride,
                         const void *w, void *c, long long c_ld, long long c_bstride) {
    GemmProblem p;
    memset(&p, 0, sizeof(p));
    p.rows = B * W; p.cols = cols; p.kdim = kdim;
    p.seg_rows = W; p.valid_rows = W;
    p.a_mode = A_ROWS; p.a = a; p.a_ld = a_ld; p.a_bstride = a_bstride;
    p.b_mode = B_ROWS; p.b0 = w; p.b_split = cols; p.b_ld = kdim;
    p.dh = 1; p.dhp = 1; p.heads = 1;
    p.epi = EPI_ROWS; p.c0 = c; p.c_ld = c_ld; p.c_bstride = c_bstride;
    return p;
}

// mem = last M rows of [mem; h]: plans the ring copy into rc (blocks workgroups)
// and advances the ring's host-side state; the copy runs in whichever launch
// carries rc, which must come after every launch that reads the old rows.
txl_status plan_mem_update(txl_dtype dt, int B, int D, txl_mem *mem, const void *h, long long h_bstride,
                           long long h_ld, int W, RingCopy &rc, int &blocks) {
    const int n = W < mem->M ? W : mem->M;
    const int pos0 = (int)(((long long)mem->head + mem->len) % mem->M);
    blocks = plan_ring_copy(dt == TXL_BF16, rc, mem->data, mem->M, D, pos0, h, h_bstride, h_ld, W - n, n, B);
    if (blocks < 0) return fail(TXL_ERR_UNSUPPORTED, "memory update of %d rows of %d elements exceeds 32-bit indexing",
                                n, D);
    if (mem->len + n <= mem->M) {
        mem->len += n;
    } else {
        mem->head = (int)(((long long)mem->head + mem->len + n - mem->M) % mem->M);
        mem->len = mem->M;
    }
    return TXL_OK;
}

txl_status enqueue_mem_update(txl_dtype dt, int B, int D, txl_mem *mem, const void *h, long long h_bstride, int W,
                              hipStream_t s) {
    RingCopy rc;
    int blocks = 0;
    txl_mem next = *mem;
    TXL_TRY(plan_mem_update(dt, B, D, &next, h, h_bstride, D, W, rc, blocks));
    TXL_TRY(hip_check(launch_ring_copy(rc, blocks, s), "memory update launch"));
    *mem = next;
    return TXL_OK;
}

// A pitched copy of `rows` rows (seg_rows per batch entry) of `cols` elements:
// src rows src_ld apart (batch stride src_bs), dst rows dst_ld apart (batch
// stride dst_bs), dst columns cols .. dst_ld-1 zeroed; src null zeroes only the
// pad columns. Element counts are even for bf16, so rows are whole words.
PitchCopy pitch_job(size_t es, const void *src, long long src_ld, long long src_bs, void *dst, long long dst_ld,
                    long long dst_bs, int rows, int seg_rows, int cols) {
    PitchCopy pc;
    memset(&pc, 0, sizeof(pc));
    auto words = [&](long long elems) { return elems * (long long)es / 4; };
    pc.src = (const uint32_t *)src;
    pc.dst = (uint32_t *)dst;
    pc.src_pitch = words(src_ld);
    pc.dst_pitch = words(dst_ld);
    pc.src_bstride = words(src_bs);
    pc.dst_bstride = words(dst_bs);
    pc.seg_rows = seg_rows;
    pc.rows = rows;
    pc.w0 = src ? 0 : (int)words(cols);
    pc.w1 = (int)words(dst_ld);
    pc.copy_w = src ? (int)words(cols) : 0;
    // whole rows per workgroup, about kPitchWords words each
    const int width = std::max(1, pc.w1 - pc.w0);
    pc.rb = std::max(1, kPitchWords / width);
    pc.blocks = std::max(1, (rows + pc.rb - 1) / pc.rb);
    return pc;
}

// One layer. h rows are h_ld elements apart and y rows are written y_ld apart.
// With `update` (the layer's own memory, the ring `mem` reads) the memory update
// mem = last M rows of [mem; h] rides along the output projection's launch,
// which comes after every read of the old rows. With a padded layout (L.pad)
// the block's activations live at the 16-byte aligned pitches Dp and Fp, h is
// first copied to that pitch unless it is there already, and W_o, W1 (to Dp)
// and W2 (to Fp) are repacked by workgroups riding along the projection
// launch, which also zero the pad columns of o, h1 and f: the output
// projection and the FFN products then reduce over Dp or Fp (the pad columns
// contribute zeros) with every operand 16-byte aligned.
txl_status enqueue_block(txl_dtype dt, int B, int W, int D, int H, int F, const void *h, long long h_bstride,
                         long long h_ld, const txl_mem *mem, const txl_layer_params *p, const void *R, void *y,
                         long long y_bstride, long long y_ld, char *ws, const Layout &L, hipStream_t s,
                         txl_mem *update = nullptr) {
    const bool bf = dt == TXL_BF16;
    const size_t es = es_of(dt);
    const int Dp = L.Dp, Fp = L.Fp;
    const long long WDp = (long long)W * Dp, WFp = (long long)W * Fp;
    const void *Wo = p->Wo, *W1 = p->W1, *W2 = p->W2;
    static_assert(kMaxPitchCopies >= 6, "the block's repacks and pad clears ride along one launch");
    PitchCopy extra[kMaxPitchCopies];
    int n_extra = 0;
    if (L.pad) {
        if (h_ld != Dp) {
            // the input rows at the padded pitch, in a launch of their own (the
            // projection reads them)
            const PitchCopy px = pitch_job(es, h, h_ld, h_bstride, ws + L.hx, Dp, WDp, B * W, W, D);
            TXL_TRY(hip_check(launch_pitch_copies(&px, 1, s), "input pitch copy launch"));
            h = ws + L.hx;
            h_ld = Dp;
            h_bstride = WDp;
        }
        // W_o and W1 reduce over d_model, W2 over F: repacked when their rows
        // are not aligned
        if (Dp != D) {
            extra[n_extra++] = pitch_job(es, p->Wo, D, 0, ws + L.wo, Dp, 0, D, D, D);
            extra[n_extra++] = pitch_job(es, p->W1, D, 0, ws + L.w1, Dp, 0, F, F, D);
            Wo = ws + L.wo;
            W1 = ws + L.w1;
        }
        if (Fp != F) {
            extra[n_extra++] = pitch_job(es, p->W2, F, 0, ws + L.w2, Fp, 0, D, D, F);
            W2 = ws + L.w2;
        }
        // pad columns of the GEMM inputs the block writes (nothing else writes them)
        extra[n_extra++] = pitch_job(es, nullptr, 0, 0, ws + L.o, Dp, WDp, B * W, W, D);
        extra[n_extra++] = pitch_job(es, nullptr, 0, 0, ws + L.h1, Dp, WDp, B * W, W, D);
        if (Fp != F) extra[n_extra++] = pitch_job(es, nullptr, 0, 0, ws + L.f, Fp, WFp, B * W, W, F);
    }
    TXL_TRY(enqueue_attention(dt, B, W, D, H, h, h_bstride, mem, nullptr, p, R, ws, L, s, nullptr, h_ld, Dp, extra,
                              n_extra));
    // z = h + O Wo^T (fp32)
    GemmProblem wo = rows_problem(B, W, Dp, D, ws + L.o, Dp, WDp, Wo, ws + L.z, Dp, WDp);
    wo.res = h; wo.res_ld = h_ld; wo.res_bstride = h_bstride; wo.out_f32 = 1;
    GemmLaunch gwo = single(wo);
    txl_mem next;
    if (update) {
        next = *update;
        TXL_TRY(plan_mem_update(dt, B, D, &next, h, h_bstride, h_ld, W, gwo.rc, gwo.copy_blocks));
    }
    TXL_TRY(hip_check(launch_gemm(bf, gwo, s), "output projection launch"));
    if (update) *update = next;
    TXL_TRY(hip_check(launch_layer_norm(bf, (const float *)(ws + L.z), nullptr, Dp, p->ln1_g, p->ln1_b, ws + L.h1, WDp,
                                        Dp, B, W, D, s),
                      "LayerNorm launch"));
    // f = ReLU(h1 W1^T + b1)
    GemmProblem f1 = rows_problem(B, W, Dp, F, ws + L.h1, Dp, WDp, W1, ws + L.f, Fp, WFp);
    f1.bias = p->b1; f1.relu = 1;
    TXL_TRY(hip_check(launch_gemm(bf, single(f1), s), "FFN1 launch"));
    // z = h1 + f W2^T + b2 (fp32), reduced over Fp when W2 was repacked (the pad
    // columns of f and of the repacked W2 are zero). A long reduction over too
    // few tiles to give every CU two (64-row tiles) is split in two at a k-tile
    // boundary when it runs on the direct-to-LDS kernel: the first half carries
    // the bias and the residual into z, the second half writes its partial sums
    // to z2, and LayerNorm adds the two (16-layer stacks: fp32 75.2 -> 72.5 ms
    // per schedule; bf16 with W2 repacked 20.1 -> 19.2 ms, where the split over
    // the caller's dword-aligned W2 on the register-staged kernel was slower).
    const int Fk = W2 == p->W2 ? F : Fp;
    GemmProblem f2 = rows_problem(B, W, Fk, D, ws + L.f, Fp, WFp, W2, ws + L.z, Dp, WDp);
    f2.bias = p->b2; f2.res = ws + L.h1; f2.res_ld = Dp; f2.res_bstride = WDp; f2.out_f32 = 1;
    const long long tiles64 = ((long long)B * W + 63) / 64 * ((D + 127) / 128);
    const float *z2 = nullptr;
    if ((dt == TXL_FP32 || Fk % 8 == 0) && F >= 1024 && tiles64 < 512) {
        const int ks = (int)round_up((Fk + 1) / 2, 64);
        GemmProblem f2b = f2;
        f2.kdim = ks;
        f2b.kdim = Fk - ks;
        f2b.a = (const char *)f2.a + (size_t)ks * es;
        f2b.b0 = (const char *)f2.b0 + (size_t)ks * es;
        f2b.bias = nullptr;
        f2b.res = nullptr;
        f2b.c0 = ws + L.z2;
        z2 = (const float *)(ws + L.z2);
        TXL_TRY(hip_check(launch_gemm(bf, grouped({f2, f2b}), s), "FFN2 launch"));
    } else {
        TXL_TRY(hip_check(launch_gemm(bf, single(f2), s), "FFN2 launch"));
    }
    TXL_TRY(hip_check(launch_layer_norm(bf, (const float *)(ws + L.z), z2, Dp, p->ln2_g, p->ln2_b, y, y_bstride, y_ld,
                                        B, W, D, s),
                      "LayerNorm launch"));
    return TXL_OK;
}


// Workspace of the backward pass (one region per operand, 256-byte aligned).
struct BwdLayout {
    size_t qu, qv, dOh, qut, qvt, dOt, ke, vk, ket, vt, rk, rt, o;   // T operands
    size_t pt, dst, dsd;                                            // T, per-(b, h) matrices
    size_t lse, drh, part;                                          // fp32
    size_t total;
    BwdDims d;
};

BwdLayout plan_bwd(txl_dtype dt, int B, int W, int m, int D, int H) {
    BwdLayout L;
    memset(&L, 0, sizeof(L));
    const size_t es = es_of(dt);
    BwdDims &d = L.d;
    d.B = B; d.H = H; d.W = W; d.m = m; d.K = m + W; d.D = D; d.dh = D / H;
    d.dp = attn_dp(d.dh);
    d.Wp = (int)round_up(W, 128);          // GEMM tiles never straddle two (b, h) entries
    d.W8 = (int)round_up(W, 8);            // reduction length of the dval, dk and dr GEMMs
    d.Kp = (int)round_up(d.K, 128);
    const size_t G = (size_t)B * H;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = (size_t)round_up((long long)(off + bytes), 256);
        return at;
    };
    const size_t qb = G * d.Wp * d.dp * es, kb = G * d.Kp * d.dp * es, sb = G * d.Kp * d.Wp * es;
    L.qu = take(qb); L.qv = take(qb); L.dOh = take(qb); L.qut = take(qb); L.qvt = take(qb); L.dOt = take(qb);
    L.ke = take(kb); L.vk = take(kb); L.ket = take(kb); L.vt = take(kb);
    L.rk = take((size_t)H * rk_table_rows(d.Kp) * d.dp * es);
    L.rt = take((size_t)H * d.dp * attn_bwd_rt_ld(d.Kp) * es);
    L.o = take((size_t)B * W * D * es);
    L.pt = take(sb); L.dst = take(sb); L.dsd = take(sb);
    L.lse = take(G * d.Wp * 4);
    L.drh = take(G * d.Kp * d.dp * 4);
    L.part = take((size_t)2 * H * bwd_parts(d) * 64 * 4);
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

size_t txl_workspace_bytes(txl_op op, txl_dtype dtype, int B, int W, int M, int D, int H, int F) {
    if (B < 1 || W < 1 || D < 2 || H < 1 || D % H || M < 0) return 0;
    if (dtype != TXL_FP32 && dtype != TXL_BF16) return 0;
    if (op == TXL_OP_REL_ATTN_BWD) return M + W > 4096 ? 0 : plan_bwd(dtype, B, W, M, D, H).total;
    if (op != TXL_OP_REL_ATTN && op != TXL_OP_LAYER && op != TXL_OP_STACK && op != TXL_OP_REL_ATTN_CACHED &&
        op != TXL_OP_ATTN_VARIANT)
        return 0;
    const bool attn_only = op == TXL_OP_REL_ATTN || op == TXL_OP_REL_ATTN_CACHED || op == TXL_OP_ATTN_VARIANT;
    if (!attn_only && F < 1) return 0;
    return plan(op, dtype, B, W, M + W, D, H, attn_only ? 0 : F).total;
}

txl_status txl_sinusoid_table(txl_dtype dtype, int R_len, int D, void *R, void *stream) {
    if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (R_len < 1 || D < 2 || D % 2) return fail(TXL_ERR_ARG, "need R_len >= 1 and an even D >= 2");
    if (!R || !al4(R)) return fail(TXL_ERR_ARG, "R must be a non-NULL 4-byte aligned pointer");
    return hip_check(launch_sinusoid(dtype == TXL_BF16, R, R_len, D, (hipStream_t)stream), "sinusoid launch");
}

namespace {

// Argument checks of txl_rel_attn_fwd and txl_rel_attn_fwd_noalloc (all but the workspace).
txl_status check_rel_attn(txl_dtype dtype, int B, int W, int D, int H, const void *h, long long h_bstride,
                          const txl_mem *mem, const txl_layer_params *p, const void *R, int R_len, const void *out,
                          long long out_bstride) {
    TXL_TRY(check_shape(dtype, B, W, D, H));
    TXL_TRY(check_rows(h, h_bstride, W, D, dtype, "h"));
    TXL_TRY(check_rows(out, out_bstride, W, D, dtype, "out"));
    TXL_TRY(check_mem(mem, W));
    TXL_TRY(check_attn_params(p));
    const int m = mem ? mem->len : 0;
    TXL_TRY(check_rows_budget(B, W, m));
    if (!R || !al4(R)) return fail(TXL_ERR_ARG, "R must be a non-NULL 4-byte aligned pointer");
    if (R_len < m + W) return fail(TXL_ERR_ARG, "R_len=%d < mem len + W = %d", R_len, m + W);
    return TXL_OK;
}

}  // namespace

txl_status txl_rel_attn_fwd(txl_dtype dtype, int B, int W, int D, int H, const void *h, long long h_bstride,
                            const txl_mem *mem, const txl_layer_params *p, const void *R, int R_len, void *out,
                            long long out_bstride, void *ws, size_t ws_bytes, void *stream) {
    TXL_TRY(check_rel_attn(dtype, B, W, D, H, h, h_bstride, mem, p, R, R_len, out, out_bstride));
    const int m = mem ? mem->len : 0;
    const Layout L = plan(TXL_OP_REL_ATTN, dtype, B, W, m + W, D, H, 0);
    if (!ws || ws_bytes < L.total) return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
    if ((uintptr_t)ws % 256) return fail(TXL_ERR_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    TXL_TRY(enqueue_attention(dtype, B, W, D, H, h, h_bstride, mem, nullptr, p, R, w, L, s));
    GemmProblem wo = rows_problem(B, W, D, D, w + L.o, D, (long long)W * D, p->Wo, out, D, out_bstride);
    return hip_check(launch_gemm(dtype == TXL_BF16, single(wo), s), "output projection launch");
}

txl_status txl_rel_attn_fwd_update(txl_dtype dtype, int B, int W, int D, int H, const void *h, long long h_bstride,
                                   txl_mem *mem, const txl_layer_params *p, const void *R, int R_len, void *out,
                                   long long out_bstride, void *ws, size_t ws_bytes, void *stream) {
    if (!mem) return fail(TXL_ERR_ARG, "memory is NULL (txl_rel_attn_fwd_update updates it)");
    TXL_TRY(check_rel_attn(dtype, B, W, D, H, h, h_bstride, mem, p, R, R_len, out, out_bstride));
    const Layout L = plan(TXL_OP_REL_ATTN, dtype, B, W, mem->len + W, D, H, 0);
    if (!ws || ws_bytes < L.total) return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
    if ((uintptr_t)ws % 256) return fail(TXL_ERR_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    txl_mem next = *mem;
    GemmLaunch gwo = single(rows_problem(B, W, D, D, w + L.o, D, (long long)W * D, p->Wo, out, D, out_bstride));
    // the copy is planned before any launch so that a refused update launches nothing
    TXL_TRY(plan_mem_update(dtype, B, D, &next, h, h_bstride, D, W, gwo.rc, gwo.copy_blocks));
    TXL_TRY(enqueue_attention(dtype, B, W, D, H, h, h_bstride, mem, nullptr, p, R, w, L, s));
    TXL_TRY(hip_check(launch_gemm(dtype == TXL_BF16, gwo, s), "output projection launch"));
    *mem = next;
    return TXL_OK;
}

// ---------------------------------------------------------------------------
// txl_rel_attn_fwd_noalloc: the same launches with the workspace in a fixed
// device array. Each GPU the library runs on holds its own copy (module-load
// memory, kept until the process ends). Host code never hands the array's name
// to a kernel or a copy: its device address comes from hipGetSymbolAddress,
// looked up once per device with that device current.
// ---------------------------------------------------------------------------
namespace {

static_assert(TXL_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");
static __device__ __align__(256) char scratch[TXL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxScratchDevices];

// Device address of the current device's copy of `scratch`.
txl_status scratch_address(void **out) {
    int dev = -1;
    TXL_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(TXL_ERR_UNSUPPORTED, "device %d: txl_rel_attn_fwd_noalloc supports devices 0..%d", dev,
                    kMaxScratchDevices - 1);
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
    if (slot.err != hipSuccess || !slot.ptr)
        return fail(TXL_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(slot.err));
    *out = slot.ptr;
    return TXL_OK;
}

}  // namespace

txl_status txl_rel_attn_fwd_noalloc(txl_dtype dtype, int B, int W, int D, int H, const void *h,
                                    long long h_bstride, const txl_mem *mem, const txl_layer_params *p,
                                    const void *R, int R_len, void *out, long long out_bstride, void *stream) {
    TXL_TRY(check_rel_attn(dtype, B, W, D, H, h, h_bstride, mem, p, R, R_len, out, out_bstride));
    const int m = mem ? mem->len : 0;
    // sized by this call's key count; every check runs before any device call
    const size_t need = plan(TXL_OP_REL_ATTN, dtype, B, W, m + W, D, H, 0).total;
    if (need > (size_t)TXL_NOALLOC_SCRATCH_BYTES)
        return fail(TXL_ERR_WORKSPACE, "txl_rel_attn_fwd_noalloc: this call needs %zu bytes of scratch, the fixed "
                    "array holds %zu (call txl_rel_attn_fwd with a workspace instead)", need,
                    (size_t)TXL_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    TXL_TRY(scratch_address(&ws));
    return txl_rel_attn_fwd(dtype, B, W, D, H, h, h_bstride, mem, p, R, R_len, out, out_bstride, ws,
                            (size_t)TXL_NOALLOC_SCRATCH_BYTES, stream);
}

txl_status txl_mem_update(txl_dtype dtype, int B, int D, txl_mem *mem, const void *h, long long h_bstride, int W,
                          void *stream) {
    if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (B < 1 || D < 2 || W < 1 || D % 2) return fail(TXL_ERR_ARG, "need B, W >= 1 and an even D >= 2");
    if (!mem) return fail(TXL_ERR_ARG, "memory is NULL");
    TXL_TRY(check_mem(mem, W));
    TXL_TRY(check_rows(h, h_bstride, W, D, dtype, "h"));
    return enqueue_mem_update(dtype, B, D, mem, h, h_bstride, W, (hipStream_t)stream);
}

txl_status txl_layer_fwd(txl_dtype dtype, int B, int W, int D, int H, int F, const void *h, long long h_bstride,
                         const txl_mem *mem, const txl_layer_params *p, const void *R, int R_len, void *y,
                         long long y_bstride, void *ws, size_t ws_bytes, void *stream) {
    TXL_TRY(check_shape(dtype, B, W, D, H));
    if (D > 1024) return fail(TXL_ERR_UNSUPPORTED, "LayerNorm supports D <= 1024 (got %d)", D);
    TXL_TRY(check_rows(h, h_bstride, W, D, dtype, "h"));
    TXL_TRY(check_rows(y, y_bstride, W, D, dtype, "y"));
    TXL_TRY(check_mem(mem, W));
    TXL_TRY(check_block_params(p, F));
    const int m = mem ? mem->len : 0;
    TXL_TRY(check_rows_budget(B, W, m));
    if (!R || !al4(R)) return fail(TXL_ERR_ARG, "R must be a non-NULL 4-byte aligned pointer");
    if (R_len < m + W) return fail(TXL_ERR_ARG, "R_len=%d < mem len + W = %d", R_len, m + W);
    const Layout L = plan(TXL_OP_LAYER, dtype, B, W, m + W, D, H, F);
    if (!ws || ws_bytes < L.total) return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
    if ((uintptr_t)ws % 256) return fail(TXL_ERR_ARG, "workspace must be 256-byte aligned");
    return enqueue_block(dtype, B, W, D, H, F, h, h_bstride, D, mem, p, R, y, y_bstride, D, (char *)ws, L,
                         (hipStream_t)stream);
}

txl_status txl_stack_fwd_segments(txl_dtype dtype, int B, int W, int D, int H, int F, int n_layers, int n_seg,
                                  const void *x, txl_mem *mems, const txl_layer_params *params, const void *R,
                                  int R_len, void *y, void *ws, size_t ws_bytes, void *stream) {
    TXL_TRY(check_shape(dtype, B, W, D, H));
    if (D > 1024) return fail(TXL_ERR_UNSUPPORTED, "LayerNorm supports D <= 1024 (got %d)", D);
    if (n_layers < 1 || n_seg < 1) return fail(TXL_ERR_ARG, "n_layers and n_seg must be >= 1");
    const long long seq = (long long)n_seg * W;
    TXL_TRY(check_rows(x, seq * D, W, D, dtype, "x"));
    TXL_TRY(check_rows(y, seq * D, W, D, dtype, "y"));
    if (!mems || !params) return fail(TXL_ERR_ARG, "mems and params must not be NULL");
    const int M = mems[0].M;
    for (int l = 0; l < n_layers; ++l) {
        TXL_TRY(check_mem(&mems[l], W));
        if (mems[l].M != M) return fail(TXL_ERR_ARG, "every memory ring must have the same M");
        TXL_TRY(check_block_params(&params[l], F));
    }
    TXL_TRY(check_rows_budget(B, W, M));
    if (!R || !al4(R)) return fail(TXL_ERR_ARG, "R must be a non-NULL 4-byte aligned pointer");
    if (R_len < M + W) return fail(TXL_ERR_ARG, "R_len=%d < M + W = %d", R_len, M + W);
    const Layout L = plan(TXL_OP_STACK, dtype, B, W, M + W, D, H, F);
    if (!ws || ws_bytes < L.total) return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
    if ((uintptr_t)ws % 256) return fail(TXL_ERR_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    const size_t es = es_of(dtype);
    for (int t = 0; t < n_seg; ++t) {
        const char *hin = (const char *)x + (size_t)t * W * D * es;
        long long hin_bs = seq * D, hin_ld = D;
        for (int l = 0; l < n_layers; ++l) {
            const bool last = l == n_layers - 1;
            // inter-layer activations at the layout's row pitch, the output in y's
            char *hout = last ? (char *)y + (size_t)t * W * D * es : w + ((l & 1) ? L.hb1 : L.hb0);
            const long long hout_ld = last ? D : L.Dp;
            const long long hout_bs = last ? seq * D : (long long)W * L.Dp;
            TXL_TRY(enqueue_block(dtype, B, W, D, H, F, hin, hin_bs, hin_ld, &mems[l], &params[l], R, hout, hout_bs,
                                  hout_ld, w, L, s, &mems[l]));
            hin = hout;
            hin_bs = hout_bs;
            hin_ld = hout_ld;
        }
    }
    return TXL_OK;
}

txl_status txl_stack_fwd_window(txl_dtype dtype, int B, int W, int D, int H, int F, int n_layers, const void *x,
                                long long x_bstride, const txl_layer_params *params, const void *R, int R_len,
                                void *y, long long y_bstride, void *ws, size_t ws_bytes, void *stream) {
    TXL_TRY(check_shape(dtype, B, W, D, H));
    if (D > 1024) return fail(TXL_ERR_UNSUPPORTED, "LayerNorm supports D <= 1024 (got %d)", D);
    if (n_layers < 1) return fail(TXL_ERR_ARG, "n_layers must be >= 1");
    TXL_TRY(check_rows(x, x_bstride, W, D, dtype, "x"));
    TXL_TRY(check_rows(y, y_bstride, W, D, dtype, "y"));
    if (!params) return fail(TXL_ERR_ARG, "params must not be NULL");
    for (int l = 0; l < n_layers; ++l) TXL_TRY(check_block_params(&params[l], F));
    TXL_TRY(check_rows_budget(B, W, 0));
    if (!R || !al4(R)) return fail(TXL_ERR_ARG, "R must be a non-NULL 4-byte aligned pointer");
    if (R_len < W) return fail(TXL_ERR_ARG, "R_len=%d < W = %d", R_len, W);
    const Layout L = plan(TXL_OP_STACK, dtype, B, W, W, D, H, F);
    if (!ws || ws_bytes < L.total) return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
    if ((uintptr_t)ws % 256) return fail(TXL_ERR_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    const char *hin = (const char *)x;
    long long hin_bs = x_bstride, hin_ld = D;
    for (int l = 0; l < n_layers; ++l) {
        const bool last = l == n_layers - 1;
        char *hout = last ? (char *)y : w + ((l & 1) ? L.hb1 : L.hb0);
        const long long hout_ld = last ? D : L.Dp;
        const long long hout_bs = last ? y_bstride : (long long)W * L.Dp;
        TXL_TRY(enqueue_block(dtype, B, W, D, H, F, hin, hin_bs, hin_ld, nullptr, &params[l], R, hout, hout_bs, hout_ld,
                              w, L, s));
        hin = hout;
        hin_bs = hout_bs;
        hin_ld = hout_ld;
    }
    return TXL_OK;
}

txl_status txl_attn_fwd_variant(txl_dtype dtype, txl_pos_variant variant, int B, int W, int D, int H,
                                const void *h, long long h_bstride, const txl_mem *mem, const txl_layer_params *p,
                                const void *aK, const void *aV, int clip, void *out, long long out_bstride,
                                void *ws, size_t ws_bytes, void *stream) {
    TXL_TRY(check_shape(dtype, B, W, D, H));
    if (variant != TXL_POS_SHAW && variant != TXL_POS_ABSOLUTE)
        return fail(TXL_ERR_ARG, "unknown encoding variant %d", (int)variant);
    TXL_TRY(check_rows(h, h_bstride, W, D, dtype, "h"));
    TXL_TRY(check_rows(out, out_bstride, W, D, dtype, "out"));
    TXL_TRY(check_mem(mem, W));
    if (!p) return fail(TXL_ERR_ARG, "params is NULL");
    {
        const void *ptrs[] = {p->Wq, p->WkE, p->Wv, p->Wo};
        const char *names[] = {"Wq", "WkE", "Wv", "Wo"};
        for (int i = 0; i < 4; ++i) {
            if (!ptrs[i]) return fail(TXL_ERR_ARG, "parameter %s is NULL", names[i]);
            if (!al4(ptrs[i])) return fail(TXL_ERR_ARG, "parameter %s must be 4-byte aligned", names[i]);
        }
    }
    if (variant == TXL_POS_SHAW) {
        if (clip < 0 || clip > shaw_max_clip())
            return fail(TXL_ERR_UNSUPPORTED, "clip=%d must be in [0, %d]", clip, shaw_max_clip());
        if (!aK || !aV || !al4(aK) || !al4(aV)) return fail(TXL_ERR_ARG, "aK and aV must be non-NULL and 4-byte aligned");
    }
    const int m = mem ? mem->len : 0;
    TXL_TRY(check_rows_budget(B, W, m));
    const Layout L = plan(TXL_OP_ATTN_VARIANT, dtype, B, W, (mem ? mem->M : 0) + W, D, H, 0);
    if (!ws || ws_bytes < L.total) return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
    if ((uintptr_t)ws % 256) return fail(TXL_ERR_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    const Variant var = {variant, aK, aV, clip};
    TXL_TRY(enqueue_attention(dtype, B, W, D, H, h, h_bstride, mem, nullptr, p, nullptr, w, L, s, &var));
    GemmProblem wo = rows_problem(B, W, D, D, w + L.o, D, (long long)W * D, p->Wo, out, D, out_bstride);
    return hip_check(launch_gemm(dtype == TXL_BF16, single(wo), s), "output projection launch");
}

txl_status txl_add_positions(txl_dtype dtype, int B, int W, int D, const void *x, long long x_bstride, int pos0,
                             void *y, long long y_bstride, void *stream) {
    if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (B < 1 || W < 1 || D < 2 || D % 2) return fail(TXL_ERR_ARG, "need B, W >= 1 and an even D >= 2");
    if (D > 1024) return fail(TXL_ERR_UNSUPPORTED, "positions support D <= 1024 (got %d)", D);
    if (pos0 < 0) return fail(TXL_ERR_ARG, "pos0=%d must be >= 0", pos0);
    TXL_TRY(check_rows(x, x_bstride, W, D, dtype, "x"));
    TXL_TRY(check_rows(y, y_bstride, W, D, dtype, "y"));
    return hip_check(launch_add_positions(dtype == TXL_BF16, x, x_bstride, y, y_bstride, B, W, D, pos0,
                                          (hipStream_t)stream), "position launch");
}

}  // extern "C"

namespace {

// C[e] = A[e] B[e]^T for batch entries e (A [rows][kdim] with row stride a_ld,
// B [cols][kdim]), fp32 output [rows][cols] per entry.
GemmProblem batched_problem(int entries, int rows, int cols, int kdim, const void *a, long long a_ld,
                            const void *b, long long b_ld, void *c) {
    GemmProblem p;
    memset(&p, 0, sizeof(p));
    p.rows = entries * rows; p.cols = cols; p.kdim = kdim;
    p.seg_rows = rows; p.valid_rows = rows;
    p.a_mode = A_ROWS; p.a = a; p.a_ld = a_ld; p.a_bstride = (long long)rows * a_ld;
    p.b_mode = B_ROWS; p.b0 = b; p.b_split = cols; p.b_ld = b_ld; p.b_bstride = (long long)cols * b_ld;
    p.dh = 1; p.dhp = 1; p.heads = 1;
    p.epi = EPI_ROWS; p.c0 = c; p.c_ld = cols; p.c_bstride = (long long)rows * cols; p.out_f32 = 1;
    return p;
}


}  // namespace

extern "C" {

txl_status txl_rel_attn_bwd(txl_dtype dtype, int B, int W, int D, int H, int m, const void *q, const void *k,
                            const void *val, const void *r, const void *u, const void *v, const void *dO,
                            float *dq, float *dk, float *dval, float *dr, float *du, float *dv, void *ws,
                            size_t ws_bytes, void *stream) {
    TXL_TRY(check_shape(dtype, B, W, D, H));
    if (m < 0) return fail(TXL_ERR_ARG, "m=%d must be >= 0", m);
    if ((long long)m + W > 4096) return fail(TXL_ERR_UNSUPPORTED, "the backward supports m + W <= 4096");
    const void *ins[] = {q, k, val, r, u, v, dO};
    const char *in_names[] = {"q", "k", "val", "r", "u", "v", "dO"};
    for (int i = 0; i < 7; ++i)
        if (!ins[i] || !al4(ins[i])) return fail(TXL_ERR_ARG, "%s must be a non-NULL 4-byte aligned pointer", in_names[i]);
    const void *outs[] = {dq, dk, dval, dr, du, dv};
    const char *out_names[] = {"dq", "dk", "dval", "dr", "du", "dv"};
    for (int i = 0; i < 6; ++i)
        if (!outs[i] || !al4(outs[i])) return fail(TXL_ERR_ARG, "%s must be a non-NULL 4-byte aligned pointer", out_names[i]);
    const BwdLayout L = plan_bwd(dtype, B, W, m, D, H);
    const BwdDims &d = L.d;
    if ((long long)B * H * d.Kp >= (1LL << 22)) return fail(TXL_ERR_UNSUPPORTED, "B * H * (m + W) too large");
    if (!ws || ws_bytes < L.total) return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
    if ((uintptr_t)ws % 256) return fail(TXL_ERR_ARG, "workspace must be 256-byte aligned");
    const bool bf = dtype == TXL_BF16;
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    const int G = B * H, Wp = d.Wp, Kp = d.Kp, dp = d.dp, W8 = d.W8;
    // packed operands: (q + u), (q + v) pre-scaled for exp2 scores as in the forward, and the
    // transposed copies the attention kernels and the GEMMs take
    const float lam = (float)(1.4426950408889634 / sqrt((double)d.dh));
    BwdPack pk;
    pk.qu = w + L.qu; pk.qv = w + L.qv; pk.dOh = w + L.dOh; pk.qut = w + L.qut; pk.qvt = w + L.qvt;
    pk.dOt = w + L.dOt; pk.ke = w + L.ke; pk.vk = w + L.vk; pk.ket = w + L.ket; pk.vt = w + L.vt;
    pk.rk = w + L.rk; pk.rt = w + L.rt;
    TXL_TRY(hip_check(launch_bwd_pack(bf, d, pk, q, k, val, r, u, v, dO, lam, s), "backward pack launch"));
    // forward once more for its output and log-sum-exp
    AttnArgs fa;
    memset(&fa, 0, sizeof(fa));
    fa.qu = w + L.qu; fa.qv = w + L.qv; fa.ke = w + L.ke; fa.vt = w + L.vt; fa.rk = w + L.rk;
    fa.o = w + L.o; fa.o_bstride = (long long)W * D;
    fa.B = B; fa.H = H; fa.W = W; fa.Wp = Wp; fa.m = m; fa.K = d.K; fa.Kp = Kp; fa.dh = d.dh; fa.dp = dp; fa.D = D;
    fa.C = Kp; fa.khead = 0; fa.rk_hstride = (long long)rk_table_rows(Kp) * dp; fa.dist = 1;
    fa.lse = (float *)(w + L.lse); fa.nsplit = 1;
    TXL_TRY(hip_check(launch_rel_attn(bf, fa, s), "attention launch"));
    // fused query side: dq, du / dv partials, p and dS key-major, dS by distance
    AttnBwdArgs ba;
    memset(&ba, 0, sizeof(ba));
    ba.qu = w + L.qu; ba.qv = w + L.qv; ba.dO = w + L.dOh; ba.ke = w + L.ke; ba.vk = w + L.vk; ba.kt = w + L.ket;
    ba.rk = w + L.rk; ba.rt = w + L.rt; ba.o = w + L.o; ba.lse = (const float *)(w + L.lse);
    ba.dq = dq; ba.part = (float *)(w + L.part);
    ba.pt = w + L.pt; ba.dst = w + L.dst; ba.dsd = w + L.dsd;
    ba.B = B; ba.H = H; ba.W = W; ba.Wp = Wp; ba.m = m; ba.K = d.K; ba.Kp = Kp; ba.dh = d.dh; ba.dp = dp;
    ba.D = D; ba.rk_hstride = fa.rk_hstride; ba.rt_ld = attn_bwd_rt_ld(Kp); ba.rt_off = attn_bwd_rt_off(m);
    ba.c = (float)(1.0 / sqrt((double)d.dh));
    TXL_TRY(hip_check(launch_rel_attn_bwd(bf, ba, s), "attention backward launch"));
    // dval = P^T dO and dk = dS^T (q+u) per (b, h), written straight into [B][K][D]; dr's part
    // dS_d^T (q+v) per (b, h); all reduced over W8 queries
    GemmProblem gv = batched_problem(G, Kp, dp, W8, w + L.pt, Wp, w + L.dOt, Wp, dval);
    GemmProblem gk = batched_problem(G, Kp, dp, W8, w + L.dst, Wp, w + L.qut, Wp, dk);
    for (GemmProblem *p : {&gv, &gk}) {
        p->epi = EPI_GROWS; p->heads = H; p->dh = d.dh; p->dhp = dp;
        p->c_ld = D; p->c_bstride = (long long)d.K * D; p->c_rows = d.K;
    }
    GemmProblem gr = batched_problem(G, Kp, dp, W8, w + L.dsd, Wp, w + L.qvt, Wp, w + L.drh);
    // key j (distance d) sees no query i < j - m (d - m): each A row is zero before that query
    for (GemmProblem *p : {&gv, &gk, &gr}) { p->kz_on = 1; p->kz_lag = m; }
    TXL_TRY(hip_check(launch_gemm(bf, grouped({gv, gk, gr}), s), "gradient GEMM launch"));
    return hip_check(launch_bwd_finish(d, (const float *)(w + L.drh), (const float *)(w + L.part), dr, du, dv, s),
                     "backward reduction launch");
}

int txl_kv_cache_capacity(int M, int W) {
    if (M < 0 || W < 1) return 0;
    return kv_capacity(M, W);
}

txl_status txl_kv_cache_append(txl_dtype dtype, int B, int D, int H, txl_kv_cache *cache,
                               const txl_layer_params *p, const void *x, long long x_bstride, int n,
                               void *stream) {
    TXL_TRY(check_shape(dtype, B, n < 1 ? 1 : n, D, H));
    if (n < 1) return fail(TXL_ERR_ARG, "n=%d must be >= 1", n);
    TXL_TRY(check_rows(x, x_bstride, n, D, dtype, "x"));
    TXL_TRY(check_attn_params(p));
    const int keep = cache && n > cache->M ? cache->M : n;      // only the last M rows can stay
    TXL_TRY(check_kv_cache(dtype, cache, keep, cache ? (long long)cache->M + 8 : 0, B, D, H));
    if ((long long)B * keep >= (1LL << 22)) return fail(TXL_ERR_UNSUPPORTED, "B * rows = %lld exceeds 2^22", (long long)B * keep);
    const char *first = (const char *)x + (size_t)(n - keep) * D * es_of(dtype);
    // Rows past the new window may reuse slots of rows that leave it (C >= M + keep).
    const GemmProblem kv = kv_cache_problem(B, keep, D, H, attn_dp(D / H), first, x_bstride, p, cache);
    TXL_TRY(hip_check(launch_gemm(dtype == TXL_BF16, single(kv), (hipStream_t)stream), "cache projection launch"));
    kv_cache_advance(cache, keep);
    return TXL_OK;
}

txl_status txl_rel_attn_fwd_cached(txl_dtype dtype, int B, int W, int D, int H, const void *h, long long h_bstride,
                                   txl_kv_cache *cache, const txl_layer_params *p, const void *R, int R_len,
                                   void *out, long long out_bstride, void *ws, size_t ws_bytes, void *stream) {
    TXL_TRY(check_shape(dtype, B, W, D, H));
    TXL_TRY(check_rows(h, h_bstride, W, D, dtype, "h"));
    TXL_TRY(check_rows(out, out_bstride, W, D, dtype, "out"));
    TXL_TRY(check_kv_cache(dtype, cache, W, cache ? (long long)cache->M + W : 0, B, D, H));
    TXL_TRY(check_attn_params(p));
    const int m = cache->len;
    TXL_TRY(check_rows_budget(B, W, m));
    if (!R || !al4(R)) return fail(TXL_ERR_ARG, "R must be a non-NULL 4-byte aligned pointer");
    if (R_len < m + W) return fail(TXL_ERR_ARG, "R_len=%d < cache len + W = %d", R_len, m + W);
    const Layout L = plan(TXL_OP_REL_ATTN_CACHED, dtype, B, W, cache->M + W, D, H, 0);
    if (!ws || ws_bytes < L.total) return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
    if ((uintptr_t)ws % 256) return fail(TXL_ERR_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    TXL_TRY(enqueue_attention(dtype, B, W, D, H, h, h_bstride, nullptr, cache, p, R, w, L, s));
    GemmProblem wo = rows_problem(B, W, D, D, w + L.o, D, (long long)W * D, p->Wo, out, D, out_bstride);
    TXL_TRY(hip_check(launch_gemm(dtype == TXL_BF16, single(wo), s), "output projection launch"));
    kv_cache_advance(cache, W);
    return TXL_OK;
}

txl_status txl_profile_begin(int max_launches) {
    if (max_launches < 1) return fail(TXL_ERR_ARG, "max_launches must be >= 1");
    if (g_prof.on) return fail(TXL_ERR_ARG, "profiling already active");
    for (size_t i = 0; i < g_prof.start.size(); ++i) {
        (void)hipEventDestroy(g_prof.start[i]);
        (void)hipEventDestroy(g_prof.stop[i]);
    }
    g_prof.start.assign(max_launches, nullptr);
    g_prof.stop.assign(max_launches, nullptr);
    for (int i = 0; i < max_launches; ++i) {
        TXL_TRY(hip_check(hipEventCreate(&g_prof.start[i]), "hipEventCreate"));
        TXL_TRY(hip_check(hipEventCreate(&g_prof.stop[i]), "hipEventCreate"));
    }
    g_prof.used = 0;
    g_prof.on = true;
    return TXL_OK;
}

txl_status txl_profile_end(double *total_ms, int *launches) {
    if (!g_prof.on) return fail(TXL_ERR_ARG, "profiling is not active");
    g_prof.on = false;
    g_prof.times.clear();
    double sum = 0.0;
    for (int i = 0; i < g_prof.used; ++i) {
        TXL_TRY(hip_check(hipEventSynchronize(g_prof.stop[i]), "hipEventSynchronize"));
        float ms = 0.f;
        TXL_TRY(hip_check(hipEventElapsedTime(&ms, g_prof.start[i], g_prof.stop[i]), "hipEventElapsedTime"));
        g_prof.times.push_back(ms);
        sum += ms;
    }
    if (total_ms) *total_ms = sum;
    if (launches) *launches = g_prof.used;
    return TXL_OK;
}

txl_status txl_profile_times(double *ms, int capacity, int *n) {
    if (g_prof.on) return fail(TXL_ERR_ARG, "profiling is still active");
    if (capacity < 0 || (capacity > 0 && !ms)) return fail(TXL_ERR_ARG, "ms must hold capacity >= 0 values");
    const int k = std::min(capacity, (int)g_prof.times.size());
    for (int i = 0; i < k; ++i) ms[i] = g_prof.times[i];
    if (n) *n = k;
    return TXL_OK;
}

const char *txl_status_string(txl_status s) {
    switch (s) {
        case TXL_OK: return "ok";
        case TXL_ERR_ARG: return "invalid argument";
        case TXL_ERR_UNSUPPORTED: return "unsupported configuration";
        case TXL_ERR_WORKSPACE: return "workspace missing or too small";
        case TXL_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *txl_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
