// api.hip -- the extern "C" entry points of libwedlm: argument checks,
// launch planning and kernel launches.  No call allocates device memory or
// synchronises the device.
#include <math.h>
#include <atomic>
#include <new>
#include <stdarg.h>
#include <stdio.h>

#include "kernels.hpp"

namespace wedlm {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

__attribute__((format(printf, 2, 3))) static int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

static int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) {
        g_err[0] = 0;
        return WEDLM_OK;
    }
    return fail(WEDLM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace wedlm


using namespace wedlm;

static int check_shape(const wedlm_shape* s) {
    if (!s) return fail(WEDLM_ERR_ARG, "shape is NULL");
    if (s->B < 1 || s->W < 1 || s->W > 64)
        return fail(WEDLM_ERR_SHAPE, "need B >= 1 and 1 <= W <= 64 (B=%d W=%d)", s->B, s->W);
    if (s->Hq < 1 || s->Hkv < 1 || s->Hq % s->Hkv != 0 || s->Hq / s->Hkv > 16)
        return fail(WEDLM_ERR_SHAPE, "need Hkv >= 1, Hq %% Hkv == 0 and Hq/Hkv <= 16 (Hq=%d Hkv=%d)", s->Hq, s->Hkv);
    if (s->D != 64 && s->D != 128) return fail(WEDLM_ERR_UNSUPPORTED, "head dim %d: built for 64 and 128", s->D);
    if (s->page_size != kPage) return fail(WEDLM_ERR_UNSUPPORTED, "page_size %d: built for 16", s->page_size);
    if (s->max_pages < 1 || s->num_pages < 1)
        return fail(WEDLM_ERR_SHAPE, "max_pages (%d) and num_pages (%d) must be >= 1", s->max_pages, s->num_pages);
    if (s->dtype != WEDLM_F32 && s->dtype != WEDLM_BF16) return fail(WEDLM_ERR_ARG, "dtype %d", s->dtype);
    // every element offset must fit the kernels' 64-bit arithmetic and the
    // 32-bit grid: keep the grid below 2^31 work-groups
    if ((int64_t)s->B * s->W > (1ll << 24)) return fail(WEDLM_ERR_SHAPE, "B*W too large");
    return WEDLM_OK;
}

// Checks of wedlm_reorder's arguments and its kernel argument block.
static int reorder_args(const wedlm_shape* s, const uint8_t* filled, const int32_t* pos, const void* q,
                        const void* k, const void* v, void* q_phys, void* k_cache, void* v_cache,
                        const int32_t* block_table, const int32_t* ctx_len, int32_t* perm, double rope_base,
                        int32_t* dev_status, ReorderArgs* a) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (!filled || !pos || !q || !k || !v || !q_phys || !k_cache || !v_cache || !block_table || !ctx_len || !perm)
        return fail(WEDLM_ERR_ARG, "wedlm_reorder: NULL device pointer");
    if (!(rope_base > 1.0) || !isfinite(rope_base)) return fail(WEDLM_ERR_ARG, "rope_base must be > 1");
    a->filled = filled; a->pos = pos; a->q = q; a->k = k; a->v = v; a->q_phys = q_phys;
    a->k_cache = k_cache; a->v_cache = v_cache; a->block_table = block_table; a->ctx_len = ctx_len;
    a->perm = perm; a->status = dev_status;
    a->B = s->B; a->W = s->W; a->Hq = s->Hq; a->Hkv = s->Hkv; a->D = s->D;
    a->max_pages = s->max_pages; a->num_pages = s->num_pages;
    a->log2_base = log2(rope_base);
    a->part = nullptr;   // q, k, v from the given tensors
    a->part_S = 0;
    a->part_N = 0;
    return WEDLM_OK;
}

extern "C" int wedlm_reorder(const wedlm_shape* s, const uint8_t* filled, const int32_t* pos, const void* q,
                             const void* k, const void* v, void* q_phys, void* k_cache, void* v_cache,
                             const int32_t* block_table, const int32_t* ctx_len, int32_t* perm,
                             double rope_base, int32_t* dev_status, void* stream) {
    ReorderArgs a;
    const int rc = reorder_args(s, filled, pos, q, k, v, q_phys, k_cache, v_cache, block_table, ctx_len, perm,
                                rope_base, dev_status, &a);
    if (rc) return rc;
    return hip_status(launch_reorder(a, s->dtype, (hipStream_t)stream), "wedlm_reorder launch");
}

// ---------------------------------------------------------------- attention plan
static std::atomic<int32_t> g_split_override{0};   // process-wide, read by every plan
static std::atomic<int32_t> g_tail_override{-1};   // tail splits: -1 automatic, 0 off, n > 0 that many

// Compute units of the current device (cached per device; 256 on MI355X).
static int device_cus() {
    static std::atomic<int> cache[64];   // 0 = not queried yet; threads may race to fill a slot
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
static const int64_t kMaxContext = 524288;  // keys incl. the window (at most 64 splits)

struct Plan {
    int nw, chunk, RT, row_tiles, nsplit, split_keys, tail, cus;
    size_t ws_bytes, off_ml, off_tail;
};

static Plan make_plan(const wedlm_shape* s, int32_t max_ctx_len) {
    Plan p;
    p.cus = (int)device_cus();
    const int G = s->Hq / s->Hkv;
    const int M = s->W * G;
    p.nw = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
    p.chunk = attn_chunk(s->dtype, p.nw);
    p.RT = 32 * p.nw;
    p.row_tiles = (M + p.RT - 1) / p.RT;
    const int64_t T = (int64_t)max_ctx_len + s->W;
    const int64_t pairs = (int64_t)s->B * s->Hkv * p.row_tiles;
    int64_t sk;
    const int32_t override_keys = g_split_override.load(std::memory_order_relaxed);
    if (override_keys > 0) {
        sk = override_keys;
    } else {
        // One round of work-groups over the device (a bf16 work-group fills a
        // CU's LDS): the key work of every (sequence, KV head, row tile) at
        // the bound is cut so that the splits number about one per CU.  At
        // least 256 bf16 keys per split so the per-split prologue and the
        // fp32 partial (RT*D*4 bytes) stay small next to the K/V a split
        // streams; the fp32 kernel spends eight times the matrix-core
        // instructions per key, so on small grids its splits go down to 64
        // keys (one fp32 sequence, window 8, a few hundred keys: 16.3 vs
        // 19.6 us per decode step; on a 2K-token bf16 prefix 128-key splits
        // were slower than 256).
        const int64_t target = device_cus();
        const int64_t min_keys = s->dtype == WEDLM_F32 ? 64 : 256;
        sk = (T * pairs + target - 1) / target;
        if (sk < min_keys) sk = min_keys;
    }
    sk = (sk + p.chunk - 1) / p.chunk * p.chunk;
    if (sk > (int64_t)kMaxSplitPages * kPage) sk = (int64_t)kMaxSplitPages * kPage;
    // the combine merges at most 64 splits per row
    if ((T + sk - 1) / sk > 64) sk = (T + 63) / 64;
    sk = (sk + p.chunk - 1) / p.chunk * p.chunk;
    if (sk >= T) sk = (T + p.chunk - 1) / p.chunk * p.chunk;  // one split covers everything
    p.split_keys = (int)sk;
    p.nsplit = (int)((T + sk - 1) / sk);
    if (p.nsplit < 1) p.nsplit = 1;
    // Tail splits: a one-split bf16 plan whose (sequence, KV head) groups
    // fill at least half of the CUs in one round is bound by its longest
    // sequences, each streaming alone on one CU after the short ones are
    // done.  The longest 3/8 of the sequences (ranked on the device from
    // ctx_len) get a second work-group for the back part of their keys
    // (where the cut falls: tail_cut); those are dispatched after the first
    // round and start on the CUs the shortest sequences free.  3/8 of the
    // batch measured best at the ragged 32-sequence shape (a quarter, a
    // half, three quarters 1-4 % slower).
    p.tail = 0;
    {
        const int32_t ov = g_tail_override.load(std::memory_order_relaxed);
        const int64_t cus = p.cus;
        const bool fits = s->dtype == WEDLM_BF16 && p.nsplit == 1 && p.row_tiles == 1 && s->B >= 2 &&
                          s->B <= kMaxSplitPages / 2 && pairs <= cus;
        if (fits && ov > 0) p.tail = ov < s->B ? ov : s->B;
        else if (fits && ov < 0 && 2 * pairs >= cus && s->B >= 4) p.tail = (3 * s->B + 7) / 8;
        if (p.tail > 0) p.nsplit = 2;
    }
    p.off_tail = 0;
    if (p.nsplit == 1) {
        p.ws_bytes = 0;
        p.off_ml = 0;
    } else {
        const size_t rows = (size_t)pairs * p.nsplit * p.RT;
        const size_t o_bytes = (rows * s->D * sizeof(float) + 255) / 256 * 256;
        p.off_ml = o_bytes;
        p.ws_bytes = o_bytes + (rows * sizeof(float2) + 255) / 256 * 256;
        if (p.tail > 0) {
            p.off_tail = p.ws_bytes;
            p.ws_bytes += ((size_t)p.tail * s->Hkv * sizeof(int32_t) + 255) / 256 * 256;
        }
    }
    return p;
}

// ---------------------------------------------------------------- Dual-Stream Masking attention
struct DualLayout {
    wedlm_shape sm, sp;   // memory windows (W = 64), prediction windows (W = b)
    size_t kc, vc, qphys, perm, filled_m, pos_m, ctx_m, bt_m, pos_p, ctx_p, bt_p, attn, attn_bytes, total;
};

static int dual_layout(const wedlm_shape* s, int32_t N, DualLayout* L) {
    if (!s) return fail(WEDLM_ERR_ARG, "shape is NULL");
    const int b = s->W;
    if (b != 16 && b != 32 && b != 64)
        return fail(WEDLM_ERR_SHAPE, "dual stream: block size (shape W) must be 16, 32 or 64, got %d", b);
    if (N < 64 || N % 64 != 0 || N > kMaxContext)
        return fail(WEDLM_ERR_SHAPE, "dual stream: N must be a multiple of 64 in [64, %lld], got %d",
                    (long long)kMaxContext, N);
    if (s->B < 1 || (int64_t)s->B * N > (1ll << 24))
        return fail(WEDLM_ERR_SHAPE, "dual stream: need 1 <= sequences and sequences*N <= 2^24");
    const int64_t S = s->B, np = N / kPage, pool = 2 * S * np;
    if (pool > INT32_MAX / 2) return fail(WEDLM_ERR_SHAPE, "dual stream: too many pages");
    L->sm = *s;
    L->sm.B = (int32_t)(S * N / 64); L->sm.W = 64;
    L->sm.max_pages = (int32_t)np; L->sm.num_pages = (int32_t)pool; L->sm.page_size = kPage;
    L->sp = L->sm;
    L->sp.B = (int32_t)(S * N / b); L->sp.W = b;
    int rc = check_shape(&L->sm);
    if (rc) return rc;
    rc = check_shape(&L->sp);
    if (rc) return rc;
    const size_t elt = s->dtype == WEDLM_F32 ? 4 : 2;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t r = o; o += up(bytes); return r; };
    L->kc = take((size_t)pool * s->Hkv * kPage * s->D * elt);
    L->vc = take((size_t)pool * s->Hkv * kPage * s->D * elt);
    L->qphys = take((size_t)S * N * s->Hq * s->D * elt);
    L->perm = take((size_t)S * N * 4);
    L->filled_m = take((size_t)S * N);
    L->pos_m = take((size_t)S * N * 4);
    L->ctx_m = take((size_t)L->sm.B * 4);
    L->bt_m = take((size_t)L->sm.B * np * 4);
    L->pos_p = take((size_t)S * N * 4);
    L->ctx_p = take((size_t)L->sp.B * 4);
    L->bt_p = take((size_t)L->sp.B * np * 4);
    const size_t wa = make_plan(&L->sm, N - 64).ws_bytes, wb = make_plan(&L->sp, N - b).ws_bytes;
    L->attn_bytes = wa > wb ? wa : wb;
    L->attn = take(L->attn_bytes);
    L->total = o;
    return WEDLM_OK;
}

extern "C" size_t wedlm_dual_stream_attn_workspace(const wedlm_shape* s, int32_t N) {
    DualLayout L;
    return dual_layout(s, N, &L) == WEDLM_OK ? L.total : 0;
}

extern "C" int wedlm_dual_stream_attn(const wedlm_shape* s, int32_t N, const void* qm, const void* km, const void* vm,
                                      const void* qp, const void* kp, const void* vp, const uint8_t* flags,
                                      void* out_m, void* out_p, double rope_base, void* workspace, size_t ws_bytes,
                                      int32_t* dev_status, void* stream) {
    DualLayout L;
    int rc = dual_layout(s, N, &L);
    if (rc) return rc;
    if (!qm || !km || !vm || !qp || !kp || !vp || !flags || !out_m || !out_p)
        return fail(WEDLM_ERR_ARG, "wedlm_dual_stream_attn: NULL device pointer");
    if (!workspace || ws_bytes < L.total)
        return fail(WEDLM_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", L.total, workspace ? ws_bytes : 0);
    char* ws = static_cast<char*>(workspace);
    auto I32 = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
    hipStream_t st = (hipStream_t)stream;
    rc = hip_status(launch_dual_layout(reinterpret_cast<uint8_t*>(ws + L.filled_m), I32(L.pos_m), I32(L.ctx_m),
                                       I32(L.bt_m), I32(L.pos_p), I32(L.ctx_p), I32(L.bt_p), s->B, N, s->W, st),
                    "wedlm_dual_stream_attn layout");
    if (rc) return rc;
    void* kc = ws + L.kc;
    void* vc = ws + L.vc;
    void* qph = ws + L.qphys;
    // memory stream: all-observed 64-token windows over the sequence's memory pages
    rc = wedlm_reorder(&L.sm, reinterpret_cast<uint8_t*>(ws + L.filled_m), I32(L.pos_m), qm, km, vm, qph, kc, vc,
                       I32(L.bt_m), I32(L.ctx_m), I32(L.perm), rope_base, dev_status, stream);
    if (rc) return rc;
    rc = wedlm_step_attn(&L.sm, qph, kc, vc, I32(L.bt_m), I32(L.ctx_m), I32(L.perm), out_m, 0.f, N - 64,
                         ws + L.attn, L.attn_bytes, dev_status, stream);
    if (rc) return rc;
    // prediction stream: block windows over the memory prefix and their own pages
    rc = wedlm_reorder(&L.sp, flags, I32(L.pos_p), qp, kp, vp, qph, kc, vc, I32(L.bt_p), I32(L.ctx_p), I32(L.perm),
                       rope_base, dev_status, stream);
    if (rc) return rc;
    return wedlm_step_attn(&L.sp, qph, kc, vc, I32(L.bt_p), I32(L.ctx_p), I32(L.perm), out_p, 0.f, N - s->W,
                           ws + L.attn, L.attn_bytes, dev_status, stream);
}

// ---------------------------------------------------------------- LM head + select / commit
struct LmheadLayout {
    size_t rows, count, part, row_stat, total;
    int nvt, nrg;
};

static bool lmhead_layout(int32_t B, int32_t W, int32_t V, int32_t Dm, LmheadLayout* L) {
    if (B < 1 || W < 1 || W > 64 || (int64_t)B * W > 4096 || V < 1 || Dm < kLmKC || Dm > 65536 ||
        Dm % kLmKC != 0)
        return false;
    const int64_t R = (int64_t)B * W;
    L->nvt = (int)((V + kLmNT - 1) / kLmNT);
    L->nrg = (int)((R + kLmMT - 1) / kLmMT);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    L->rows = 0;
    L->count = up((size_t)R * 4);
    L->part = L->count + 256;
    L->row_stat = L->part + up((size_t)R * L->nvt * sizeof(float4));
    L->total = L->row_stat + up((size_t)R * sizeof(float4));
    return true;
}

extern "C" size_t wedlm_lmhead_select_commit_workspace(int32_t B, int32_t W, int32_t V, int32_t Dm) {
    LmheadLayout L;
    return lmhead_layout(B, W, V, Dm, &L) ? L.total : 0;
}

extern "C" int wedlm_lmhead_select_commit(int32_t B, int32_t W, int32_t V, int32_t Dm, const void* hidden,
                                          const void* lm_head, int32_t* tok, uint8_t* filled, int32_t* pos,
                                          int32_t* ctx_len, int32_t* n_commit, int32_t* committed,
                                          int32_t* argmax_out, float* entropy_out, int64_t* counters, float alpha,
                                          float tau, int32_t mask_id, void* workspace, size_t ws_bytes,
                                          void* stream) {
    LmheadLayout L;
    if (!lmhead_layout(B, W, V, Dm, &L))
        return fail(WEDLM_ERR_SHAPE,
                    "need B >= 1, 1 <= W <= 64, B*W <= 4096, V >= 1, Dm a multiple of %d in [%d, 65536] "
                    "(B=%d W=%d V=%d Dm=%d)", kLmKC, kLmKC, B, W, V, Dm);
    if (!hidden || !lm_head || !tok || !filled || !pos || !ctx_len || !n_commit || !committed)
        return fail(WEDLM_ERR_ARG, "wedlm_lmhead_select_commit: NULL device pointer");
    if (reinterpret_cast<uintptr_t>(hidden) % 16 || reinterpret_cast<uintptr_t>(lm_head) % 16)
        return fail(WEDLM_ERR_ARG, "hidden and lm_head must be 16-byte aligned");
    if (!isfinite(alpha) || !isfinite(tau)) return fail(WEDLM_ERR_ARG, "alpha and tau must be finite");
    if (!workspace || ws_bytes < L.total)
        return fail(WEDLM_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", L.total, workspace ? ws_bytes : 0);
    char* ws = static_cast<char*>(workspace);
    LmheadArgs g;
    g.hidden = static_cast<const bf16_t*>(hidden);
    g.lm_head = static_cast<const bf16_t*>(lm_head);
    g.filled = filled;
    g.rows = reinterpret_cast<int32_t*>(ws + L.rows);
    g.count = reinterpret_cast<int32_t*>(ws + L.count);
    g.part = reinterpret_cast<float4*>(ws + L.part);
    g.row_stat = reinterpret_cast<float4*>(ws + L.row_stat);
    g.R = B * W; g.Dm = Dm; g.V = V; g.nvt = L.nvt; g.nrg = L.nrg;
    hipStream_t st = (hipStream_t)stream;
    int rc = hip_status(launch_lmhead(g, st), "wedlm_lmhead_select_commit launch");
    if (rc != WEDLM_OK) return rc;
    SelectArgs a;
    a.logits = nullptr; a.tok = tok; a.filled = filled; a.pos = pos; a.ctx_len = ctx_len;
    a.n_commit = n_commit; a.committed = committed; a.argmax_out = argmax_out; a.entropy_out = entropy_out;
    a.counters = counters;
    a.part = g.row_stat;
    a.B = B; a.W = W; a.V = V; a.nparts = 1; a.part_len = V;
    a.alpha = alpha; a.tau = tau; a.mask_id = mask_id;
    return hip_status(launch_commit(a, st), "wedlm_lmhead_select_commit launch");
}

// ---------------------------------------------------------------- synthetic decoder step
struct ModelLayout {
    size_t x_res, h, qphys, perm, o, act, P, attn, lm, total;
    size_t attn_bytes, lm_bytes;
    int Sqkv, So, Sgu, Sd;
};

static int model_layout(const wedlm_model* m, const wedlm_shape* s, int32_t max_ctx_len, ModelLayout* L) {
    if (!m || !s) return fail(WEDLM_ERR_ARG, "model or shape is NULL");
    int rc = check_shape(s);
    if (rc) return rc;
    if (s->dtype != WEDLM_BF16) return fail(WEDLM_ERR_UNSUPPORTED, "wedlm_model_step runs in bf16");
    if (m->n_layers < 1 || !m->layers || !m->embed || !m->final_norm || !m->lm_head)
        return fail(WEDLM_ERR_ARG, "model: need n_layers >= 1 and embed, final_norm, lm_head, layers");
    if (m->d_model != s->Hq * s->D || m->d_model % 256 || m->d_ff < 256 || m->d_ff % 256 || m->vocab < 1)
        return fail(WEDLM_ERR_SHAPE, "model: need d_model = Hq*D, d_model and d_ff multiples of 256, vocab >= 1");
    if (!(m->rms_eps > 0.f) || !isfinite(m->rms_eps)) return fail(WEDLM_ERR_ARG, "model: rms_eps must be > 0");
    const int64_t M = (int64_t)s->B * s->W;
    if (M > 4096) return fail(WEDLM_ERR_SHAPE, "model: B*W must be <= 4096");
    if (max_ctx_len < 0 || (int64_t)max_ctx_len + s->W > kMaxContext)
        return fail(WEDLM_ERR_UNSUPPORTED, "context beyond %lld tokens", (long long)kMaxContext);
    LmheadLayout LL;
    if (!lmhead_layout(s->B, s->W, m->vocab, m->d_model, &LL))
        return fail(WEDLM_ERR_SHAPE, "model: LM head shape not supported");
    const int d = m->d_model, F = m->d_ff, HqD = s->Hq * s->D, HkvD = s->Hkv * s->D;
    const int Nqkv = HqD + 2 * HkvD;
    L->Sqkv = gemm_splits((int)M, Nqkv, d);
    L->So = gemm_splits((int)M, d, HqD);
    L->Sgu = gemm_splits((int)M, 2 * F, d);
    L->Sd = gemm_splits((int)M, d, F);
    size_t pmax = 0;
    for (size_t x : {(size_t)L->Sqkv * Nqkv, (size_t)L->So * d, (size_t)L->Sgu * 2 * F, (size_t)L->Sd * d})
        pmax = x > pmax ? x : pmax;
    pmax *= (size_t)M * 4;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t r = o; o += up(bytes); return r; };
    L->x_res = take((size_t)M * d * 4);
    L->h = take((size_t)M * d * 2);
    L->qphys = take((size_t)M * HqD * 2);
    L->perm = take((size_t)M * 4);
    L->o = take((size_t)M * HqD * 2);
    L->act = take((size_t)M * F * 2);
    L->P = take(pmax);
    L->attn_bytes = make_plan(s, max_ctx_len).ws_bytes;
    L->attn = take(L->attn_bytes);
    L->lm_bytes = LL.total;
    L->lm = take(L->lm_bytes);
    L->total = o;
    return WEDLM_OK;
}

extern "C" size_t wedlm_model_step_workspace(const wedlm_model* m, const wedlm_shape* s, int32_t max_ctx_len) {
    ModelLayout L;
    return model_layout(m, s, max_ctx_len, &L) == WEDLM_OK ? L.total : 0;
}

extern "C" int wedlm_model_step(const wedlm_model* m, const wedlm_shape* s, const int32_t* block_table, int32_t* tok,
                                uint8_t* filled, int32_t* pos, int32_t* ctx_len, int32_t* n_commit, int32_t* committed,
                                int32_t* argmax_out, float* entropy_out, int64_t* counters, void* hidden_out,
                                float alpha, float tau,
                                double rope_base, int32_t max_ctx_len, void* workspace, size_t ws_bytes,
                                int32_t* dev_status, void* stream) {
    ModelLayout L;
    int rc = model_layout(m, s, max_ctx_len, &L);
    if (rc) return rc;
    if (!block_table || !tok || !filled || !pos || !ctx_len || !n_commit || !committed)
        return fail(WEDLM_ERR_ARG, "wedlm_model_step: NULL device pointer");
    for (int l = 0; l < m->n_layers; ++l) {
        const wedlm_layer_weights& w = m->layers[l];
        if (!w.attn_norm || !w.wq || !w.wk || !w.wv || !w.wo || !w.mlp_norm || !w.w_gate || !w.w_up || !w.w_down ||
            !w.k_cache || !w.v_cache)
            return fail(WEDLM_ERR_ARG, "wedlm_model_step: layer %d has a NULL pointer", l);
        for (const void* p : {w.attn_norm, w.wq, w.wk, w.wv, w.wo, w.mlp_norm, w.w_gate, w.w_up, w.w_down})
            if (reinterpret_cast<uintptr_t>(p) % 16)
                return fail(WEDLM_ERR_ARG, "wedlm_model_step: layer %d weights must be 16-byte aligned", l);
    }
    for (const void* p : {m->embed, m->final_norm, m->lm_head})
        if (reinterpret_cast<uintptr_t>(p) % 16)
            return fail(WEDLM_ERR_ARG, "wedlm_model_step: embed, final_norm and lm_head must be 16-byte aligned");
    if (!workspace || ws_bytes < L.total)
        return fail(WEDLM_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", L.total, workspace ? ws_bytes : 0);
    char* ws = static_cast<char*>(workspace);
    hipStream_t st = (hipStream_t)stream;
    const int M = s->B * s->W, d = m->d_model, F = m->d_ff, HqD = s->Hq * s->D, HkvD = s->Hkv * s->D;
    auto bf = [&](size_t off) { return reinterpret_cast<bf16_t*>(ws + off); };
    auto f32 = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    auto cbf = [](const void* p) { return static_cast<const bf16_t*>(p); };
    // y = X W^T over up to three weight matrices stacked along the output
    // dimension (rows [0, n1) of W0, [n1, n2) of W1, [n2, N) of W2)
    auto gemm = [&](const void* W0, const void* W1, const void* W2, int n1, int n2, const bf16_t* X, int N, int K,
                    int S, bf16_t* act = nullptr) {
        GemmArgs g{cbf(W0), cbf(W1), cbf(W2), n1, n2, X, f32(L.P), M, N, K, S, 1, act};
        return hip_status(launch_gemm(g, st), "wedlm_model_step gemm");
    };
    const bool swiglu_fused = gemm_swiglu_fused(M, L.Sgu);
    auto rows = [&](bf16_t* out, int N, int S, const void* norm) {
        ModelRowArgs r{};
        r.x_res = f32(L.x_res); r.h = out; r.g = cbf(norm); r.P = f32(L.P);
        r.M = M; r.N = N; r.S = S; r.eps = m->rms_eps; r.status = dev_status;
        return r;
    };
    {
        ModelRowArgs r = rows(bf(L.h), d, 0, m->layers[0].attn_norm);
        r.tok = tok; r.embed = cbf(m->embed); r.n_embed = m->vocab + 1;
        rc = hip_status(launch_embed_rmsnorm(r, st), "wedlm_model_step embed");
        if (rc) return rc;
    }
    const int Nqkv = HqD + 2 * HkvD;
    for (int l = 0; l < m->n_layers; ++l) {
        const wedlm_layer_weights& w = m->layers[l];
        const void* next_norm = l + 1 < m->n_layers ? m->layers[l + 1].attn_norm : m->final_norm;
        // q, k, v of the normalised window rows: one launch over [Wq; Wk; Wv]
        if ((rc = gemm(w.wq, w.wk, w.wv, HqD, HqD + HkvD, bf(L.h), Nqkv, d, L.Sqkv))) return rc;
        // reorder + RoPE + append into this layer's cache straight from the
        // projection's split partials (their bf16-rounded sums are the q, k,
        // v a separate finish launch would store), then attention
        {
            ReorderArgs ra;
            const void* part = ws + L.P;   // q, k, v come from the partials (non-null for the checks)
            if ((rc = reorder_args(s, filled, pos, part, part, part, ws + L.qphys, w.k_cache,
                                   w.v_cache, block_table, ctx_len, reinterpret_cast<int32_t*>(ws + L.perm),
                                   rope_base, dev_status, &ra)))
                return rc;
            ra.part = f32(L.P);
            ra.part_S = L.Sqkv;
            ra.part_N = Nqkv;
            if ((rc = hip_status(launch_reorder_from_partials(ra, st), "wedlm_model_step reorder"))) return rc;
        }
        rc = wedlm_step_attn(s, ws + L.qphys, w.k_cache, w.v_cache, block_table, ctx_len,
                             reinterpret_cast<int32_t*>(ws + L.perm), ws + L.o, 0.f, max_ctx_len, ws + L.attn,
                             L.attn_bytes, dev_status, stream);
        if (rc) return rc;
        // x += o Wo^T; h = RMSNorm(x) * mlp_norm
        if ((rc = gemm(w.wo, w.wo, w.wo, d, d, bf(L.o), d, HqD, L.So))) return rc;
        if ((rc = hip_status(launch_add_rmsnorm(rows(bf(L.h), d, L.So, w.mlp_norm), st), "wedlm_model_step norm")))
            return rc;
        // act = silu(h Wg^T) * (h Wu^T): one launch over [Wg; Wu]; with one
        // K split the launch writes act itself, otherwise a finish sums splits
        if (swiglu_fused) {
            if ((rc = gemm(w.w_gate, w.w_up, w.w_up, F, 2 * F, bf(L.h), 2 * F, d, 1, bf(L.act)))) return rc;
        } else {
            if ((rc = gemm(w.w_gate, w.w_up, w.w_up, F, 2 * F, bf(L.h), 2 * F, d, L.Sgu))) return rc;
            if ((rc = hip_status(launch_finish_swiglu(rows(bf(L.act), 2 * F, L.Sgu, nullptr), st),
                                 "wedlm_model_step finish")))
                return rc;
        }
        // x += act Wd^T; h = RMSNorm(x) * next norm
        if ((rc = gemm(w.w_down, w.w_down, w.w_down, d, d, bf(L.act), d, F, L.Sd))) return rc;
        if ((rc = hip_status(launch_add_rmsnorm(rows(bf(L.h), d, L.Sd, next_norm), st), "wedlm_model_step norm")))
            return rc;
    }
    if (hidden_out) {
        rc = hip_status(hipMemcpyAsync(hidden_out, ws + L.h, (size_t)M * d * 2, hipMemcpyDeviceToDevice, st),
                        "wedlm_model_step hidden copy");
        if (rc) return rc;
    }
    return wedlm_lmhead_select_commit(s->B, s->W, m->vocab, d, ws + L.h, m->lm_head, tok, filled, pos, ctx_len,
                                      n_commit, committed, argmax_out, entropy_out, counters, alpha, tau, m->vocab,
                                      ws + L.lm, L.lm_bytes, stream);
}

extern "C" int wedlm_attn_plan(const wedlm_shape* s, int32_t max_ctx_len, int32_t* nsplit, int32_t* split_keys) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (max_ctx_len < 0) return fail(WEDLM_ERR_ARG, "max_ctx_len must be >= 0");
    if ((int64_t)max_ctx_len + s->W > kMaxContext)
        return fail(WEDLM_ERR_UNSUPPORTED, "context beyond %lld tokens", (long long)kMaxContext);
    Plan p = make_plan(s, max_ctx_len);
    if (nsplit) *nsplit = p.nsplit;
    if (split_keys) *split_keys = p.split_keys;
    g_err[0] = 0;
    return WEDLM_OK;
}

extern "C" int wedlm_set_attn_split_keys(int32_t keys) {
    if (keys != 0 && (keys < 64 || keys > kMaxSplitPages * kPage || keys % 64 != 0))
        return fail(WEDLM_ERR_ARG, "split keys must be 0 or a multiple of 64 in [64, %d]", kMaxSplitPages * kPage);
    g_split_override.store(keys, std::memory_order_relaxed);
    g_err[0] = 0;
    return WEDLM_OK;
}

extern "C" int32_t wedlm_attn_tail(const wedlm_shape* s, int32_t max_ctx_len) {
    if (check_shape(s) || max_ctx_len < 0 || (int64_t)max_ctx_len + s->W > kMaxContext) return -1;
    g_err[0] = 0;
    return make_plan(s, max_ctx_len).tail;
}

extern "C" int wedlm_set_attn_tail(int32_t n) {
    if (n < -1) return fail(WEDLM_ERR_ARG, "tail must be -1 (automatic), 0 (off) or a sequence count");
    g_tail_override.store(n, std::memory_order_relaxed);
    g_err[0] = 0;
    return WEDLM_OK;
}

extern "C" size_t wedlm_step_attn_workspace(const wedlm_shape* s, int32_t max_ctx_len) {
    if (check_shape(s) || max_ctx_len < 0) return 0;
    return make_plan(s, max_ctx_len).ws_bytes;
}

static int step_attn(const wedlm_shape* s, const void* q_phys, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* ctx_len, const int32_t* perm, void* out, float scale,
                     int32_t max_ctx_len, void* workspace, size_t ws_bytes, int32_t* dev_status, void* stream);

extern "C" int wedlm_step_attn(const wedlm_shape* s, const void* q_phys, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_len, const int32_t* perm, void* out,
                               float scale, int32_t max_ctx_len, void* workspace, size_t ws_bytes,
                               int32_t* dev_status, void* stream) {
    return step_attn(s, q_phys, k_cache, v_cache, block_table, ctx_len, perm, out, scale, max_ctx_len, workspace,
                     ws_bytes, dev_status, stream);
}

// ---------------------------------------------------------------- attention without a caller workspace
// The split partials of wedlm_step_attn_noalloc live in this file-scope
// device array (one copy per GPU, kept until the process ends).  In host
// code `scratch` only names the symbol: its device address on the current
// GPU comes from hipGetSymbolAddress, taken once per device and cached.
static constexpr size_t kAttnScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

static void* scratch_ptr(int* err_dev) {
    static std::atomic<void*> cache[64];   // per device; threads may race to fill a slot with the same value
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        *err_dev = dev;
        return nullptr;
    }
    void* p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            *err_dev = dev;
            return nullptr;
        }
        cache[dev].store(p, std::memory_order_release);
    }
    return p;
}

extern "C" size_t wedlm_step_attn_noalloc_limit(void) { return kAttnScratchBytes; }

extern "C" int wedlm_step_attn_noalloc(const wedlm_shape* s, const void* q_phys, const void* k_cache,
                                       const void* v_cache, const int32_t* block_table, const int32_t* ctx_len,
                                       const int32_t* perm, void* out, float scale, int32_t max_ctx_len,
                                       int32_t* dev_status, void* stream) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (max_ctx_len < 0) return fail(WEDLM_ERR_ARG, "max_ctx_len must be >= 0");
    if ((int64_t)max_ctx_len + s->W > kMaxContext)
        return fail(WEDLM_ERR_UNSUPPORTED, "context of %lld tokens: built for up to %lld",
                    (long long)max_ctx_len + s->W, (long long)kMaxContext);
    const size_t need = make_plan(s, max_ctx_len).ws_bytes;
    if (need > kAttnScratchBytes)
        return fail(WEDLM_ERR_WORKSPACE,
                    "wedlm_step_attn_noalloc: this shape needs %zu bytes of split partials, the built-in scratch "
                    "holds %zu; use wedlm_step_attn with a workspace", need, kAttnScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        int dev = -1;
        ws = scratch_ptr(&dev);
        if (!ws) return fail(WEDLM_ERR_HIP, "wedlm_step_attn_noalloc: no scratch address on device %d", dev);
    }
    return step_attn(s, q_phys, k_cache, v_cache, block_table, ctx_len, perm, out, scale, max_ctx_len, ws, need,
                     dev_status, stream);
}

// Checks of wedlm_step_attn's arguments, its plan and its kernel argument
// block.
static int attn_args(const wedlm_shape* s, const void* q_phys, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* ctx_len, const int32_t* perm, void* out, float scale,
                     int32_t max_ctx_len, void* workspace, size_t ws_bytes, int32_t* dev_status, AttnArgs* ap,
                     Plan* pp) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (!q_phys || !k_cache || !v_cache || !block_table || !ctx_len || !perm || !out)
        return fail(WEDLM_ERR_ARG, "wedlm_step_attn: NULL device pointer");
    if (max_ctx_len < 0 || (int64_t)max_ctx_len + s->W > (int64_t)s->max_pages * kPage)
        return fail(WEDLM_ERR_SHAPE, "max_ctx_len %d + W exceeds max_pages * page_size", max_ctx_len);
    if ((int64_t)max_ctx_len + s->W > kMaxContext)
        return fail(WEDLM_ERR_UNSUPPORTED, "context of %lld tokens: built for up to %lld (64 splits of 8192 keys)",
                    (long long)max_ctx_len + s->W, (long long)kMaxContext);
    if (!(scale >= 0.f) || !isfinite(scale)) return fail(WEDLM_ERR_ARG, "scale must be finite and >= 0");
    Plan p = make_plan(s, max_ctx_len);
    if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes))
        return fail(WEDLM_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", p.ws_bytes, workspace ? ws_bytes : 0);
    AttnArgs& a = *ap;
    a.q = q_phys; a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
    a.ctx_len = ctx_len; a.perm = perm; a.out = out;
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = p.ws_bytes ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + p.off_ml) : nullptr;
    a.tail = p.tail;
    a.tail_free = p.tail ? (int)(p.cus > (int64_t)s->B * s->Hkv ? p.cus - (int64_t)s->B * s->Hkv : 0) : 0;
    a.tail_seq = p.tail ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.off_tail) : nullptr;
    a.status = dev_status;
    a.B = s->B; a.W = s->W; a.Hq = s->Hq; a.Hkv = s->Hkv; a.G = s->Hq / s->Hkv; a.M = s->W * a.G;
    a.max_pages = s->max_pages; a.num_pages = s->num_pages;
    a.RT = p.RT; a.row_tiles = p.row_tiles; a.nsplit = p.nsplit; a.split_keys = p.split_keys;
    a.split_align = p.chunk;
    a.max_ctx = max_ctx_len;
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)s->D);
    a.scale_log2 = sc * kLog2e;
    *pp = p;
    return WEDLM_OK;
}

static int step_attn(const wedlm_shape* s, const void* q_phys, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* ctx_len, const int32_t* perm, void* out, float scale,
                     int32_t max_ctx_len, void* workspace, size_t ws_bytes, int32_t* dev_status, void* stream) {
    AttnArgs a;
    Plan p;
    const int rc = attn_args(s, q_phys, k_cache, v_cache, block_table, ctx_len, perm, out, scale, max_ctx_len,
                             workspace, ws_bytes, dev_status, &a, &p);
    if (rc) return rc;
    return hip_status(launch_attn(a, s->dtype, s->D, p.nw, (hipStream_t)stream), "wedlm_step_attn launch");
}

// ---------------------------------------------------------------- select / commit
static const int kPartLen = 16384;   // most logits per work-group: 256 threads x 16 float4
static std::atomic<int32_t> g_parts_override{0};   // process-wide, read by every select plan

// Parts of a row: as few as kPartLen allows.  A vocab_stats work-group's
// time is mostly latency (the slot flag, then one round of 16 loads per
// thread), so more, shorter parts only add work-groups: on a 151936-logit
// vocabulary 10 parts beat 16 to 64 at every window size measured (1 x 16
// up to 64 x 16 slots).  Equal lengths (multiples of 4) so that no
// work-group is left with a short tail.
static void select_plan(int32_t B, int32_t W, int32_t V, int* nparts, int* part_len) {
    (void)B; (void)W;
    int np = (V + kPartLen - 1) / kPartLen;
    const int32_t forced = g_parts_override.load(std::memory_order_relaxed);
    if (forced > np) np = forced;
    if (np > (V + 3) / 4) np = (V + 3) / 4;                 // at least 4 logits per part
    if (np < 1) np = 1;
    const int pl = ((V + np - 1) / np + 3) / 4 * 4;
    *part_len = pl;
    *nparts = (V + pl - 1) / pl;
}

extern "C" int wedlm_set_select_parts(int32_t parts) {
    if (parts < 0 || parts > 4096) return fail(WEDLM_ERR_ARG, "select parts must be 0 or in [1, 4096], got %d", parts);
    g_parts_override.store(parts, std::memory_order_relaxed);
    g_err[0] = 0;
    return WEDLM_OK;
}

extern "C" size_t wedlm_select_commit_workspace(int32_t B, int32_t W, int32_t V) {
    if (B < 1 || W < 1 || W > 64 || V < 1) return 0;
    int np, pl;
    select_plan(B, W, V, &np, &pl);
    return ((size_t)B * W * np * sizeof(float4) + 255) / 256 * 256;
}

// Checks of wedlm_select_commit's arguments and its kernel argument block.
static int select_args(int32_t B, int32_t W, int32_t V, const float* logits, int32_t* tok, uint8_t* filled,
                       int32_t* pos, int32_t* ctx_len, int32_t* n_commit, int32_t* committed, int32_t* argmax_out,
                       float* entropy_out, int64_t* counters, float alpha, float tau, int32_t mask_id,
                       void* workspace, size_t ws_bytes, SelectArgs* ap) {
    if (B < 1 || W < 1 || W > 64 || V < 1)
        return fail(WEDLM_ERR_SHAPE, "need B >= 1, 1 <= W <= 64, V >= 1 (B=%d W=%d V=%d)", B, W, V);
    int np, pl;
    select_plan(B, W, V, &np, &pl);
    // the dispatch counts work-items in 32 bits: at most 2^24 - 1 work-groups of 256
    if ((int64_t)B * W * np > (1ll << 24) - 1 || V > (1 << 30))
        return fail(WEDLM_ERR_SHAPE, "grid too large (B=%d W=%d parts=%d)", B, W, np);
    if (!logits || !tok || !filled || !pos || !ctx_len || !n_commit || !committed)
        return fail(WEDLM_ERR_ARG, "wedlm_select_commit: NULL device pointer");
    if (!isfinite(alpha) || !isfinite(tau)) return fail(WEDLM_ERR_ARG, "alpha and tau must be finite");
    const size_t need = wedlm_select_commit_workspace(B, W, V);
    if (!workspace || ws_bytes < need)
        return fail(WEDLM_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace ? ws_bytes : 0);
    SelectArgs& a = *ap;
    a.logits = logits; a.tok = tok; a.filled = filled; a.pos = pos; a.ctx_len = ctx_len;
    a.n_commit = n_commit; a.committed = committed; a.argmax_out = argmax_out; a.entropy_out = entropy_out;
    a.counters = counters;
    a.part = static_cast<float4*>(workspace);
    a.B = B; a.W = W; a.V = V; a.nparts = np; a.part_len = pl;
    a.alpha = alpha; a.tau = tau; a.mask_id = mask_id;
    return WEDLM_OK;
}

extern "C" int wedlm_select_commit(int32_t B, int32_t W, int32_t V, const float* logits, int32_t* tok,
                                   uint8_t* filled, int32_t* pos, int32_t* ctx_len, int32_t* n_commit,
                                   int32_t* committed, int32_t* argmax_out, float* entropy_out, int64_t* counters,
                                   float alpha, float tau, int32_t mask_id, void* workspace, size_t ws_bytes,
                                   void* stream) {
    SelectArgs a;
    const int rc = select_args(B, W, V, logits, tok, filled, pos, ctx_len, n_commit, committed, argmax_out,
                               entropy_out, counters, alpha, tau, mask_id, workspace, ws_bytes, &a);
    if (rc) return rc;
    return hip_status(launch_select(a, (hipStream_t)stream), "wedlm_select_commit launch");
}

// ---------------------------------------------------------------- whole decode step
// Workspace of wedlm_decode_step: the attention's split partials, then the
// vocabulary partials, each on a 256-byte boundary.
static size_t step_attn_bytes(const wedlm_shape* s, int32_t max_ctx_len) {
    return (make_plan(s, max_ctx_len).ws_bytes + 255) / 256 * 256;
}

extern "C" size_t wedlm_decode_step_workspace(const wedlm_shape* s, int32_t max_ctx_len, int32_t V) {
    if (check_shape(s) || max_ctx_len < 0 || (int64_t)max_ctx_len + s->W > kMaxContext) return 0;
    const size_t sel = wedlm_select_commit_workspace(s->B, s->W, V);
    return sel ? step_attn_bytes(s, max_ctx_len) + sel : 0;
}

static int decode_step(const wedlm_shape* s, const wedlm_step_io* io, void* workspace, size_t ws_bytes,
                       void* stream, const LaunchTiming* tm);

extern "C" int wedlm_decode_step(const wedlm_shape* s, const wedlm_step_io* io, void* workspace, size_t ws_bytes,
                                 void* stream) {
    return decode_step(s, io, workspace, ws_bytes, stream, nullptr);
}

extern "C" int wedlm_decode_step_timed(const wedlm_shape* s, const wedlm_step_io* io, void* workspace,
                                       size_t ws_bytes, void* stream, void* attn_start, void* attn_stop) {
    LaunchTiming tm;
    tm.start = static_cast<hipEvent_t>(attn_start);
    tm.stop = static_cast<hipEvent_t>(attn_stop);
    return decode_step(s, io, workspace, ws_bytes, stream, (attn_start || attn_stop) ? &tm : nullptr);
}

static int decode_step(const wedlm_shape* s, const wedlm_step_io* io, void* workspace, size_t ws_bytes,
                       void* stream, const LaunchTiming* tm) {
    if (!io) return fail(WEDLM_ERR_ARG, "wedlm_decode_step: io is NULL");
    int rc = check_shape(s);
    if (rc) return rc;
    if (io->max_ctx_len < 0) return fail(WEDLM_ERR_ARG, "max_ctx_len must be >= 0");
    if ((int64_t)io->max_ctx_len + s->W > kMaxContext)
        return fail(WEDLM_ERR_UNSUPPORTED, "context of %lld tokens: built for up to %lld",
                    (long long)io->max_ctx_len + s->W, (long long)kMaxContext);
    const size_t need = wedlm_decode_step_workspace(s, io->max_ctx_len, io->V);
    if (need == 0) return fail(WEDLM_ERR_SHAPE, "need V >= 1 (V=%d)", io->V);
    if (!workspace || ws_bytes < need)
        return fail(WEDLM_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace ? ws_bytes : 0);
    char* ws = static_cast<char*>(workspace);
    const size_t attn_bytes = step_attn_bytes(s, io->max_ctx_len);
    ReorderArgs ra;
    AttnArgs aa;
    Plan p;
    SelectArgs sa;
    if ((rc = reorder_args(s, io->filled, io->pos, io->q, io->k, io->v, io->q_phys, io->k_cache, io->v_cache,
                           io->block_table, io->ctx_len, io->perm, io->rope_base, io->dev_status, &ra)))
        return rc;
    if ((rc = attn_args(s, io->q_phys, io->k_cache, io->v_cache, io->block_table, io->ctx_len, io->perm, io->out,
                        io->scale, io->max_ctx_len, attn_bytes ? ws : nullptr, attn_bytes, io->dev_status, &aa,
                        &p)))
        return rc;
    if ((rc = select_args(s->B, s->W, io->V, io->logits, io->tok, io->filled, io->pos, io->ctx_len, io->n_commit,
                          io->committed, io->argmax_out, io->entropy_out, io->counters, io->alpha, io->tau,
                          io->mask_id, ws + attn_bytes, ws_bytes - attn_bytes, &sa)))
        return rc;
    // the front launch is one-dimensional with 256 work-items per work-group
    // (one per slot, then one per vocabulary unit): its work-item count must
    // fit the dispatch's 32 bits
    if ((int64_t)s->B * s->W + (int64_t)s->B * s->W * sa.nparts >= (1ll << 24))
        return fail(WEDLM_ERR_SHAPE, "wedlm_decode_step: grid too large (B=%d W=%d parts=%d)", s->B, s->W, sa.nparts);
    hipStream_t st = (hipStream_t)stream;
    if ((rc = hip_status(launch_step_front(ra, sa, s->dtype, st), "wedlm_decode_step front launch"))) return rc;
    if ((rc = hip_status(launch_attn_split(aa, s->dtype, s->D, p.nw, st, tm),
                         "wedlm_decode_step attention launch")))
        return rc;
    return hip_status(launch_step_back(aa, sa, s->dtype, s->D, st), "wedlm_decode_step back launch");
}

// ---------------------------------------------------------------- graph capture
struct wedlm_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

extern "C" int wedlm_graph_begin(void* stream) {
    if (!stream) return fail(WEDLM_ERR_ARG, "graph capture needs a created stream, not the default stream");
    return hip_status(hipStreamBeginCapture((hipStream_t)stream, hipStreamCaptureModeThreadLocal),
                      "wedlm_graph_begin");
}

extern "C" int wedlm_graph_end(void* stream, wedlm_graph** out) {
    if (!stream || !out) return fail(WEDLM_ERR_ARG, "wedlm_graph_end: NULL stream or output");
    *out = nullptr;
    hipGraph_t g = nullptr;
    int rc = hip_status(hipStreamEndCapture((hipStream_t)stream, &g), "wedlm_graph_end capture");
    if (rc) return rc;
    hipGraphExec_t e = nullptr;
    rc = hip_status(hipGraphInstantiate(&e, g, nullptr, nullptr, 0), "wedlm_graph_end instantiate");
    if (rc) {
        (void)hipGraphDestroy(g);
        return rc;
    }
    wedlm_graph* w = new (std::nothrow) wedlm_graph{g, e};
    if (!w) {
        (void)hipGraphExecDestroy(e);
        (void)hipGraphDestroy(g);
        return fail(WEDLM_ERR_ARG, "wedlm_graph_end: out of host memory");
    }
    *out = w;
    g_err[0] = 0;
    return WEDLM_OK;
}

extern "C" int wedlm_graph_launch(const wedlm_graph* g, void* stream) {
    if (!g) return fail(WEDLM_ERR_ARG, "wedlm_graph_launch: NULL graph");
    return hip_status(hipGraphLaunch(g->exec, (hipStream_t)stream), "wedlm_graph_launch");
}

extern "C" int wedlm_graph_nodes(const wedlm_graph* g, size_t* kernels, size_t* others) {
    if (!g || !kernels || !others) return fail(WEDLM_ERR_ARG, "wedlm_graph_nodes: NULL argument");
    size_t n = 0;
    int rc = hip_status(hipGraphGetNodes(g->graph, nullptr, &n), "wedlm_graph_nodes");
    if (rc) return rc;
    *kernels = *others = 0;
    if (n == 0) return WEDLM_OK;
    hipGraphNode_t* nodes = new (std::nothrow) hipGraphNode_t[n];
    if (!nodes) return fail(WEDLM_ERR_ARG, "wedlm_graph_nodes: out of host memory");
    rc = hip_status(hipGraphGetNodes(g->graph, nodes, &n), "wedlm_graph_nodes");
    for (size_t i = 0; rc == WEDLM_OK && i < n; ++i) {
        hipGraphNodeType t;
        rc = hip_status(hipGraphNodeGetType(nodes[i], &t), "wedlm_graph_nodes");
        if (rc == WEDLM_OK) ++(t == hipGraphNodeTypeKernel ? *kernels : *others);
    }
    delete[] nodes;
    return rc;
}

extern "C" void wedlm_graph_destroy(wedlm_graph* g) {
    if (!g) return;
    (void)hipGraphExecDestroy(g->exec);
    (void)hipGraphDestroy(g->graph);
    delete g;
}

extern "C" const char* wedlm_last_error(void) { return g_err; }

extern "C" const char* wedlm_version(void) { return "wedlm-mi355x 0.1 (gfx950)"; }
