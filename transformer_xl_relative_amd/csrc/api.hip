// api.hip -- C ABI of libxlrel: host-side validation, workspace layout and the
// launch sequence of the relative attention layer. Declarations and the
// contract of every entry point are in include/xl_rel.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/xl_rel.h"
#include "xl_internal.hpp"

// Workspace of xl_segment_step_noalloc: one copy per GPU, resident from the
// library's load until the process ends. Host code never passes this name to a
// kernel or a copy: it is a host-side stand-in, and the device address comes
// from hipGetSymbolAddress (scratch_ptr below).
static __device__ __attribute__((aligned(256))) unsigned char scratch[XL_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;
thread_local void* g_ev_begin = nullptr;
thread_local void* g_ev_end = nullptr;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(XL_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kI32 = 2147483647;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t esize(int dt) { return dt == XL_BF16 ? 2 : 4; }

// longest context the bf16 attention's LDS bias table covers (80 KB of tiles
// and rings plus 4 bytes per table entry, mlen + qlen + 384 entries, <= 160 KB)
constexpr int64_t kMaxBiasKlen = (80 * 1024) / 4 - 384;

// Validate the shape part of a descriptor (mlen given separately).
int check_desc(const xl_attn_desc* d, int64_t mlen, bool need_dmodel) {
    if (!d) return fail(XL_NULL_ARG, "desc is NULL");
    if (d->batch < 1 || d->n_head < 1 || d->qlen < 1 || mlen < 0)
        return fail(XL_BAD_SHAPE, "batch, n_head, qlen must be >= 1 and mlen >= 0 (got %lld, %lld, %lld, %lld)",
                    (long long)d->batch, (long long)d->n_head, (long long)d->qlen, (long long)mlen);
    // every size on its own first, so that the products below cannot overflow
    if (d->batch > kI32 || d->n_head > kI32 || d->qlen > kI32 || mlen > kI32)
        return fail(XL_UNSUPPORTED, "batch, n_head, qlen and mlen must each be below 2^31");
    if (d->dtype != XL_BF16 && d->dtype != XL_F32) return fail(XL_BAD_SHAPE, "dtype must be XL_F32 or XL_BF16");
    if (!((d->dtype == XL_BF16 && d->d_head == 64) || (d->dtype == XL_F32 && d->d_head == 8)))
        return fail(XL_UNSUPPORTED, "supported (dtype, d_head): (bf16, 64), (f32, 8); got (%d, %lld)", (int)d->dtype,
                    (long long)d->d_head);
    if (need_dmodel) {
        if (d->d_model < 2 || (d->d_model & 1)) return fail(XL_BAD_SHAPE, "d_model must be even and >= 2");
        // the projection GEMMs advance K in whole 64-byte stages
        const int64_t mult = d->dtype == XL_BF16 ? 32 : 16;
        if (d->d_model % mult) return fail(XL_UNSUPPORTED, "d_model must be a multiple of %lld", (long long)mult);
        if ((d->n_head * d->d_head) % mult)
            return fail(XL_UNSUPPORTED, "n_head * d_head must be a multiple of %lld", (long long)mult);
        if (d->out_dtype != XL_BF16 && d->out_dtype != XL_F32) return fail(XL_BAD_SHAPE, "bad out_dtype");
        if (d->d_model > 65536) return fail(XL_UNSUPPORTED, "d_model above 65536");
        if (!(d->base == 0.0 || (d->base > 0.0 && isfinite(d->base)))) return fail(XL_BAD_SHAPE, "base must be > 0");
        if (!isfinite(d->scale)) return fail(XL_BAD_SHAPE, "scale must be finite");
    }
    if (d->bias_clamp > 65535) return fail(XL_UNSUPPORTED, "bias_clamp above 65535");
    if (d->bias_kind != XL_BIAS_CLAMP && d->bias_kind != XL_BIAS_T5)
        return fail(XL_BAD_SHAPE, "bias_kind must be XL_BIAS_CLAMP or XL_BIAS_T5");
    if (d->flags & ~XL_REUSE_TABLE) return fail(XL_BAD_SHAPE, "unknown flags 0x%x", (unsigned)d->flags);
    if (d->attn_splits < 0 || d->attn_splits > xl::kMaxAttnSplits)
        return fail(XL_BAD_SHAPE, "attn_splits must be in [0, %d]", xl::kMaxAttnSplits);
    const int64_t klen = mlen + d->qlen;
    const int64_t hd = d->n_head * d->d_head;
    // every element count a kernel indexes with 32-bit arithmetic must fit
    if (klen > kI32 / 128 || d->batch > kI32 / 2 / klen || hd > 65536 || d->batch > kI32 / 64 / d->n_head)
        return fail(XL_UNSUPPORTED, "problem too large for the 32-bit element offsets of the kernels");
    // the keys (and the memory rows) beyond 2^40 elements would not fit any
    // device; below it every tile count of the projection launches fits an int
    constexpr double kMaxElems = 1099511627776.0;   // 2^40
    if ((double)d->batch * d->n_head * klen * d->d_head > kMaxElems ||
        (need_dmodel && (double)d->batch * klen * d->d_model > kMaxElems))
        return fail(XL_UNSUPPORTED, "problem larger than 2^40 elements per tensor");
    if (d->batch * d->n_head * ((d->qlen + 127) / 128) > kI32) return fail(XL_UNSUPPORTED, "grid too large");
    // the bf16 attention keeps the bias table of a workgroup's distances in LDS
    if (d->bias_clamp >= 0 && d->dtype == XL_BF16 && klen > kMaxBiasKlen)
        return fail(XL_UNSUPPORTED, "with a bias table, mlen + qlen must be <= %lld", (long long)kMaxBiasKlen);
    return XL_OK;
}

// key splits of the fused attention (bf16 only)
xl::SplitPlan splits_of(const xl_attn_desc* d, int64_t mlen) {
    if (d->dtype != XL_BF16) return {0, 1};
    return xl::attn_bf16_split_plan(d->batch, d->n_head, d->qlen, mlen, d->attn_splits);
}
// (sized for every memory length up to mlen: a caller may size one workspace
// for its longest memory and run shorter ones in it)
size_t part_bytes_of(const xl_attn_desc* d, int64_t mlen) {
    (void)mlen;
    return d->dtype == XL_BF16 ? xl::attn_bf16_part_bytes_bound(d->batch, d->n_head, d->qlen, d->attn_splits) : 0;
}

int64_t n_rel_of(const xl_attn_desc* d, int64_t klen) {
    return d->clamp_len < 0 ? klen : (klen < d->clamp_len + 1 ? klen : d->clamp_len + 1);
}

// kv_ring: the keys and values live in the caller's key ring (no k, vt regions)
void fill_layout(const xl_attn_desc* d, int64_t mlen, xl_ws_layout* L, bool kv_ring = false) {
    const size_t es = esize(d->dtype);
    const int64_t B = d->batch, H = d->n_head, dh = d->d_head, q = d->qlen, D = d->d_model;
    const int64_t klen = mlen + q;
    const int64_t ldv = (klen + 63) / 64 * 64;
    const int64_t n_rel = n_rel_of(d, klen);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    L->q = take((size_t)(B * H * q * dh) * es);
    L->k = take(kv_ring ? 0 : (size_t)(B * H * klen * dh) * es);
    L->vt = take(kv_ring ? 0 : (size_t)(B * H * dh * ldv) * es);
    L->rel = take((size_t)(n_rel * D) * es);
    L->r = take((size_t)(H * n_rel * dh) * es);
    L->attn = take((size_t)(B * q * H * dh) * es);
    L->part = take(part_bytes_of(d, mlen));
    L->total = off;
    L->klen = klen;
    L->ldv = ldv;
    L->n_rel = n_rel;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* pa = (const char*)a;
    const char* pb = (const char*)b;
    return pa < pb + nb && pb < pa + na;
}

int run_core(const xl::AttnArgs& a, bool bf16, int dh, hipStream_t s) {
    // with timing events set, the runtime timestamps the kernel itself
    const bool timed = g_ev_begin && g_ev_end;
    hipError_t e = xl::launch_attn(a, bf16, dh, s, timed ? (hipEvent_t)g_ev_begin : nullptr,
                                   timed ? (hipEvent_t)g_ev_end : nullptr);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return XL_OK;
}

// The layer forward (residual, when not null: [B, qlen, D] in desc->dtype,
// added to the output projection) on a memory that is either a plain [B, mlen, D] tensor
// (ring_len == mlen, ring_head == 0) or a FIFO ring; fifo_write (may be null)
// is the ring update, carried out by the output projection's launch (after
// every read of the ring). With kv (not null) the memory is a key ring of
// projected keys and values instead: only the segment's rows are projected,
// straight into the ring after the memory keys, and the attention reads all
// keys from it (mem, ring_len, ring_head unused).
int layer_forward(const xl_attn_desc* d, const xl_attn_weights* w, const void* h, const void* mem, int64_t mlen,
                  int64_t ring_len, int64_t ring_head, void* out, void* ws, size_t ws_bytes, hipStream_t s,
                  const xl::RowCopy* fifo_write, const xl_kv_fifo* kv = nullptr, const void* residual = nullptr,
                  bool table_ready = false) {
    xl_ws_layout L;
    fill_layout(d, mlen, &L, kv != nullptr);
    if (ws_bytes < L.total)
        return fail(XL_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
    if (((uintptr_t)ws) % kAlign) return fail(XL_UNSUPPORTED, "workspace must be 256-byte aligned");
    const bool bf = d->dtype == XL_BF16;
    const int64_t B = d->batch, H = d->n_head, dh = d->d_head, q = d->qlen, D = d->d_model, HD = H * dh;
    const int64_t klen = L.klen;
    const float scale = d->scale == 0.f ? (float)(1.0 / sqrt((double)dh)) : d->scale;
    const double base = d->base == 0.0 ? 10000.0 : d->base;
    char* W = (char*)ws;
    hipError_t e;

    // 1. sinusoid rows R_n, n < n_rel (a distance uses row min(delta, n_rel-1)),
    // unless the caller vouches that the workspace holds this table already
    // (XL_REUSE_TABLE: then r as well), or the previous layer of a stack step
    // wrote it for the same key count (table_ready: r is still projected)
    const bool reuse = (d->flags & XL_REUSE_TABLE) != 0;
    if (!reuse && !table_ready) {
        e = xl::launch_relpos(0, L.n_rel, D, -1, base, bf ? 1 : 0, W + L.rel, s);
        if (e != hipSuccess) return hip_fail(e, "relpos launch");
    }

    // 2-4. the input projections as one grid: r = R W_r^T, q, and k, v over
    // [memory ; segment] (the attention folds u and v into q as it loads it)
    xl::GemmArgs g[4];
    memset(g, 0, sizeof g);
    int ng = 0;
    auto base_args = [&](xl::GemmArgs& a) {
        a.H = (int)H;
        a.dh = (int)dh;
        a.b_split = 1 << 30;
    };
    if (!reuse) {   // r = R W_r^T -> [H, n_rel, dh]
        xl::GemmArgs& a = g[ng++];
        base_args(a);
        a.M = (int)L.n_rel; a.N = (int)HD; a.K = (int)D;
        a.a0 = W + L.rel; a.lda = D;
        a.b0 = w->w_r; a.epi = xl::EPI_R; a.out0 = W + L.r; a.seq = (int)L.n_rel;
    }
    {   // q projection -> q [B, H, qlen, dh]
        xl::GemmArgs& a = g[ng++];
        base_args(a);
        a.M = (int)(B * q); a.N = (int)HD; a.K = (int)D;
        a.a0 = h; a.lda = D;
        a.b0 = w->w_q; a.epi = xl::EPI_K; a.out0 = W + L.q;
        a.seq = (int)q;
    }
    void* k_out = kv ? kv->k : (void*)(W + L.k);
    void* vt_out = kv ? kv->vt : (void*)(W + L.vt);
    auto kv_rows = [&](xl::GemmArgs& a) {
        if (kv) {
            // the segment's rows only, into ring rows (head + len + t) mod cap
            a.M = (int)(B * q); a.K = (int)D;
            a.a0 = h; a.lda = D; a.a_seq = 0;
            a.seq = (int)q; a.ldv = (int)kv->cap;
            a.out_rows = (int)kv->cap;
            a.out_pos0 = (int)((kv->head + kv->len) % kv->cap);
            return;
        }
        a.M = (int)(B * klen); a.K = (int)D;
        a.a0 = mlen ? mem : h; a.a1 = h; a.lda = D;
        a.a0_bstride = ring_len * D; a.a1_bstride = q * D;
        a.a_seq = (int)klen; a.a_split = (int)mlen; a.ring_len = (int)(ring_len > 0 ? ring_len : 1);
        a.ring_head = (int)ring_head;
        a.seq = (int)klen; a.ldv = (int)L.ldv;
    };
    if (HD % 128 == 0) {   // k and v share the A rows: one problem, weight rows [W_k ; W_v]
        xl::GemmArgs& a = g[ng++];
        base_args(a);
        kv_rows(a);
        a.N = (int)(2 * HD);
        a.b0 = w->w_k; a.b1 = w->w_v; a.b_split = (int)HD;
        a.epi = xl::EPI_KV; a.out0 = k_out; a.out1 = vt_out;
    } else {
        xl::GemmArgs& a = g[ng++];
        base_args(a);
        kv_rows(a);
        a.N = (int)HD;
        a.b0 = w->w_k; a.epi = xl::EPI_K; a.out0 = k_out;
        xl::GemmArgs& c = g[ng++];
        c = a;
        c.b0 = w->w_v; c.epi = xl::EPI_VT; c.out0 = vt_out;
    }
    if ((e = xl::launch_gemms(g, ng, bf, s)) != hipSuccess) return hip_fail(e, "projection launch");
    // 5. fused relative attention
    xl::AttnArgs a;
    a.q = W + L.q; a.u = w->u; a.v = w->v; a.scale = scale;
    a.k = k_out; a.vt = vt_out; a.r = W + L.r;
    a.bias = d->bias_clamp >= 0 ? w->bias_table : nullptr;
    a.out = W + L.attn;
    a.B = (int)B; a.H = (int)H; a.qlen = (int)q; a.mlen = (int)mlen; a.klen = (int)klen;
    a.ldv = (int)L.ldv; a.n_rel = (int)L.n_rel; a.r_rows = (int)L.n_rel;
    a.bias_clamp = (int)(d->bias_clamp >= 0 ? d->bias_clamp : 0);
    a.bias_kind = d->bias_kind;
    if (kv) {
        a.ldv = (int)kv->cap;
        a.kv_rows = (int)kv->cap;
        a.kv_head = (int)kv->head;
    }
    const xl::SplitPlan sp = splits_of(d, mlen);
    a.split_steps = sp.steps;
    a.split_max = sp.max;
    a.part = W + L.part;
    int st = run_core(a, bf, (int)dh, s);
    if (st != XL_OK) return st;
    // 6. output projection
    xl::GemmArgs go;
    memset(&go, 0, sizeof go);
    go.M = (int)(B * q); go.N = (int)D; go.K = (int)HD;
    go.a0 = W + L.attn; go.lda = HD; go.a_seq = 0;
    go.b0 = w->w_o; go.b_split = 1 << 30; go.epi = xl::EPI_OUT; go.out0 = out;
    go.out_bf16 = d->out_dtype == XL_BF16;
    go.res = residual;
    go.H = (int)H; go.dh = (int)dh;
    if ((e = xl::launch_gemm(go, bf, s, fifo_write)) != hipSuccess) return hip_fail(e, "output projection launch");
    return XL_OK;
}

int check_weights(const xl_attn_desc* d, const xl_attn_weights* w) {
    if (!w) return fail(XL_NULL_ARG, "weights is NULL");
    if (!w->w_q || !w->w_k || !w->w_v || !w->w_r || !w->w_o || !w->u || !w->v)
        return fail(XL_NULL_ARG, "a weight pointer is NULL");
    if (d->bias_clamp >= 0 && !w->bias_table) return fail(XL_NULL_ARG, "bias_clamp >= 0 but bias_table is NULL");
    return XL_OK;
}

// ---- the pre-LN decoder layer around the attention ----------------------------------------------

struct DecLayout {
    size_t attn_total;                    // the attention layer's workspace, at offset 0
    size_t xm, xs, h1, x2, y1, buf0, buf1, total;
};

// stack: two more [B, qlen, D] buffers for the outputs of the inner layers;
// kv: the memory is a key ring (no normalised memory rows, no k or vt regions)
void dec_layout(const xl_attn_desc* d, int64_t mlen, int64_t d_inner, bool stack, DecLayout* L, bool kv = false) {
    xl_ws_layout A;
    fill_layout(d, mlen, &A, kv);
    const size_t es = esize(d->dtype);
    const int64_t B = d->batch, q = d->qlen, D = d->d_model;
    size_t off = align_up(A.total);
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    L->attn_total = A.total;
    L->xm = take(kv ? 0 : (size_t)(B * mlen * D) * es);
    L->xs = take((size_t)(B * q * D) * es);
    L->h1 = take((size_t)(B * q * D) * 4);   // fp32 for either element type
    L->x2 = take((size_t)(B * q * D) * es);
    L->y1 = take((size_t)(B * q * d_inner) * es);
    L->buf0 = take(stack ? (size_t)(B * q * D) * es : 0);
    L->buf1 = take(stack ? (size_t)(B * q * D) * es : 0);
    L->total = off;
}

int check_decoder(const xl_attn_desc* d, int64_t d_inner, float eps, const xl_decoder_weights* w) {
    if (!w) return fail(XL_NULL_ARG, "weights is NULL");
    if (d->flags & XL_REUSE_TABLE)
        return fail(XL_UNSUPPORTED, "XL_REUSE_TABLE: every decoder layer writes its own table into the workspace");
    int st = check_weights(d, &w->attn);
    if (st != XL_OK) return st;
    if (!w->ln1_g || !w->ln1_b || !w->ln2_g || !w->ln2_b || !w->w1 || !w->b1 || !w->w2 || !w->b2)
        return fail(XL_NULL_ARG, "a layer norm or feed-forward weight pointer is NULL");
    const int64_t mult = d->dtype == XL_BF16 ? 32 : 16;
    if (d_inner < 1 || d_inner % mult) return fail(XL_BAD_SHAPE, "d_inner must be a positive multiple of %lld", (long long)mult);
    if (d_inner > 262144) return fail(XL_UNSUPPORTED, "d_inner above 262144");
    if (d->batch * d->qlen * d_inner > kI32) return fail(XL_UNSUPPORTED, "batch * qlen * d_inner too large");
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(XL_BAD_SHAPE, "ln_eps must be finite and >= 0");
    // the bf16 epilogue reads the biases 16 bytes at a time
    if (((uintptr_t)w->b1 | (uintptr_t)w->b2) % 16) return fail(XL_UNSUPPORTED, "b1 and b2 must be 16-byte aligned");
    return XL_OK;
}

// One decoder layer on a memory that is a plain tensor or a FIFO ring (as in
// layer_forward); fifo_write (may be null) copies h into the ring after every
// read of it.
//   xm, xs = LN1(mem), LN1(h); h1 = h + RelAttn(xs over [xm ; xs]);
//   out = h1 + W2 relu(W1 LN2(h1) + b1) + b2
// h1 stays fp32 in the workspace: out adds it back after the feed-forward
// network, and a bf16 copy would put half an ulp of h1 (0.016 at |h1| >= 4)
// into out however small out is after that sum.
int decoder_forward(const xl_attn_desc* d, int64_t d_inner, float eps, const xl_decoder_weights* w, const void* h,
                    const void* mem, int64_t mlen, int64_t ring_len, int64_t ring_head, void* out, void* ws,
                    size_t ws_bytes, hipStream_t s, const xl::RowCopy* fifo_write, const xl_kv_fifo* kv = nullptr,
                    bool table_ready = false) {
    DecLayout L;
    dec_layout(d, mlen, d_inner, false, &L, kv != nullptr);
    if (ws_bytes < L.total)
        return fail(XL_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
    if (((uintptr_t)ws) % kAlign) return fail(XL_UNSUPPORTED, "workspace must be 256-byte aligned");
    const bool bf = d->dtype == XL_BF16;
    const int64_t B = d->batch, q = d->qlen, D = d->d_model;
    char* W = (char*)ws;
    hipError_t e;
    // 1. LN1 of every row of [memory ; segment]; with a key ring only the
    // segment's (the memory's keys and values were projected from their
    // normalised rows when those were the segment)
    xl::LnArgs ln;
    memset(&ln, 0, sizeof ln);
    const int64_t mrows = kv ? 0 : mlen;
    ln.a0 = mrows ? mem : h; ln.a1 = h;
    ln.a0_bstride = ring_len * D; ln.a1_bstride = q * D;
    ln.a_seq = (int)(mrows + q); ln.a_split = (int)mrows; ln.ring_len = (int)(ring_len > 0 ? ring_len : 1);
    ln.ring_head = (int)ring_head;
    ln.y0 = W + L.xm; ln.y1 = W + L.xs;
    ln.gamma = w->ln1_g; ln.beta = w->ln1_b;
    ln.rows = (int)(B * (mrows + q)); ln.D = (int)D; ln.eps = eps;
    if ((e = xl::launch_layer_norm(ln, bf, s)) != hipSuccess) return hip_fail(e, "layer norm launch");
    // 2. attention sublayer with the residual: h1 = h + RelAttn(...)
    xl_attn_desc da = *d;
    da.mlen = mlen;
    da.out_dtype = XL_F32;
    int st = layer_forward(&da, &w->attn, W + L.xs, kv ? nullptr : W + L.xm, mlen, mlen, 0, W + L.h1, W, L.attn_total,
                           s, fifo_write, kv, h, table_ready);
    if (st != XL_OK) return st;
    // 3. LN2(h1)
    ln.a0 = W + L.h1; ln.a1 = W + L.h1;
    ln.a0_bstride = q * D; ln.a1_bstride = q * D;
    ln.a_seq = (int)q; ln.a_split = 0; ln.ring_len = 1; ln.ring_head = 0;
    ln.y0 = W + L.x2; ln.y1 = W + L.x2;
    ln.gamma = w->ln2_g; ln.beta = w->ln2_b;
    ln.rows = (int)(B * q);
    ln.x_f32 = 1;
    if ((e = xl::launch_layer_norm(ln, bf, s)) != hipSuccess) return hip_fail(e, "layer norm launch");
    // 4-5. the feed-forward network with its residual
    xl::GemmArgs g;
    memset(&g, 0, sizeof g);
    g.M = (int)(B * q); g.N = (int)d_inner; g.K = (int)D;
    g.a0 = W + L.x2; g.lda = D; g.a_seq = 0;
    g.b0 = w->w1; g.b_split = 1 << 30; g.epi = xl::EPI_OUT; g.out0 = W + L.y1; g.out_bf16 = bf ? 1 : 0;
    g.H = (int)d->n_head; g.dh = (int)d->d_head;
    g.bias_n = w->b1; g.relu = 1;
    if ((e = xl::launch_gemm(g, bf, s)) != hipSuccess) return hip_fail(e, "feed-forward launch");
    g.N = (int)D; g.K = (int)d_inner;
    g.a0 = W + L.y1; g.lda = d_inner;
    g.b0 = w->w2; g.out0 = out; g.out_bf16 = d->out_dtype == XL_BF16;
    g.bias_n = w->b2; g.relu = 0; g.res = W + L.h1; g.res_f32 = 1;
    if ((e = xl::launch_gemm(g, bf, s)) != hipSuccess) return hip_fail(e, "feed-forward launch");
    return XL_OK;
}

int check_fifo(const xl_mem_fifo* f) {
    if (!f) return fail(XL_NULL_ARG, "fifo is NULL");
    if (!f->buf) return fail(XL_NULL_ARG, "fifo->buf is NULL");
    if (f->mlen_max < 1 || f->len < 0 || f->len > f->mlen_max || f->head < 0 || f->head >= f->mlen_max)
        return fail(XL_BAD_SHAPE, "fifo state invalid (mlen_max %lld, len %lld, head %lld)", (long long)f->mlen_max,
                    (long long)f->len, (long long)f->head);
    if (f->mlen_max > kI32 / 64) return fail(XL_UNSUPPORTED, "mlen_max too large");
    return XL_OK;
}

// a FIFO's rows across the batch, bounded like the key rows (after check_desc)
int check_fifo_rows(const xl_attn_desc* d, const xl_mem_fifo* f) {
    if (f->mlen_max > kI32 / 2 / d->batch) return fail(XL_UNSUPPORTED, "batch * fifo->mlen_max too large");
    return XL_OK;
}

// the FIFO update of a segment step: row t of h lands at ring row
// (head + len + t) % mlen_max; only the last min(qlen, mlen_max) rows survive
xl::RowCopy fifo_copy(const xl_attn_desc* d, const xl_mem_fifo* f, const void* h) {
    const int64_t M = f->mlen_max, q = d->qlen;
    const int64_t n_w = q < M ? q : M;
    const int64_t src0 = q - n_w;
    const int64_t dst0 = (f->head + f->len + src0) % M;
    return xl::RowCopy{h, f->buf, q, M, dst0, src0, n_w, d->batch, d->d_model * (int64_t)esize(d->dtype)};
}
void fifo_advance(const xl_attn_desc* d, xl_mem_fifo* f) {
    const int64_t M = f->mlen_max, q = d->qlen;
    const int64_t new_len = f->len + q < M ? f->len + q : M;
    f->head = (f->head + f->len + q - new_len) % M;
    f->len = new_len;
}

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // guarded by g_scratch_mu

int scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(XL_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p || (uintptr_t)p % kAlign) return fail(XL_HIP_ERROR, "scratch is not 256-byte aligned");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return XL_OK;
}

}  // namespace

extern "C" {

const char* xl_status_string(int status) {
    switch (status) {
        case XL_OK: return "ok";
        case XL_NULL_ARG: return "null argument";
        case XL_BAD_SHAPE: return "bad shape";
        case XL_UNSUPPORTED: return "unsupported";
        case XL_WORKSPACE_TOO_SMALL: return "workspace too small";
        case XL_HIP_ERROR: return "HIP error";
        default: return "unknown status";
    }
}

const char* xl_last_error(void) { return g_last_error.c_str(); }

int xl_set_core_events(void* ev_begin, void* ev_end) {
    g_ev_begin = ev_begin;
    g_ev_end = ev_end;
    return XL_OK;
}

int xl_relpos_embed(int64_t delta0, int64_t n_rows, int64_t d_model, int64_t clamp_len, double base, int out_dtype,
                    void* out, void* stream) {
    g_last_error.clear();
    if (n_rows < 0 || d_model < 2 || (d_model & 1)) return fail(XL_BAD_SHAPE, "n_rows >= 0 and even d_model >= 2 required");
    if (out_dtype != XL_F32 && out_dtype != XL_BF16) return fail(XL_BAD_SHAPE, "bad out_dtype");
    if (base == 0.0) base = 10000.0;
    if (!(base > 0.0) || !isfinite(base)) return fail(XL_BAD_SHAPE, "base must be > 0");
    if (n_rows > kI32 || d_model > kI32 || n_rows * (d_model / 2) > ((int64_t)1 << 40))
        return fail(XL_UNSUPPORTED, "table too large");
    if (n_rows == 0) return XL_OK;
    if (!out) return fail(XL_NULL_ARG, "out is NULL");
    if (((uintptr_t)out) % 8) return fail(XL_UNSUPPORTED, "out must be 8-byte aligned");
    hipError_t e = xl::launch_relpos(delta0, n_rows, d_model, clamp_len, base, out_dtype == XL_BF16, out,
                                     (hipStream_t)stream);
    return e == hipSuccess ? XL_OK : hip_fail(e, "relpos launch");
}

size_t xl_rel_attn_workspace_size(const xl_attn_desc* desc) {
    if (check_desc(desc, desc ? desc->mlen : 0, true) != XL_OK) return 0;
    xl_ws_layout L;
    fill_layout(desc, desc->mlen, &L);
    return L.total;
}

int xl_rel_attn_workspace_layout(const xl_attn_desc* desc, xl_ws_layout* layout) {
    g_last_error.clear();
    int st = check_desc(desc, desc ? desc->mlen : 0, true);
    if (st != XL_OK) return st;
    if (!layout) return fail(XL_NULL_ARG, "layout is NULL");
    fill_layout(desc, desc->mlen, layout);
    return XL_OK;
}

int xl_rel_attn_fwd(const xl_attn_desc* desc, const xl_attn_weights* w, const void* h, const void* mem, void* out,
                    void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    int st = check_desc(desc, desc ? desc->mlen : 0, true);
    if (st != XL_OK) return st;
    if ((st = check_weights(desc, w)) != XL_OK) return st;
    if (!h || !out || !ws) return fail(XL_NULL_ARG, "h, out and ws must be non-NULL");
    if (desc->mlen > 0 && !mem) return fail(XL_NULL_ARG, "mem is NULL with mlen > 0");
    const size_t es = esize(desc->dtype);
    const size_t out_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * esize(desc->out_dtype);
    const size_t h_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * es;
    if (overlaps(out, out_bytes, h, h_bytes) ||
        (desc->mlen > 0 && overlaps(out, out_bytes, mem, (size_t)(desc->batch * desc->mlen * desc->d_model) * es)) ||
        overlaps(out, out_bytes, ws, ws_bytes))
        return fail(XL_BAD_SHAPE, "out aliases an input or the workspace");
    return layer_forward(desc, w, h, mem, desc->mlen, desc->mlen, 0, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

size_t xl_rel_attn_core_workspace_size(const xl_attn_desc* desc) {
    if (check_desc(desc, desc ? desc->mlen : 0, false) != XL_OK) return 0;
    return part_bytes_of(desc, desc->mlen);
}

int xl_rel_attn_core(const xl_attn_desc* desc, const void* q, const void* k, const void* vt, int64_t ldv,
                     const void* r, int64_t n_rel, const void* u, const void* v, const void* bias_table, void* attn,
                     void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    int st = check_desc(desc, desc ? desc->mlen : 0, false);
    if (st != XL_OK) return st;
    if (!q || !k || !vt || !r || !u || !v || !attn) return fail(XL_NULL_ARG, "a core operand is NULL");
    if (!isfinite(desc->scale)) return fail(XL_BAD_SHAPE, "scale must be finite");
    const int64_t klen = desc->mlen + desc->qlen;
    if (ldv < klen || ldv % 8) return fail(XL_BAD_SHAPE, "ldv must be >= klen and a multiple of 8");
    if (ldv > kI32 / 64) return fail(XL_UNSUPPORTED, "ldv too large");
    const int64_t need = n_rel_of(desc, klen);
    if (n_rel < need) return fail(XL_BAD_SHAPE, "r has %lld rows, needs %lld", (long long)n_rel, (long long)need);
    if (n_rel > kI32 / 64) return fail(XL_UNSUPPORTED, "r has too many rows");
    if (desc->bias_clamp >= 0 && !bias_table) return fail(XL_NULL_ARG, "bias_clamp >= 0 but bias_table is NULL");
    xl::AttnArgs a;
    a.q = q; a.u = u; a.v = v;
    a.scale = desc->scale == 0.f ? (float)(1.0 / sqrt((double)desc->d_head)) : desc->scale;
    a.k = k; a.vt = vt; a.r = r;
    a.bias = desc->bias_clamp >= 0 ? bias_table : nullptr;
    a.out = attn;
    a.B = (int)desc->batch; a.H = (int)desc->n_head; a.qlen = (int)desc->qlen; a.mlen = (int)desc->mlen;
    a.klen = (int)klen; a.ldv = (int)ldv; a.n_rel = (int)need; a.r_rows = (int)n_rel;
    a.bias_clamp = (int)(desc->bias_clamp >= 0 ? desc->bias_clamp : 0);
    a.bias_kind = desc->bias_kind;
    const xl::SplitPlan sp = splits_of(desc, desc->mlen);
    a.split_steps = sp.steps;
    a.split_max = sp.max;
    const size_t need_ws = part_bytes_of(desc, desc->mlen);
    if (need_ws > 0) {
        if (!ws) return fail(XL_NULL_ARG, "ws is NULL but the split attention needs %zu bytes", need_ws);
        if (ws_bytes < need_ws)
            return fail(XL_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, need_ws);
        if (((uintptr_t)ws) % kAlign) return fail(XL_UNSUPPORTED, "workspace must be 256-byte aligned");
        const size_t ab = (size_t)(desc->batch * desc->qlen * desc->n_head * desc->d_head) * esize(desc->dtype);
        if (overlaps(ws, need_ws, attn, ab)) return fail(XL_BAD_SHAPE, "ws aliases attn");
        a.part = ws;
    }
    return run_core(a, desc->dtype == XL_BF16, (int)desc->d_head, (hipStream_t)stream);
}

int xl_segment_step(const xl_attn_desc* desc, const xl_attn_weights* w, const void* h, xl_mem_fifo* fifo, void* out,
                    void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    int st = check_fifo(fifo);
    if (st != XL_OK) return st;
    if ((st = check_desc(desc, fifo->len, true)) != XL_OK) return st;
    if ((st = check_fifo_rows(desc, fifo)) != XL_OK) return st;
    if ((st = check_weights(desc, w)) != XL_OK) return st;
    if (!h || !out || !ws) return fail(XL_NULL_ARG, "h, out and ws must be non-NULL");
    const size_t es = esize(desc->dtype);
    const size_t h_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * es;
    const size_t ring_bytes = (size_t)(desc->batch * fifo->mlen_max * desc->d_model) * es;
    const size_t out_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * esize(desc->out_dtype);
    if (overlaps(h, h_bytes, fifo->buf, ring_bytes)) return fail(XL_BAD_SHAPE, "h aliases fifo->buf");
    if (overlaps(out, out_bytes, fifo->buf, ring_bytes) || overlaps(out, out_bytes, h, h_bytes) ||
        overlaps(out, out_bytes, ws, ws_bytes))
        return fail(XL_BAD_SHAPE, "out aliases an input, the memory or the workspace");
    xl_attn_desc d = *desc;
    d.mlen = fifo->len;
    hipStream_t s = (hipStream_t)stream;
    const xl::RowCopy cp = fifo_copy(desc, fifo, h);
    st = layer_forward(&d, w, h, fifo->buf, fifo->len, fifo->mlen_max, fifo->head, out, ws, ws_bytes, s, &cp);
    if (st != XL_OK) return st;
    fifo_advance(desc, fifo);
    return XL_OK;
}

int xl_segment_step_noalloc(const xl_attn_desc* desc, const xl_attn_weights* w, const void* h, xl_mem_fifo* fifo,
                            void* out, void* stream) {
    g_last_error.clear();
    int st = check_fifo(fifo);
    if (st != XL_OK) return st;
    if ((st = check_desc(desc, fifo->len, true)) != XL_OK) return st;
    xl_ws_layout L;
    fill_layout(desc, fifo->len, &L);
    if (L.total > XL_NOALLOC_SCRATCH_BYTES)
        return fail(XL_WORKSPACE_TOO_SMALL, "this step needs %zu bytes of scratch; the allocation-free step holds %zu",
                    L.total, (size_t)XL_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((st = scratch_ptr(&ws)) != XL_OK) return st;
    return xl_segment_step(desc, w, h, fifo, out, ws, XL_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

namespace {
// a key ring's state against desc (its len as the memory length)
int check_kv_ring(const xl_attn_desc* desc, const xl_kv_fifo* kv) {
    if (!kv) return fail(XL_NULL_ARG, "kv is NULL");
    if (!kv->k || !kv->vt) return fail(XL_NULL_ARG, "kv->k and kv->vt must be non-NULL");
    int st = check_desc(desc, kv->len >= 0 ? kv->len : 0, true);
    if (st != XL_OK) return st;
    if (desc->dtype != XL_BF16) return fail(XL_UNSUPPORTED, "the key ring path is bf16 only");
    const int64_t q = desc->qlen, M = kv->mlen_max, C = kv->cap;
    if (M > kI32 / 128 || C > kI32 / 128) return fail(XL_UNSUPPORTED, "cap or mlen_max too large");
    if (M < 1 || kv->len < 0 || kv->len > M || kv->head < 0 || kv->head >= C || C < M + q)
        return fail(XL_BAD_SHAPE, "kv state invalid (cap %lld, mlen_max %lld, len %lld, head %lld, qlen %lld)",
                    (long long)C, (long long)M, (long long)kv->len, (long long)kv->head, (long long)q);
    if (C % 8 || M % 8 || q % 8 || kv->len % 8 || kv->head % 8)
        return fail(XL_UNSUPPORTED, "the key ring needs cap, mlen_max, len, head and qlen multiples of 8");
    if (C > kI32 / 2 / desc->batch) return fail(XL_UNSUPPORTED, "batch * cap too large");
    return XL_OK;
}

// the segment's keys now follow the memory keys: keep the last mlen_max
void kv_advance(const xl_attn_desc* desc, xl_kv_fifo* kv) {
    const int64_t total = kv->len + desc->qlen;
    const int64_t new_len = total < kv->mlen_max ? total : kv->mlen_max;
    kv->head = (kv->head + total - new_len) % kv->cap;
    kv->len = new_len;
}
}  // namespace

extern "C" {

size_t xl_segment_step_kv_workspace_size(const xl_attn_desc* desc) {
    if (check_desc(desc, desc ? desc->mlen : 0, true) != XL_OK || desc->dtype != XL_BF16) return 0;
    xl_ws_layout L;
    fill_layout(desc, desc->mlen, &L, true);
    return L.total;
}

int xl_segment_step_kv(const xl_attn_desc* desc, const xl_attn_weights* w, const void* h, xl_kv_fifo* kv,
                       void* out, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    int st = check_kv_ring(desc, kv);
    if (st != XL_OK) return st;
    const int64_t q = desc->qlen, C = kv->cap;
    if ((st = check_weights(desc, w)) != XL_OK) return st;
    if (!h || !out || !ws) return fail(XL_NULL_ARG, "h, out and ws must be non-NULL");
    const size_t es = esize(desc->dtype);
    const size_t h_bytes = (size_t)(desc->batch * q * desc->d_model) * es;
    const size_t ring_bytes = (size_t)(desc->batch * desc->n_head * C * desc->d_head) * es;
    const size_t out_bytes = (size_t)(desc->batch * q * desc->d_model) * esize(desc->out_dtype);
    if (overlaps(kv->k, ring_bytes, kv->vt, ring_bytes)) return fail(XL_BAD_SHAPE, "kv->k aliases kv->vt");
    for (const void* p : {kv->k, kv->vt})
        if (overlaps(p, ring_bytes, h, h_bytes) || overlaps(p, ring_bytes, out, out_bytes) ||
            overlaps(p, ring_bytes, ws, ws_bytes))
            return fail(XL_BAD_SHAPE, "the key ring aliases h, out or the workspace");
    if (overlaps(out, out_bytes, h, h_bytes) || overlaps(out, out_bytes, ws, ws_bytes))
        return fail(XL_BAD_SHAPE, "out aliases h or the workspace");
    xl_attn_desc d = *desc;
    d.mlen = kv->len;
    st = layer_forward(&d, w, h, nullptr, kv->len, 0, 0, out, ws, ws_bytes, (hipStream_t)stream, nullptr, kv);
    if (st != XL_OK) return st;
    kv_advance(desc, kv);
    return XL_OK;
}

size_t xl_rel_attn_core_bwd_workspace_size(const xl_attn_desc* desc) {
    if (!desc || check_desc(desc, desc->mlen, false) != XL_OK) return 0;
    const int64_t rows = desc->batch * desc->n_head * desc->qlen;
    const int64_t klen = desc->mlen + desc->qlen;
    if (rows > (((int64_t)1 << 40) / klen)) return 0;   // the call rejects it too
    const int64_t dr_rows = n_rel_of(desc, klen) - 1;   // per-batch-element partial sums of dr
    return 2 * align_up((size_t)(rows * klen) * 4) + 2 * align_up((size_t)(rows * desc->d_head) * 4) +
           align_up((size_t)(desc->batch * desc->n_head * dr_rows * desc->d_head) * 4) +
           align_up((size_t)(rows * 3) * 4);
}

int xl_rel_attn_core_bwd(const xl_attn_desc* desc, const void* q, const void* k, const void* vt, int64_t ldv,
                         const void* r, int64_t n_rel, const void* u, const void* v, const void* bias_table,
                         const void* dout, float* dq, float* dk, float* dv, float* dr, float* du, float* dv_bias,
                         float* dbias, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    int st = check_desc(desc, desc ? desc->mlen : 0, false);
    if (st != XL_OK) return st;
    if (!q || !k || !vt || !r || !u || !v || !dout) return fail(XL_NULL_ARG, "an input pointer is NULL");
    if (!dq || !dk || !dv || !dr || !du || !dv_bias) return fail(XL_NULL_ARG, "an output pointer is NULL");
    if (desc->bias_clamp >= 0 && (!bias_table || !dbias))
        return fail(XL_NULL_ARG, "bias_clamp >= 0 but bias_table or dbias is NULL");
    const int64_t klen = desc->mlen + desc->qlen;
    if (ldv < klen || ldv % 8) return fail(XL_BAD_SHAPE, "ldv must be >= klen and a multiple of 8");
    if (ldv > kI32 / 64) return fail(XL_UNSUPPORTED, "ldv too large");
    const int64_t need = n_rel_of(desc, klen);
    if (n_rel < need) return fail(XL_BAD_SHAPE, "r has %lld rows, needs %lld", (long long)n_rel, (long long)need);
    if (n_rel > kI32 / 64) return fail(XL_UNSUPPORTED, "r has too many rows");
    const int64_t rows = desc->batch * desc->n_head * desc->qlen;
    if (rows > (((int64_t)1 << 40) / klen)) return fail(XL_UNSUPPORTED, "problem too large for the plain backward");
    const size_t need_ws = xl_rel_attn_core_bwd_workspace_size(desc);
    if (!ws || ws_bytes < need_ws)
        return fail(XL_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws ? ws_bytes : 0, need_ws);
    if (((uintptr_t)ws) % kAlign) return fail(XL_UNSUPPORTED, "workspace must be 256-byte aligned");
    const size_t es = esize(desc->dtype);
    const int64_t dh = desc->d_head, H = desc->n_head;
    const size_t qb = (size_t)(rows * dh), kb = (size_t)(desc->batch * H * klen * dh);
    // no output may overlap an input, another output or the workspace
    const void* outs[] = {dq, dk, dv, dr, du, dv_bias};
    const size_t osz[] = {qb * 4, kb * 4, kb * 4, (size_t)(H * n_rel * dh) * 4, (size_t)(H * dh) * 4,
                          (size_t)(H * dh) * 4};
    const void* ins[] = {q, k, vt, r, dout, ws};
    const size_t isz[] = {qb * es, kb * es, (size_t)(desc->batch * H * dh * ldv) * es, (size_t)(H * n_rel * dh) * es,
                          qb * es, ws_bytes};
    for (int x = 0; x < 6; ++x) {
        for (int y = 0; y < 6; ++y)
            if (overlaps(outs[x], osz[x], ins[y], isz[y])) return fail(XL_BAD_SHAPE, "a gradient aliases an input");
        for (int y = 0; y < x; ++y)
            if (overlaps(outs[x], osz[x], outs[y], osz[y])) return fail(XL_BAD_SHAPE, "two gradients overlap");
    }
    xl::AttnBwdArgs a;
    memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.vt = vt; a.r = r; a.u = u; a.v = v;
    a.bias = desc->bias_clamp >= 0 ? bias_table : nullptr;
    a.dout = dout;
    a.scale = desc->scale == 0.f ? (float)(1.0 / sqrt((double)dh)) : desc->scale;
    a.B = (int)desc->batch; a.H = (int)H; a.qlen = (int)desc->qlen; a.mlen = (int)desc->mlen; a.klen = (int)klen;
    a.ldv = (int)ldv; a.n_rel = (int)need; a.r_rows = (int)n_rel;
    a.bias_clamp = (int)(desc->bias_clamp >= 0 ? desc->bias_clamp : 0);
    a.bias_kind = desc->bias_kind;
    a.bias_rows = desc->bias_kind == XL_BIAS_T5 ? XL_T5_BUCKETS : 2 * a.bias_clamp + 1;
    char* W = (char*)ws;
    size_t off = 0;
    a.P = (float*)(W + off); off += align_up((size_t)(rows * klen) * 4);
    a.dS = (float*)(W + off); off += align_up((size_t)(rows * klen) * 4);
    a.dqu = (float*)(W + off); off += align_up(qb * 4);
    a.dqv = (float*)(W + off); off += align_up(qb * 4);
    a.drp = (float*)(W + off); off += align_up((size_t)(desc->batch * H * (need - 1) * dh) * 4);
    if (dh == 64) a.rstat = (float*)(W + off);   // the tiled path: the rows' softmax statistics
    a.uvp = a.dqu;   // the tiled path's du/dv partials (2 x 64 floats per 64 queries) reuse the dq_u, dq_v regions
    a.dr_first = dh == 64 ? a.n_rel - 1 : 0;   // the tiled dr path (d_head 64) takes the rows below the last
    a.dq = dq; a.dk = dk; a.dv = dv; a.dr = dr; a.du = du; a.dvb = dv_bias; a.dbias = dbias;
    const hipError_t e = xl::launch_attn_bwd(a, desc->dtype == XL_BF16, (int)dh, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return XL_OK;
}

// d_inner as check_decoder bounds it (the size functions have no weights to check)
bool d_inner_ok(const xl_attn_desc* d, int64_t d_inner) {
    return d_inner >= 1 && d_inner <= 262144 && d->batch * d->qlen * d_inner <= kI32;
}

size_t xl_decoder_layer_workspace_size(const xl_attn_desc* desc, int64_t d_inner) {
    if (!desc || check_desc(desc, desc->mlen, true) != XL_OK || !d_inner_ok(desc, d_inner)) return 0;
    DecLayout L;
    dec_layout(desc, desc->mlen, d_inner, false, &L);
    return L.total;
}

int xl_decoder_layer_fwd(const xl_attn_desc* desc, int64_t d_inner, float ln_eps, const xl_decoder_weights* w,
                         const void* h, const void* mem, void* out, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    int st = check_desc(desc, desc ? desc->mlen : 0, true);
    if (st != XL_OK) return st;
    const float eps = ln_eps == 0.f ? 1e-5f : ln_eps;
    if ((st = check_decoder(desc, d_inner, eps, w)) != XL_OK) return st;
    if (!h || !out || !ws) return fail(XL_NULL_ARG, "h, out and ws must be non-NULL");
    if (desc->mlen > 0 && !mem) return fail(XL_NULL_ARG, "mem is NULL with mlen > 0");
    if ((uintptr_t)h % 16) return fail(XL_UNSUPPORTED, "h must be 16-byte aligned");
    const size_t es = esize(desc->dtype);
    const size_t out_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * esize(desc->out_dtype);
    const size_t h_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * es;
    if (overlaps(out, out_bytes, h, h_bytes) ||
        (desc->mlen > 0 && overlaps(out, out_bytes, mem, (size_t)(desc->batch * desc->mlen * desc->d_model) * es)) ||
        overlaps(out, out_bytes, ws, ws_bytes))
        return fail(XL_BAD_SHAPE, "out aliases an input or the workspace");
    return decoder_forward(desc, d_inner, eps, w, h, mem, desc->mlen, desc->mlen, 0, out, ws, ws_bytes,
                           (hipStream_t)stream, nullptr);
}

size_t xl_decoder_stack_workspace_size(const xl_attn_desc* desc, int64_t d_inner) {
    if (!desc || check_desc(desc, desc->mlen, true) != XL_OK || !d_inner_ok(desc, d_inner)) return 0;
    DecLayout L;
    dec_layout(desc, desc->mlen, d_inner, true, &L);
    return L.total;
}

int xl_decoder_stack_step(const xl_attn_desc* desc, int64_t d_inner, float ln_eps, int64_t n_layer,
                          const xl_decoder_weights* w, const void* h, xl_mem_fifo* fifos, void* out, void* ws,
                          size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (!desc) return fail(XL_NULL_ARG, "desc is NULL");
    if (n_layer < 1 || n_layer > 4096) return fail(XL_BAD_SHAPE, "n_layer must be in [1, 4096]");
    if (!w || !fifos) return fail(XL_NULL_ARG, "weights and fifos must be non-NULL");
    if (!h || !out || !ws) return fail(XL_NULL_ARG, "h, out and ws must be non-NULL");
    if ((uintptr_t)h % 16) return fail(XL_UNSUPPORTED, "h must be 16-byte aligned");
    int st = check_desc(desc, desc->mlen, true);   // the sizes, before any product of them
    if (st != XL_OK) return st;
    const float eps = ln_eps == 0.f ? 1e-5f : ln_eps;
    const size_t es = esize(desc->dtype);
    const size_t h_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * es;
    const size_t out_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * esize(desc->out_dtype);
    for (int64_t n = 0; n < n_layer; ++n) {
        if ((st = check_fifo(&fifos[n])) != XL_OK) return st;
        if ((st = check_fifo_rows(desc, &fifos[n])) != XL_OK) return st;
        if (fifos[n].len > desc->mlen)
            return fail(XL_BAD_SHAPE, "fifo %lld holds %lld rows, more than desc->mlen = %lld", (long long)n,
                        (long long)fifos[n].len, (long long)desc->mlen);
        if ((st = check_desc(desc, fifos[n].len, true)) != XL_OK) return st;
        if ((st = check_decoder(desc, d_inner, eps, &w[n])) != XL_OK) return st;
        const size_t ring_bytes = (size_t)(desc->batch * fifos[n].mlen_max * desc->d_model) * es;
        if (overlaps(h, h_bytes, fifos[n].buf, ring_bytes) || overlaps(out, out_bytes, fifos[n].buf, ring_bytes) ||
            overlaps(ws, ws_bytes, fifos[n].buf, ring_bytes))
            return fail(XL_BAD_SHAPE, "fifo %lld's ring aliases h, out or the workspace", (long long)n);
        for (int64_t k = 0; k < n; ++k)
            if (overlaps(fifos[k].buf, (size_t)(desc->batch * fifos[k].mlen_max * desc->d_model) * es, fifos[n].buf,
                         ring_bytes))
                return fail(XL_BAD_SHAPE, "the rings of fifos %lld and %lld overlap", (long long)k, (long long)n);
    }
    if (overlaps(out, out_bytes, h, h_bytes) || overlaps(out, out_bytes, ws, ws_bytes))
        return fail(XL_BAD_SHAPE, "out aliases h or the workspace");
    DecLayout L;
    dec_layout(desc, desc->mlen, d_inner, true, &L);
    if (ws_bytes < L.total)
        return fail(XL_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
    hipStream_t s = (hipStream_t)stream;
    char* W = (char*)ws;
    // layer n reads the output of layer n-1 and keeps that input in its own
    // ring; the sinusoid table in the workspace serves every layer after the
    // first whose memory length (hence key count) equals the previous one's
    const void* x = h;
    int64_t prev_len = -1;   // the memory length the previous layer ran with
    for (int64_t n = 0; n < n_layer; ++n) {
        const bool last = n == n_layer - 1;
        void* y = last ? out : (void*)(W + ((n & 1) ? L.buf1 : L.buf0));
        xl_attn_desc d = *desc;
        d.mlen = fifos[n].len;
        if (!last) d.out_dtype = desc->dtype;
        const bool table_ready = fifos[n].len == prev_len;
        prev_len = fifos[n].len;
        const xl::RowCopy cp = fifo_copy(desc, &fifos[n], x);
        st = decoder_forward(&d, d_inner, eps, &w[n], x, fifos[n].buf, fifos[n].len, fifos[n].mlen_max, fifos[n].head,
                             y, W, L.buf0, s, &cp, nullptr, table_ready);
        if (st != XL_OK) return st;
        fifo_advance(desc, &fifos[n]);
        x = y;
    }
    return XL_OK;
}

size_t xl_decoder_stack_kv_workspace_size(const xl_attn_desc* desc, int64_t d_inner) {
    if (!desc || check_desc(desc, desc->mlen, true) != XL_OK || !d_inner_ok(desc, d_inner) || desc->dtype != XL_BF16)
        return 0;
    DecLayout L;
    dec_layout(desc, desc->mlen, d_inner, true, &L, true);
    return L.total;
}

int xl_decoder_stack_step_kv(const xl_attn_desc* desc, int64_t d_inner, float ln_eps, int64_t n_layer,
                             const xl_decoder_weights* w, const void* h, xl_kv_fifo* rings, void* out, void* ws,
                             size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (!desc) return fail(XL_NULL_ARG, "desc is NULL");
    if (n_layer < 1 || n_layer > 4096) return fail(XL_BAD_SHAPE, "n_layer must be in [1, 4096]");
    if (!w || !rings) return fail(XL_NULL_ARG, "weights and rings must be non-NULL");
    if (!h || !out || !ws) return fail(XL_NULL_ARG, "h, out and ws must be non-NULL");
    if ((uintptr_t)h % 16) return fail(XL_UNSUPPORTED, "h must be 16-byte aligned");
    int st = check_desc(desc, desc->mlen, true);   // the sizes, before any product of them
    if (st != XL_OK) return st;
    if (desc->dtype != XL_BF16) return fail(XL_UNSUPPORTED, "the key ring path is bf16 only");
    const float eps = ln_eps == 0.f ? 1e-5f : ln_eps;
    const size_t es = esize(desc->dtype);
    const size_t h_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * es;
    const size_t out_bytes = (size_t)(desc->batch * desc->qlen * desc->d_model) * esize(desc->out_dtype);
    // every layer is checked before any runs, so that on an error no ring has moved
    for (int64_t n = 0; n < n_layer; ++n) {
        if ((st = check_kv_ring(desc, &rings[n])) != XL_OK) return st;
        if (rings[n].len > desc->mlen)
            return fail(XL_BAD_SHAPE, "ring %lld holds %lld keys, more than desc->mlen = %lld", (long long)n,
                        (long long)rings[n].len, (long long)desc->mlen);
        if ((st = check_decoder(desc, d_inner, eps, &w[n])) != XL_OK) return st;
        const size_t rb = (size_t)(desc->batch * desc->n_head * rings[n].cap * desc->d_head) * es;
        if (overlaps(rings[n].k, rb, rings[n].vt, rb)) return fail(XL_BAD_SHAPE, "ring %lld: k aliases vt", (long long)n);
        for (const void* p : {rings[n].k, rings[n].vt}) {
            if (overlaps(p, rb, h, h_bytes) || overlaps(p, rb, out, out_bytes) || overlaps(p, rb, ws, ws_bytes))
                return fail(XL_BAD_SHAPE, "ring %lld aliases h, out or the workspace", (long long)n);
            for (int64_t k = 0; k < n; ++k) {
                const size_t rk = (size_t)(desc->batch * desc->n_head * rings[k].cap * desc->d_head) * es;
                if (overlaps(p, rb, rings[k].k, rk) || overlaps(p, rb, rings[k].vt, rk))
                    return fail(XL_BAD_SHAPE, "the rings of layers %lld and %lld overlap", (long long)k, (long long)n);
            }
        }
    }
    if (overlaps(out, out_bytes, h, h_bytes) || overlaps(out, out_bytes, ws, ws_bytes))
        return fail(XL_BAD_SHAPE, "out aliases h or the workspace");
    DecLayout L;
    dec_layout(desc, desc->mlen, d_inner, true, &L, true);
    if (ws_bytes < L.total)
        return fail(XL_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
    hipStream_t s = (hipStream_t)stream;
    char* W = (char*)ws;
    // layer n reads the output of layer n-1; its ring takes that input's
    // projected keys and values. The sinusoid table in the workspace serves
    // every layer after the first whose memory length equals the previous one's
    const void* x = h;
    int64_t prev_len = -1;   // the memory length the previous layer ran with
    for (int64_t n = 0; n < n_layer; ++n) {
        const bool last = n == n_layer - 1;
        void* y = last ? out : (void*)(W + ((n & 1) ? L.buf1 : L.buf0));
        xl_attn_desc d = *desc;
        d.mlen = rings[n].len;
        if (!last) d.out_dtype = desc->dtype;
        const bool table_ready = rings[n].len == prev_len;
        prev_len = rings[n].len;
        st = decoder_forward(&d, d_inner, eps, &w[n], x, nullptr, rings[n].len, 0, 0, y, W, L.buf0, s, nullptr,
                             &rings[n], table_ready);
        if (st != XL_OK) return st;
        kv_advance(desc, &rings[n]);
        x = y;
    }
    return XL_OK;
}

}  // extern "C"
