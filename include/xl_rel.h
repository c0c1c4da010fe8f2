/*
 * xl_rel.h -- C ABI of libxlrel.so: the Transformer-XL relative multi-head
 * attention forward over [cached memory ; current segment] on AMD MI355X
 * (gfx950).
 *
 * The method (pages by title/host and section):
 *  - score of query i and key j, for one head:
 *      A_rel(i,j) = q_i.k_j + q_i.r_{i-j} + u.k_j + v.r_{i-j}
 *    (qidao123.com thread-401555 "Transformer-XL cross-window RPE" §3;
 *     felixzhao.cn article 118 "Transformer-XL 和相对位置编码" §2.3.2;
 *     2kiu.com/news/5253360 TransformerXL relative-position tutorial §2.2),
 *    computed here in the folded form (q_i+u).k_j + (q_i+v).r_{i-j};
 *  - r_delta = R_delta W_r^T with the sinusoid R_delta (thread-401555 §2,
 *    felixzhao.cn §2.3.2), distances clamped to [-C, C] (2kiu.com §2.4);
 *  - queries from the segment, keys/values over [memory ; segment], memory
 *    first (felixzhao.cn §2.3.1; intelliparadigm.com 2238855
 *    "Transformer-XL架构解析" §2.1); causal mask after the whole sum
 *    (2kiu.com §4.2), softmax, P.V, output projection (2kiu.com §3.1);
 *  - optional per-head scalar bias b_{clamp(i-j, +-k)} added after scaling
 *    (jsqmd.com 1364567 "Transformer偏置型相对位置编码" §2.2, §3.1-§3.4),
 *    or, instead of the clamped distance, its T5 log-scale bucket (same
 *    page, §4.2);
 *  - FIFO memory update: the newest states push out the oldest
 *    (intelliparadigm.com §1.1), memory is a detached copy (felixzhao.cn
 *    §2.3.1).
 *
 * Conventions for every entry point
 *  - All tensors are dense, row-major, on the device of the current HIP
 *    device, owned by the caller. The library allocates no device memory:
 *    scratch space comes from the caller's workspace (xl_segment_step_noalloc
 *    alone uses a static device array the library holds instead).
 *  - 'stream' is a hipStream_t (NULL: the null stream). Work is enqueued
 *    asynchronously; device-side results are valid once the stream reaches
 *    that point. Host-side outputs (status, FIFO bookkeeping) are final on
 *    return.
 *  - Arguments are validated on the host before anything is enqueued; on
 *    error nothing is launched and a status code is returned, with a
 *    human-readable reason available from xl_last_error() (per thread).
 *  - No output may alias an input.
 *  - A call enqueues kernel launches only (no allocation, copy, fill or
 *    synchronisation), so a caller may capture it in a HIP graph; a replay
 *    recomputes from the buffers' contents at replay time. The segment steps
 *    advance their FIFO or ring positions on the host when called, so a
 *    captured step keeps the positions it was captured with.
 *  - Weight layout is nn.Linear's [out_features, in_features]: a projection
 *    is y = x W^T.
 */
#ifndef XL_REL_H
#define XL_REL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    XL_OK = 0,
    XL_NULL_ARG = 1,             /* a required pointer is NULL */
    XL_BAD_SHAPE = 2,            /* sizes inconsistent or out of range */
    XL_UNSUPPORTED = 3,          /* valid but outside the supported envelope */
    XL_WORKSPACE_TOO_SMALL = 4,  /* ws_bytes below xl_rel_attn_workspace_size() */
    XL_HIP_ERROR = 5             /* a HIP launch/runtime call failed */
};

/*
 * The supported envelope (outside it a call returns XL_UNSUPPORTED, or
 * XL_BAD_SHAPE where a size is not meaningful at all), with klen = mlen + qlen:
 *   (dtype, d_head) = (XL_BF16, 64) or (XL_F32, 8);
 *   d_model <= 65536, a multiple of 32 (bf16) or 16 (f32); n_head * d_head
 *     <= 65536 and a multiple of 32 (bf16) or 16 (f32);
 *   klen <= (2^31 - 1) / 128 (a head's keys within 32-bit byte offsets),
 *     batch * klen < 2^30, batch * n_head < 2^25, every tensor of the call
 *     (keys, values, memory rows) at most 2^40 elements;
 *   with a bias table in bf16: klen <= 20096 (the table of a workgroup's
 *     distances sits in LDS); bias_clamp <= 65535; attn_splits <= 64;
 *   FIFO memory: mlen_max < 2^25 and batch * mlen_max < 2^30; key ring:
 *     cap and mlen_max <= (2^31 - 1) / 128, batch * cap < 2^30, cap,
 *     mlen_max, len, head and qlen multiples of 8;
 *   decoder: d_inner <= 262144 and batch * qlen * d_inner < 2^31.
 * Every limit is checked before any product of caller sizes is formed.
 */

/* Element types. */
enum { XL_F32 = 0, XL_BF16 = 1 };

/* Rows of the scalar bias table (xl_attn_desc.bias_kind), by the distance
 * delta = i - j of a visible pair (delta >= 0):
 *  XL_BIAS_CLAMP: row clamp(delta, -k, k) + k of 2k+1 rows, k = bias_clamp
 *                 (jsqmd.com 1364567 §3.1);
 *  XL_BIAS_T5:    row bucket(delta) of XL_T5_BUCKETS rows, on the log-scale
 *                 boundaries 1, 2, 4, ..., 1024 (same page, §4.2): bucket 0
 *                 holds delta <= 1, bucket b in 1..10 holds
 *                 2^(b-1) < delta <= 2^b, bucket 11 every delta > 1024. */
enum { XL_BIAS_CLAMP = 0, XL_BIAS_T5 = 1 };
enum { XL_T5_BUCKETS = 12 };

/* Human-readable name of a status code (static string). */
const char* xl_status_string(int status);
/* Detail of the last error on the calling thread ("" if none). */
const char* xl_last_error(void);

/*
 * Sinusoidal relative embedding (thread-401555 §2; felixzhao.cn §2.3.2).
 * Row n (0 <= n < n_rows) of out [n_rows, d_model] is R_delta for
 * delta = delta0 + n, first clamped to [-clamp_len, clamp_len] when
 * clamp_len >= 0 (2kiu.com §2.4):
 *     R_delta[2t]   = sin(delta * base^(-2t/d_model))
 *     R_delta[2t+1] = cos(delta * base^(-2t/d_model)),  t < d_model/2.
 * Computed in fp64 and rounded once (to nearest even) to out_dtype.
 * d_model must be even and positive; base > 0 (0 selects 10000);
 * n_rows >= 0 (0 launches nothing). delta0 may be negative: delta0 = -2,
 * n_rows = 1, d_model = 4 gives approximately [-0.909, -0.416, -0.020,
 * 0.999], the example the page works through.
 */
int xl_relpos_embed(int64_t delta0, int64_t n_rows, int64_t d_model, int64_t clamp_len,
                    double base, int out_dtype, void* out, void* stream);

/* Shape and numerics of one relative-attention layer call. */
typedef struct {
    int64_t batch;       /* B >= 1 */
    int64_t d_model;     /* D: multiple of 32 for bf16, of 16 for f32 */
    int64_t n_head;      /* H >= 1; H*d_head a multiple of 32 (bf16) / 16 (f32) */
    int64_t d_head;      /* 64 (bf16) or 8 (f32) */
    int64_t qlen;        /* segment length, >= 1 */
    int64_t mlen;        /* memory length, >= 0 (ignored by xl_segment_step) */
    int64_t clamp_len;   /* < 0: no clamp; else distances clamp to [-C, C] */
    int64_t bias_clamp;  /* < 0: no scalar bias table; else the table is on,
                            with 2k+1 rows (k = bias_clamp) for
                            XL_BIAS_CLAMP, XL_T5_BUCKETS rows for XL_BIAS_T5 */
    double base;         /* sinusoid base; 0 selects 10000 */
    float scale;         /* score scale; 0 selects 1/sqrt(d_head) */
    int32_t dtype;       /* XL_BF16 (d_head 64) or XL_F32 (d_head 8): h, mem,
                            weights, u, v, bias table and every intermediate */
    int32_t out_dtype;   /* XL_F32 or XL_BF16 for the layer output */
    int32_t attn_splits; /* bf16 fused attention: how many workgroups may share
                            one 128-query tile's keys. 0 lets the library
                            choose (it splits only when the tiles leave compute
                            units without a second workgroup); 1..64 caps every
                            tile at that count (and at its number of 32-key
                            steps). Results agree to rounding for every value.
                            f32: ignored. */
    int32_t bias_kind;   /* XL_BIAS_CLAMP (0) or XL_BIAS_T5: how a distance
                            picks its bias table row; ignored when
                            bias_clamp < 0 */
    int32_t flags;       /* 0 or XL_REUSE_TABLE (below) */
} xl_attn_desc;

/* xl_attn_desc.flags. XL_REUSE_TABLE: the rel and r regions of the workspace
 * already hold this call's table rows -- an earlier xl_rel_attn_fwd /
 * xl_segment_step / xl_segment_step_kv / xl_segment_step_noalloc call wrote
 * them into the same workspace (for xl_segment_step_noalloc: the same GPU's
 * scratch) with the same d_model, n_head, clamp_len, base, w_r contents and
 * the same number of table rows n_rel = min(mlen + qlen, clamp_len + 1)
 * (for a segment run: once the memory is full). The sinusoid and the R
 * projection are then skipped: the table depends on the distance alone
 * (felixzhao.cn article 118 §2.3.2), so a recurrent run with fixed weights
 * computes it once. The library cannot check this promise; a stale table
 * gives wrong outputs. Not accepted by the decoder entry points (every layer
 * writes its own table into the shared workspace). */
enum { XL_REUSE_TABLE = 1 };

/* Weights of one layer; all device pointers in desc->dtype. */
typedef struct {
    const void* w_q;         /* [H*d_head, D] */
    const void* w_k;         /* [H*d_head, D] */
    const void* w_v;         /* [H*d_head, D] */
    const void* w_r;         /* [H*d_head, D]  position projection W_{k,R} */
    const void* w_o;         /* [D, H*d_head] */
    const void* u;           /* [H, d_head]  content bias */
    const void* v;           /* [H, d_head]  position bias */
    const void* bias_table;  /* [2*bias_clamp+1, H] (XL_BIAS_CLAMP) or
                                [XL_T5_BUCKETS, H] (XL_BIAS_T5); NULL when
                                bias_clamp < 0 */
} xl_attn_weights;

/*
 * Workspace layout of xl_rel_attn_fwd / xl_segment_step: byte offsets
 * (from the workspace base, each 256-byte aligned) of the intermediates the
 * call leaves behind, in desc->dtype:
 *   q       [B, H, qlen, d_head]  projected queries (u and v are added by the
 *                                 attention as it loads them)
 *   k       [B, H, klen, d_head]  keys over [memory ; segment]
 *   vt      [B, H, d_head, ldv]   values, transposed; columns >= klen unused
 *   rel     [n_rel, D]            sinusoid rows R_n, n = 0..n_rel-1
 *   r       [H, n_rel, d_head]    projected table r_n = R_n W_r^T
 *   attn    [B, qlen, H*d_head]   attention output before W_o
 *   part    scratch of the key-split attention (see xl_rel_attn_core)
 * with klen = mlen + qlen and n_rel = min(klen, clamp_len + 1) (klen when
 * there is no clamp).
 */
typedef struct {
    size_t q, k, vt, rel, r, attn;
    size_t part;             /* split partial results (fp32), 0 bytes unless split */
    size_t total;            /* == xl_rel_attn_workspace_size() */
    int64_t klen, ldv, n_rel;
} xl_ws_layout;

/* Workspace bytes needed by xl_rel_attn_fwd for desc (0 on invalid desc). */
size_t xl_rel_attn_workspace_size(const xl_attn_desc* desc);
/* Fill *layout for desc. Returns a status code. */
int xl_rel_attn_workspace_layout(const xl_attn_desc* desc, xl_ws_layout* layout);

/*
 * One relative-attention layer forward (the whole hot path):
 *   h   [B, qlen, D]  current segment (desc->dtype)
 *   mem [B, mlen, D]  cached memory, oldest first; NULL iff mlen == 0
 *   out [B, qlen, D]  (desc->out_dtype)
 * Steps: sinusoid rows -> r = R W_r^T -> q-projection -> k/v projection of
 * [mem ; h] -> fused relative attention (scores from s*(q+u) and s*(q+v))
 * -> W_o.
 * ws must hold xl_rel_attn_workspace_size(desc) bytes, 256-byte aligned.
 */
int xl_rel_attn_fwd(const xl_attn_desc* desc, const xl_attn_weights* w,
                    const void* h, const void* mem, void* out,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * The fused attention kernel alone (score, rel-shift, mask, softmax, P.V),
 * on projected operands in desc->dtype, laid out as in xl_ws_layout:
 *   q [B, H, qlen, d_head] projected queries; k [B, H, klen, d_head];
 *   vt [B, H, d_head, ldv] (ldv >= klen, multiple of 8);
 *   r [H, n_rel, d_head] with row n the projection of distance n, n_rel at
 *     least min(klen, clamp_len + 1) (klen without a clamp); a distance
 *     delta uses row min(delta, C) (C = clamp_len, or klen - 1 unclamped);
 *   u, v [H, d_head] content and position biases;
 *   bias_table [2*bias_clamp+1, H], [XL_T5_BUCKETS, H] (desc->bias_kind
 *       XL_BIAS_T5) or NULL;
 *   attn [B, qlen, H*d_head] output (desc->dtype).
 * The scores are s*(q_i+u).k_j + s*(q_i+v).r + bias with s = desc->scale
 * (0 selects 1/sqrt(d_head)); the sums q+u and q+v are rounded to desc->dtype
 * once, as the kernel loads the queries. desc->d_model, base, out_dtype are
 * ignored.
 * ws: xl_rel_attn_core_workspace_size(desc) bytes, 256-byte aligned, for the
 * partial results of a key split (may be NULL when that size is 0). With S
 * the largest split count of a tile it holds S*B*H*qlen*(d_head+2) floats:
 * per split, the unnormalised output, then (running maximum, sum) per query;
 * a second kernel merges them into attn.
 */
size_t xl_rel_attn_core_workspace_size(const xl_attn_desc* desc);
int xl_rel_attn_core(const xl_attn_desc* desc, const void* q, const void* k,
                     const void* vt, int64_t ldv, const void* r, int64_t n_rel,
                     const void* u, const void* v, const void* bias_table, void* attn,
                     void* ws, size_t ws_bytes, void* stream);

/* Caller-owned FIFO memory of one layer: a ring of mlen_max rows per
 * batch element. Logical row t (0 = oldest, t < len) of batch b is at
 * buf[b, (head + t) % mlen_max, :]. */
typedef struct {
    void* buf;          /* [B, mlen_max, D] in desc->dtype */
    int64_t mlen_max;   /* >= 1 */
    int64_t len;        /* rows in use, 0 <= len <= mlen_max */
    int64_t head;       /* physical row of the oldest entry, 0 <= head < mlen_max */
} xl_mem_fifo;

/*
 * One segment of a segment-recurrent run (felixzhao.cn §2.3.1,
 * intelliparadigm.com §1.1): the layer forward of h over
 * [memory ; h] with mlen = fifo->len (desc->mlen is ignored), then the FIFO
 * update: the memory becomes the last min(len + qlen, mlen_max) rows of
 * [memory ; h] (the layer *input* states, copied). h must not alias
 * fifo->buf. On success fifo->len and fifo->head are updated on return;
 * the ring contents are written on 'stream' after the layer has read them.
 * ws: xl_rel_attn_workspace_size() of desc with mlen = fifo->len.
 */
int xl_segment_step(const xl_attn_desc* desc, const xl_attn_weights* w, const void* h,
                    xl_mem_fifo* fifo, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * xl_segment_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same step, with the workspace taken from a static device array of
 * XL_NOALLOC_SCRATCH_BYTES held by the library on each GPU it runs on (from
 * the library's load until the process ends) instead of a caller's buffer.
 * The call allocates nothing; the first call on a device looks up that
 * device's array address once. Limit: a step whose
 * xl_rel_attn_workspace_size() (desc with mlen = fifo->len) exceeds
 * XL_NOALLOC_SCRATCH_BYTES returns XL_WORKSPACE_TOO_SMALL and leaves the fifo
 * untouched. Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (nothing in it needs to start at zero): calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller. Arguments, outputs and errors otherwise as
 * xl_segment_step.
 */
#define XL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int xl_segment_step_noalloc(const xl_attn_desc* desc, const xl_attn_weights* w, const void* h,
                            xl_mem_fifo* fifo, void* out, void* stream);

/* Caller-owned key ring of one layer, for evaluation with fixed weights: the
 * projected keys and values of the memory are kept instead of its input
 * states, so a segment step projects only its own rows (the cache reuse of
 * intelliparadigm.com §3.2 and felixzhao.cn §2.3.1). Key t of the memory
 * (0 = oldest, t < len) of batch b, head h is row (head + t) % cap of
 * k[b, h] and column (head + t) % cap of vt[b, h]. */
typedef struct {
    void* k;            /* [B, H, cap, d_head] bf16 */
    void* vt;           /* [B, H, d_head, cap] bf16 (values, transposed) */
    int64_t cap;        /* ring rows per head, >= mlen_max + qlen */
    int64_t mlen_max;   /* memory keys kept, >= 1 */
    int64_t len;        /* memory keys in use, 0 <= len <= mlen_max */
    int64_t head;       /* ring row of the oldest memory key */
} xl_kv_fifo;

/*
 * One segment step on a key ring: the same layer forward as
 * xl_segment_step with the memory given by its projected keys and values
 * (mlen = kv->len; desc->mlen is ignored). The segment's keys and values are
 * projected into the ring right after the memory keys, the attention runs
 * over all of them, and on return len and head describe the last
 * min(len + qlen, mlen_max) keys. For the same inputs the keys and values are
 * those xl_segment_step computes from the stored states, so the outputs
 * agree. bf16 only; cap, mlen_max, len, head and qlen must be multiples of
 * 8 (else XL_UNSUPPORTED). ws: xl_segment_step_kv_workspace_size() of desc
 * with mlen = kv->len (no k or vt regions: they live in the ring).
 */
size_t xl_segment_step_kv_workspace_size(const xl_attn_desc* desc);
int xl_segment_step_kv(const xl_attn_desc* desc, const xl_attn_weights* w, const void* h,
                       xl_kv_fifo* kv, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Gradients of xl_rel_attn_core for an upstream gradient dout [B, qlen,
 * H*d_head] (desc->dtype) of its output. The inputs are those of the forward
 * call (same layouts, desc->mlen keys of memory). With the logits l of the
 * forward and P = softmax(l): dP = dout . v, D_i = sum_j P_ij dP_ij,
 * dS = P (dP - D), then (s = desc->scale)
 *   dq_i = s sum_j dS_ij (k_j + r_ij),   dk_j = s sum_i dS_ij (q_i + u),
 *   dv_j = sum_i P_ij dout_i,            dr_c = s sum_{pairs of row c} dS_ij (q_i + v),
 *   du = s sum_ij dS_ij k_j,             dv_bias = s sum_ij dS_ij r_ij,
 *   dbias[row, h] = sum_{pairs of row} dS_ij
 * (the chain rule through the softmax and the four dot products of
 * qidao123.com thread-401555 §3; dr gathers the band back per distance, the
 * transpose of the relative shift). Rows of r at or beyond the rows in use
 * get zero. All gradients are fp32 and overwritten: dq [B, H, qlen, d_head],
 * dk, dv [B, H, klen, d_head], dr [H, n_rel, d_head], du, dv_bias
 * [H, d_head], dbias like bias_table (needed when desc->bias_clamp >= 0).
 * The memory keys receive gradients like any key; a caller that detaches the
 * memory drops those rows. Gradients accumulate in fp32 (for bf16 operands
 * the products run on the bf16 matrix cores with fp32 operands split into a
 * high and a low bf16 part, about 16 bits of mantissa), P and dS are
 * materialised in the workspace (xl_rel_attn_core_bwd_workspace_size():
 * 8 bytes per (query, key) pair, 8 per query element, 4 per element of
 * batch x n_head x (table rows in use - 1) x d_head for per-batch-element
 * partial sums of dr, and 12 per query row for the softmax statistics), no
 * atomics.
 * Errors as xl_rel_attn_core; gradients must not overlap inputs, each other
 * or the workspace (XL_BAD_SHAPE).
 */
size_t xl_rel_attn_core_bwd_workspace_size(const xl_attn_desc* desc);
int xl_rel_attn_core_bwd(const xl_attn_desc* desc, const void* q, const void* k, const void* vt, int64_t ldv,
                         const void* r, int64_t n_rel, const void* u, const void* v, const void* bias_table,
                         const void* dout, float* dq, float* dk, float* dv, float* dr, float* du, float* dv_bias,
                         float* dbias, void* ws, size_t ws_bytes, void* stream);

/*
 * ---- The decoder layer around the attention, and the stacked layers ----
 * A decoder layer is one module of masked self-attention and a position-wise
 * feed-forward network; N of them are stacked, each module's output feeding
 * the next, and layer n keeps as its memory its own input states of the
 * previous segments (felixzhao.cn article 118 §1, §2.3.1). The attention
 * input is layer-normalised (2kiu.com §3.4), i.e. the layer is pre-LN:
 *     a   = RelAttn(queries LN1(h), keys and values over [LN1(mem) ; LN1(h)])
 *     h1  = h + a
 *     out = h1 + W2 relu(W1 LN2(h1) + b1) + b2
 * where LN is the row-wise layer normalisation (population variance,
 * y = (x - mean) / sqrt(var + eps) * gamma + beta; eps: ln_eps, 0 selects
 * 1e-5, the value intelliparadigm.com §4.2 names) and RelAttn is the layer of
 * xl_rel_attn_fwd. The pages name two linear layers around a nonlinearity
 * for the feed-forward network; the biases and the ReLU are readings taken
 * where they are silent. h1 is rounded to desc->dtype; out is in
 * desc->out_dtype. Every weight is in desc->dtype, on the device.
 */
typedef struct {
    xl_attn_weights attn;    /* the attention sublayer (its bias table too) */
    const void* ln1_g;       /* [D] LN1 gain */
    const void* ln1_b;       /* [D] LN1 shift */
    const void* ln2_g;       /* [D] LN2 gain */
    const void* ln2_b;       /* [D] LN2 shift */
    const void* w1;          /* [d_inner, D] */
    const void* b1;          /* [d_inner] */
    const void* w2;          /* [D, d_inner] */
    const void* b2;          /* [D] */
} xl_decoder_weights;

/*
 * One decoder layer on h [B, qlen, D] with the memory mem [B, mlen, D]
 * (desc->mlen; may be NULL when 0). d_inner: the feed-forward width, a
 * multiple of 32 (bf16) or 16 (f32). ws: xl_decoder_layer_workspace_size()
 * bytes (0 for an invalid desc), 256-byte aligned. out must not alias h, mem
 * or ws. Errors as xl_rel_attn_fwd, plus XL_BAD_SHAPE for d_inner or ln_eps.
 */
size_t xl_decoder_layer_workspace_size(const xl_attn_desc* desc, int64_t d_inner);
int xl_decoder_layer_fwd(const xl_attn_desc* desc, int64_t d_inner, float ln_eps, const xl_decoder_weights* w,
                         const void* h, const void* mem, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * One segment of an n_layer stack (w[n_layer], fifos[n_layer]): layer n runs
 * on its input (h for layer 0, else layer n-1's output) over
 * [memory of fifos[n] ; input], then fifos[n] takes that input as in
 * xl_segment_step (its ring is written after the layer has read it; len and
 * head are updated on return). The last layer writes out (desc->out_dtype);
 * the inner layers' outputs stay in the workspace (desc->dtype). Every
 * fifo's len must be <= desc->mlen; the rings must not overlap each other,
 * h, out or ws. ws: xl_decoder_stack_workspace_size() of desc with mlen the
 * largest fifo len of the call. On an error no fifo has been advanced unless
 * the status is XL_HIP_ERROR.
 */
size_t xl_decoder_stack_workspace_size(const xl_attn_desc* desc, int64_t d_inner);
int xl_decoder_stack_step(const xl_attn_desc* desc, int64_t d_inner, float ln_eps, int64_t n_layer,
                          const xl_decoder_weights* w, const void* h, xl_mem_fifo* fifos, void* out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * The same segment of an n_layer stack with each layer's memory kept as a
 * key ring of projected keys and values (rings[n_layer], xl_kv_fifo): the
 * cache reuse of intelliparadigm.com §3.2 applied to every layer of the
 * stack of felixzhao.cn §2.3.1. A layer's memory enters it only through LN1
 * and the key and value projections, and those rows were normalised and
 * projected with the same weights when they were that layer's input, so
 * layer n normalises and projects only its input's rows, straight into
 * rings[n] after the memory keys, and attends over the ring. For the same
 * inputs the outputs are those of xl_decoder_stack_step bit for bit. On
 * return each ring's len and head describe its last min(len + qlen,
 * mlen_max) keys. bf16 only; every ring as in xl_segment_step_kv (cap,
 * mlen_max, len, head and qlen multiples of 8), len <= desc->mlen; the rings
 * must not overlap each other, h, out or ws. ws:
 * xl_decoder_stack_kv_workspace_size() of desc with mlen the largest ring
 * len of the call (no normalised memory rows, no k or vt regions). On an
 * error no ring has been advanced unless the status is XL_HIP_ERROR.
 */
size_t xl_decoder_stack_kv_workspace_size(const xl_attn_desc* desc, int64_t d_inner);
int xl_decoder_stack_step_kv(const xl_attn_desc* desc, int64_t d_inner, float ln_eps, int64_t n_layer,
                             const xl_decoder_weights* w, const void* h, xl_kv_fifo* rings, void* out, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Timing hook: when both are non-NULL, the hipEvent_t handles ev_begin/ev_end
 * take the start and end timestamps of the fused attention kernel itself
 * (passed to the runtime with the kernel launch) in the next calls of
 * xl_rel_attn_fwd, xl_segment_step and xl_rel_attn_core on this thread, on the
 * launch stream. NULL, NULL switches it off. Returns XL_OK.
 */
int xl_set_core_events(void* ev_begin, void* ev_end);

#ifdef __cplusplus
}
#endif
#endif /* XL_REL_H */
