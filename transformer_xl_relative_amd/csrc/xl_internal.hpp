// xl_internal.hpp -- launchers shared between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xl {

hipError_t launch_relpos(int64_t delta0, int64_t n_rows, int64_t d_model, int64_t clamp_len,
                         double base, int out_bf16, void* out, hipStream_t s);

// Epilogues of the projection GEMM C = A B^T (A rows: activations, B rows: weights).
enum EpiKind : int {
    EPI_K = 1,    // q or k [B,H,seq,dh]
    EPI_VT = 2,   // vt [B,H,dh,ldv]
    EPI_R = 3,    // r [H, seq, dh] (seq = n_rel rows)
    EPI_OUT = 4,  // out [M, N] row-major, f32 or bf16
    EPI_KV = 5,   // columns n < b_split: k (out0), the others: vt (out1)
};

// One projection C = A B^T with its epilogue.
struct GemmArgs {
    int M, N, K;
    // A-operand rows. Row m of a "concat" problem (a_seq > 0) is token j = m % a_seq
    // of batch b = m / a_seq: j < a_split comes from the ring a0 (row
    // (ring_head + j) % ring_len of batch b), otherwise row j - a_split of a1.
    // With a_seq == 0 row m is a0 + m * lda.
    const void* a0;
    const void* a1;
    int64_t lda;             // elements between consecutive rows
    int64_t a0_bstride;      // elements between batches of a0
    int64_t a1_bstride;      // elements between batches of a1
    int a_seq, a_split, ring_len, ring_head;
    // B-operand rows ([out, in] weights): row n < b_split is b0[n], else b1[n - b_split]
    const void* b0;
    const void* b1;
    int b_split;
    // epilogue
    int epi;
    void* out0;
    void* out1;
    int H, dh, seq, ldv;
    int out_bf16;            // EPI_OUT: 1 bf16, 0 f32
    // K and V^T outputs into a key ring (EPI_KV, bf16): token j of a batch
    // lands at ring row (out_pos0 + j) mod out_rows of its head (k: out_rows
    // rows per head; V^T: ldv == out_rows columns). out_rows 0: no ring (k has
    // seq rows per head, token j at row j).
    int out_rows = 0;
    int out_pos0 = 0;
    // EPI_OUT extras: out = act(acc + bias_n[n]) + res[m, n], act the ReLU when
    // relu; bias_n [N] and res [M, N] (row-major) in the operand type, or null;
    // res_f32: res is fp32 also for bf16 operands
    const void* bias_n = nullptr;
    const void* res = nullptr;
    int relu = 0;
    int res_f32 = 0;
};

constexpr int kMaxGemms = 4;

// The FIFO ring write (see launch_fifo_write), carried by a GEMM launch whose
// tiles leave compute units idle: extra workgroups of the same grid copy the
// rows meanwhile. Nothing the GEMMs read or write may overlap src or ring.
struct RowCopy {
    const void* src;
    void* ring;
    int64_t qlen, ring_len, dst0, src0, n, B, row_bytes;
};

// Launch up to kMaxGemms independent projections as one grid (their tiles
// share the machine), and the row copy cp if not null. K of every problem
// must be a multiple of 64 bytes.
hipError_t launch_gemms(const GemmArgs* g, int count, bool bf16, hipStream_t s, const RowCopy* cp = nullptr);
// the bf16 kernels (gemm_bf16.hip); launch_gemms forwards bf16 problems here
hipError_t launch_gemms_bf16(const GemmArgs* g, int count, hipStream_t s, const RowCopy* cp);
inline hipError_t launch_gemm(const GemmArgs& g, bool bf16, hipStream_t s, const RowCopy* cp = nullptr) {
    return launch_gemms(&g, 1, bf16, s, cp);
}

struct AttnArgs {
    const void* q;        // [B, H, qlen, dh] projected queries
    const void* u;        // [H, dh] content bias
    const void* v;        // [H, dh] position bias
    float scale;          // score scale, applied as scale*(q+u), scale*(q+v)
    const void* k;
    const void* vt;
    const void* r;
    const void* bias;     // [2*bias_clamp+1, H], [12, H] (bias_kind 1) or nullptr
    void* out;            // [B, qlen, H*dh]
    int B, H, qlen, mlen, klen, ldv;
    int n_rel;            // distance delta uses row min(delta, n_rel - 1)
    int r_rows;           // rows per head in r (>= n_rel)
    // keys in a ring (bf16 kernel): key j of a head is ring row
    // (kv_head + j) mod kv_rows of k ([B,H,kv_rows,dh]) and column of vt
    // (ldv == kv_rows); kv_rows 0: k has klen rows per head, key j at row j
    int kv_rows = 0;
    int kv_head = 0;
    int bias_clamp;
    int bias_kind = 0;    // 0: row clamp(delta, +-bias_clamp) + bias_clamp; 1: t5_bucket(delta)
    // key splits of the bf16 kernel: a query tile with ts key steps is shared by
    // min(ceil(ts / split_steps), split_max) workgroups (split_steps 0: none).
    // part holds split_max * B*H*qlen * (d_head + 2) floats of partial results.
    int split_steps = 0;
    int split_max = 1;
    void* part = nullptr;
};

// T5 bucket of a distance on the boundaries 1, 2, 4, ..., 1024: 0 for
// delta <= 1, b for 2^(b-1) < delta <= 2^b (b <= 10), 11 beyond 1024.
__host__ __device__ inline int t5_bucket(int delta) {
    if (delta <= 1) return 0;
    const int b = 32 - __builtin_clz((unsigned)(delta - 1));
    return b < 11 ? b : 11;
}
// bias table row of a distance
__host__ __device__ inline int bias_row(int delta, int bias_kind, int bias_clamp) {
    if (bias_kind) return t5_bucket(delta);
    return (delta < -bias_clamp ? -bias_clamp : delta > bias_clamp ? bias_clamp : delta) + bias_clamp;
}

constexpr int kMaxAttnSplits = 64;
// The split plan of a bf16 problem (forced > 0: up to `forced` workgroups per
// tile), and the bytes of its partial results.
struct SplitPlan {
    int steps, max;
};
SplitPlan attn_bf16_split_plan(int64_t B, int64_t H, int64_t qlen, int64_t mlen, int forced);
size_t attn_bf16_part_bytes(int64_t B, int64_t H, int64_t qlen, const SplitPlan& p);
// bytes of the split partials for every memory length at once (a bound on the
// split count that does not depend on mlen, so workspace sizes grow with mlen)
size_t attn_bf16_part_bytes_bound(int64_t B, int64_t H, int64_t qlen, int forced);

// fused attention for bf16 operands and d_head 64 (attn_bf16.hip)
// ev0/ev1 (may be null): events the runtime timestamps at the start and end of
// the attention kernel itself
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_attn(const AttnArgs& a, bool bf16, int dh, hipStream_t s, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr);

// Gradients of the attention core (attn_bwd.hip). Inputs as AttnArgs (q, k,
// vt, r with r_rows rows per head, u, v, bias) in the element type, dout
// [B, qlen, H*dh] likewise; P and dS are workspace [B, H, qlen, klen] fp32,
// dqu and dqv workspace [B, H, qlen, dh] fp32. Outputs fp32: dq [B,H,qlen,dh],
// dk, dv [B,H,klen,dh], dr [H, r_rows, dh], du, dvb [H, dh], dbias
// [bias_rows, H] (when bias).
struct AttnBwdArgs {
    const void* q;
    const void* k;
    const void* vt;
    const void* r;
    const void* u;
    const void* v;
    const void* bias;
    const void* dout;
    float scale;
    int B, H, qlen, mlen, klen, ldv, n_rel, r_rows;
    int bias_clamp, bias_kind, bias_rows;
    float* P;
    float* dS;
    float* dqu;
    float* dqv;
    float* dq;
    float* dk;
    float* dv;
    float* dr;
    float* du;
    float* dvb;
    float* dbias;
    float* drp;     // per-batch-element partial sums of dr for rows c < dr_first
    float* uvp;     // tiled path: per (b, h, query block) column sums for du, dv
    float* rstat;   // tiled path: per query row (m, 1/s, D); P and dS then hold l and dP
    int dr_first;   // rows c >= dr_first of dr come from the per-row kernel
};
hipError_t launch_attn_bwd(const AttnBwdArgs& a, bool bf16, int dh, hipStream_t s);

// Layer normalisation of rows (b, j), j < a_seq, b < rows / a_seq: row j <
// a_split of batch b is ring row (ring_head + j) % ring_len of a0 (batch
// stride a0_bstride elements) and goes to y0 [B, a_split, D]; the others are
// row j - a_split of a1 (batch stride a1_bstride) and go to y1
// [B, a_seq - a_split, D]. gamma, beta [D]; every tensor in one element type;
// D a multiple of 8 (bf16) or 4 (f32).
struct LnArgs {
    const void* a0;
    const void* a1;
    int64_t a0_bstride, a1_bstride;
    int a_seq, a_split, ring_len, ring_head;
    void* y0;
    void* y1;
    const void* gamma;
    const void* beta;
    int rows, D;
    float eps;
    int x_f32;   // bf16: the rows read (a0, a1) are fp32; gamma, beta and y stay bf16
};
hipError_t launch_layer_norm(const LnArgs& a, bool bf16, hipStream_t s);

// FIFO write: copies rows h[b, src0 + t, :] (t < n) to ring row
// (dst0 + t) % ring_len of batch b.
hipError_t launch_fifo_write(const void* h, int64_t qlen, void* ring, int64_t ring_len, int64_t dst0,
                             int64_t src0, int64_t n, int64_t B, int64_t row_bytes, hipStream_t s);

}  // namespace xl
