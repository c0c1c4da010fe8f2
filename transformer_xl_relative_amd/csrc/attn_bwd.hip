// attn_bwd.hip -- gradients of the fused relative attention core.
//
// For one head and the logits l_ij = (qu_i . k_j + qv_i . r_c) + beta[row]
// of the forward (qu = scale*(q+u), qv = scale*(q+v), c the table row of the
// distance delta = mlen + i - j clamped to n_rel - 1, causal: j <= mlen + i),
// P = softmax_j(l), and an upstream gradient dO of o = P.V:
//   dP_ij = dO_i . v_j,  D_i = sum_j P_ij dP_ij,  dS_ij = P_ij (dP_ij - D_i)
//   dq_i = scale * sum_j dS_ij (k_j + r_c)        (qu and qv both carry q)
//   dk_j = sum_i dS_ij qu_i,   dv_j = sum_i P_ij dO_i
//   dr_c = sum over pairs of row c of dS_ij qv_i  (the transpose of the shift)
//   du = scale * sum_i sum_j dS_ij k_j,  dv = scale * sum_i sum_j dS_ij r_c
//   dbeta[row] = sum over pairs of that row of dS_ij
// (the chain rule through the softmax and the four dot products of
// qidao123.com thread-401555 §3; the shift's transpose gathers the band
// back per distance, felixzhao.cn article 118 §2.3.2).
//
// P and dS are materialised in the workspace ([B, H, qlen, klen] fp32 each),
// every output is written by one thread (no atomics). For bf16 operands with
// d_head 64 the work runs in 64 x 64 blocks staged through LDS, the products
// on the bf16 matrix cores with fp32 operands split into a high and a low
// bf16 part (fp32 accumulation, about 16 bits of mantissa per operand):
//   logits: one workgroup per 64 queries walks their key blocks: l and dP
//           per pair, and the row statistics (m, 1/s, D)
//   dk/dv:  rows keys, summed over queries; its loader turns l, dP into
//           P, dS and writes dS back in place for the kernels after it
//   dq:     rows queries, summed over keys and over distances; it also
//           leaves per-block column sums for du, dv
//   dr:     rows table rows below the last in use, summed over the queries
//           of one batch element; a reduce adds the elements
//   small:  the last table row in use (every clamped distance), du, dv and
//           the bias table gradient
// For fp32 operands (d_head 8) a plain form: one wave per query row (logits,
// softmax, dP, dS; then dq), per key (dk, dv) and per table row (dr), d_head
// or keys across the lanes, rows re-read from the caches for every pair.
#include "xl_common.hpp"
#include "xl_internal.hpp"

namespace xl {
namespace {

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    return Elem<T>::to_f(((const T*)p)[i]);
}

// the bias table row of a visible distance (delta >= 0)
__device__ __forceinline__ int brow(const AttnBwdArgs& a, int delta) {
    return bias_row(delta, a.bias_kind, a.bias_clamp);
}

// XCD-aware block order for the blocked kernels: workgroups are dealt
// round-robin to the 8 XCDs (workgroup w runs on XCD w % 8), so numbering
// them such that XCD x takes the x-th eighth of the n blocks keeps the rows
// of one head within one L2. Grids are padded to a multiple of 8; a result
// >= n is padding.
__device__ __forceinline__ int xcd_block(int n) {
    const int w = (int)__builtin_amdgcn_workgroup_id_x(), per = (n + 7) / 8;
    return (w & 7) * per + (w >> 3);
}
__host__ __forceinline__ unsigned xcd_grid(int64_t n) { return (unsigned)((n + 7) / 8 * 8); }

// dS_ij of a visible pair, once final (after the row kernel of the plain
// path, after the dk/dv kernel of the tiled path)
__device__ __forceinline__ float ds_at(const AttnBwdArgs& a, int64_t row, int j) { return a.dS[row * a.klen + j]; }

template <typename T, int DH>
__global__ void __launch_bounds__(256) bwd_rows_kernel(AttnBwdArgs a) {
    __shared__ float sh[4][3][DH];   // per wave: qu, qv, dO of its row
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int wave = (int)__builtin_amdgcn_workitem_id_x() >> 6;
    const int64_t row = (int64_t)__builtin_amdgcn_workgroup_id_x() * 4 + wave;
    if (row >= (int64_t)a.B * a.H * a.qlen) return;
    const int i = (int)(row % a.qlen);
    const int bh = (int)(row / a.qlen);
    const int h = bh % a.H, b = bh / a.H;
    if (lane < DH) {
        const float qd = ld<T>(a.q, row * DH + lane);
        sh[wave][0][lane] = a.scale * (qd + ld<T>(a.u, h * DH + lane));
        sh[wave][1][lane] = a.scale * (qd + ld<T>(a.v, h * DH + lane));
        sh[wave][2][lane] = ld<T>(a.dout, ((int64_t)b * a.qlen + i) * a.H * DH + h * DH + lane);
    }
    __builtin_amdgcn_wave_barrier();
    const float* qu = sh[wave][0];
    const float* qv = sh[wave][1];
    const float* go = sh[wave][2];
    const int nv = a.mlen + i + 1;
    float* P = a.P + row * a.klen;
    float* S = a.dS + row * a.klen;
    const int64_t kbase = (int64_t)bh * a.klen;
    float m = -INFINITY;
    for (int j = lane; j < nv; j += 64) {
        const int delta = a.mlen + i - j;
        const int c = delta < a.n_rel - 1 ? delta : a.n_rel - 1;
        const int64_t kr = (kbase + j) * DH, rr = ((int64_t)h * a.r_rows + c) * DH;
        float l = 0.f;
#pragma unroll 8
        for (int d = 0; d < DH; ++d) l += qu[d] * ld<T>(a.k, kr + d) + qv[d] * ld<T>(a.r, rr + d);
        if (a.bias) l += ld<T>(a.bias, (int64_t)brow(a, delta) * a.H + h);
        P[j] = l;
        m = fmaxf(m, l);
    }
    m = wmax(m);
    float s = 0.f;
    for (int j = lane; j < nv; j += 64) {
        const float e = __expf(P[j] - m);
        P[j] = e;
        s += e;
    }
    const float inv = 1.f / wsum(s);
    const int64_t vbase = (int64_t)bh * DH * a.ldv;
    float dsum = 0.f;
    for (int j = lane; j < nv; j += 64) {
        const float p = P[j] * inv;
        float dp = 0.f;
#pragma unroll 8
        for (int d = 0; d < DH; ++d) dp += go[d] * ld<T>(a.vt, vbase + (int64_t)d * a.ldv + j);
        P[j] = p;
        S[j] = dp;
        dsum += p * dp;
    }
    const float D = wsum(dsum);
    for (int j = lane; j < nv; j += 64) S[j] = P[j] * (S[j] - D);
}

// waves per workgroup of the dq, dk/dv and dr kernels: neighbouring rows of
// one head in one workgroup share their key, query and table rows in L1
constexpr int BW = 4;
constexpr int ILP = 4;   // independent partial sums per lane in their loops

template <typename T, int DH>
__global__ void __launch_bounds__(64 * BW) bwd_dq_kernel(AttnBwdArgs a) {
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int64_t row = (int64_t)__builtin_amdgcn_workgroup_id_x() * BW + ((int)__builtin_amdgcn_workitem_id_x() >> 6);
    if (row >= (int64_t)a.B * a.H * a.qlen || lane >= DH) return;
    const int i = (int)(row % a.qlen);
    const int bh = (int)(row / a.qlen);
    const int h = bh % a.H;
    const int nv = a.mlen + i + 1;
    const float* S = a.dS + row * a.klen;
    const int64_t kbase = (int64_t)bh * a.klen;
    // ILP partial sums: four keys in flight per iteration
    float pu[ILP] = {}, pv[ILP] = {};
    int j = 0;
    for (; j + ILP <= nv; j += ILP) {
#pragma unroll
        for (int x = 0; x < ILP; ++x) {
            const int delta = a.mlen + i - (j + x);
            const int c = delta < a.n_rel - 1 ? delta : a.n_rel - 1;
            const float ds = S[j + x];
            pu[x] += ds * ld<T>(a.k, (kbase + j + x) * DH + lane);
            pv[x] += ds * ld<T>(a.r, ((int64_t)h * a.r_rows + c) * DH + lane);
        }
    }
    for (; j < nv; ++j) {
        const int delta = a.mlen + i - j;
        const int c = delta < a.n_rel - 1 ? delta : a.n_rel - 1;
        const float ds = S[j];
        pu[0] += ds * ld<T>(a.k, (kbase + j) * DH + lane);
        pv[0] += ds * ld<T>(a.r, ((int64_t)h * a.r_rows + c) * DH + lane);
    }
    float cu = 0.f, cv = 0.f;
#pragma unroll
    for (int x = 0; x < ILP; ++x) {
        cu += pu[x];
        cv += pv[x];
    }
    a.dq[row * DH + lane] = a.scale * (cu + cv);
    a.dqu[row * DH + lane] = cu;
    a.dqv[row * DH + lane] = cv;
}

template <typename T, int DH>
__global__ void __launch_bounds__(64 * BW) bwd_dkdv_kernel(AttnBwdArgs a) {
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int64_t key = (int64_t)__builtin_amdgcn_workgroup_id_x() * BW + ((int)__builtin_amdgcn_workitem_id_x() >> 6);
    if (key >= (int64_t)a.B * a.H * a.klen || lane >= DH) return;
    const int j = (int)(key % a.klen);
    const int bh = (int)(key / a.klen);
    const int h = bh % a.H, b = bh / a.H;
    const float ud = ld<T>(a.u, h * DH + lane);
    float gk = 0.f, gv = 0.f;
    const int i0 = j > a.mlen ? j - a.mlen : 0;
#pragma unroll 4
    for (int i = i0; i < a.qlen; ++i) {
        const int64_t row = (int64_t)bh * a.qlen + i;
        const float ds = a.dS[row * a.klen + j];
        const float p = a.P[row * a.klen + j];
        gk += ds * a.scale * (ld<T>(a.q, row * DH + lane) + ud);
        gv += p * ld<T>(a.dout, ((int64_t)b * a.qlen + i) * a.H * DH + h * DH + lane);
    }
    a.dk[key * DH + lane] = gk;
    a.dv[key * DH + lane] = gv;
}

// one wave per (head, table row c); rows >= n_rel (unused by any pair) get 0
template <typename T, int DH>
__global__ void __launch_bounds__(64 * BW) bwd_dr_kernel(AttnBwdArgs a) {
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int64_t w = (int64_t)__builtin_amdgcn_workgroup_id_x() * BW + ((int)__builtin_amdgcn_workitem_id_x() >> 6);
    const int nr = a.r_rows - a.dr_first;
    if (w >= (int64_t)a.H * nr || lane >= DH) return;
    const int c = a.dr_first + (int)(w % nr), h = (int)(w / nr);
    float acc = 0.f;
    if (c < a.n_rel) {
        const int d_hi = c < a.n_rel - 1 ? c : a.klen - 1;   // distances of row c: [c, d_hi]
        const float vd = ld<T>(a.v, h * DH + lane);
        for (int delta = c; delta <= d_hi; ++delta) {
            // the pairs of distance delta: (batch element b, query i0 + k) for
            // k < rows, taken as one flat range u = b rows + k, so that ILP
            // independent loads are in flight also when each element has few
            const int i0 = delta > a.mlen ? delta - a.mlen : 0;
            const int rows = a.qlen - i0, nu = a.B * rows;
            auto term = [&](int u) __attribute__((always_inline)) {
                const int b = u / rows, i = i0 + (u - b * rows);
                const int64_t row = ((int64_t)b * a.H + h) * a.qlen + i;
                return ds_at(a, row, a.mlen + i - delta) * (ld<T>(a.q, row * DH + lane) + vd);
            };
            float pa[ILP] = {};
            int u = 0;
            for (; u + ILP <= nu; u += ILP) {
#pragma unroll
                for (int x = 0; x < ILP; ++x) pa[x] += term(u + x);
            }
            for (; u < nu; ++u) pa[0] += term(u);
#pragma unroll
            for (int x = 0; x < ILP; ++x) acc += a.scale * pa[x];
        }
    }
    a.dr[((int64_t)h * a.r_rows + c) * DH + lane] = acc;
}

// the eight bf16 of a 16-byte piece as floats
__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
}

// merge two (max, sum of exp(x - max), sum of exp(x - max) y) triples of one row
__device__ __forceinline__ void merge_stats(float& m, float& s, float& e, float m2, float s2, float e2) {
    const float mx = fmaxf(m, m2);
    if (mx == -INFINITY) return;   // both empty
    const float w1 = __expf(m - mx), w2 = __expf(m2 - mx);
    s = s * w1 + s2 * w2;
    e = e * w1 + e2 * w2;
    m = mx;
}

// ---- Logits, dP and the row statistics, one workgroup per 64 queries ----
// A workgroup takes queries i0..i0+63 of one head and walks the key blocks of
// 64 that they see, so the query operands are loaded and split once, the
// next block's keys, values and table rows load while the current block is
// computed, and the softmax statistics of each row stay in registers. Wave
// (wq, wk) computes the 32 x 32 quarter of queries i0 + 32 wq .. and keys
// j0 + 32 wk .. of every block, transposed (keys or distances on the MFMA
// rows, queries on the columns: a lane owns one query), on the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   content  k . qu      qu = s (q + u) enters as a high and a low bf16 part
//                        (hi = bf16(qu), lo = bf16(qu - hi): 16 bits of
//                        mantissa), k is exact: two products
//   dP       v . dO      both exact bf16: one product
//   position r . qv      qv split like qu, over the 63 distances the quarter
//                        spans (two blocks of 32 table rows), then gathered
//                        through LDS: pair (i, j) takes band row 31 + i - j
// The logits of visible pairs (plus the bias table entry) go to the P buffer
// and dP to the dS buffer. Each lane keeps (m, sum exp(l - m), sum exp(l - m) dP) of its query over its keys,
// merged at the end with the other half-wave and the other key wave into
// (m, 1/s, D) per row.
constexpr int LRP = 64 * 2 + 16;     // bytes per staged row of 64 bf16 (conflict-free 16-byte reads)
constexpr int BSP = 40;              // floats per row of a wave's band scratch
constexpr int LR_STG = 256 * LRP;    // staged K rows (64), V rows (64), table rows (128)
constexpr int LR_SCR = 64 * BSP * 4; // per wave: the band quarter (64 rows of 32 queries)

__global__ void __launch_bounds__(256, 2) bwd_logits_rows_kernel(AttnBwdArgs a) {
    constexpr int DH = 64;
    constexpr int KS = 0, VS = 64, RS = 128;   // staged rows
    extern __shared__ __attribute__((aligned(16))) char lsm[];
    char* stg = lsm;
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63, wave = tid >> 6, hf = lane >> 5, li = lane & 31;
    const int wq = wave >> 1, wk = wave & 1;
    float* scr = (float*)(lsm + LR_STG + wave * LR_SCR);
    const int BH = a.B * a.H, nit = (a.qlen + 63) / 64;
    // heaviest query blocks first; with BH a multiple of 8 a head stays on XCD g % 8
    const int w = (int)__builtin_amdgcn_workgroup_id_x();
    if (w >= BH * nit) return;
    const int it = nit - 1 - w / BH, g = w % BH;
    const int h = g % a.H, b = g / a.H;
    const int i0 = 64 * it;
    const int ilast = i0 + 63 < a.qlen ? i0 + 63 : a.qlen - 1;
    const int njt = (a.klen + 63) / 64;
    int jt_last = (a.mlen + ilast) / 64;
    if (jt_last > njt - 1) jt_last = njt - 1;
    const int64_t rb = (int64_t)g * a.qlen;
    const bf16_t* kp = (const bf16_t*)a.k;
    const bf16_t* vp = (const bf16_t*)a.vt;
    const bf16_t* rp = (const bf16_t*)a.r;
    const u32x4 z = {0u, 0u, 0u, 0u};

    // ---- query operands (MFMA B): lane owns query iq, d_head 16 kk + 8 hf .. + 7
    const int iq = i0 + 32 * wq + li;
    const bool qok = iq < a.qlen;
    bf16x8 quh[4], qul[4], qvh[4], qvl[4], dob[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int d = 16 * kk + 8 * hf;
        const u32x4 fq = qok ? *(const u32x4*)((const bf16_t*)a.q + (rb + iq) * DH + d) : z;
        const u32x4 fo = qok ? *(const u32x4*)((const bf16_t*)a.dout + (((int64_t)b * a.qlen + iq) * a.H + h) * DH + d) : z;
        const u32x4 fu = *(const u32x4*)((const bf16_t*)a.u + h * DH + d);
        const u32x4 fv = *(const u32x4*)((const bf16_t*)a.v + h * DH + d);
        float x[8], uu[8], vv[8];
        unpack8(fq, x);
        unpack8(fu, uu);
        unpack8(fv, vv);
        u32x4 uh, ul, wh, wl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float hu[2], lu[2], hw[2], lw[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float qu = qok ? a.scale * (x[2 * e + k] + uu[2 * e + k]) : 0.f;
                const float qv = qok ? a.scale * (x[2 * e + k] + vv[2 * e + k]) : 0.f;
                hu[k] = bf2f(f2bf(qu));
                lu[k] = qu - hu[k];
                hw[k] = bf2f(f2bf(qv));
                lw[k] = qv - hw[k];
            }
            uh[e] = pack2bf(hu[0], hu[1]);
            ul[e] = pack2bf(lu[0], lu[1]);
            wh[e] = pack2bf(hw[0], hw[1]);
            wl[e] = pack2bf(lw[0], lw[1]);
        }
        quh[kk] = as_bf16x8(uh);
        qul[kk] = as_bf16x8(ul);
        qvh[kk] = as_bf16x8(wh);
        qvl[kk] = as_bf16x8(wl);
        dob[kk] = as_bf16x8(fo);
    }

    // ---- staging of key block jt: K rows and V rows (by key, from V^T) of keys
    // j0 .., table rows of distances dlo + rho, rho < 128, dlo = mlen + i0 - j0 - 63
    // (clamped to the table). Thread: K chunks (row, 16 bytes) tid, tid + 256;
    // V^T pieces (d_head row, 8 keys) tid, tid + 256; table chunks tid + 256 t.
    u32x4 fk[2], fvt[2], fr[4];
    auto fetch = [&](int jt) __attribute__((always_inline)) {
        const int j0 = 64 * jt, dlo = a.mlen + i0 - j0 - 63;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int c = tid + 256 * t, row = c >> 3, ch = c & 7;
            fk[t] = j0 + row < a.klen ? *(const u32x4*)(kp + ((int64_t)g * a.klen + j0 + row) * DH + 8 * ch) : z;
            const int d = c & 63, kc = c >> 6, jj = j0 + 8 * kc;
            fvt[t] = jj < a.ldv ? *(const u32x4*)(vp + ((int64_t)g * DH + d) * a.ldv + jj) : z;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = tid + 256 * t, row = c >> 3, ch = c & 7;
            int dist = dlo + row;
            dist = dist < 0 ? 0 : (dist > a.n_rel - 1 ? a.n_rel - 1 : dist);
            fr[t] = *(const u32x4*)(rp + ((int64_t)h * a.r_rows + dist) * DH + 8 * ch);
        }
    };
    auto stash = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int c = tid + 256 * t, row = c >> 3, ch = c & 7;
            *(u32x4*)(stg + (KS + row) * LRP + 16 * ch) = fk[t];
            const int d = c & 63, kc = c >> 6;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *(bf16_t*)(stg + (VS + 8 * kc + e) * LRP + 2 * d) = (bf16_t)((fvt[t][e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = tid + 256 * t, row = c >> 3, ch = c & 7;
            *(u32x4*)(stg + (RS + row) * LRP + 16 * ch) = fr[t];
        }
    };
    auto rd = [&](int r, int off) __attribute__((always_inline)) {
        return as_bf16x8(*(const u32x4*)(stg + r * LRP + off));
    };

    // running statistics of query iq over this lane's keys
    float m = -INFINITY, s = 0.f, sd = 0.f;
    const int rho0 = 32 + 32 * wq - 32 * wk;   // first staged table row of the quarter
    const bool vec = (a.klen & 3) == 0;        // rows of P and dS are 16-byte aligned
    fetch(0);
    stash();
    __syncthreads();
    for (int jt = 0; jt <= jt_last; ++jt) {
        if (jt < jt_last) fetch(jt + 1);
        const int j0 = 64 * jt, jq = j0 + 32 * wk;   // first key of the quarter
        // the quarter sees a pair when its first key is visible to its last query
        const int iql = i0 + 32 * wq + 31 < a.qlen ? i0 + 32 * wq + 31 : a.qlen - 1;
        if (jq <= a.mlen + iql) {
            // in phases, so that at most two accumulator blocks are live: the
            // band (then parked in LDS), the content with the gathered band,
            // then dP
            f32x16 ab0, ab1;
#pragma unroll
            for (int v = 0; v < 16; ++v) ab0[v] = ab1[v] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int off = 32 * kk + 16 * hf;
                const bf16x8 r0 = rd(RS + rho0 + li, off), r1 = rd(RS + rho0 + 32 + li, off);
                ab0 = mfma32(r0, qvh[kk], ab0);
                ab1 = mfma32(r1, qvh[kk], ab1);
                ab0 = mfma32(r0, qvl[kk], ab0);
                ab1 = mfma32(r1, qvl[kk], ab1);
            }
            // band rows t (distance dlo + rho0 + t) of query li, then the pairs:
            // key jq + kj takes band row 31 + li - kj
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = 8 * (v >> 2) + 4 * hf + (v & 3);
                scr[t * BSP + li] = ab0[v];
                scr[(32 + t) * BSP + li] = ab1[v];
            }
            __builtin_amdgcn_wave_barrier();
            __asm__ __volatile__("" ::: "memory");
            f32x16 ac;
#pragma unroll
            for (int v = 0; v < 16; ++v) ac[v] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int off = 32 * kk + 16 * hf;
                const bf16x8 kv = rd(KS + 32 * wk + li, off);
                ac = mfma32(kv, quh[kk], ac);
                ac = mfma32(kv, qul[kk], ac);
            }
            // every pair of the quarter visible (its last key to its first
            // query, all queries in range): no test per pair
            const bool full = i0 + 32 * wq + 31 < a.qlen && jq + 31 <= a.mlen + i0 + 32 * wq;
            float lv[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int kj = 8 * (v >> 2) + 4 * hf + (v & 3);
                const int j = jq + kj;
                const bool vis = full || (qok && j <= a.mlen + iq);
                float l = ac[v] + scr[(31 + li - kj) * BSP + li];
                if (a.bias && vis) l += bf2f(((const bf16_t*)a.bias)[(int64_t)brow(a, a.mlen + iq - j) * a.H + h]);
                lv[v] = vis ? l : -INFINITY;
            }
            __builtin_amdgcn_wave_barrier();
            __asm__ __volatile__("" ::: "memory");
            f32x16 ap;
#pragma unroll
            for (int v = 0; v < 16; ++v) ap[v] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) ap = mfma32(rd(VS + 32 * wk + li, 32 * kk + 16 * hf), dob[kk], ap);
            // stores: four consecutive keys per register group
            float* pl = a.P + (rb + iq) * a.klen;
            float* pd = a.dS + (rb + iq) * a.klen;
            if (full && vec) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int j = jq + 8 * gq + 4 * hf;
                    *(f32x4*)(pl + j) = (f32x4){lv[4 * gq], lv[4 * gq + 1], lv[4 * gq + 2], lv[4 * gq + 3]};
                    *(f32x4*)(pd + j) = (f32x4){ap[4 * gq], ap[4 * gq + 1], ap[4 * gq + 2], ap[4 * gq + 3]};
                }
            } else if (qok) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int j = jq + 8 * gq + 4 * hf;
                    if (vec && j + 3 <= a.mlen + iq) {
                        *(f32x4*)(pl + j) = (f32x4){lv[4 * gq], lv[4 * gq + 1], lv[4 * gq + 2], lv[4 * gq + 3]};
                        *(f32x4*)(pd + j) = (f32x4){ap[4 * gq], ap[4 * gq + 1], ap[4 * gq + 2], ap[4 * gq + 3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (j + e <= a.mlen + iq) {
                                pl[j + e] = lv[4 * gq + e];
                                pd[j + e] = ap[4 * gq + e];
                            }
                    }
                }
            }
            // statistics: rescale to a grown maximum, then add the block
            float mb = lv[0];
#pragma unroll
            for (int v = 1; v < 16; ++v) mb = fmaxf(mb, lv[v]);
            if (mb > m) {
                const float sc = __expf(m - mb);
                s *= sc;
                sd *= sc;
                m = mb;
            }
            if (full) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float e = __expf(lv[v] - m);
                    s += e;
                    sd += e * ap[v];
                }
            } else if (m != -INFINITY) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    // masked pairs add nothing (dP past klen may be anything)
                    const float e = lv[v] != -INFINITY ? __expf(lv[v] - m) : 0.f;
                    s += e;
                    sd += lv[v] != -INFINITY ? e * ap[v] : 0.f;
                }
            }
        }
        __syncthreads();   // every wave is done with block jt's operands
        if (jt < jt_last) {
            stash();
            __syncthreads();
        }
    }
    // merge the half-waves (the same query), then the two key waves
    merge_stats(m, s, sd, __shfl_xor(m, 32, 64), __shfl_xor(s, 32, 64), __shfl_xor(sd, 32, 64));
    float* xs = (float*)(lsm + LR_STG);   // the wave scratch is free now
    if (wk == 1 && hf == 0) {
        xs[(wq * 32 + li) * 3] = m;
        xs[(wq * 32 + li) * 3 + 1] = s;
        xs[(wq * 32 + li) * 3 + 2] = sd;
    }
    __syncthreads();
    if (wk == 0 && hf == 0 && qok) {
        merge_stats(m, s, sd, xs[(wq * 32 + li) * 3], xs[(wq * 32 + li) * 3 + 1], xs[(wq * 32 + li) * 3 + 2]);
        a.rstat[(rb + iq) * 3] = m;
        a.rstat[(rb + iq) * 3 + 1] = 1.f / s;
        a.rstat[(rb + iq) * 3 + 2] = sd / s;
    }
}

// ---- Tiled products for d_head 64 ----
// With P and dS stored, the dq, dk/dv and dr sums are products of a
// [rows x t] slice of dS or P with a [t x 64] slice of query, key, table or
// dO rows, causal entries masked out:
//   dk/dv: rows keys j,  t queries i:   dS_ij (q_i + u),  P_ij dO_i
//   dq:    rows queries i, t keys j:    dS_ij k_j, and with t a distance
//          delta = mlen + i - j:        dS_i(mlen+i-delta) r_min(delta, n_rel-1)
//   dr:    rows table rows c < n_rel - 1, t queries i of one batch element:
//          dS_i(mlen+i-c) (q_i + v)
// A workgroup of 4 waves computes a 64 x 64 block of one head's output, a
// 32 x 32 quarter per wave on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation), and stages 32 values of t of each operand through LDS
// as bf16, both operands t-contiguous per row (80-byte rows): lane (li, half)
// feeds row li with t = 16 kk + 8 half .. + 7. The fp32 operands (dS, P, and
// q + u, q + v) enter as a high and a low bf16 part (hi = bf16(x),
// lo = bf16(x - hi): 16 bits of mantissa); key, table and dO rows are exact
// bf16. A product of two split operands takes hi.hi + hi.lo + lo.hi (the
// dropped lo.lo is below 2^-16 of it), one split and one exact operand two
// instructions. The next stage's operands are loaded into registers while
// this one is computed. dr splits over the batch elements (partial sums per element,
// added by bwd_dr_reduce_kernel) so that its grid fills the chip.
enum : int { TP_DKDV = 0, TP_DQ = 1, TP_DR = 2 };
constexpr int TM = 64, TT = 32, TPB = TT * 2 + 16;   // TPB: bytes per staged bf16 row

// (dq fits 4 waves per SIMD without spilling; dk/dv would spill)
template <int MODE>
__global__ void __launch_bounds__(256, MODE == TP_DQ ? 4 : 1) bwd_tile_kernel(AttnBwdArgs a) {
    constexpr int DH = 64;
    constexpr int NP = MODE == TP_DR ? 1 : 2;   // products per block
    // per product: A high and low parts (rows m), B high and low parts (rows d)
    __shared__ __attribute__((aligned(16))) char sA[NP][2][TM * TPB];
    __shared__ __attribute__((aligned(16))) char sB[NP][2][DH * TPB];
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int nrows = MODE == TP_DKDV ? a.klen : (MODE == TP_DQ ? a.qlen : a.dr_first);
    const int nmt = (nrows + TM - 1) / TM;
    int wg = xcd_block(a.B * a.H * nmt);
    if (wg >= a.B * a.H * nmt) return;
    int b = 0;
    if (MODE == TP_DR) {   // grid: (batch element, head, row tile)
        b = wg / (a.H * nmt);
        wg -= b * a.H * nmt;
    }
    const int g = wg / nmt, m0 = (wg - g * nmt) * TM;   // g: b*H + h, or h for dr
    const int h = MODE == TP_DR ? g : g % a.H;
    if (MODE != TP_DR) b = g / a.H;
    const int64_t rb = ((int64_t)b * a.H + h) * a.qlen;   // first query row of the head
    // t range
    int t_lo = 0, t_hi;
    if (MODE == TP_DQ) {
        const int last = m0 + TM < a.qlen ? m0 + TM - 1 : a.qlen - 1;
        t_hi = a.mlen + last + 1;
    } else {
        t_lo = m0 > a.mlen ? m0 - a.mlen : 0;
        t_hi = a.qlen;
    }
    // the stage operands of this thread
    float bias8[8];
    {
        const int d8 = tid >> 5;
        const bf16_t* bv = (const bf16_t*)(MODE == TP_DKDV ? a.u : a.v) + h * DH + 8 * d8;
#pragma unroll
        for (int e = 0; e < 8; ++e) bias8[e] = (MODE == TP_DQ) ? 0.f : bf2f(bv[e]);
    }
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    float ra[NP][8];
    float rs[MODE == TP_DKDV ? 8 : 1][3];   // dk/dv: the row statistics of the fetched pairs
    u32x4 rbv[NP];
    int ft0 = 0;                            // first t of the fetched stage
    auto fetch = [&](int t0) __attribute__((always_inline)) {
        ft0 = t0;
        // pair k of this thread: (m, t) as below. Whether it is a visible pair
        // inside the block is monotone in k for each bound, so when the first
        // and the last are, all eight are: then the loads go without a
        // condition each (one branch per thread instead of eight)
        auto pair = [&](int k, int& m, int& t) __attribute__((always_inline)) {
            if (MODE == TP_DQ) {
                t = t0 + (tid & 31);
                m = m0 + (tid >> 5) + 8 * k;
            } else {
                m = m0 + (tid & 63);   // lanes along m: coalesced rows of dS and P
                t = t0 + 8 * wv + k;   // 8 consecutive t per lane: one 16-byte LDS write
            }
        };
        auto visible = [&](int k) __attribute__((always_inline)) {
            int m, t;
            pair(k, m, t);
            if (MODE == TP_DKDV) return m < a.klen && t < a.qlen && m <= a.mlen + t;
            if (MODE == TP_DQ) return m < a.qlen && t <= a.mlen + m;
            return m < a.dr_first && t < a.qlen && m <= a.mlen + t;
        };
        auto load = [&](int k) __attribute__((always_inline)) {
            int m, t;
            pair(k, m, t);
            if (MODE == TP_DKDV) {   // l and dP, raw: stash() turns them into P and dS
                const int64_t o = (rb + t) * a.klen + m;
                ra[0][k] = a.P[o];
                ra[NP - 1][k] = a.dS[o];
            } else if (MODE == TP_DQ) {   // dS is final by now
                const int64_t o = (rb + m) * a.klen;
                ra[0][k] = a.dS[o + t];
                ra[NP - 1][k] = a.dS[o + (a.mlen + m - t)];
            } else {
                ra[0][k] = a.dS[(rb + t) * a.klen + (a.mlen + t - m)];
            }
        };
        if (visible(0) && visible(7)) {
#pragma unroll
            for (int k = 0; k < 8; ++k) load(k);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                ra[0][k] = 0.f;
                ra[NP - 1][k] = 0.f;
                if (visible(k)) load(k);
            }
        }
        if (MODE == TP_DKDV) {
            // the rows' statistics (t is uniform across the wave, so they come
            // through scalar loads)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int t = t0 + 8 * wv + k;
                float s0 = 0.f, s1 = 0.f, s2 = 0.f;
                if (t < a.qlen) {
                    const float* st = a.rstat + (rb + t) * 3;
                    s0 = st[0];
                    s1 = st[1];
                    s2 = st[2];
                }
                rs[k][0] = s0;
                rs[k][1] = s1;
                rs[k][2] = s2;
            }
        }
        // the [t x 64] rows: lane t of 32 consecutive rows, 8 columns per lane;
        // each wave covers 32 rows x 16 columns, so that its transposed 2-byte
        // LDS writes (rows by column, t-contiguous) fall on 32 distinct banks
        const int t = t0 + (tid & 31), c = 8 * (tid >> 5);
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (MODE == TP_DKDV) {
            rbv[0] = t < a.qlen ? *(const u32x4*)((const bf16_t*)a.q + (rb + t) * DH + c) : z;
            rbv[NP - 1] = t < a.qlen ? *(const u32x4*)((const bf16_t*)a.dout + (((int64_t)b * a.qlen + t) * a.H + h) * DH + c) : z;
        } else if (MODE == TP_DQ) {
            const int rr = t < a.n_rel - 1 ? t : a.n_rel - 1;
            rbv[0] = t < a.klen ? *(const u32x4*)((const bf16_t*)a.k + ((int64_t)g * a.klen + t) * DH + c) : z;
            rbv[NP - 1] = t < a.klen ? *(const u32x4*)((const bf16_t*)a.r + ((int64_t)h * a.r_rows + rr) * DH + c) : z;
        } else {
            rbv[0] = t < a.qlen ? *(const u32x4*)((const bf16_t*)a.q + (rb + t) * DH + c) : z;
        }
    };
    auto stash = [&]() __attribute__((always_inline)) {
        if (MODE == TP_DKDV) {
            // P = exp(l - m) / s, dS = P (dP - D); this block is the only
            // reader of the pair, so it leaves dS final in place (the kernels
            // after it read dS only)
            const int m = m0 + (tid & 63), tb = ft0 + 8 * wv;
            // all eight pairs visible (the first and the last are): no
            // condition per pair
            const bool all = m < a.klen && tb + 7 < a.qlen && m <= a.mlen + tb;
            float* dsr = a.dS + (rb + tb) * a.klen + m;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float pv = 0.f, dv = 0.f;
                if (all || (m < a.klen && tb + k < a.qlen && m <= a.mlen + tb + k)) {
                    pv = __expf(ra[0][k] - rs[k][0]) * rs[k][1];
                    dv = pv * (ra[NP - 1][k] - rs[k][2]);
                }
                ra[0][k] = dv;
                ra[NP - 1][k] = pv;
            }
            if (all) {
#pragma unroll
                for (int k = 0; k < 8; ++k) dsr[(int64_t)k * a.klen] = ra[0][k];
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (m < a.klen && tb + k < a.qlen && m <= a.mlen + tb + k) dsr[(int64_t)k * a.klen] = ra[0][k];
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (MODE == TP_DQ) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int m = (tid >> 5) + 8 * k, t = tid & 31;
                    const bf16_t hi = f2bf(ra[p][k]);
                    *(bf16_t*)(sA[p][0] + m * TPB + 2 * t) = hi;
                    *(bf16_t*)(sA[p][1] + m * TPB + 2 * t) = f2bf(ra[p][k] - bf2f(hi));
                }
            } else {
                // row m, t = 8 (tid / 64) .. + 7: high and low parts, 16 bytes each
                u32x4 wh, wl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = ra[p][2 * e], x1 = ra[p][2 * e + 1];
                    const bf16_t h0 = f2bf(x0), h1 = f2bf(x1);
                    wh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                    wl[e] = pack2bf(x0 - bf2f(h0), x1 - bf2f(h1));
                }
                const int off = (tid & 63) * TPB + 16 * (tid >> 6);
                *(u32x4*)(sA[p][0] + off) = wh;
                *(u32x4*)(sA[p][1] + off) = wl;
            }
            // the [t x 64] operand: the first product of dk/dv and dr adds its
            // bias vector (then it is split); t past the range hold zeros
            // (their A entries are zero too)
            const bool add = (MODE == TP_DKDV && p == 0) || MODE == TP_DR;
            const int t = tid & 31;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 8 * (tid >> 5) + e;
                const uint32_t raw = (rbv[p][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                if (add) {
                    const float x = bf2f((bf16_t)raw) + bias8[e];
                    const bf16_t hi = f2bf(x);
                    *(bf16_t*)(sB[p][0] + d * TPB + 2 * t) = hi;
                    *(bf16_t*)(sB[p][1] + d * TPB + 2 * t) = f2bf(x - bf2f(hi));
                } else {
                    *(bf16_t*)(sB[p][0] + d * TPB + 2 * t) = (bf16_t)raw;
                }
            }
        }
    };
    const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, li = lane & 31;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;   // this wave's quarter of the block
    f32x16 acc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[p][v] = 0.f;
    if (t_lo < t_hi) fetch(t_lo);
    for (int t0 = t_lo; t0 < t_hi; t0 += TT) {
        __syncthreads();
        stash();
        __syncthreads();
        if (t0 + TT < t_hi) fetch(t0 + TT);
#pragma unroll
        for (int kk = 0; kk < TT / 16; ++kk) {
            const int off = 32 * kk + 16 * half;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const bool split_b = (MODE == TP_DKDV && p == 0) || MODE == TP_DR;
                const bf16x8 ah = as_bf16x8(*(const u32x4*)(sA[p][0] + (wm + li) * TPB + off));
                const bf16x8 al = as_bf16x8(*(const u32x4*)(sA[p][1] + (wm + li) * TPB + off));
                const bf16x8 bh = as_bf16x8(*(const u32x4*)(sB[p][0] + (wn + li) * TPB + off));
                acc[p] = mfma32(ah, bh, acc[p]);
                acc[p] = mfma32(al, bh, acc[p]);
                if (split_b) {
                    const bf16x8 bl = as_bf16x8(*(const u32x4*)(sB[p][1] + (wn + li) * TPB + off));
                    acc[p] = mfma32(ah, bl, acc[p]);
                }
            }
        }
    }
    // accumulator v of lane (li, half): row wm + 8 (v / 4) + 4 half + v % 4, column wn + li
    const int d = wn + li;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm + 8 * (v >> 2) + 4 * half + (v & 3);
        if (m >= nrows) continue;
        if (MODE == TP_DKDV) {
            const int64_t o = ((int64_t)g * a.klen + m) * DH + d;
            a.dk[o] = a.scale * acc[0][v];
            a.dv[o] = acc[NP - 1][v];
        } else if (MODE == TP_DQ) {
            a.dq[(rb + m) * DH + d] = a.scale * (acc[0][v] + acc[NP - 1][v]);
        } else {
            a.drp[(((int64_t)b * a.H + h) * a.dr_first + m) * DH + d] = acc[0][v];
        }
    }
    if (MODE == TP_DQ) {
        // du, dv: the block's column sums of the two products (rows past
        // qlen are zero): a lane's 16 rows, the other half's, then the two
        // waves of each column half added in LDS; one partial per block
        float* red = (float*)&sA[0][0][0];   // 2 products x 2 row halves x 64 floats, within sA
        float cs[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float x = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) x += acc[p][v];
            cs[p] = x + __shfl_xor(x, 32, 64);
        }
        __syncthreads();
        if (half == 0)
#pragma unroll
            for (int p = 0; p < NP; ++p) red[(p * 2 + (wave >> 1)) * DH + d] = cs[p];
        __syncthreads();
        if (tid < 2 * DH) {
            const int p = tid >> 6, col = tid & 63;
            a.uvp[((int64_t)g * nmt + m0 / TM) * 2 * DH + tid] = red[(p * 2) * DH + col] + red[(p * 2 + 1) * DH + col];
        }
    }
}

// du, dv on the tiled path: one workgroup per head adds the dq blocks'
// partial column sums (2 x 64 per batch element and 64-query block). Eight
// groups of 128 threads take every eighth partial, their loads issued
// together (UVG in flight per thread), then the groups' sums are added in a
// fixed order through LDS.
constexpr int UVG = 8;

__global__ void __launch_bounds__(128 * UVG) bwd_uv_tiled_kernel(AttnBwdArgs a) {
    constexpr int DH = 64;
    __shared__ float part[UVG][2 * DH];
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int col = tid & (2 * DH - 1), grp = tid >> 7;
    const int h = (int)__builtin_amdgcn_workgroup_id_x();
    const int nmt = (a.qlen + TM - 1) / TM;
    const int n = a.B * nmt;
    float sum = 0.f;
    for (int x0 = grp; x0 < n; x0 += UVG * UVG) {
        float v[UVG];
#pragma unroll
        for (int k = 0; k < UVG; ++k) {
            const int x = x0 + UVG * k;
            const int b = x / nmt, mt = x - b * nmt;
            v[k] = x < n ? a.uvp[(((int64_t)b * a.H + h) * nmt + mt) * 2 * DH + col] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < UVG; ++k) sum += v[k];
    }
    part[grp][col] = sum;
    __syncthreads();
    if (grp == 0) {
        float t = 0.f;
#pragma unroll
        for (int g = 0; g < UVG; ++g) t += part[g][col];
        float* out = col < DH ? a.du : a.dvb;
        out[h * DH + (col & (DH - 1))] = a.scale * t;
    }
}

// dr rows c < dr_first: the sum of the batch elements' partial sums, scaled
__global__ void __launch_bounds__(256) bwd_dr_reduce_kernel(AttnBwdArgs a) {
    constexpr int DH = 64;
    const int64_t n = (int64_t)a.H * a.dr_first * DH;
    const int64_t e = (int64_t)__builtin_amdgcn_workgroup_id_x() * 256 + (int)__builtin_amdgcn_workitem_id_x();
    if (e >= n) return;
    float s = 0.f;
    for (int b = 0; b < a.B; ++b) s += a.drp[b * n + e];
    const int64_t h = e / ((int64_t)a.dr_first * DH), rest = e - h * a.dr_first * DH;
    a.dr[(h * a.r_rows) * DH + rest] = a.scale * s;
}

// du, dv: one workgroup of UVW waves per head, d_head across the lanes; wave
// w sums the query rows w, w + UVW, ... of the head, then the waves' sums add
// up in LDS. The bias table gradient: one wave per (head, table row), the
// lanes split the (b, i) pairs of each distance of the row.
constexpr int UVW = 16;

template <int DH>
__global__ void __launch_bounds__(64 * UVW) bwd_uv_kernel(AttnBwdArgs a) {
    __shared__ float part[2][UVW][DH];
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int wave = (int)__builtin_amdgcn_workitem_id_x() >> 6;
    const int h = (int)__builtin_amdgcn_workgroup_id_x();
    float su = 0.f, sv = 0.f;
    if (lane < DH) {
        const int n = a.B * a.qlen;
#pragma unroll 4
        for (int t = wave; t < n; t += UVW) {
            const int b = t / a.qlen, i = t - b * a.qlen;
            const int64_t row = ((int64_t)b * a.H + h) * a.qlen + i;
            su += a.dqu[row * DH + lane];
            sv += a.dqv[row * DH + lane];
        }
        part[0][wave][lane] = su;
        part[1][wave][lane] = sv;
    }
    __syncthreads();
    if (wave == 0 && lane < DH) {
        float tu = 0.f, tv = 0.f;
        for (int x = 0; x < UVW; ++x) {
            tu += part[0][x][lane];
            tv += part[1][x][lane];
        }
        a.du[h * DH + lane] = a.scale * tu;
        a.dvb[h * DH + lane] = a.scale * tv;
    }
}

__global__ void __launch_bounds__(64) bwd_bias_kernel(AttnBwdArgs a) {
    const int lane = (int)__builtin_amdgcn_workitem_id_x();
    const int w = (int)__builtin_amdgcn_workgroup_id_x();
    const int rowb = w / a.H, h = w % a.H;
    // the visible distances [lo, hi] whose table row is rowb
    int lo, hi;
    if (a.bias_kind == 1) {
        lo = rowb == 0 ? 0 : (1 << (rowb - 1)) + 1;
        hi = rowb == 0 ? 1 : (rowb < 11 ? 1 << rowb : a.klen - 1);
    } else {
        const int t = rowb - a.bias_clamp;          // clamped distance of the row
        lo = t;
        hi = t < a.bias_clamp ? t : a.klen - 1;
    }
    if (hi > a.klen - 1) hi = a.klen - 1;
    float s = 0.f;
    if (lo >= 0)
        for (int delta = lo; delta <= hi; ++delta) {
            const int i0 = delta > a.mlen ? delta - a.mlen : 0;
            const int n = a.B * (a.qlen - i0);
            for (int t = lane; t < n; t += 64) {
                const int b = t / (a.qlen - i0), i = i0 + t % (a.qlen - i0);
                const int64_t row = ((int64_t)b * a.H + h) * a.qlen + i;
                s += ds_at(a, row, a.mlen + i - delta);
            }
        }
    s = wsum(s);
    if (lane == 0) a.dbias[(int64_t)rowb * a.H + h] = s;
}

template <typename T, int DH>
hipError_t launch_t(const AttnBwdArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.H * a.qlen, keys = (int64_t)a.B * a.H * a.klen;
    AttnBwdArgs f = a;   // the arguments once P and dS are final
    (void)hipGetLastError();
    if constexpr (DH == 64) {
        // the LDS limit is raised once per process (a function-local static is
        // initialised exactly once, also under concurrent launches)
        constexpr int lds = LR_STG + 4 * LR_SCR;
        static const hipError_t attr =
            hipFuncSetAttribute((const void*)bwd_logits_rows_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (attr != hipSuccess) return attr;
        (void)hipGetLastError();
        const int64_t nwg = (int64_t)a.B * a.H * ((a.qlen + 63) / 64);
        hipLaunchKernelGGL(bwd_logits_rows_kernel, dim3((unsigned)nwg), dim3(256), lds, s, a);
    } else {
        hipLaunchKernelGGL((bwd_rows_kernel<T, DH>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    }
    if constexpr (DH == 64) {
        const int64_t BH = (int64_t)a.B * a.H;
        // dk/dv first: it turns l, dP into P, dS in place, which the later kernels read
        hipLaunchKernelGGL(bwd_tile_kernel<TP_DKDV>, dim3(xcd_grid(BH * ((a.klen + TM - 1) / TM))), dim3(256), 0, s, a);
        f.rstat = nullptr;
        hipLaunchKernelGGL(bwd_tile_kernel<TP_DQ>, dim3(xcd_grid(BH * ((a.qlen + TM - 1) / TM))), dim3(256), 0, s, f);
        if (a.dr_first > 0) {
            hipLaunchKernelGGL(bwd_tile_kernel<TP_DR>, dim3(xcd_grid(BH * ((a.dr_first + TM - 1) / TM))), dim3(256), 0, s,
                               f);
            hipLaunchKernelGGL(bwd_dr_reduce_kernel,
                               dim3((unsigned)(((int64_t)a.H * a.dr_first * DH + 255) / 256)), dim3(256), 0, s, f);
        }
    } else {
        hipLaunchKernelGGL((bwd_dq_kernel<T, DH>), dim3((unsigned)((rows + BW - 1) / BW)), dim3(64 * BW), 0, s, a);
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, DH>), dim3((unsigned)((keys + BW - 1) / BW)), dim3(64 * BW), 0, s, a);
    }
    const int64_t nr = a.r_rows - a.dr_first;   // the last table row in use and the unused rows
    hipLaunchKernelGGL((bwd_dr_kernel<T, DH>), dim3((unsigned)((a.H * nr + BW - 1) / BW)), dim3(64 * BW), 0, s, f);
    if constexpr (DH == 64) hipLaunchKernelGGL(bwd_uv_tiled_kernel, dim3((unsigned)a.H), dim3(128 * UVG), 0, s, f);
    else hipLaunchKernelGGL((bwd_uv_kernel<DH>), dim3((unsigned)a.H), dim3(64 * UVW), 0, s, f);
    if (a.bias) hipLaunchKernelGGL(bwd_bias_kernel, dim3((unsigned)(a.bias_rows * a.H)), dim3(64), 0, s, f);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const AttnBwdArgs& a, bool bf16, int dh, hipStream_t s) {
    if ((int64_t)a.B * a.H * a.qlen == 0) return hipSuccess;
    if (bf16 && dh == 64) return launch_t<bf16_t, 64>(a, s);
    if (!bf16 && dh == 8) return launch_t<float, 8>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace xl
