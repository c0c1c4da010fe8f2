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
//   logits: l and dP per block of (queries, keys), with per-block softmax
//           partials; row stats combines them into (m, 1/s, D) per row
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
        for (int b = 0; b < a.B; ++b) {
            const int64_t rbase = ((int64_t)b * a.H + h) * a.qlen;
            for (int delta = c; delta <= d_hi; ++delta) {
                const int i0 = delta > a.mlen ? delta - a.mlen : 0;
                float pa[ILP] = {};
                int i = i0;
                for (; i + ILP <= a.qlen; i += ILP) {
#pragma unroll
                    for (int x = 0; x < ILP; ++x) {
                        const int64_t row = rbase + i + x;
                        pa[x] += ds_at(a, row, a.mlen + i + x - delta) * (ld<T>(a.q, row * DH + lane) + vd);
                    }
                }
                for (; i < a.qlen; ++i) {
                    const int64_t row = rbase + i;
                    pa[0] += ds_at(a, row, a.mlen + i - delta) * (ld<T>(a.q, row * DH + lane) + vd);
                }
#pragma unroll
                for (int x = 0; x < ILP; ++x) acc += a.scale * pa[x];
            }
        }
    }
    a.dr[((int64_t)h * a.r_rows + c) * DH + lane] = acc;
}



// ---- Logits and dP in 64 x 64 blocks (d_head 64) ----
// A workgroup takes queries i0..i0+63 and keys j0..j0+63 of one head
// (blocks with no visible pair exit at once); each of its 4 waves computes a
// 32 x 32 quarter (queries wm.., keys wn..) on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   content  qu . k      qu = s (q + u) enters as a high and a low bf16 part
//                        (hi = bf16(qu), lo = bf16(qu - hi): 16 bits of
//                        mantissa), k is exact: two products
//   dP       dO . v      both exact bf16: one product
//   position qv . r      qv split like qu, over the 64 distances the quarter
//                        spans, n = 32 + wm - wn + (0..63) counted from
//                        dlo = mlen + i0 - j0 - 63: four products, then
//                        gathered through LDS: pair (i, j) takes distance
//                        column 31 + i - j
// Operands are staged as bf16, 32 of d_head at a time, d-contiguous per row
// (80-byte rows: the lanes' 16-byte reads of 16 rows fall on distinct bank
// groups); lane (li, half) feeds row li with d = 16 kk + 8 half .. + 7. V is
// stored transposed (V^T rows by d_head) and staged by key. The logits of
// visible pairs (plus the bias table entry) go to the P buffer, dP to the dS
// buffer, and per row and half block of 32 keys the softmax partials (max
// m_t, sum of exp(l - m_t), sum of exp(l - m_t) dP) to those that
// bwd_row_stats_kernel combines.
constexpr int LDC = 32;              // d_head per stage
constexpr int LRB = LDC * 2 + 16;    // bytes per staged bf16 row
constexpr int BDP = 64 + 4;

__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
}

// (three workgroups per compute unit: the registers fit 3 waves per SIMD
// without spilling, and the LDS 3 x 45 KB)
__global__ void __launch_bounds__(256, 3) bwd_logits_tile_kernel(AttnBwdArgs a) {
    constexpr int DH = 64;
    // staged rows: qu high, qu low, qv high, qv low, dO (64 queries each), k, v
    // (64 keys each), the table rows of 128 distances
    constexpr int QH = 0, QL = 64, VH = 128, VL = 192, OR = 256, KR = 320, VR = 384, RR = 448, NROW = 576;
    __shared__ __attribute__((aligned(16))) char stg[NROW * LRB];
    float* ops = (float*)stg;   // reused by the epilogue
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int nit = (a.qlen + 63) / 64, njt = (a.klen + 63) / 64, nh = (a.klen + 31) / 32;
    int wg = xcd_block(a.B * a.H * nit * njt);
    if (wg >= a.B * a.H * nit * njt) return;
    const int g = wg / (nit * njt);
    wg -= g * nit * njt;
    const int it = wg / njt, jt = wg - it * njt;
    const int i0 = 64 * it, j0 = 64 * jt;
    const int ilast = i0 + 63 < a.qlen ? i0 + 63 : a.qlen - 1;
    if (j0 > a.mlen + ilast) return;   // no visible pair in the block
    const int h = g % a.H, b = g / a.H;
    const int64_t rb = (int64_t)g * a.qlen;
    const int dlo = a.mlen + i0 - j0 - 63;
    const bf16_t* qp = (const bf16_t*)a.q;
    const bf16_t* op = (const bf16_t*)a.dout;
    const bf16_t* kp = (const bf16_t*)a.k;
    const bf16_t* vp = (const bf16_t*)a.vt;
    const bf16_t* rp = (const bf16_t*)a.r;
    const u32x4 z = {0u, 0u, 0u, 0u};
    // per stage a thread loads 16 bytes (8 of d_head) of a q, dO and k row,
    // of u and v, 8 keys of a V^T row, and 16 bytes of two table rows
    const int row = tid >> 2, pc = tid & 3;
    // V^T: lane d of 32 rows, 8 keys each; consecutive lanes then write
    // consecutive bytes of a key row when V is staged by key
    const int vd = tid & 31, vj = tid >> 5;
    int dist0 = dlo + row, dist1 = dlo + 64 + row;
    dist0 = dist0 < 0 ? 0 : (dist0 > a.n_rel - 1 ? a.n_rel - 1 : dist0);
    dist1 = dist1 < 0 ? 0 : (dist1 > a.n_rel - 1 ? a.n_rel - 1 : dist1);
    u32x4 fq, fo, fk, fvt, fr0, fr1, fu, fv;
    auto fetch = [&](int d0) __attribute__((always_inline)) {
        const int d = d0 + 8 * pc, i = i0 + row, j = j0 + row;
        fq = i < a.qlen ? *(const u32x4*)(qp + (rb + i) * DH + d) : z;
        fo = i < a.qlen ? *(const u32x4*)(op + (((int64_t)b * a.qlen + i) * a.H + h) * DH + d) : z;
        fk = j < a.klen ? *(const u32x4*)(kp + ((int64_t)g * a.klen + j) * DH + d) : z;
        fu = *(const u32x4*)((const bf16_t*)a.u + h * DH + d);
        fv = *(const u32x4*)((const bf16_t*)a.v + h * DH + d);
        const int jj = j0 + 8 * vj;
        fvt = jj < a.ldv ? *(const u32x4*)(vp + ((int64_t)g * DH + d0 + vd) * a.ldv + jj) : z;
        fr0 = *(const u32x4*)(rp + ((int64_t)h * a.r_rows + dist0) * DH + d);
        fr1 = *(const u32x4*)(rp + ((int64_t)h * a.r_rows + dist1) * DH + d);
    };
    auto put = [&](int r, const u32x4 w) __attribute__((always_inline)) {
        *(u32x4*)(stg + r * LRB + 16 * pc) = w;
    };
    auto stash = [&]() __attribute__((always_inline)) {
        float x[8], uu[8], vv[8];
        unpack8(fq, x);
        unpack8(fu, uu);
        unpack8(fv, vv);
        u32x4 uh, ul, wh, wl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float hv[2], lv[2], hw[2], lw[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float qu = a.scale * (x[2 * e + k] + uu[2 * e + k]);
                const float qv = a.scale * (x[2 * e + k] + vv[2 * e + k]);
                hv[k] = bf2f(f2bf(qu));
                lv[k] = qu - hv[k];
                hw[k] = bf2f(f2bf(qv));
                lw[k] = qv - hw[k];
            }
            uh[e] = pack2bf(hv[0], hv[1]);
            ul[e] = pack2bf(lv[0], lv[1]);
            wh[e] = pack2bf(hw[0], hw[1]);
            wl[e] = pack2bf(lw[0], lw[1]);
        }
        put(QH + row, uh);
        put(QL + row, ul);
        put(VH + row, wh);
        put(VL + row, wl);
        put(OR + row, fo);
        put(KR + row, fk);
        put(RR + row, fr0);
        put(RR + 64 + row, fr1);
        // V^T -> key rows: key 8 vj + e, d_head offset vd
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *(bf16_t*)(stg + (VR + 8 * vj + e) * LRB + 2 * vd) = (bf16_t)((fvt[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    };
    const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, li = lane & 31;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
    const int nb = 32 + wm - wn;   // first staged distance row of this quarter
    f32x16 ac, ap, ab0, ab1;
#pragma unroll
    for (int v = 0; v < 16; ++v) ac[v] = ap[v] = ab0[v] = ab1[v] = 0.f;
    auto rd = [&](int r, int off) __attribute__((always_inline)) {
        return as_bf16x8(*(const u32x4*)(stg + r * LRB + off));
    };
    fetch(0);
    for (int d0 = 0; d0 < DH; d0 += LDC) {
        __syncthreads();
        stash();
        __syncthreads();
        if (d0 + LDC < DH) fetch(d0 + LDC);
#pragma unroll
        for (int kk = 0; kk < LDC / 16; ++kk) {
            const int off = 32 * kk + 16 * half;
            const bf16x8 qh = rd(QH + wm + li, off), ql = rd(QL + wm + li, off);
            const bf16x8 vh = rd(VH + wm + li, off), vl = rd(VL + wm + li, off);
            const bf16x8 ov = rd(OR + wm + li, off);
            const bf16x8 kv = rd(KR + wn + li, off), vv = rd(VR + wn + li, off);
            const bf16x8 r0 = rd(RR + nb + li, off), r1 = rd(RR + nb + 32 + li, off);
            ac = mfma32(qh, kv, ac);
            ab0 = mfma32(vh, r0, ab0);
            ab1 = mfma32(vh, r1, ab1);
            ap = mfma32(ov, vv, ap);
            ac = mfma32(ql, kv, ac);
            ab0 = mfma32(vl, r0, ab0);
            ab1 = mfma32(vl, r1, ab1);
        }
    }
    // the positional quarter through LDS (reusing the operand area, 4 x 32 x BDP floats)
    float (*bd)[BDP] = (float (*)[BDP])(ops + wave * 32 * BDP);
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3);
        bd[r][li] = ab0[v];
        bd[r][32 + li] = ab1[v];
    }
    __syncthreads();
    // accumulator v of lane (li, half): query row wm + r, r = 8 (v / 4) + 4 half + v % 4; key wn + li
    const int j = j0 + wn + li;
    float lv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3);
        const int i = i0 + wm + r;
        const bool vis = i < a.qlen && j <= a.mlen + i;
        float l = ac[v] + bd[r][31 + r - li];
        if (vis && a.bias) l += bf2f(((const bf16_t*)a.bias)[(int64_t)brow(a, a.mlen + i - j) * a.H + h]);
        if (vis) {
            const int64_t o = (rb + i) * a.klen + j;
            a.P[o] = l;
            a.dS[o] = ap[v];
        }
        lv[v] = vis ? l : -INFINITY;
    }
    // the softmax partials from l and dP laid out by row in LDS: thread
    // (row, q) reduces keys 16 q .. 16 q + 15, two threads per half block
    float (*ls)[BDP] = (float (*)[BDP])(ops);
    float (*dps)[BDP] = (float (*)[BDP])(ops + 64 * BDP);
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * half + (v & 3);
        ls[wm + r][wn + li] = lv[v];
        dps[wm + r][wn + li] = ap[v];
    }
    __syncthreads();
    {
        const int rr = tid >> 2, q = tid & 3;
        float lx[16], px[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f32x4 x = *(const f32x4*)&ls[rr][16 * q + 4 * k];
            const f32x4 y = *(const f32x4*)&dps[rr][16 * q + 4 * k];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lx[4 * k + e] = x[e];
                px[4 * k + e] = y[e];
            }
        }
        float m = lx[0];
#pragma unroll
        for (int k = 1; k < 16; ++k) m = fmaxf(m, lx[k]);
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        float se = 0.f, sd = 0.f;
        if (m != -INFINITY)   // a half block with no visible pair in this row contributes nothing
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const float e = __expf(lx[k] - m);
                se += e;
                sd += e * px[k];
            }
        se += __shfl_xor(se, 1, 64);
        sd += __shfl_xor(sd, 1, 64);
        const int i = i0 + rr, hb = q >> 1;
        if ((q & 1) == 0 && i < a.qlen && j0 + 32 * hb < a.klen) {   // half blocks past klen have no partials
            float* pt = a.rpart + ((rb + i) * nh + 2 * jt + hb) * 3;
            pt[0] = m;
            pt[1] = se;
            pt[2] = sd;
        }
    }
}

// per query row: m = max of the half blocks' maxima, s = sum of their exp
// sums rescaled to m, D = (rescaled sum of exp(l - m_t) dP) / s; stored
// (m, 1/s, D). RSL lanes share a row: lane x takes half blocks x, x + RSL,
// ..., and the lanes' (m, s, e) merge by rescaling to the larger maximum.
constexpr int RSL = 8;

__device__ __forceinline__ void merge_stats(float& m, float& s, float& e, float m2, float s2, float e2) {
    const float mx = fmaxf(m, m2);
    if (mx == -INFINITY) return;   // both empty
    const float w1 = __expf(m - mx), w2 = __expf(m2 - mx);
    s = s * w1 + s2 * w2;
    e = e * w1 + e2 * w2;
    m = mx;
}

__global__ void __launch_bounds__(256) bwd_row_stats_kernel(AttnBwdArgs a) {
    const int64_t idx = (int64_t)__builtin_amdgcn_workgroup_id_x() * 256 + (int)__builtin_amdgcn_workitem_id_x();
    const int64_t row = idx / RSL;
    const int x = (int)(idx % RSL);
    const int64_t rows = (int64_t)a.B * a.H * a.qlen;
    const bool live = row < rows;   // every lane takes part in the shuffles
    const int i = live ? (int)(row % a.qlen) : 0;
    const int nh = (a.klen + 31) / 32, nt = live ? (a.mlen + i) / 32 + 1 : 0;
    const float* pt = a.rpart + (live ? row : 0) * nh * 3;
    float m = -INFINITY, s = 0.f, e = 0.f;
    for (int t = x; t < nt; t += RSL) merge_stats(m, s, e, pt[3 * t], pt[3 * t + 1], pt[3 * t + 2]);
#pragma unroll
    for (int o = 1; o < RSL; o <<= 1)
        merge_stats(m, s, e, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64), __shfl_xor(e, o, 64));
    if (live && x == 0) {
        a.rstat[row * 3] = m;
        a.rstat[row * 3 + 1] = 1.f / s;
        a.rstat[row * 3 + 2] = e / s;
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
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            int m, t;
            if (MODE == TP_DQ) {
                t = t0 + (tid & 31);
                m = m0 + (tid >> 5) + 8 * k;
            } else {
                m = m0 + (tid & 63);   // lanes along m: coalesced rows of dS and P
                t = t0 + 8 * wv + k;   // 8 consecutive t per lane: one 16-byte LDS write
            }
            float x0 = 0.f, x1 = 0.f;
            if (MODE == TP_DKDV) {
                // l, dP and the row's statistics, raw: stash() turns them into
                // P and dS once this stage's products have been issued
                // (t is uniform across the wave, so the statistics come
                // through scalar loads)
                float s0 = 0.f, s1 = 0.f, s2 = 0.f;
                if (t < a.qlen) {
                    const float* st = a.rstat + (rb + t) * 3;
                    s0 = st[0];
                    s1 = st[1];
                    s2 = st[2];
                }
                if (m < a.klen && t < a.qlen && m <= a.mlen + t) {
                    const int64_t o = (rb + t) * a.klen + m;
                    x0 = a.P[o];
                    x1 = a.dS[o];
                }
                rs[k][0] = s0;
                rs[k][1] = s1;
                rs[k][2] = s2;
            } else if (MODE == TP_DQ) {   // dS is final by now
                if (m < a.qlen && t <= a.mlen + m) {
                    const int64_t o = (rb + m) * a.klen;
                    x0 = a.dS[o + t];
                    x1 = a.dS[o + (a.mlen + m - t)];
                }
            } else {
                if (m < a.dr_first && t < a.qlen && m <= a.mlen + t) x0 = a.dS[(rb + t) * a.klen + (a.mlen + t - m)];
            }
            ra[0][k] = x0;
            if (NP > 1) ra[NP - 1][k] = x1;
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
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int m = m0 + (tid & 63), t = ft0 + 8 * wv + k;
                float pv = 0.f, dv = 0.f;
                if (m < a.klen && t < a.qlen && m <= a.mlen + t) {
                    pv = __expf(ra[0][k] - rs[k][0]) * rs[k][1];
                    dv = pv * (ra[NP - 1][k] - rs[k][2]);
                    a.dS[(rb + t) * a.klen + m] = dv;
                }
                ra[0][k] = dv;
                ra[NP - 1][k] = pv;
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
// partial column sums over the batch elements and query blocks
__global__ void __launch_bounds__(128) bwd_uv_tiled_kernel(AttnBwdArgs a) {
    constexpr int DH = 64;
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int h = (int)__builtin_amdgcn_workgroup_id_x();
    const int nmt = (a.qlen + TM - 1) / TM;
    const int n = a.B * nmt;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int x = 0; x < n; ++x) {
        const int b = x / nmt, mt = x - b * nmt;
        s4[x & 3] += a.uvp[(((int64_t)b * a.H + h) * nmt + mt) * 2 * DH + tid];
    }
    const float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    float* out = tid < DH ? a.du : a.dvb;
    out[h * DH + (tid & 63)] = a.scale * sum;
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
        const int64_t nblk = (int64_t)a.B * a.H * ((a.qlen + 63) / 64) * ((a.klen + 63) / 64);
        hipLaunchKernelGGL(bwd_logits_tile_kernel, dim3(xcd_grid(nblk)), dim3(256), 0, s, a);
        hipLaunchKernelGGL(bwd_row_stats_kernel, dim3((unsigned)((rows * RSL + 255) / 256)), dim3(256), 0, s, a);
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
    if constexpr (DH == 64) hipLaunchKernelGGL(bwd_uv_tiled_kernel, dim3((unsigned)a.H), dim3(128), 0, s, f);
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
