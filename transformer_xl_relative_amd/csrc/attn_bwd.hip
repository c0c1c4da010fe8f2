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
// A first, plain form: fp32 vector arithmetic, P and dS materialised in the
// workspace ([B, H, qlen, klen] fp32 each), every output written by exactly
// one wave (no atomics):
//   rows:  one wave per query row, keys across the lanes: logits, softmax,
//          dP, D, dS
//   dq:    one wave per query row, d_head across the lanes
//   dk/dv: one wave per key, d_head across the lanes
//   dr:    one wave per table row, d_head across the lanes, over the pairs of
//          that distance (the last row takes every clamped distance)
//   small: du, dv and the bias table gradient
// The row, dq, dk/dv and dr kernels re-read key, table and query rows from
// the caches for every pair (no tile reuse): a correct baseline, bound by
// cache bandwidth and latency rather than arithmetic.
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

// The same for bf16 operands and d_head 64, with the key, table and value
// rows shared through LDS: a workgroup takes RQ consecutive queries of one
// (b, h) (one wave each) and walks the keys in chunks of RK; each chunk's K
// rows, the table rows of its RK + RQ - 1 distances, and later its V rows
// (transposed from V^T as they are stored) are read from memory once for
// the RQ queries. Rows are padded to 144 bytes so that the lanes' 16-byte
// reads of their own rows fall on distinct banks.
constexpr int RQ = 8, RK = 64, KP = 64 * 2 + 16;

__device__ __forceinline__ float dot8(const float* a, const u32x4 w) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        s += a[2 * e] * __uint_as_float(w[e] << 16) + a[2 * e + 1] * __uint_as_float(w[e] & 0xFFFF0000u);
    return s;
}

__global__ void __launch_bounds__(RQ * 64) bwd_rows_tiled_kernel(AttnBwdArgs a) {
    constexpr int DH = 64;
    __shared__ __attribute__((aligned(16))) char kt[RK * KP];
    __shared__ __attribute__((aligned(16))) char rt[(RK + RQ - 1) * KP];
    __shared__ __attribute__((aligned(16))) float sh[RQ][3][DH];   // per wave: qu, qv, dO
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63, wave = tid >> 6;
    const int nqb = (a.qlen + RQ - 1) / RQ;
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int bh = wg / nqb, i0 = (wg - bh * nqb) * RQ;
    const int h = bh % a.H, b = bh / a.H;
    const int i = i0 + wave;
    const bool live = i < a.qlen;
    const int64_t row = (int64_t)bh * a.qlen + (live ? i : a.qlen - 1);
    {
        const float qd = bf2f(((const bf16_t*)a.q)[row * DH + lane]);
        sh[wave][0][lane] = a.scale * (qd + bf2f(((const bf16_t*)a.u)[h * DH + lane]));
        sh[wave][1][lane] = a.scale * (qd + bf2f(((const bf16_t*)a.v)[h * DH + lane]));
        sh[wave][2][lane] = bf2f(((const bf16_t*)a.dout)[((int64_t)b * a.qlen + (row - (int64_t)bh * a.qlen)) * a.H * DH +
                                                         h * DH + lane]);
    }
    const int nv = live ? a.mlen + i + 1 : 0;                      // visible keys of this wave's query
    const int jend = a.mlen + (i0 + RQ < a.qlen ? i0 + RQ : a.qlen); // keys any query of the block sees
    float* P = a.P + row * a.klen;
    float* S = a.dS + row * a.klen;
    const bf16_t* kb = (const bf16_t*)a.k + (int64_t)bh * a.klen * DH;
    const bf16_t* rb = (const bf16_t*)a.r + (int64_t)h * a.r_rows * DH;
    const bf16_t* vb = (const bf16_t*)a.vt + (int64_t)bh * DH * a.ldv;
    const float* qu = sh[wave][0];
    const float* qv = sh[wave][1];
    const float* go = sh[wave][2];
    float m = -INFINITY;
    for (int j0 = 0; j0 < jend; j0 += RK) {
        // K rows j0 .. j0+RK-1: RK*8 pieces of 16 bytes, one per thread
        {
            const int key = tid >> 3, c = tid & 7, jj = j0 + key;
            const u32x4 w = jj < a.klen ? *(const u32x4*)(kb + (int64_t)jj * DH + 8 * c) : (u32x4){0u, 0u, 0u, 0u};
            *(u32x4*)(kt + key * KP + 16 * c) = w;
        }
        // table rows of distances dlo + n, n < RK + RQ - 1 (clamped into the table)
        const int dlo = a.mlen + i0 - (j0 + RK - 1);
        for (int t = tid; t < (RK + RQ - 1) * 8; t += RQ * 64) {
            const int n = t >> 3, c = t & 7;
            int dist = dlo + n;
            dist = dist < 0 ? 0 : (dist > a.n_rel - 1 ? a.n_rel - 1 : dist);
            const u32x4 w = *(const u32x4*)(rb + (int64_t)dist * DH + 8 * c);
            *(u32x4*)(rt + n * KP + 16 * c) = w;
        }
        __syncthreads();
        const int j = j0 + lane;
        if (j < nv) {
            const int delta = a.mlen + i - j;
            const int n = delta - dlo;
            float l = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const u32x4 kw = *(const u32x4*)(kt + lane * KP + 16 * c);
                const u32x4 rw = *(const u32x4*)(rt + n * KP + 16 * c);
                l += dot8(qu + 8 * c, kw) + dot8(qv + 8 * c, rw);
            }
            if (a.bias) l += bf2f(((const bf16_t*)a.bias)[(int64_t)brow(a, delta) * a.H + h]);
            P[j] = l;
            m = fmaxf(m, l);
        }
        __syncthreads();
    }
    m = wmax(m);
    float s = 0.f;
    for (int j = lane; j < nv; j += 64) {
        const float e = __expf(P[j] - m);
        P[j] = e;
        s += e;
    }
    const float inv = 1.f / wsum(s);
    float dsum = 0.f;
    for (int j0 = 0; j0 < jend; j0 += RK) {
        // V rows of keys j0 .. j0+RK-1, transposed from V^T: a thread reads 8
        // keys of one d_head row and writes them to 8 key rows
        {
            const int d = tid >> 3, c = tid & 7, jj = j0 + 8 * c;
            const u32x4 w = jj < a.ldv ? *(const u32x4*)(vb + (int64_t)d * a.ldv + jj) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t half = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                *(bf16_t*)(kt + (8 * c + e) * KP + 2 * d) = (bf16_t)half;
            }
        }
        __syncthreads();
        const int j = j0 + lane;
        if (j < nv) {
            float dp = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c)
                dp += dot8(go + 8 * c, *(const u32x4*)(kt + lane * KP + 16 * c));
            const float p = P[j] * inv;
            P[j] = p;
            S[j] = dp;
            dsum += p * dp;
        }
        __syncthreads();
    }
    const float D = wsum(dsum);
    for (int j = lane; j < nv; j += 64) S[j] = P[j] * (S[j] - D);
}

template <typename T, int DH>
__global__ void __launch_bounds__(256) bwd_dq_kernel(AttnBwdArgs a) {
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int64_t row = (int64_t)__builtin_amdgcn_workgroup_id_x() * 4 + ((int)__builtin_amdgcn_workitem_id_x() >> 6);
    if (row >= (int64_t)a.B * a.H * a.qlen || lane >= DH) return;
    const int i = (int)(row % a.qlen);
    const int bh = (int)(row / a.qlen);
    const int h = bh % a.H;
    const int nv = a.mlen + i + 1;
    const float* S = a.dS + row * a.klen;
    const int64_t kbase = (int64_t)bh * a.klen;
    float cu = 0.f, cv = 0.f;
#pragma unroll 4
    for (int j = 0; j < nv; ++j) {
        const int delta = a.mlen + i - j;
        const int c = delta < a.n_rel - 1 ? delta : a.n_rel - 1;
        const float ds = S[j];
        cu += ds * ld<T>(a.k, (kbase + j) * DH + lane);
        cv += ds * ld<T>(a.r, ((int64_t)h * a.r_rows + c) * DH + lane);
    }
    a.dq[row * DH + lane] = a.scale * (cu + cv);
    a.dqu[row * DH + lane] = cu;
    a.dqv[row * DH + lane] = cv;
}

template <typename T, int DH>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(AttnBwdArgs a) {
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int64_t key = (int64_t)__builtin_amdgcn_workgroup_id_x() * 4 + ((int)__builtin_amdgcn_workitem_id_x() >> 6);
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
__global__ void __launch_bounds__(256) bwd_dr_kernel(AttnBwdArgs a) {
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int64_t w = (int64_t)__builtin_amdgcn_workgroup_id_x() * 4 + ((int)__builtin_amdgcn_workitem_id_x() >> 6);
    if (w >= (int64_t)a.H * a.r_rows || lane >= DH) return;
    const int c = (int)(w % a.r_rows), h = (int)(w / a.r_rows);
    float acc = 0.f;
    if (c < a.n_rel) {
        const int d_hi = c < a.n_rel - 1 ? c : a.klen - 1;   // distances of row c: [c, d_hi]
        const float vd = ld<T>(a.v, h * DH + lane);
        for (int b = 0; b < a.B; ++b) {
            const int64_t rbase = ((int64_t)b * a.H + h) * a.qlen;
            for (int delta = c; delta <= d_hi; ++delta) {
                const int i0 = delta > a.mlen ? delta - a.mlen : 0;
#pragma unroll 4
                for (int i = i0; i < a.qlen; ++i) {
                    const int64_t row = rbase + i;
                    const float ds = a.dS[row * a.klen + (a.mlen + i - delta)];
                    acc += ds * a.scale * (ld<T>(a.q, row * DH + lane) + vd);
                }
            }
        }
    }
    a.dr[w * DH + lane] = acc;
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
                s += a.dS[row * a.klen + (a.mlen + i - delta)];
            }
        }
    s = wsum(s);
    if (lane == 0) a.dbias[(int64_t)rowb * a.H + h] = s;
}

template <typename T, int DH>
hipError_t launch_t(const AttnBwdArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.H * a.qlen, keys = (int64_t)a.B * a.H * a.klen;
    (void)hipGetLastError();
    if constexpr (DH == 64) {
        const int64_t nqb = (a.qlen + RQ - 1) / RQ;
        hipLaunchKernelGGL(bwd_rows_tiled_kernel, dim3((unsigned)((int64_t)a.B * a.H * nqb)), dim3(RQ * 64), 0, s, a);
    } else {
        hipLaunchKernelGGL((bwd_rows_kernel<T, DH>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL((bwd_dq_kernel<T, DH>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, DH>), dim3((unsigned)((keys + 3) / 4)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bwd_dr_kernel<T, DH>), dim3((unsigned)(((int64_t)a.H * a.r_rows + 3) / 4)), dim3(256), 0, s,
                       a);
    hipLaunchKernelGGL((bwd_uv_kernel<DH>), dim3((unsigned)a.H), dim3(64 * UVW), 0, s, a);
    if (a.bias) hipLaunchKernelGGL(bwd_bias_kernel, dim3((unsigned)(a.bias_rows * a.H)), dim3(64), 0, s, a);
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
