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
    hipLaunchKernelGGL((bwd_rows_kernel<T, DH>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
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
