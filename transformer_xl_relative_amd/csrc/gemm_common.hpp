// gemm_common.hpp -- operand row addressing and epilogues shared by the
// projection GEMM kernels (C = A B^T, both operands K-contiguous).
#pragma once

#include "xl_common.hpp"
#include "xl_internal.hpp"

#include <type_traits>

namespace xl {
namespace gemm {

// Row copy done by the workgroups after the last tile: rows (b, t), t < n,
// of src (row b*qlen + src0 + t) go to ring row b*ring_len + (dst0 + t) % ring_len;
// workgroup w of wgs copies flattened rows [w*rows_per, (w+1)*rows_per).
struct CopyJob {
    const char* src;
    char* ring;
    int qlen, ring_len, dst0, src0, n, rows, rows_per, chunks;   // chunks: 16-byte pieces per row
    int first_wg;                // workgroups from this one on copy (past the tiles)
};

struct GemmBatch {
    GemmArgs p[kMaxGemms];
    int tile_start[kMaxGemms + 1];
    int tiles_n[kMaxGemms];
    int tiles_real[kMaxGemms];   // tiles of a problem (its range in the grid may be padded)
    int count;
    CopyJob cp;
};

// The row copy part of workgroup w (nt threads): its rows' 16-byte pieces,
// eight per thread in flight at a time (all loads before the stores).
__device__ __forceinline__ void copy_rows(const CopyJob cp, int w, int nt) {
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int r0 = w * cp.rows_per;
    const int r1 = min(r0 + cp.rows_per, cp.rows);
    if (r1 <= r0) return;
    const int units = (r1 - r0) * cp.chunks;
    constexpr int U = 8;
    for (int u0 = tid; u0 < units; u0 += U * nt) {
        u32x4 v[U];
        int64_t doff[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int u = u0 + k * nt;
            doff[k] = -1;
            if (u < units) {
                const int rl = u / cp.chunks, c = u - rl * cp.chunks;
                const int row = r0 + rl;
                const int b = row / cp.n, t = row - b * cp.n;
                int pr = cp.dst0 + t;
                pr = pr >= cp.ring_len ? pr % cp.ring_len : pr;
                v[k] = *(const u32x4*)(cp.src + (((int64_t)b * cp.qlen + cp.src0 + t) * cp.chunks + c) * 16);
                doff[k] = (((int64_t)b * cp.ring_len + pr) * cp.chunks + c) * 16;
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (doff[k] >= 0) *(u32x4*)(cp.ring + doff[k]) = v[k];
    }
}


template <typename T>
__device__ __forceinline__ const T* a_row_ptr(const GemmArgs& g, int m) {
    const T* a0 = (const T*)g.a0;
    if (g.a_seq == 0) return a0 + (int64_t)m * g.lda;
    const int b = m / g.a_seq, j = m - b * g.a_seq;
    if (j < g.a_split) {
        int pr = g.ring_head + j;
        if (pr >= g.ring_len) pr -= g.ring_len;
        return a0 + (int64_t)b * g.a0_bstride + (int64_t)pr * g.lda;
    }
    return (const T*)g.a1 + (int64_t)b * g.a1_bstride + (int64_t)(j - g.a_split) * g.lda;
}

template <typename T>
__device__ __forceinline__ const T* b_row_ptr(const GemmArgs& g, int n) {
    return n < g.b_split ? (const T*)g.b0 + (int64_t)n * g.K : (const T*)g.b1 + (int64_t)(n - g.b_split) * g.K;
}

// EPI_OUT extras on the outputs (m, n..n+3), for m < M: bias, ReLU, residual
template <typename T>
__device__ __forceinline__ void out_extras(const GemmArgs& g, int m, int n, f32x4& w) {
    if (!g.bias_n && !g.res && !g.relu) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (n + e >= g.N) break;
        float t = w[e];
        if (g.bias_n) t += Elem<T>::to_f(((const T*)g.bias_n)[n + e]);
        if (g.relu) t = fmaxf(t, 0.f);
        if (g.res) t += Elem<T>::to_f(((const T*)g.res)[(int64_t)m * g.N + n + e]);
        w[e] = t;
    }
}

// the same for 8 outputs (m, n..n+7) of the bf16 kernel, n a multiple of 8
// and N of 32: bias_n and a bf16 res are read 16 bytes at a time, an fp32 res
// (res_f32) 32 bytes
__device__ __forceinline__ void out_extras8(const GemmArgs& g, int m, int n, float* f) {
    if (g.bias_n) {
        const u32x4 b = *(const u32x4*)((const bf16_t*)g.bias_n + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) { f[2 * e] += bf2f(b[e] & 0xFFFF); f[2 * e + 1] += bf2f(b[e] >> 16); }
    }
    if (g.relu) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = fmaxf(f[e], 0.f);
    }
    if (g.res && g.res_f32) {
        const float* r = (const float*)g.res + (int64_t)m * g.N + n;
        const f32x4 r0 = *(const f32x4*)r, r1 = *(const f32x4*)(r + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { f[e] += r0[e]; f[4 + e] += r1[e]; }
    } else if (g.res) {
        const u32x4 r = *(const u32x4*)((const bf16_t*)g.res + (int64_t)m * g.N + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) { f[2 * e] += bf2f(r[e] & 0xFFFF); f[2 * e + 1] += bf2f(r[e] >> 16); }
    }
}

// Store 4 consecutive outputs: row_out -> (m, n..n+3), else (m..m+3, n).
template <typename T>
__device__ __forceinline__ void store4(const GemmArgs& g, int m, int n, const f32x4 v) {
    constexpr bool BF = Elem<T>::kBf16;
    int epi = g.epi;
    void* out = g.out0;
    if (epi == EPI_KV) {
        if (n < g.b_split) {
            epi = EPI_K;
        } else {
            epi = EPI_VT;
            n -= g.b_split;
            out = g.out1;
        }
    }
    if (epi == EPI_OUT) {
        if (m >= g.M) return;
        f32x4 w = v;
        out_extras<T>(g, m, n, w);
        if (g.out_bf16) {
            bf16_t* o = (bf16_t*)out + (int64_t)m * g.N + n;
            if (n + 3 < g.N) {
                *(u32x2*)o = (u32x2){pack2bf(w[0], w[1]), pack2bf(w[2], w[3])};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) if (n + e < g.N) o[e] = f2bf(w[e]);
            }
        } else {
            float* o = (float*)out + (int64_t)m * g.N + n;
            if (n + 3 < g.N) *(f32x4*)o = (f32x4){w[0], w[1], w[2], w[3]};
            else {
#pragma unroll
                for (int e = 0; e < 4; ++e) if (n + e < g.N) o[e] = w[e];
            }
        }
        return;
    }
    const int ncols = g.epi == EPI_KV ? g.b_split : g.N;
    if (epi == EPI_VT) {
        // column n = (h, d); rows m..m+3 = tokens of (possibly) different batches
        if (n >= ncols) return;
        const int hh = n / g.dh, d = n - hh * g.dh;
        const int b = m / g.seq, j = m - b * g.seq;
        T* o = (T*)out + ((int64_t)(b * g.H + hh) * g.dh + d) * g.ldv + j;
        if (m + 3 < g.M && j + 3 < g.seq && (j & 3) == 0) {
            if constexpr (BF) *(u32x2*)o = (u32x2){pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
            else *(f32x4*)o = (f32x4){v[0], v[1], v[2], v[3]};
            return;
        }
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int mm = m + e;
            if (mm >= g.M) break;
            const int bb = mm / g.seq, jj = mm - bb * g.seq;
            T* oe = (T*)out + ((int64_t)(bb * g.H + hh) * g.dh + d) * g.ldv + jj;
            if constexpr (BF) *oe = f2bf(v[e]); else *oe = v[e];
        }
        return;
    }
    // row-major-per-head outputs: (m, n..n+3) with n..n+3 inside one head
    if (m >= g.M || n >= ncols) return;
    const int hh = n / g.dh, d = n - hh * g.dh;
    int64_t off;
    if (epi == EPI_R) {
        off = ((int64_t)hh * g.seq + m) * g.dh + d;
    } else {
        const int b = m / g.seq, j = m - b * g.seq;
        off = ((int64_t)(b * g.H + hh) * g.seq + j) * g.dh + d;
    }
    T* o = (T*)out + off;
    if constexpr (BF) *(u32x2*)o = (u32x2){pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
    else *(f32x4*)o = (f32x4){v[0], v[1], v[2], v[3]};
}

// s_waitcnt with vmcnt = N and the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most ahead * PER vector loads are outstanding, for a runtime
// ahead in [0, MAXA] (each count is an immediate of its own)
template <int MAXA, int PER>
__device__ __forceinline__ void wait_stages(int ahead) {
    if constexpr (MAXA == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= MAXA) wait_vmcnt<MAXA * PER>();
        else wait_stages<MAXA - 1, PER>(ahead);
    }
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}


}  // namespace gemm
}  // namespace xl
