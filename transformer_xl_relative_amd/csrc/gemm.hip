// gemm.hip -- projection GEMM C = A B^T on MFMA for the Q, K, V, R and output
// projections of the relative attention layer (nn.Linear weights [out, in]).
//
// Tile 128 x 128 per workgroup of 4 waves (2 x 2 waves of 64 x 64), K-step of
// 128 bytes per row (64 bf16 / 32 f32), two LDS stages. Both operands are
// K-contiguous, so the MFMA A/B roles can be swapped per epilogue: with
// kRowOut the weight rows feed the MFMA A operand and each lane ends up owning
// one output row and 4 consecutive output columns (row-major stores); without
// it each lane owns one output column and 4 consecutive rows (used for the
// transposed value layout).
#include "xl_common.hpp"
#include "xl_internal.hpp"

namespace xl {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int ROWB = 144;                 // LDS row pitch: 128 data bytes + 16 pad
constexpr int TILEB = 128 * ROWB;         // one operand tile in LDS
constexpr int GEMM_LDS = 4 * TILEB;       // 2 stages x (A, B)

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
__device__ __forceinline__ void store4(const GemmArgs& g, int m, int n, const float* v, bool row_out) {
    // row_out: v[e] belongs to (m, n+e); otherwise to (m+e, n).
    constexpr bool BF = Elem<T>::kBf16;
    if (g.epi == EPI_OUT) {
        if (m >= g.M) return;
        if (g.out_bf16) {
            bf16_t* o = (bf16_t*)g.out0 + (int64_t)m * g.N + n;
            if (n + 3 < g.N) {
                *(u32x2*)o = (u32x2){pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
            } else {
                for (int e = 0; e < 4; ++e) if (n + e < g.N) o[e] = f2bf(v[e]);
            }
        } else {
            float* o = (float*)g.out0 + (int64_t)m * g.N + n;
            if (n + 3 < g.N) *(f32x4*)o = (f32x4){v[0], v[1], v[2], v[3]};
            else for (int e = 0; e < 4; ++e) if (n + e < g.N) o[e] = v[e];
        }
        return;
    }
    if (g.epi == EPI_VT) {
        // column n = (h, d); rows m..m+3 = tokens of (possibly) different batches
        if (n >= g.N) return;
        const int hh = n / g.dh, d = n - hh * g.dh;
        for (int e = 0; e < 4; ++e) {
            const int mm = m + e;
            if (mm >= g.M) break;
            const int b = mm / g.seq, j = mm - b * g.seq;
            T* o = (T*)g.out0 + ((int64_t)(b * g.H + hh) * g.dh + d) * g.ldv + j;
            if constexpr (BF) *o = f2bf(v[e]); else *o = v[e];
        }
        return;
    }
    // row-major-per-head outputs: (m, n..n+3) with n..n+3 inside one head
    if (m >= g.M || n >= g.N) return;
    const int hh = n / g.dh, d = n - hh * g.dh;
    int64_t off;
    if (g.epi == EPI_R) {
        off = ((int64_t)hh * g.seq + m) * g.dh + d;
    } else {
        const int b = m / g.seq, j = m - b * g.seq;
        off = ((int64_t)(b * g.H + hh) * g.seq + j) * g.dh + d;
    }
    if (g.epi == EPI_Q) {
        const T* u = (const T*)g.bias0 + hh * g.dh + d;
        const T* vb = (const T*)g.bias1 + hh * g.dh + d;
        float a[4], c[4];
        for (int e = 0; e < 4; ++e) {
            a[e] = g.scale * (v[e] + Elem<T>::to_f(u[e]));
            c[e] = g.scale * (v[e] + Elem<T>::to_f(vb[e]));
        }
        T* o0 = (T*)g.out0 + off;
        T* o1 = (T*)g.out1 + off;
        if constexpr (BF) {
            *(u32x2*)o0 = (u32x2){pack2bf(a[0], a[1]), pack2bf(a[2], a[3])};
            *(u32x2*)o1 = (u32x2){pack2bf(c[0], c[1]), pack2bf(c[2], c[3])};
        } else {
            *(f32x4*)o0 = (f32x4){a[0], a[1], a[2], a[3]};
            *(f32x4*)o1 = (f32x4){c[0], c[1], c[2], c[3]};
        }
        return;
    }
    T* o = (T*)g.out0 + off;
    if constexpr (BF) *(u32x2*)o = (u32x2){pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
    else *(f32x4*)o = (f32x4){v[0], v[1], v[2], v[3]};
}

template <typename T, bool kRowOut>
__global__ void __launch_bounds__(256, 2) gemm_kernel(GemmArgs g) {
    constexpr bool BF = Elem<T>::kBf16;
    constexpr int EPC = 16 / sizeof(T);    // elements per 16-byte chunk
    constexpr int BK = 128 / sizeof(T);    // elements per K-step
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

    // loader: thread owns chunk (tid % 8) of rows tid/8 + 32p, p = 0..3
    const int lc = tid & 7, lr = tid >> 3;
    const T* arow[4];
    const T* brow[4];
    bool aok[4], bok[4];
    for (int p = 0; p < 4; ++p) {
        const int m = m0 + lr + 32 * p, n = n0 + lr + 32 * p;
        aok[p] = m < g.M;
        bok[p] = n < g.N;
        arow[p] = aok[p] ? a_row_ptr<T>(g, m) : nullptr;
        brow[p] = bok[p] ? (const T*)g.b + (int64_t)n * g.K : nullptr;
    }
    u32x4 ra[4], rb[4];
    auto gload = [&](int k0) {
        const int kk = k0 + lc * EPC;
        const bool kin = kk < g.K;
        for (int p = 0; p < 4; ++p) {
            ra[p] = (aok[p] && kin) ? *(const u32x4*)(arow[p] + kk) : (u32x4){0, 0, 0, 0};
            rb[p] = (bok[p] && kin) ? *(const u32x4*)(brow[p] + kk) : (u32x4){0, 0, 0, 0};
        }
    };
    auto sstore = [&](int stage) {
        char* A = smem + stage * 2 * TILEB;
        char* B = A + TILEB;
        for (int p = 0; p < 4; ++p) {
            *(u32x4*)(A + (lr + 32 * p) * ROWB + lc * 16) = ra[p];
            *(u32x4*)(B + (lr + 32 * p) * ROWB + lc * 16) = rb[p];
        }
    };

    f32x16 acc[2][2];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (g.K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const char* A = smem + (kt & 1) * 2 * TILEB;
        const char* B = A + TILEB;
        if constexpr (BF) {
            for (int kc = 0; kc < 4; ++kc) {
                bf16x8 av[2], bv[2];
                for (int i = 0; i < 2; ++i)
                    av[i] = as_bf16x8(*(const u32x4*)(A + (wm * 64 + i * 32 + l32) * ROWB + (2 * kc + hf) * 16));
                for (int j = 0; j < 2; ++j)
                    bv[j] = as_bf16x8(*(const u32x4*)(B + (wn * 64 + j * 32 + l32) * ROWB + (2 * kc + hf) * 16));
                for (int i = 0; i < 2; ++i)
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = kRowOut ? mfma32(bv[j], av[i], acc[i][j]) : mfma32(av[i], bv[j], acc[i][j]);
            }
        } else {
            for (int kc = 0; kc < BK / 2; ++kc) {
                float av[2], bv[2];
                for (int i = 0; i < 2; ++i)
                    av[i] = *(const float*)(A + (wm * 64 + i * 32 + l32) * ROWB + (2 * kc + hf) * 4);
                for (int j = 0; j < 2; ++j)
                    bv[j] = *(const float*)(B + (wn * 64 + j * 32 + l32) * ROWB + (2 * kc + hf) * 4);
                for (int i = 0; i < 2; ++i)
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = kRowOut ? mfma32(bv[j], av[i], acc[i][j]) : mfma32(av[i], bv[j], acc[i][j]);
            }
        }
        if (kt + 1 < nk) sstore((kt + 1) & 1);
        __syncthreads();
    }

    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
            for (int gq = 0; gq < 4; ++gq) {
                float v[4] = {acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]};
                if (kRowOut) {
                    const int m = m0 + wm * 64 + i * 32 + l32;
                    const int n = n0 + wn * 64 + j * 32 + 8 * gq + 4 * hf;
                    store4<T>(g, m, n, v, true);
                } else {
                    const int m = m0 + wm * 64 + i * 32 + 8 * gq + 4 * hf;
                    const int n = n0 + wn * 64 + j * 32 + l32;
                    store4<T>(g, m, n, v, false);
                }
            }
}

}  // namespace

template <typename T, bool kRowOut>
hipError_t set_lds_attr() {
    static bool done = false;
    if (!done) {
        hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<T, kRowOut>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS);
        if (e != hipSuccess) return e;
        done = true;
    }
    return hipSuccess;
}

hipError_t launch_gemm(const GemmArgs& g, bool bf16, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    hipError_t e = bf16 ? (g.epi != EPI_VT ? set_lds_attr<bf16_t, true>() : set_lds_attr<bf16_t, false>())
                        : (g.epi != EPI_VT ? set_lds_attr<float, true>() : set_lds_attr<float, false>());
    if (e != hipSuccess) return e;
    dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM);
    (void)hipGetLastError();   // drop a stale error of an earlier runtime call
    const bool row_out = g.epi != EPI_VT;
    if (bf16) {
        if (row_out) hipLaunchKernelGGL((gemm_kernel<bf16_t, true>), grid, dim3(256), GEMM_LDS, s, g);
        else hipLaunchKernelGGL((gemm_kernel<bf16_t, false>), grid, dim3(256), GEMM_LDS, s, g);
    } else {
        if (row_out) hipLaunchKernelGGL((gemm_kernel<float, true>), grid, dim3(256), GEMM_LDS, s, g);
        else hipLaunchKernelGGL((gemm_kernel<float, false>), grid, dim3(256), GEMM_LDS, s, g);
    }
    return hipGetLastError();
}

}  // namespace xl
