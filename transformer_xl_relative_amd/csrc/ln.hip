// ln.hip -- row-wise layer normalisation of the pre-LN decoder layer.
//
// y = (x - mean) / sqrt(var + eps) * gamma + beta over each row of D values,
// with the population variance (felixzhao.cn article 118 §2.3.1 for the
// stacked attention + FFN modules; 2kiu.com/news/5253360 §3.4 for the
// normalised attention input). Statistics accumulate in fp32; the output is
// rounded once to the element type. Under a bf16 output the rows read may be
// fp32 (the decoder layer's residual stream after attention).
//
// One wave owns one row: 16-byte pieces, 64 lanes across the row. Rows of up
// to MAXP pieces per lane stay in registers (the loads of the row, gamma and
// beta issued before the first sum, then the squared deviations and the
// output from the registers); longer
// rows take three passes whose second and third re-read the row from the
// caches. HBM-bound: every element is read from memory once and written once.
#include "xl_common.hpp"
#include "xl_internal.hpp"

namespace xl {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <typename T>
struct Piece;
template <>
struct Piece<bf16_t> {
    static constexpr int N = 8;   // elements per 16-byte piece
    __device__ static void load(const bf16_t* p, float* v) {
        const u32x4 w = *(const u32x4*)p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
    }
    __device__ static void store(bf16_t* p, const float* v) {
        *(u32x4*)p = (u32x4){pack2bf(v[0], v[1]), pack2bf(v[2], v[3]), pack2bf(v[4], v[5]), pack2bf(v[6], v[7])};
    }
};
template <>
struct Piece<float> {
    static constexpr int N = 4;
    __device__ static void load(const float* p, float* v) {
        const f32x4 w = *(const f32x4*)p;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = w[e];
    }
    __device__ static void store(float* p, const float* v) { *(f32x4*)p = (f32x4){v[0], v[1], v[2], v[3]}; }
};

// N row values of type X: one piece, or (fp32 rows under a bf16 output) N / 4
// 16-byte loads
template <typename X, int N>
__device__ __forceinline__ void load_row(const X* p, float* v) {
    if constexpr (Piece<X>::N == N) {
        Piece<X>::load(p, v);
    } else {
#pragma unroll
        for (int e = 0; e < N; e += 4) Piece<float>::load((const float*)p + e, v + e);
    }
}

constexpr int MAXP = 4;   // pieces per lane kept in registers (D <= 2048 bf16, 1024 f32)

// T: gamma, beta and the output; X: the rows read (T, or fp32 under a bf16 output)
template <typename T, typename X>
__global__ void __launch_bounds__(256) ln_kernel(LnArgs a) {
    const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63;
    const int row = (int)__builtin_amdgcn_workgroup_id_x() * 4 + ((int)__builtin_amdgcn_workitem_id_x() >> 6);
    if (row >= a.rows) return;
    // source and destination rows of (b, j)
    const int b = row / a.a_seq, j = row - b * a.a_seq;
    const X* x;
    T* y;
    if (j < a.a_split) {
        int pr = a.ring_head + j;
        if (pr >= a.ring_len) pr -= a.ring_len;
        x = (const X*)a.a0 + (int64_t)b * a.a0_bstride + (int64_t)pr * a.D;
        y = (T*)a.y0 + ((int64_t)b * a.a_split + j) * a.D;
    } else {
        const int n1 = a.a_seq - a.a_split;
        x = (const X*)a.a1 + (int64_t)b * a.a1_bstride + (int64_t)(j - a.a_split) * a.D;
        y = (T*)a.y1 + ((int64_t)b * n1 + (j - a.a_split)) * a.D;
    }
    constexpr int N = Piece<T>::N;
    const int stride = 64 * N;
    const T* g = (const T*)a.gamma;
    const T* bt = (const T*)a.beta;
    if (a.D <= MAXP * stride) {
        // the row, gamma and beta all requested before the first use
        float r[MAXP][N], gv[MAXP][N], bv[MAXP][N];
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            const int k = p * stride + lane * N;
            if (k < a.D) {
                load_row<X, N>(x + k, r[p]);
                Piece<T>::load(g + k, gv[p]);
                Piece<T>::load(bt + k, bv[p]);
            } else {
#pragma unroll
                for (int e = 0; e < N; ++e) r[p][e] = gv[p][e] = bv[p][e] = 0.f;
            }
        }
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < MAXP; ++p)
#pragma unroll
            for (int e = 0; e < N; ++e) s += r[p][e];
        const float mean = wave_sum(s) / (float)a.D;
        float q = 0.f;
#pragma unroll
        for (int p = 0; p < MAXP; ++p)
            if (p * stride + lane * N < a.D) {
#pragma unroll
                for (int e = 0; e < N; ++e) q += (r[p][e] - mean) * (r[p][e] - mean);
            }
        const float inv = 1.f / sqrtf(wave_sum(q) / (float)a.D + a.eps);
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            const int k = p * stride + lane * N;
            if (k < a.D) {
#pragma unroll
                for (int e = 0; e < N; ++e) r[p][e] = (r[p][e] - mean) * inv * gv[p][e] + bv[p][e];
                Piece<T>::store(y + k, r[p]);
            }
        }
        return;
    }
    float v[N];
    float s = 0.f;
    for (int k = lane * N; k < a.D; k += stride) {
        load_row<X, N>(x + k, v);
#pragma unroll
        for (int e = 0; e < N; ++e) s += v[e];
    }
    const float mean = wave_sum(s) / (float)a.D;
    float q = 0.f;
    for (int k = lane * N; k < a.D; k += stride) {
        load_row<X, N>(x + k, v);
#pragma unroll
        for (int e = 0; e < N; ++e) q += (v[e] - mean) * (v[e] - mean);
    }
    const float inv = 1.f / sqrtf(wave_sum(q) / (float)a.D + a.eps);
    for (int k = lane * N; k < a.D; k += stride) {
        float gv[N], bv[N];
        load_row<X, N>(x + k, v);
        Piece<T>::load(g + k, gv);
        Piece<T>::load(bt + k, bv);
#pragma unroll
        for (int e = 0; e < N; ++e) v[e] = (v[e] - mean) * inv * gv[e] + bv[e];
        Piece<T>::store(y + k, v);
    }
}

}  // namespace

hipError_t launch_layer_norm(const LnArgs& a, bool bf16, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)((a.rows + 3) / 4));
    (void)hipGetLastError();
    if (bf16 && a.x_f32) hipLaunchKernelGGL((ln_kernel<bf16_t, float>), grid, dim3(256), 0, s, a);
    else if (bf16) hipLaunchKernelGGL((ln_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ln_kernel<float, float>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace xl
