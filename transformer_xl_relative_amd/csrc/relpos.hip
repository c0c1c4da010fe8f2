// relpos.hip -- sinusoidal relative embedding rows and the FIFO ring write.
//
// Relative embedding (qidao123.com thread-401555 §2; felixzhao.cn article 118
// §2.3.2): row n holds R_delta, delta = delta0 + n clamped to [-C, C]
// (2kiu.com/news/5253360 §2.4), with R[2t] = sin(delta * base^(-2t/D)) and
// R[2t+1] = cos(same). The angle and both trigonometric values are evaluated
// in fp64 and rounded once to the output type. Small: the launch writes
// n_rows * D elements.
#include "xl_common.hpp"
#include "xl_internal.hpp"

namespace xl {
namespace {

// A thread owns frequency pair t of RPT consecutive rows: the inverse
// frequency is evaluated once, the angles and their sin/cos per row.
constexpr int RPT = 4;

template <bool kBf16>
__global__ void __launch_bounds__(256) relpos_kernel(int64_t delta0, int64_t n_rows, int64_t d_model,
                                                     int64_t clamp_len, double base, void* out) {
    const int half = (int)(d_model >> 1);
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ngroups = (n_rows + RPT - 1) / RPT;
    if (idx >= ngroups * half) return;
    const int64_t grp = idx / half;
    const int t = (int)(idx - grp * half);
    const double inv_freq = pow(base, -(2.0 * (double)t) / (double)d_model);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int64_t n = grp * RPT + k;
        if (n >= n_rows) break;
        int64_t delta = delta0 + n;
        if (clamp_len >= 0) delta = delta < -clamp_len ? -clamp_len : (delta > clamp_len ? clamp_len : delta);
        double sv, cv;
        sincos((double)delta * inv_freq, &sv, &cv);
        if constexpr (kBf16) {
            ((uint32_t*)out)[n * half + t] = (uint32_t)d2bf(sv) | ((uint32_t)d2bf(cv) << 16);
        } else {
            ((float2*)out)[n * half + t] = make_float2((float)sv, (float)cv);
        }
    }
}

// Ring write of the segment-recurrent memory: rows are independent copies of
// row_bytes each (16-byte multiples); batch b row t of h goes to ring row
// (dst0 + t) % ring_len. A workgroup copies whole rows (its threads stride
// over the row's 16-byte chunks), so the row arithmetic is per row.
__global__ void __launch_bounds__(256) fifo_kernel(const char* h, int qlen, char* ring, int ring_len, int dst0,
                                                   int src0, int n, int row_bytes) {
    const int b = blockIdx.y;
    const int chunks = row_bytes >> 4;
    for (int t = blockIdx.x; t < n; t += gridDim.x) {
        int pr = dst0 + t;
        pr = pr >= ring_len ? pr % ring_len : pr;
        const u32x4* src = (const u32x4*)(h + ((int64_t)b * qlen + src0 + t) * row_bytes);
        u32x4* dst = (u32x4*)(ring + ((int64_t)b * ring_len + pr) * row_bytes);
        for (int w = threadIdx.x; w < chunks; w += blockDim.x) dst[w] = src[w];
    }
}
}  // namespace

hipError_t launch_relpos(int64_t delta0, int64_t n_rows, int64_t d_model, int64_t clamp_len, double base,
                         int out_bf16, void* out, hipStream_t s) {
    const int64_t work = (n_rows + RPT - 1) / RPT * (d_model / 2);
    if (work <= 0) return hipSuccess;
    const int64_t blocks = (work + 255) / 256;
    (void)hipGetLastError();   // drop a stale error of an earlier runtime call
    if (out_bf16) hipLaunchKernelGGL(relpos_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, delta0, n_rows, d_model, clamp_len, base, out);
    else hipLaunchKernelGGL(relpos_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, delta0, n_rows, d_model, clamp_len, base, out);
    return hipGetLastError();
}

hipError_t launch_fifo_write(const void* h, int64_t qlen, void* ring, int64_t ring_len, int64_t dst0, int64_t src0,
                             int64_t n, int64_t B, int64_t row_bytes, hipStream_t s) {
    if (n <= 0 || B <= 0) return hipSuccess;
    // the callers keep every count below 2^31 (validated on the host)
    const int blocks = (int)(n < 4096 ? n : 4096);
    (void)hipGetLastError();
    hipLaunchKernelGGL(fifo_kernel, dim3((unsigned)blocks, (unsigned)B), dim3(256), 0, s, (const char*)h, (int)qlen,
                       (char*)ring, (int)ring_len, (int)dst0, (int)src0, (int)n, (int)row_bytes);
    return hipGetLastError();
}

}  // namespace xl
