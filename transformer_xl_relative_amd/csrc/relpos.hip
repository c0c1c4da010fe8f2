// relpos.hip -- sinusoidal relative embedding rows and the FIFO ring write.
//
// Relative embedding (qidao123.com thread-401555 §2; felixzhao.cn article 118
// §2.3.2): row n holds R_delta, delta = delta0 + n clamped to [-C, C]
// (2kiu.com/news/5253360 §2.4), with R[2t] = sin(delta * base^(-2t/D)) and
// R[2t+1] = cos(same). One thread per (row, t) pair; the angle and both
// trigonometric values are evaluated in fp64 and rounded once to the output
// type. HBM-bound and tiny: the launch writes n_rows * D elements.
#include "xl_common.hpp"
#include "xl_internal.hpp"

namespace xl {
namespace {

template <bool kBf16>
__global__ void __launch_bounds__(256) relpos_kernel(int64_t delta0, int64_t n_rows, int64_t d_model,
                                                     int64_t clamp_len, double base, void* out) {
    const int64_t half = d_model >> 1;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_rows * half) return;
    const int64_t n = idx / half, t = idx - n * half;
    int64_t delta = delta0 + n;
    if (clamp_len >= 0) delta = delta < -clamp_len ? -clamp_len : (delta > clamp_len ? clamp_len : delta);
    const double inv_freq = pow(base, -(2.0 * (double)t) / (double)d_model);
    const double ang = (double)delta * inv_freq;
    double sv, cv;
    sincos(ang, &sv, &cv);
    if constexpr (kBf16) {
        const uint32_t packed = (uint32_t)d2bf(sv) | ((uint32_t)d2bf(cv) << 16);
        ((uint32_t*)out)[n * half + t] = packed;
    } else {
        float2 v = make_float2((float)sv, (float)cv);
        ((float2*)out)[n * half + t] = v;
    }
}

// Ring write of the segment-recurrent memory: rows are independent copies of
// row_bytes each (16-byte multiples), batch b row t of h goes to ring row
// (dst0 + t) % ring_len.
__global__ void __launch_bounds__(256) fifo_kernel(const char* h, int64_t qlen, char* ring, int64_t ring_len,
                                                   int64_t dst0, int64_t src0, int64_t n, int64_t row_bytes) {
    const int64_t b = blockIdx.y;
    const int64_t chunks = row_bytes >> 4;
    const int64_t total = n * chunks;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = c / chunks, w = c - t * chunks;
        int64_t pr = (dst0 + t) % ring_len;
        const u32x4 v = *(const u32x4*)(h + ((b * qlen + src0 + t) * row_bytes) + w * 16);
        *(u32x4*)(ring + ((b * ring_len + pr) * row_bytes) + w * 16) = v;
    }
}

}  // namespace

hipError_t launch_relpos(int64_t delta0, int64_t n_rows, int64_t d_model, int64_t clamp_len, double base,
                         int out_bf16, void* out, hipStream_t s) {
    const int64_t work = n_rows * (d_model / 2);
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
    const int64_t total = n * (row_bytes >> 4);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    (void)hipGetLastError();
    hipLaunchKernelGGL(fifo_kernel, dim3((unsigned)blocks, (unsigned)B), dim3(256), 0, s, (const char*)h, qlen,
                       (char*)ring, ring_len, dst0, src0, n, row_bytes);
    return hipGetLastError();
}

}  // namespace xl
