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

// sin and cos of x in fp64, for |x| < 2^30 (the library routine beyond).
// Reduction by pi/2 after Cody and Waite: k = rint(2x/pi), r = x - k pi/2
// with pi/2 split into three doubles and fused multiply-adds (each product
// k * part is exact inside the fma), so |r| <= pi/4 up to a rounding of k.
// Then the Taylor series of sin r and cos r through r^17 and r^18 (the next
// terms are below 1e-19 on that interval), evaluated by Horner's rule, and the
// quadrant k mod 4. The constants: pi/2 = 0x1.921fb54442d18p+0
// + 0x1.1a62633145c07p-54 - 0x1.f1976b7ed8fbcp-110 (to 160 bits), and
// 2/pi = 0x1.45f306dc9c883p-1; the coefficients are 1/n! with n! exact.
__device__ __forceinline__ void sincos_f64(double x, double* sp, double* cp) {
    if (!(fabs(x) < 0x1p30)) {
        sincos(x, sp, cp);
        return;
    }
    const double k = rint(x * 0x1.45f306dc9c883p-1);
    double r = fma(-k, 0x1.921fb54442d18p+0, x);
    r = fma(-k, 0x1.1a62633145c07p-54, r);
    r = fma(-k, -0x1.f1976b7ed8fbcp-110, r);
    const double z = r * r;
    double ps = 1.0 / 355687428096000.0;             // 1/17!
    ps = fma(ps, z, -1.0 / 1307674368000.0);         // 1/15!
    ps = fma(ps, z, 1.0 / 6227020800.0);             // 1/13!
    ps = fma(ps, z, -1.0 / 39916800.0);              // 1/11!
    ps = fma(ps, z, 1.0 / 362880.0);                 // 1/9!
    ps = fma(ps, z, -1.0 / 5040.0);                  // 1/7!
    ps = fma(ps, z, 1.0 / 120.0);                    // 1/5!
    ps = fma(ps, z, -1.0 / 6.0);                     // 1/3!
    const double sr = fma(r * z, ps, r);
    double pc = -1.0 / 6402373705728000.0;           // 1/18!
    pc = fma(pc, z, 1.0 / 20922789888000.0);         // 1/16!
    pc = fma(pc, z, -1.0 / 87178291200.0);           // 1/14!
    pc = fma(pc, z, 1.0 / 479001600.0);              // 1/12!
    pc = fma(pc, z, -1.0 / 3628800.0);               // 1/10!
    pc = fma(pc, z, 1.0 / 40320.0);                  // 1/8!
    pc = fma(pc, z, -1.0 / 720.0);                   // 1/6!
    pc = fma(pc, z, 1.0 / 24.0);                     // 1/4!
    pc = fma(pc, z, -0.5);                           // 1/2!
    const double cr = fma(z, pc, 1.0);
    const int q = (int)(int64_t)k & 3;
    *sp = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
    *cp = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
}

// A workgroup owns 64 frequency pairs t (blockIdx.x * 64 + lane) of 4 * RPT
// consecutive rows, wave w rows RPT w .. RPT w + RPT - 1. Wave 0 evaluates
// the 64 inverse frequencies (fp64 pow, the costliest step) into LDS for all
// four waves; each thread then takes the sin and cos of its RPT angles, which
// are independent, so their latencies overlap. Lanes run along t: each row's
// stores are consecutive.
constexpr int RPT = 2;
constexpr int RPW = 4 * RPT;   // rows per workgroup

template <bool kBf16>
__global__ void __launch_bounds__(256) relpos_kernel(int64_t delta0, int64_t n_rows, int64_t d_model,
                                                     int64_t clamp_len, double base, void* out) {
    __shared__ double inv_freq_s[64];
    const int half = (int)(d_model >> 1);
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int t = (int)blockIdx.x * 64 + lane;
    if (wave == 0)
        inv_freq_s[lane] = t < half ? pow(base, -(2.0 * (double)t) / (double)d_model) : 0.0;
    __syncthreads();
    if (t >= half) return;
    const double inv_freq = inv_freq_s[lane];
    const int64_t ngroups = (n_rows + RPW - 1) / RPW;
    for (int64_t grp = blockIdx.y; grp < ngroups; grp += gridDim.y) {
        double sv[RPT], cv[RPT];
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int64_t n = min(grp * RPW + RPT * wave + k, n_rows - 1);
            int64_t delta = delta0 + n;
            if (clamp_len >= 0) delta = delta < -clamp_len ? -clamp_len : (delta > clamp_len ? clamp_len : delta);
            sincos_f64((double)delta * inv_freq, &sv[k], &cv[k]);
        }
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int64_t n = grp * RPW + RPT * wave + k;
            if (n < n_rows) {
                if constexpr (kBf16) {
                    ((uint32_t*)out)[n * half + t] = (uint32_t)d2bf(sv[k]) | ((uint32_t)d2bf(cv[k]) << 16);
                } else {
                    ((float2*)out)[n * half + t] = make_float2((float)sv[k], (float)cv[k]);
                }
            }
        }
    }
}

// Ring write of the segment-recurrent memory: rows are independent copies of
// `chunks` 16-byte chunks each; batch b row t of h goes to ring row
// (dst0 + t) % ring_len. The n * chunks chunks of a batch are numbered
// row-major; a workgroup moves CPT * 256 consecutive chunks (lane-consecutive,
// so every wave touches whole cache lines), all loads before the stores.
constexpr int CPT = 4;

__global__ void __launch_bounds__(256) fifo_kernel(const char* h, int qlen, char* ring, int ring_len, int dst0,
                                                   int src0, uint32_t total, uint32_t chunks, int B) {
    const uint32_t c0 = blockIdx.x * (256u * CPT) + threadIdx.x;
    for (int b = blockIdx.y; b < B; b += gridDim.y) {
        const u32x4* src = (const u32x4*)h + ((int64_t)b * qlen + src0) * chunks;
        u32x4* dst = (u32x4*)ring + (int64_t)b * ring_len * chunks;
        u32x4 v[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const uint32_t c = c0 + 256u * k;
            if (c < total) v[k] = src[c];
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const uint32_t c = c0 + 256u * k;
            if (c < total) {
                const uint32_t t = c / chunks, w = c - t * chunks;
                uint32_t pr = (uint32_t)dst0 + t;
                pr = pr >= (uint32_t)ring_len ? pr % (uint32_t)ring_len : pr;
                dst[(int64_t)pr * chunks + w] = v[k];
            }
        }
    }
}
}  // namespace

hipError_t launch_relpos(int64_t delta0, int64_t n_rows, int64_t d_model, int64_t clamp_len, double base,
                         int out_bf16, void* out, hipStream_t s) {
    if (n_rows <= 0 || d_model < 2) return hipSuccess;
    const int64_t half = d_model / 2, groups = (n_rows + RPW - 1) / RPW;
    const dim3 grid((unsigned)((half + 63) / 64), (unsigned)(groups < 65535 ? groups : 65535));
    (void)hipGetLastError();   // drop a stale error of an earlier runtime call
    if (out_bf16) hipLaunchKernelGGL(relpos_kernel<true>, grid, dim3(256), 0, s, delta0, n_rows, d_model, clamp_len, base, out);
    else hipLaunchKernelGGL(relpos_kernel<false>, grid, dim3(256), 0, s, delta0, n_rows, d_model, clamp_len, base, out);
    return hipGetLastError();
}

hipError_t launch_fifo_write(const void* h, int64_t qlen, void* ring, int64_t ring_len, int64_t dst0, int64_t src0,
                             int64_t n, int64_t B, int64_t row_bytes, hipStream_t s) {
    if (n <= 0 || B <= 0) return hipSuccess;
    // the callers keep row and batch counts below 2^31 and row_bytes a multiple
    // of 16 (validated on the host); rows go in pieces of fewer than 2^31 chunks
    const int64_t chunks = row_bytes / 16;
    const int64_t rows_per = ((int64_t)1 << 30) / chunks;
    (void)hipGetLastError();
    for (int64_t t0 = 0; t0 < n; t0 += rows_per) {
        const int64_t nn = n - t0 < rows_per ? n - t0 : rows_per;
        const int64_t total = nn * chunks;
        const int64_t blocks = (total + 256 * CPT - 1) / (256 * CPT);
        hipLaunchKernelGGL(fifo_kernel, dim3((unsigned)blocks, (unsigned)(B < 65535 ? B : 65535)), dim3(256), 0, s,
                           (const char*)h, (int)qlen, (char*)ring, (int)ring_len, (int)((dst0 + t0) % ring_len),
                           (int)(src0 + t0), (uint32_t)total, (uint32_t)chunks, (int)B);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace xl
