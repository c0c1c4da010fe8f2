// gemm.hip -- projection GEMMs C = A B^T on MFMA for the Q, K, V, R and output
// projections of the relative attention layer (nn.Linear weights [out, in]).
//
// Up to four independent projections run as one grid: each workgroup owns a
// 128 x 128 output tile of one of them (4 waves, 2 x 2 waves of 64 x 64).
// K advances 64 bytes per stage (32 bf16 / 16 f32); operand tiles move from
// global memory straight into LDS (global_load_lds, 16 bytes per lane) and are
// issued three stages ahead through a ring of four LDS stages, so the loads of
// later stages are in flight while a stage is multiplied. Tile rows are 64
// bytes; the four 16-byte chunks of row r are stored XOR-swizzled by
// (r >> 2) & 3. A 16-byte LDS read is served 16 lanes at a time, and those
// lanes must hit 16 distinct 16-byte bank groups: the MFMA operand reads of
// 16 consecutive rows (4 per 256 bytes) then fall on 16 distinct groups. Rows past the end of A or B are clamped to the last row
// (their products land in outputs that are never stored).
//
// Both operands are K-contiguous, so the MFMA A/B roles are chosen per tile:
// for row-major outputs the weight rows feed the MFMA A operand and a lane
// owns one output row and 4 consecutive output columns; for the transposed
// value layout a lane owns one output column and 4 consecutive rows.
#include "xl_common.hpp"
#include "xl_internal.hpp"

namespace xl {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int STAGES = 4;
constexpr int ROWB = 64;                       // bytes per tile row per stage
constexpr int OPB = 128 * ROWB;                // one operand tile per stage
constexpr int STAGEB = 2 * OPB;                // A and B
constexpr int GEMM_LDS = STAGES * STAGEB;      // 64 KiB

struct GemmBatch {
    GemmArgs p[kMaxGemms];
    int tile_start[kMaxGemms + 1];
    int tiles_n[kMaxGemms];
    int count;
};

__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

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
        if (g.out_bf16) {
            bf16_t* o = (bf16_t*)out + (int64_t)m * g.N + n;
            if (n + 3 < g.N) {
                *(u32x2*)o = (u32x2){pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) if (n + e < g.N) o[e] = f2bf(v[e]);
            }
        } else {
            float* o = (float*)out + (int64_t)m * g.N + n;
            if (n + 3 < g.N) *(f32x4*)o = (f32x4){v[0], v[1], v[2], v[3]};
            else {
#pragma unroll
                for (int e = 0; e < 4; ++e) if (n + e < g.N) o[e] = v[e];
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
    if (epi == EPI_Q) {
        const T* u = (const T*)g.bias0 + hh * g.dh + d;
        const T* vb = (const T*)g.bias1 + hh * g.dh + d;
        float a[4], c[4];
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = g.scale * (v[e] + Elem<T>::to_f(u[e]));
            c[e] = g.scale * (v[e] + Elem<T>::to_f(vb[e]));
        }
        T* o0 = (T*)out + off;
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

template <typename T, bool kRowOut>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int m0, int n0, char* smem) {
    constexpr bool BF = Elem<T>::kBf16;
    constexpr int EPC = 16 / (int)sizeof(T);      // elements per 16-byte chunk
    constexpr int BKE = ROWB / (int)sizeof(T);    // elements per stage row
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;

    // loader: instruction i of this wave fills the 64 chunks (2*wave+i)*64 + lane
    // of an operand tile: row r = chunk / 4, stored chunk sc = chunk % 4, which
    // holds logical chunk sc ^ swz(r)
    const T* asrc[2];
    const T* bsrc[2];
    for (int i = 0; i < 2; ++i) {
        const int chunk = (2 * wave + i) * 64 + lane;
        const int r = chunk >> 2, lc = (chunk & 3) ^ swz(r);
        asrc[i] = a_row_ptr<T>(g, min(m0 + r, g.M - 1)) + lc * EPC;
        bsrc[i] = b_row_ptr<T>(g, min(n0 + r, g.N - 1)) + lc * EPC;
    }
    auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
        char* base = smem + stage * STAGEB;
        for (int i = 0; i < 2; ++i) {
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(asrc[i] + kt * BKE),
                                             (__attribute__((address_space(3))) void*)(base + (2 * wave + i) * 1024),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(bsrc[i] + kt * BKE),
                                             (__attribute__((address_space(3))) void*)(base + OPB + (2 * wave + i) * 1024),
                                             16, 0, 0);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // operand rows of this lane in a stage
    int arow[2], brow[2];
    for (int i = 0; i < 2; ++i) {
        arow[i] = wm * 64 + i * 32 + l32;
        brow[i] = wn * 64 + i * 32 + l32;
    }
    auto compute = [&](int stage) __attribute__((always_inline)) {
        const char* A = smem + stage * STAGEB;
        const char* B = A + OPB;
        if constexpr (BF) {
            for (int kc = 0; kc < 2; ++kc) {
                bf16x8 av[2], bv[2];
                for (int i = 0; i < 2; ++i)
                    av[i] = as_bf16x8(*(const u32x4*)(A + arow[i] * ROWB + (((2 * kc + hf) ^ swz(arow[i])) << 4)));
                for (int j = 0; j < 2; ++j)
                    bv[j] = as_bf16x8(*(const u32x4*)(B + brow[j] * ROWB + (((2 * kc + hf) ^ swz(brow[j])) << 4)));
                for (int i = 0; i < 2; ++i)
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = kRowOut ? mfma32(bv[j], av[i], acc[i][j]) : mfma32(av[i], bv[j], acc[i][j]);
            }
        } else {
            for (int kc = 0; kc < BKE / 2; ++kc) {
                const int k = 2 * kc + hf;
                float av[2], bv[2];
                for (int i = 0; i < 2; ++i)
                    av[i] = *(const float*)(A + arow[i] * ROWB + (((k >> 2) ^ swz(arow[i])) << 4) + (k & 3) * 4);
                for (int j = 0; j < 2; ++j)
                    bv[j] = *(const float*)(B + brow[j] * ROWB + (((k >> 2) ^ swz(brow[j])) << 4) + (k & 3) * 4);
                for (int i = 0; i < 2; ++i)
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = kRowOut ? mfma32(bv[j], av[i], acc[i][j]) : mfma32(av[i], bv[j], acc[i][j]);
            }
        }
    };

    const int nk = g.K / BKE;
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < nk) issue(st, st);
    for (int kt = 0; kt < nk; ++kt) {
        // the loads of stage kt are complete once at most those of the
        // (up to two) later stages already issued are outstanding
        const int later = min(nk - 1 - kt, STAGES - 2);
        if (later >= 2) wait_vmcnt<8>();
        else if (later == 1) wait_vmcnt<4>();
        else wait_vmcnt<0>();
        // Each wave has its own loads of stage kt and its LDS reads of stage
        // kt-1 complete; after the barrier every wave's are, so stage kt is
        // whole and stage kt-1 (refilled below) is no longer read. A bare
        // s_barrier: a fence would also wait for the loads still in flight
        // for the later stages.
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt unchanged
        __builtin_amdgcn_s_barrier();
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
        compute(kt % STAGES);
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 v = {acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]};
                if (kRowOut) {
                    const int m = m0 + wm * 64 + i * 32 + l32;
                    const int n = n0 + wn * 64 + j * 32 + 8 * gq + 4 * hf;
                    store4<T>(g, m, n, v);
                } else {
                    const int m = m0 + wm * 64 + i * 32 + 8 * gq + 4 * hf;
                    const int n = n0 + wn * 64 + j * 32 + l32;
                    store4<T>(g, m, n, v);
                }
            }
}

template <typename T>
__global__ void __launch_bounds__(256, 2) gemm_kernel(GemmBatch gb) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tile = blockIdx.x;
    // the problem of this tile: uniform selects on constant indices (a dynamic
    // index into the argument array would copy it to scratch)
    int k = 0;
    if (gb.count > 1 && tile >= gb.tile_start[1]) k = 1;
    if (gb.count > 2 && tile >= gb.tile_start[2]) k = 2;
    if (gb.count > 3 && tile >= gb.tile_start[3]) k = 3;
    GemmArgs g = gb.p[0];
    int start = gb.tile_start[0], tiles_n = gb.tiles_n[0];
    if (k == 1) { g = gb.p[1]; start = gb.tile_start[1]; tiles_n = gb.tiles_n[1]; }
    if (k == 2) { g = gb.p[2]; start = gb.tile_start[2]; tiles_n = gb.tiles_n[2]; }
    if (k == 3) { g = gb.p[3]; start = gb.tile_start[3]; tiles_n = gb.tiles_n[3]; }
    const int t = tile - start;
    const int tm = t / tiles_n, tn = t - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const bool col_out = g.epi == EPI_VT || (g.epi == EPI_KV && n0 >= g.b_split);
    if (col_out) gemm_tile<T, false>(g, m0, n0, smem);
    else gemm_tile<T, true>(g, m0, n0, smem);
}

template <typename T>
hipError_t set_lds_attr() {
    static bool done = false;
    if (!done) {
        hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           GEMM_LDS);
        if (e != hipSuccess) return e;
        done = true;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemms(const GemmArgs* g, int count, bool bf16, hipStream_t s) {
    if (count < 1 || count > kMaxGemms) return hipErrorInvalidValue;
    GemmBatch gb;
    gb.count = 0;
    int tiles = 0;
    for (int i = 0; i < count; ++i) {
        if (g[i].M <= 0 || g[i].N <= 0) continue;
        const int k = gb.count++;
        gb.p[k] = g[i];
        gb.tiles_n[k] = (g[i].N + BN - 1) / BN;
        gb.tile_start[k] = tiles;
        tiles += gb.tiles_n[k] * ((g[i].M + BM - 1) / BM);
    }
    gb.tile_start[gb.count] = tiles;
    if (tiles == 0) return hipSuccess;
    hipError_t e = bf16 ? set_lds_attr<bf16_t>() : set_lds_attr<float>();
    if (e != hipSuccess) return e;
    (void)hipGetLastError();   // drop a stale error of an earlier runtime call
    if (bf16) hipLaunchKernelGGL(gemm_kernel<bf16_t>, dim3(tiles), dim3(256), GEMM_LDS, s, gb);
    else hipLaunchKernelGGL(gemm_kernel<float>, dim3(tiles), dim3(256), GEMM_LDS, s, gb);
    return hipGetLastError();
}

}  // namespace xl
