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
#include "gemm_common.hpp"

namespace xl {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int STAGES = 4;
constexpr int ROWB = 64;                       // bytes per tile row per stage
constexpr int OPB = 128 * ROWB;                // one operand tile per stage
constexpr int STAGEB = 2 * OPB;                // A and B
constexpr int GEMM_LDS = STAGES * STAGEB;      // 64 KiB

using namespace gemm;

__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

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

// The LDS limit is raised once per process; a function-local static is
// initialised exactly once even when several threads launch at the same time.
template <typename T>
hipError_t set_lds_attr() {
    static const hipError_t e =
        hipFuncSetAttribute((const void*)gemm_kernel<T>, hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS);
    return e;
}

}  // namespace

hipError_t launch_gemms(const GemmArgs* g, int count, bool bf16, hipStream_t s, const RowCopy* cp) {
    if (bf16) return launch_gemms_bf16(g, count, s, cp);
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
    if (tiles > 0) {
        hipError_t e = set_lds_attr<float>();
        if (e != hipSuccess) return e;
        (void)hipGetLastError();   // drop a stale error of an earlier runtime call
        hipLaunchKernelGGL(gemm_kernel<float>, dim3(tiles), dim3(256), GEMM_LDS, s, gb);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // the f32 path copies the rows with a launch of its own
    return cp ? launch_fifo_write(cp->src, cp->qlen, cp->ring, cp->ring_len, cp->dst0, cp->src0, cp->n, cp->B,
                                  cp->row_bytes, s)
              : hipSuccess;
}

}  // namespace xl
