// gemm_bf16.hip -- projection GEMMs C = A B^T for bf16 operands on MFMA (the
// Q, K|V, R and output projections of the relative attention layer;
// nn.Linear weights [out, in]).
//
// Up to four independent projections run as one grid; each workgroup owns a
// square output tile of one of them: 256 x 256 (sixteen waves, 4 x 4, each
// holding 64 x 64 in 2 x 2 accumulator blocks of 32 x 32; four waves per SIMD,
// which hide the operand loads better than eight waves of 64 x 128)
// or 128 x 128 (sixteen waves, each 32 x 32, three stages; eight waves of
// 64 x 32 with two stages where two workgroups share a CU) for grids that the
// large tile would leave too small, or 64 x 64 (four waves, each 32 x 32, eight LDS
// stages) for small problems whose time is set by the latency of each stage.
//
// K advances 64 elements (128 bytes, whole cache lines, per operand row) per
// stage. Operand tiles move from global memory straight into LDS
// (global_load_lds, 16 bytes per lane) one to seven stages ahead; the eight
// 16-byte chunks of row r are stored XOR-swizzled by (r >> 1) & 7 so that the
// MFMA operand reads of 16 consecutive rows fall on 16 distinct bank groups.
// A wave reads the fragments of the next k-step while the MFMAs of the
// current one run (two register sets), so LDS latency hides behind the
// matrix work. Rows past
// the end of A or B are clamped to the last row (their products land in
// outputs that are never stored).
//
// Both operands are K-contiguous, so the MFMA roles are chosen per tile: for
// row-major outputs the weight rows feed the MFMA A operand and a lane owns
// one output row and 4 consecutive columns; for the transposed value layout a
// lane owns one output column and 4 consecutive rows.
#include "gemm_common.hpp"

#include <type_traits>

namespace xl {
namespace {

using namespace gemm;

// WM x WN waves, each holding WTM x WTN accumulator blocks of 32 x 32; NST LDS
// stages of RB bytes per operand row (128: 64 K elements, whole cache lines;
// 64: 32 K elements, for deeper pipelines in the same LDS)
template <int WM_, int WN_, int WTM_, int WTN_, int NST_, int RB_ = 128>
struct Tile {
    static constexpr int WM = WM_, WN = WN_, WTM = WTM_, WTN = WTN_, NST = NST_;
    static constexpr int ROWB = RB_;              // bytes per operand row per stage
    static constexpr int KST = ROWB / 2;          // K elements per stage
    static constexpr int KC = KST / 16;           // MFMA k-steps per stage
    static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
    static constexpr int SWS = CPR == 8 ? 1 : 2;  // swizzle of row r: (r >> SWS) & (CPR - 1)
    static_assert(RB_ == 128 || RB_ == 64, "row bytes per stage");
    static constexpr int NT = 64 * WM * WN;       // threads
    static constexpr int BTM = 32 * WM * WTM;     // workgroup tile rows (M)
    static constexpr int BTN = 32 * WN * WTN;     // workgroup tile columns (N)
    static constexpr int OPA = BTM * ROWB;        // the A tile of a stage, then
    static constexpr int OPB = BTN * ROWB;        // the B tile
    static constexpr int STAGEB = OPA + OPB;
    static constexpr int LDS = NST * STAGEB;
    static constexpr int NIA = BTM * CPR / NT;    // loads per thread per stage: A, B
    static constexpr int NIB = BTN * CPR / NT;
    static_assert(NIA * NT == BTM * CPR && NIB * NT == BTN * CPR, "whole loads per thread");
};
using Big = Tile<4, 4, 2, 2, 2>;     // 256 x 256, 16 waves (each 64 x 64), 2 stages (128 KiB)
using Small = Tile<4, 4, 1, 1, 3>;   // 128 x 128, 16 waves (each 32 x 32), 3 stages (96 KiB): one per CU
using Small2 = Tile<2, 4, 2, 1, 2>;  // 128 x 128, 8 waves, 2 stages (64 KiB): two per CU
using Tiny = Tile<2, 2, 1, 1, 8>;    // 64 x 64, 4 waves, 8 stages (128 KiB): seven stages in flight
using Tall = Tile<2, 4, 3, 2, 2>;    // 192 x 256, 8 waves (each 96 x 64), 2 stages (112 KiB)

template <typename T, bool kRowOut, bool kHalf>
__device__ __forceinline__ void tile_bf16(const GemmArgs& g, int m0, int n0, char* smem) {
    constexpr int WTM = T::WTM, WTN = T::WTN, NW = T::NT / 64;
    constexpr int ROWB = T::ROWB, KST = T::KST, KC = T::KC, CPR = T::CPR;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int wm = wave / T::WN, wn = wave % T::WN;

    // loader: instruction i of this wave fills the 64 chunks (i*NW+wave)*64 + lane
    // of an operand tile: row r = chunk / CPR, stored chunk chunk % CPR, which
    // holds logical chunk (chunk % CPR) ^ ((r >> SWS) & (CPR - 1)), so that the
    // operand reads of 16 consecutive rows fall on 16 distinct bank groups
    // A K of KST/2 (mod KST) leaves a last stage of half width: there the lanes of
    // the upper half of the logical chunks load chunk lc - CPR/2 again (in bounds), and the B
    // fragments of those columns are zeroed before they are multiplied, so every
    // stage issues the same load instructions
    const int nk = (g.K + KST - 1) / KST;
    const bool khalf = kHalf && (g.K % KST) != 0;   // kHalf: some problem of the launch has such a K
    const bf16_t* asrc[T::NIA];
    const bf16_t* bsrc[T::NIB];
    int aback[T::NIA], bback[T::NIB];
    // (the chunk's row and its logical chunk; the back step of a half-width stage)
    auto chunk_of = [&](int i, int& r, int& lc) __attribute__((always_inline)) {
        const int chunk = (i * NW + wave) * 64 + lane;
        r = chunk / CPR;
        lc = (chunk % CPR) ^ ((r >> T::SWS) & (CPR - 1));
    };
#pragma unroll
    for (int i = 0; i < T::NIA; ++i) {
        int r, lc;
        chunk_of(i, r, lc);
        asrc[i] = a_row_ptr<bf16_t>(g, min(m0 + r, g.M - 1)) + lc * 8;
        aback[i] = lc >= CPR / 2 ? KST / 2 : 0;
    }
#pragma unroll
    for (int i = 0; i < T::NIB; ++i) {
        int r, lc;
        chunk_of(i, r, lc);
        bsrc[i] = b_row_ptr<bf16_t>(g, min(n0 + r, g.N - 1)) + lc * 8;
        bback[i] = lc >= CPR / 2 ? KST / 2 : 0;
    }
    auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
        char* base = smem + stage * T::STAGEB;
        const bool half = khalf && kt == nk - 1;
#pragma unroll
        for (int i = 0; i < (T::NIA > T::NIB ? T::NIA : T::NIB); ++i) {
            if (i < T::NIA)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(asrc[i] + kt * KST - (half ? aback[i] : 0)),
                    (__attribute__((address_space(3))) void*)(base + (i * NW + wave) * 1024), 16, 0, 0);
            if (i < T::NIB)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(bsrc[i] + kt * KST - (half ? bback[i] : 0)),
                    (__attribute__((address_space(3))) void*)(base + T::OPA + (i * NW + wave) * 1024), 16, 0, 0);
        }
    };

    // fragment rows of this lane: A rows 32 (wm*WTM + i) + l32, B rows 32 (wn*WTN + j) + l32;
    // their swizzle depends on the row mod 16 only, so it is that of l32
    const int sw = (l32 >> T::SWS) & (CPR - 1);
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;
    uint32_t aoff[KC], boff[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        aoff[kc] = lds0 + (uint32_t)((32 * wm * WTM + l32) * ROWB + (((2 * kc + hf) ^ sw) << 4));
        boff[kc] = lds0 + (uint32_t)(T::OPA + (32 * wn * WTN + l32) * ROWB + (((2 * kc + hf) ^ sw) << 4));
    }
    // fragments of one k-step (16 K elements): two register sets, one being
    // multiplied while the other is filled
    u32x4 fa[2][WTM], fb[2][WTN];
    auto load_frags = [&](int stage, int kc, u32x4 (&a)[WTM], u32x4 (&b)[WTN]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WTM; ++i)
            a[i] = *(const __attribute__((address_space(3))) u32x4*)(size_t)(aoff[kc] + stage * T::STAGEB + i * 32 * ROWB);
#pragma unroll
        for (int j = 0; j < WTN; ++j)
            b[j] = *(const __attribute__((address_space(3))) u32x4*)(size_t)(boff[kc] + stage * T::STAGEB + j * 32 * ROWB);
    };

    f32x16 acc[WTM][WTN];
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    auto compute = [&](const u32x4 (&a)[WTM], const u32x4 (&b)[WTN]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WTM; ++i)
#pragma unroll
            for (int j = 0; j < WTN; ++j)
                acc[i][j] = kRowOut ? mfma32(as_bf16x8(b[j]), as_bf16x8(a[i]), acc[i][j])
                                    : mfma32(as_bf16x8(a[i]), as_bf16x8(b[j]), acc[i][j]);
    };

    constexpr int NST = T::NST;
    constexpr int PER = T::NIA + T::NIB;   // loads per thread per stage
#pragma unroll
    for (int st = 0; st < NST - 1; ++st)
        if (st < nk) issue(st, st);

    // one stage; U = kt % NST (constant), so LDS stages are constants
    auto stage_step = [&](auto u_c, int kt) __attribute__((always_inline)) {
        constexpr int U = decltype(u_c)::value;
        // stage kt complete (this wave's loads): later stages already issued may
        // still be in flight
        static_assert(NST >= 2 && NST <= 8 && (NST - 2) * PER < 64, "stage count");
        const int ahead = min(NST - 2, nk - 1 - kt);    // later stages already issued
        wait_stages<NST - 2, PER>(ahead);
        // after the barrier every wave's loads of stage kt have landed, and no
        // wave reads stage kt-1 any more, so its slot can be refilled
        __asm__ __volatile__("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
        if (kt + NST - 1 < nk) issue(kt + NST - 1, (U + NST - 1) % NST);
        // in a half-width last stage the B fragments of k-steps KC/2.. are zeroed
        const bool half = khalf && kt == nk - 1;
        load_frags(U, 0, fa[0], fb[0]);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            if (kc + 1 < KC) {
                load_frags(U, kc + 1, fa[(kc + 1) & 1], fb[(kc + 1) & 1]);
                if constexpr (kHalf) {
                    if (kc + 1 >= KC / 2 && half) {
#pragma unroll
                        for (int j = 0; j < WTN; ++j) fb[(kc + 1) & 1][j] = u32x4{0u, 0u, 0u, 0u};
                    }
                }
            }
            // the reads of the next k-step stay ahead of these products (two
            // register sets), so that their latency hides behind them
            __builtin_amdgcn_sched_barrier(0);
            compute(fa[kc & 1], fb[kc & 1]);
        }
    };
    // NST stages per pass, so that every stage index is a constant
    for (int kt = 0;;) {
        bool done = false;
        static_for<NST>([&](auto u_c) __attribute__((always_inline)) {
            if (!done) {
                stage_step(u_c, kt);
                done = ++kt >= nk;
            }
        });
        if (done) break;
    }

    // ---- epilogue (d_head 64: the head and offset of a column n are n >> 6 and
    // n & 63). Each wave stages 32 rows of its tile at a time in its own LDS
    // region as bf16 (rows padded by 16 bytes against bank conflicts), then
    // writes them with 16-byte stores that cover whole row segments.
    constexpr int TC = 32 * WTN;                  // wave tile columns (N)
    __builtin_amdgcn_s_waitcnt(0xC07F);           // this wave's fragment reads are done
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();                 // ... and every wave's: the stages can be reused
    __asm__ __volatile__("" ::: "memory");
    const int mw = m0 + 32 * wm * WTM, nw = n0 + 32 * wn * WTN;   // first row / column of the wave tile
    auto lds_st64 = [&](uint32_t adr, float v0, float v1, float v2, float v3) __attribute__((always_inline)) {
        *(__attribute__((address_space(3))) u32x2*)(size_t)adr = (u32x2){pack2bf(v0, v1), pack2bf(v2, v3)};
    };
    auto lds_ld128 = [&](uint32_t adr) __attribute__((always_inline)) {
        return *(const __attribute__((address_space(3))) u32x4*)(size_t)adr;
    };
    if (kRowOut && g.epi == EPI_OUT && (!g.out_bf16 || g.bias_n || g.res || g.relu)) {
        // fp32 outputs, or bias / ReLU / residual: the fp32 accumulators are
        // staged, one 32 x 32 block at a time, and rounded once after the
        // extras (a product rounded before its residual is added keeps that
        // rounding however far the sum cancels)
        constexpr int PF = 32 * 4 + 16;            // bytes per staged row
        static_assert(NW * 32 * PF <= T::LDS, "fp32 epilogue staging fits in LDS");
        const uint32_t fbuf = lds0 + (uint32_t)(wave * 32 * PF);
        const int fc = lane & 3, fr = lane >> 2;   // lane -> columns 8 fc .. 8 fc + 7 of rows fr and fr + 16
#pragma unroll
        for (int i = 0; i < WTM; ++i)
#pragma unroll
            for (int j = 0; j < WTN; ++j) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    *(__attribute__((address_space(3))) f32x4*)(size_t)(fbuf + l32 * PF + (8 * gq + 4 * hf) * 4) =
                        (f32x4){acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]};
                const int n = nw + 32 * j + 8 * fc;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int m = mw + 32 * i + fr + 16 * k;
                    const uint32_t src = fbuf + (fr + 16 * k) * PF + fc * 32;
                    const f32x4 lo = *(const __attribute__((address_space(3))) f32x4*)(size_t)src;
                    const f32x4 hi = *(const __attribute__((address_space(3))) f32x4*)(size_t)(src + 16);
                    if (m < g.M && n < g.N) {
                        float f[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        out_extras8(g, m, n, f);
                        if (g.out_bf16) {
                            *(u32x4*)((bf16_t*)g.out0 + (int64_t)m * g.N + n) =
                                (u32x4){pack2bf(f[0], f[1]), pack2bf(f[2], f[3]), pack2bf(f[4], f[5]), pack2bf(f[6], f[7])};
                        } else {
                            float* o = (float*)g.out0 + (int64_t)m * g.N + n;
                            *(f32x4*)o = (f32x4){f[0], f[1], f[2], f[3]};
                            *(f32x4*)(o + 4) = (f32x4){f[4], f[5], f[6], f[7]};
                        }
                    }
                }
            }
    } else if constexpr (kRowOut) {
        constexpr int PITCH = TC * 2 + 16;         // bytes per staged row
        constexpr int CPR = TC / 8;                // 16-byte chunks per row
        constexpr int RPI = 64 / CPR;              // rows per wave instruction in the copy
        static_assert(NW * 32 * PITCH <= T::LDS, "epilogue staging fits in LDS");
        const uint32_t wbuf = lds0 + (uint32_t)(wave * 32 * PITCH);
        int epi = g.epi;
        int ncols = g.N;
        if (epi == EPI_KV) { epi = EPI_K; ncols = g.b_split; }   // row-output tiles of K|V are K tiles
        // rows per head of a q/k output; a key ring wraps token j to row (pos0 + j) mod rows
        const int krows = g.out_rows > 0 ? g.out_rows : g.seq;
        const int64_t headstride = (int64_t)krows * 64;
        const int ch = lane % CPR, rl = lane / CPR;
        const int n = nw + 8 * ch;
        bf16_t* out = (bf16_t*)g.out0;
#pragma unroll
        for (int i = 0; i < WTM; ++i) {
#pragma unroll
            for (int j = 0; j < WTN; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int c = 32 * j + 8 * gq + 4 * hf;
                    lds_st64(wbuf + l32 * PITCH + c * 2, acc[i][j][4 * gq], acc[i][j][4 * gq + 1],
                             acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
                }
            // copy out rows 32 i .. 32 i + 31: lane -> chunk ch of rows rl + RPI k
            int m = mw + 32 * i + rl;
            int bb = 0, jj = 0;
            if (epi == EPI_K) { bb = m / g.seq; jj = m - bb * g.seq; }
            int jp = jj + g.out_pos0;              // ring row of token jj
            if (jp >= krows) jp -= krows;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const u32x4 w = lds_ld128(wbuf + (rl + RPI * k) * PITCH + ch * 16);
                if (m < g.M && n < ncols) {
                    if (epi == EPI_OUT) {   // bf16 results without extras
                        *(u32x4*)((bf16_t*)g.out0 + (int64_t)m * g.N + n) = w;
                    } else {
                        const int64_t rowoff = epi == EPI_R ? (int64_t)m * 64 : ((int64_t)bb * g.H * krows + jp) * 64;
                        *(u32x4*)(out + rowoff + (int64_t)(n >> 6) * headstride + (n & 63)) = w;
                    }
                }
                m += RPI;
                if (epi == EPI_K) {
                    jj += RPI;
                    jp += RPI;
                    while (jj >= g.seq) { jj -= g.seq; ++bb; jp = jj + g.out_pos0; }
                    if (jp >= krows) jp -= krows;
                }
            }
        }
    } else {
        // transposed values (V^T [B, H, 64, ldv]); column c is head c >> 6,
        // offset c & 63. Staging: column c of the tile holds 32 tokens.
        constexpr int PITCH = 32 * 2 + 16;         // bytes per staged column
        constexpr int CPI = 16;                    // columns per wave instruction in the copy (4 chunks each)
        static_assert(NW * TC * PITCH <= T::LDS, "epilogue staging fits in LDS");
        const uint32_t wbuf = lds0 + (uint32_t)(wave * TC * PITCH);
        bf16_t* out = (bf16_t*)g.out0;
        int c0 = nw, ncols = g.N;
        if (g.epi == EPI_KV) { out = (bf16_t*)g.out1; c0 = nw - g.b_split; ncols = g.N - g.b_split; }
        const int t = lane & 3, cl = lane >> 2;
#pragma unroll
        for (int i = 0; i < WTM; ++i) {
#pragma unroll
            for (int j = 0; j < WTN; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    lds_st64(wbuf + (32 * j + l32) * PITCH + (8 * gq + 4 * hf) * 2, acc[i][j][4 * gq],
                             acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
            // copy out: lane -> token chunk t (8 tokens) of columns cl + CPI k
            const int m = mw + 32 * i + 8 * t;     // first of the chunk's 8 tokens
            const int bb = m / g.seq, jj = m - bb * g.seq;
            // column of token jj: (out_pos0 + jj) mod ldv in a key ring
            int jc = jj + g.out_pos0;
            if (jc >= g.ldv) jc -= g.ldv;
            const bool whole = m + 7 < g.M && jj + 7 < g.seq && (jc & 7) == 0 && jc + 7 < g.ldv && (g.ldv & 7) == 0;
#pragma unroll
            for (int k = 0; k < TC / CPI; ++k) {
                const int c = cl + CPI * k;
                const int cg = c0 + c;
                const u32x4 w = lds_ld128(wbuf + c * PITCH + t * 16);
                if (cg >= ncols || m >= g.M) continue;
                if (whole) {
                    *(u32x4*)(out + ((int64_t)bb * g.H * 64 + cg) * g.ldv + jc) = w;
                } else {
                    int b2 = bb, j2 = jj;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (m + e < g.M) {
                            const uint32_t wd = w[e >> 1];
                            int c2 = j2 + g.out_pos0;
                            if (c2 >= g.ldv) c2 -= g.ldv;
                            out[((int64_t)b2 * g.H * 64 + cg) * g.ldv + c2] = (bf16_t)((e & 1) ? (wd >> 16) : (wd & 0xFFFF));
                        }
                        if (++j2 == g.seq) { j2 = 0; ++b2; }
                    }
                }
            }
        }
    }
}

template <typename T, bool kHalf>
__global__ void __launch_bounds__(T::NT, 1) gemm_bf16_kernel(GemmBatch gb) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tile = (int)__builtin_amdgcn_workgroup_id_x();
    // workgroups past the tiles copy rows
    if (tile >= gb.cp.first_wg) {
        copy_rows(gb.cp, tile - gb.cp.first_wg, T::NT);
        return;
    }
    // the problem of this tile: uniform selects on constant indices
    int k = 0;
    if (gb.count > 1 && tile >= gb.tile_start[1]) k = 1;
    if (gb.count > 2 && tile >= gb.tile_start[2]) k = 2;
    if (gb.count > 3 && tile >= gb.tile_start[3]) k = 3;
    GemmArgs g = gb.p[0];
    int start = gb.tile_start[0], tiles_n = gb.tiles_n[0];
    int end = gb.tile_start[1], real = gb.tiles_real[0];
    if (k == 1) { g = gb.p[1]; start = gb.tile_start[1]; tiles_n = gb.tiles_n[1]; end = gb.tile_start[2]; real = gb.tiles_real[1]; }
    if (k == 2) { g = gb.p[2]; start = gb.tile_start[2]; tiles_n = gb.tiles_n[2]; end = gb.tile_start[3]; real = gb.tiles_real[2]; }
    if (k == 3) { g = gb.p[3]; start = gb.tile_start[3]; tiles_n = gb.tiles_n[3]; end = gb.tile_start[4]; real = gb.tiles_real[3]; }
    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs
    // (workgroup w runs on XCD w % 8) and every problem starts at a multiple
    // of 8, so XCD x takes the x-th eighth of the problem's tiles in row-major
    // order: tiles that share A row panels (and neighbouring B panels) share
    // that XCD's L2. Padding workgroups exit at once.
    const int t = tile - start;
    const int tr = (t & 7) * ((end - start) >> 3) + (t >> 3);
    if (tr >= real) return;
    const int tm = tr / tiles_n, tn = tr - tm * tiles_n;
    const int m0 = tm * T::BTM, n0 = tn * T::BTN;
    const bool col_out = g.epi == EPI_VT || (g.epi == EPI_KV && n0 >= g.b_split);
    if (col_out) tile_bf16<T, false, kHalf>(g, m0, n0, smem);
    else tile_bf16<T, true, kHalf>(g, m0, n0, smem);
}

template <typename T>
hipError_t launch_tiles(const GemmArgs* g, int count, hipStream_t s, const RowCopy* cp) {
    GemmBatch gb;
    gb.count = 0;
    int tiles = 0;
    for (int i = 0; i < count; ++i) {
        if (g[i].M <= 0 || g[i].N <= 0) continue;
        const int k = gb.count++;
        gb.p[k] = g[i];
        gb.tiles_n[k] = (g[i].N + T::BTN - 1) / T::BTN;
        gb.tiles_real[k] = gb.tiles_n[k] * ((g[i].M + T::BTM - 1) / T::BTM);
        gb.tile_start[k] = tiles;
        tiles += (gb.tiles_real[k] + 7) / 8 * 8;     // each problem's range is a multiple of 8
    }
    gb.tile_start[gb.count] = tiles;
    // the row copy: on the compute units the tiles leave idle (one workgroup
    // per unit at this tile size), else on 32 extra workgroups
    int copy_wgs = 0;
    gb.cp = CopyJob{};
    gb.cp.first_wg = tiles;
    if (cp && cp->n > 0 && cp->B > 0) {
        const int64_t rows = cp->B * cp->n;
        int64_t want = tiles < 256 ? 256 - tiles : 32;
        want = want > rows ? rows : want;
        gb.cp.src = (const char*)cp->src;
        gb.cp.ring = (char*)cp->ring;
        gb.cp.qlen = (int)cp->qlen;
        gb.cp.ring_len = (int)cp->ring_len;
        gb.cp.dst0 = (int)cp->dst0;
        gb.cp.src0 = (int)cp->src0;
        gb.cp.n = (int)cp->n;
        gb.cp.rows = (int)rows;
        gb.cp.rows_per = (int)((rows + want - 1) / want);
        gb.cp.chunks = (int)(cp->row_bytes / 16);
        copy_wgs = (int)((rows + gb.cp.rows_per - 1) / gb.cp.rows_per);
    }
    if (tiles + copy_wgs == 0) return hipSuccess;
    bool half = false;
    for (int i = 0; i < gb.count; ++i) half = half || gb.p[i].K % T::KST != 0;
    const auto kern = half ? gemm_bf16_kernel<T, true> : gemm_bf16_kernel<T, false>;
    // the LDS limit of each variant is raised once per process (function-local
    // statics are initialised exactly once, also under concurrent launches)
    static const hipError_t attr_full =
        hipFuncSetAttribute((const void*)gemm_bf16_kernel<T, false>, hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
    static const hipError_t attr_half =
        hipFuncSetAttribute((const void*)gemm_bf16_kernel<T, true>, hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
    if ((half ? attr_half : attr_full) != hipSuccess) return half ? attr_half : attr_full;
    (void)hipGetLastError();   // drop a stale error of an earlier runtime call
    hipLaunchKernelGGL(kern, dim3(tiles + copy_wgs), dim3(T::NT), T::LDS, s, gb);
    return hipGetLastError();
}

}  // namespace

// Large tiles when they still give most CUs a tile, else 128 x 128 tiles.
hipError_t launch_gemms_bf16(const GemmArgs* g, int count, hipStream_t s, const RowCopy* cp) {
    if (count < 1 || count > kMaxGemms) return hipErrorInvalidValue;
    // the epilogues address heads with d_head 64 (the only bf16 head size)
    for (int i = 0; i < count; ++i)
        if (g[i].epi != EPI_OUT && g[i].dh != 64) return hipErrorInvalidValue;
    // 256 x 256 tiles when they nearly fill the machine; else 128 x 128 tiles,
    // with three LDS stages while one workgroup per compute unit suffices and
    // two stages (two workgroups per compute unit) beyond that; 64 x 64 tiles
    // for small problems
    int big = 0, small = 0, tall = 0;
    for (int i = 0; i < count; ++i)
        if (g[i].M > 0 && g[i].N > 0) {
            big += ((g[i].M + 255) / 256) * ((g[i].N + 255) / 256);
            small += ((g[i].M + 127) / 128) * ((g[i].N + 127) / 128);
            tall += ((g[i].M + 191) / 192) * ((g[i].N + 255) / 256);
        }
    if (cp && (cp->row_bytes % 16 || cp->B * cp->n > 0x7FFFFFFF || cp->row_bytes / 16 * (cp->B * cp->n) > 0x7FFFFFFF))
        return hipErrorInvalidValue;
    // where 256 x 256 tiles leave compute units idle and 192 x 256 tiles
    // still fit one round, the latter (the decoder's first feed-forward
    // product at the measured workload: 192 tiles against 256)
    if (big >= 192 && big < 240 && tall > big && tall <= 256) return launch_tiles<Tall>(g, count, s, cp);
    if (big >= 192) return launch_tiles<Big>(g, count, s, cp);
    if (small > 256) return launch_tiles<Small2>(g, count, s, cp);
    // few tiles: their stage latency, not the machine, sets the time; 64 x 64
    // tiles with seven stages in flight cut it and fill more compute units
    if (small < 128) return launch_tiles<Tiny>(g, count, s, cp);
    return launch_tiles<Small>(g, count, s, cp);
}

}  // namespace xl
