// attn_bf16.hip -- fused Transformer-XL relative attention forward, bf16
// operands, d_head 64, fp32 accumulation on MFMA.
//
// For one head, query i (segment position; absolute position mlen+i) and key
// j over [memory ; segment] (qidao123.com thread-401555 §3; felixzhao.cn
// article 118 §2.3.2; 2kiu.com/news/5253360 §2.2, §4.3):
//   s(i,j) = qu_i.k_j + qv_i.r[min(delta, n_rel-1)] (+ beta_h[min(delta, bc)])
//   with qu = scale*(q+u), qv = scale*(q+v), delta = mlen + i - j,
//   masked to -inf for j > mlen + i (2kiu.com §4.2), softmax over j, o = P.V.
//
// Work decomposition: one workgroup = (batch, head, 128 queries), four waves
// of 32 queries; keys advance 32 per step. Workgroups are issued longest
// first (query tiles near the end of the segment see more keys). When there
// are too few query tiles to fill the machine (long memory, short segment),
// each tile's key steps are split over several workgroups, each writing its
// unnormalised output with its running maximum and sum; a second kernel
// merges the splits (the softmax of a union of key sets is the
// max-rescaled combination of the parts). Split boundaries lie among the
// steps whose first key every query of the tile sees, so that no query has
// an empty key set in any non-empty split.
//
// Products are computed transposed (keys or distances on the MFMA rows,
// queries on the columns): a lane owns one query, and the softmax
// reductions stay in the lane plus one swap of the half-waves. MFMA row m of
// the content product holds key pi(m) (bits 2 and 3 of m swapped), so that a
// lane's eight consecutive score registers of a half step are eight
// consecutive keys: the P.V product then reads V^T with 16-byte loads.
//
// Relative shift: the position term depends on delta only. Position block
// beta of a wave is the 32x32 product of its queries with 32 consecutive
// band rows of r (descending distance); for query ii it holds the terms of
// keys 32*beta - 31 + ii .. 32*beta + ii. Blocks go into a per-wave LDS ring
// indexed by absolute key (mod 64, rows rotated against bank conflicts); the
// scores of a step start from the ring (blocks s and s+1) as the initial
// accumulator of the content product, so one MFMA chain sums the terms. Every
// band row is multiplied once per query, and no L x L matrix is formed.
//
// Software pipeline: step s issues the content product of step s+1 and the
// position block s+3, which the matrix cores run while the vector unit does
// the softmax of step s, then P.V of step s.
//
// Data movement: K tiles (32 keys x 128 B), V^T tiles (64 rows x 32 keys)
// and band blocks (32 distances x 128 B) move from global memory straight
// into LDS (buffer loads with the LDS destination, 16 bytes per lane, one
// instruction per wave per tile), two steps ahead, and are shared by the four
// waves; the band is shared because wave w needs block beta when wave w-1
// needed it one step earlier. Tiles are XOR-swizzled on 16-byte chunks so
// that the MFMA operand reads are conflict-free; loads past the end of a
// buffer return zeros (buffer range checking), which keeps the load count per
// step fixed and the waits exact.
#include "xl_common.hpp"
#include <hip/hip_ext.h>
#include "xl_internal.hpp"

#include <type_traits>

namespace xl {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// buffer_load_dwordx4 ... lds: the 16 bytes of each lane land at LDS
// address (M0 = lds) + 16 * lane.
__device__ void raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size, int voffset,
                                    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace {


// raw buffer resource over [base, base + bytes): loads at or past the end return 0
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
    const uint64_t p = (uint64_t)base;
    i32x4 r;
    r[0] = (int)(uint32_t)p;
    r[1] = (int)(uint32_t)(p >> 32);                // stride 0
    r[2] = (int)(bytes < 0 ? 0 : bytes);
    r[3] = 0x00020000;                              // raw 32-bit data format
    return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier after this wave's LDS accesses and its DMAs older than the
// newest N have completed. The empty asm statements keep the compiler from
// moving memory accesses across the barrier; a fence would instead wait for
// every load in flight, including the prefetches of later steps.
template <int N>
__device__ __forceinline__ void block_sync() {
    wait_vmcnt<N>();
    wait_lgkm0();
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

constexpr int NW = 4, WQ = 32, BQ = NW * WQ, BKY = 32, DH = 64, NT = NW * 64;
constexpr int TILE = 4096;                         // bytes of one K tile, V^T tile or band block
constexpr int RROW = 256;                          // ring row: 64 fp32 key slots of one query
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_TH = 5.5451774444795623f;  // 8 ln 2: rescale only when the max grows by 2^8

// LDS slots: K tile of step s in slot s % 3 (K(s+3) is loaded during step s),
// V^T tile of step s in slot s % 3 (V(s+2) loaded during step s), band block g
// in slot g % 6 (block g+8 loaded during step s = g); then the per-wave rings
// and, with the bias table, the table.
constexpr int OFF_K = 0;
constexpr int OFF_V = OFF_K + 3 * TILE;
constexpr int OFF_B = OFF_V + 3 * TILE;
constexpr int OFF_RING = OFF_B + 6 * TILE;
constexpr int OFF_TBL = OFF_RING + NW * WQ * RROW;
static_assert(OFF_TBL == 80 * 1024, "two workgroups per CU without the bias table");
constexpr int INFLIGHT = 3;     // loads of a step that the next step does not read
constexpr int kCUs = 256;       // compute units of the GPU

// key steps of query tile qt, and the number of workgroups that share them
__host__ __device__ inline int tile_steps(int qt, int qlen, int mlen) {
    const int qend = (qt + 1) * BQ < qlen ? (qt + 1) * BQ : qlen;
    return (mlen + qend + BKY - 1) / BKY;
}
__host__ __device__ inline int tile_splits(int ts, int split_steps, int split_max) {
    if (split_steps <= 0) return 1;
    const int n = (ts + split_steps - 1) / split_steps;
    return n < split_max ? n : split_max;
}

__device__ __forceinline__ int pi_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename V>
__device__ __forceinline__ V lds_ld(uint32_t addr) {
    return *(const __attribute__((address_space(3))) V*)(size_t)addr;
}
__device__ __forceinline__ void lds_st(uint32_t addr, float v) {
    *(__attribute__((address_space(3))) float*)(size_t)addr = v;
}
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(uint32_t addr) {
    return (__attribute__((address_space(3))) void*)(size_t)addr;
}

template <bool HAS_BIAS, bool RING>
__global__ void __launch_bounds__(NT, 2) attn_bf16_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;

    const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;

    // ---- work item (wave-uniform values kept in scalar registers)
    const int nbh = a.B * a.H;
    const int nqt = (a.qlen + BQ - 1) / BQ;
    // workgroups by decreasing query tile (decreasing work), each tile's
    // splits (split index slower than batch-head) together. Without splits and
    // with n2 = tiles - 256 in (0, 256], workgroup 256 + i becomes the second
    // resident of the compute unit that runs workgroup i, so the first n2
    // workgroups are made the lightest of the heaviest 256: the heaviest tiles
    // then run alone and the lighter ones in pairs.
    int qt = nqt - 1, nsplit = 1, widx = (int)__builtin_amdgcn_workgroup_id_x();
    if (a.split_steps == 0) {
        const int n2 = nbh * nqt - kCUs;
        if (n2 > 0 && n2 <= kCUs) widx = widx < n2 ? widx + kCUs - n2 : (widx < kCUs ? widx - n2 : widx);
        qt = nqt - 1 - widx / nbh;
        widx %= nbh;
    } else {
        for (;; --qt) {
            nsplit = tile_splits(tile_steps(qt, a.qlen, a.mlen), a.split_steps, a.split_max);
            if (widx < nbh * nsplit || qt == 0) break;
            widx -= nbh * nsplit;
        }
    }
    qt = __builtin_amdgcn_readfirstlane(qt);
    nsplit = __builtin_amdgcn_readfirstlane(nsplit);
    const int sp = __builtin_amdgcn_readfirstlane(widx / nbh);
    const int bh = __builtin_amdgcn_readfirstlane(widx % nbh);
    const int h = __builtin_amdgcn_readfirstlane(bh % a.H);
    const int b = __builtin_amdgcn_readfirstlane(bh / a.H);
    const int i0 = qt * BQ;
    const int iw = i0 + wave * WQ;
    // key steps of the tile; this workgroup's split covers steps [S0, S1). The
    // loop counts steps from S0 (LDS slots and ring halves follow that local
    // count); addresses, distances and the mask use the absolute step S0 + s.
    const int tsteps = tile_steps(qt, a.qlen, a.mlen);
    int S0 = 0, S1 = tsteps;
    if (nsplit > 1) {
        const int full = min((a.mlen + i0) / BKY + 1, tsteps);   // steps whose first key all queries see
        auto bnd = [&](int k) { return k >= nsplit ? tsteps : min((int)((int64_t)k * tsteps / nsplit), full - 1); };
        S0 = bnd(sp);
        S1 = bnd(sp + 1);
    }
    S0 = __builtin_amdgcn_readfirstlane(S0);
    const int nsteps = __builtin_amdgcn_readfirstlane(S1 - S0);
    const int wlast = iw < a.qlen ? a.mlen + min(iw + WQ, a.qlen) - 1 : -1;
    const int wsteps = __builtin_amdgcn_readfirstlane(wlast >= 0 ? max(min(wlast / BKY + 1, S1) - S0, 0) : 0);

    // keys in a ring: key j at ring row (kv_head + j) mod kv_rows (one
    // conditional subtraction covers every key below klen <= kv_rows)
    const int krows = RING ? a.kv_rows : a.klen;
    const int kcap = RING ? a.kv_rows : 0x7FFFFFFF;
    const int kv_head = RING ? a.kv_head : 0;
    const char* kb = (const char*)a.k + (int64_t)bh * krows * (DH * 2);
    const char* vb = (const char*)a.vt + (int64_t)bh * DH * a.ldv * 2;
    const char* rb = (const char*)a.r + (int64_t)h * a.r_rows * (DH * 2);
    const i32x4 krs = make_rsrc(kb, (int64_t)krows * (DH * 2));
    const i32x4 vrs = make_rsrc(vb, (int64_t)DH * a.ldv * 2);
    const i32x4 rrs = make_rsrc(rb, (int64_t)a.r_rows * (DH * 2));

    // ---- DMA lane constants. K tiles and band blocks: LDS row rho = 8*wave +
    // lane/8 of 128 bytes, stored chunk lane%8 holds chunk (lane%8)^((rho>>1)&7).
    // V^T tiles: row rho = 16*wave + lane/4 of 64 bytes, stored chunk lane%4
    // holds chunk (lane%4)^((rho>>2)&3).
    const int krho = 8 * wave + (lane >> 3);
    const int kvoff = krho * 128 + (((lane & 7) ^ ((krho >> 1) & 7)) << 4);
    const int kj0 = BKY * S0 + krho + kv_head;                      // ring row of this lane's key in step 0
    const int vrho = 16 * wave + (lane >> 2);
    // (byte offsets within a head's V^T reach 128 ldv, past 2^31 for the
    // largest accepted ldv: unsigned, as the instruction's offset is)
    const uint32_t vvoff = (uint32_t)vrho * (uint32_t)a.ldv * 2u;
    const int vj0 = BKY * S0 + 8 * ((lane & 3) ^ ((vrho >> 2) & 3)) + kv_head;     // first of its 8 keys
    // shared band block g (local) holds distances gs - 32 g - row, gs = mlen + i0 + 127 - 32 S0;
    // wave w's position block beta is band block beta + 3 - w
    const int gtop = a.mlen + i0 + BQ - 1;
    const int gs = gtop - BKY * S0;
    const int rmax = a.n_rel - 1;

    // one 16-byte piece per lane; M0 (the LDS destination) is this wave's kilobyte of the slot
    auto dma_k = [&](int s, int slot) __attribute__((always_inline)) {
        int voff;
        if constexpr (RING) {
            int p = kj0 + BKY * s;
            p -= p >= kcap ? kcap : 0;
            voff = p * 128 + (kvoff & 127);
        } else {
            voff = kvoff + BKY * S0 * 128 + s * (BKY * DH * 2);
        }
        raw_buffer_load_lds(krs, lds_ptr(lds0 + OFF_K + slot * TILE + wave * 1024), 16, voff, 0, 0, 0);
    };
    // (the 8 keys of a piece are consecutive ring columns: kv_head and
    // kv_rows are multiples of 8)
    auto dma_v = [&](int s, int slot) __attribute__((always_inline)) {
        uint32_t voff;
        if constexpr (RING) {
            int p = vj0 + BKY * s;
            p -= p >= kcap ? kcap : 0;
            voff = vvoff + 2u * (uint32_t)p;
        } else {
            voff = vvoff + 2u * (uint32_t)(vj0 + BKY * s);
        }
        raw_buffer_load_lds(vrs, lds_ptr(lds0 + OFF_V + slot * TILE + wave * 1024), 16, (int)voff, 0, 0, 0);
    };
    // band block g into the 4 KB slot at LDS offset `at`
    auto dma_band_at = [&](int g, int at) __attribute__((always_inline)) {
        const int d = min(max(gs - BKY * g - krho, 0), rmax);
        raw_buffer_load_lds(rrs, lds_ptr(lds0 + at + wave * 1024), 16, d * 128 + (kvoff & 127), 0, 0, 0);
    };
    auto dma_band = [&](int g, int slot) __attribute__((always_inline)) { dma_band_at(g, OFF_B + slot * TILE); };
    // keys past klen of the last tile: their weight is 0, but the values there
    // (padding columns of V^T) must be finite; each wave zeroes the piece its
    // own load wrote, after that load has landed
    const int vtail_abs = BKY * tsteps > a.klen ? tsteps - 1 : -1;
    const int vtail = vtail_abs >= S0 && vtail_abs < S1 ? vtail_abs - S0 : -1;
    auto fix_v_tail = [&](int slot) __attribute__((always_inline)) {
        const int lc = (lane & 3) ^ ((vrho >> 2) & 3);          // chunk of 8 keys this lane loaded
        const int nval = a.klen - (BKY * vtail_abs + 8 * lc);   // keys of the chunk below klen
        if (nval < 8) {
            const uint32_t adr = lds0 + OFF_V + slot * TILE + wave * 1024 + lane * 16;
            u32x4 w = lds_ld<u32x4>(adr);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] &= (2 * e < nval ? 0xFFFFu : 0u) | (2 * e + 1 < nval ? 0xFFFF0000u : 0u);
            *(__attribute__((address_space(3))) u32x4*)(size_t)adr = w;
        }
    };

    // ---- query operands (MFMA B operand): lane owns query iw + l32, d_head chunk 16 kc + 8 hf
    const int iq = iw + l32;
    const bool qok = iq < a.qlen;
    // the queries now; u and v of the head reach LDS with the first DMAs (one
    // instruction each per wave instead of four loads each per lane), and the
    // biases fold into the query operands once they have landed
    u32x4 qraw[4];
    {
        const int64_t row = ((int64_t)bh * a.qlen + (qok ? iq : a.qlen - 1)) * DH;
        const bf16_t* qrow = (const bf16_t*)a.q + row;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) qraw[kc] = *(const u32x4*)(qrow + 16 * kc + 8 * hf);
    }
    bf16x8 quB[4], qvB[4];
    // u at byte 0 and v at byte 1024 of this wave's ring, before the ring is first written
    const uint32_t uv_lds = lds0 + OFF_RING + (uint32_t)(wave * WQ * RROW);
    auto fold_uv = [&]() __attribute__((always_inline)) {
        // scale*(q+u) and scale*(q+v), rounded once to bf16
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const u32x4 uw = lds_ld<u32x4>(uv_lds + 32 * kc + 16 * hf);
            const u32x4 vw = lds_ld<u32x4>(uv_lds + 1024 + 32 * kc + 16 * hf);
            const u32x4 qw = qraw[kc];
            u32x4 a_u, a_v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q0 = __uint_as_float(qw[e] << 16), q1 = __uint_as_float(qw[e] & 0xFFFF0000u);
                const float u0 = __uint_as_float(uw[e] << 16), u1 = __uint_as_float(uw[e] & 0xFFFF0000u);
                const float v0 = __uint_as_float(vw[e] << 16), v1 = __uint_as_float(vw[e] & 0xFFFF0000u);
                a_u[e] = pack2bf(a.scale * (q0 + u0), a.scale * (q1 + u1));
                a_v[e] = pack2bf(a.scale * (q0 + v0), a.scale * (q1 + v1));
            }
            quB[kc] = as_bf16x8(a_u);
            qvB[kc] = as_bf16x8(a_v);
        }
    };
    const int dtop = a.mlen + iw + WQ - 1;

    // ---- prologue DMAs, ordered by when they are needed. Position blocks 0..2
    // of wave w are band blocks 3-w .. 5-w, so the prologue needs band blocks
    // 0..5; blocks 0 and 1 go to the K and V slots that K(2) and V(1) take
    // after the prologue (their band slots hold blocks 6 and 7 by then).
    //   u, v, band 0..4 | K(0), band 5 | K(1), V(0), band 6 | band 7
    // (an empty split issues none and writes the neutral partial result)
    auto band0_at = [&](int g) { return g == 0 ? OFF_V + TILE : g == 1 ? OFF_K + 2 * TILE : OFF_B + (g % 6) * TILE; };
    if (nsteps > 0) {
        // (lanes past the 128 bytes of a head read zeros: the range check)
        raw_buffer_load_lds(make_rsrc((const char*)a.u + h * (DH * 2), DH * 2), lds_ptr(uv_lds), 16, lane * 16, 0, 0, 0);
        raw_buffer_load_lds(make_rsrc((const char*)a.v + h * (DH * 2), DH * 2), lds_ptr(uv_lds + 1024), 16, lane * 16,
                            0, 0, 0);
#pragma unroll
        for (int g = 0; g <= 4; ++g) dma_band_at(g, band0_at(g));
        dma_k(0, 0);
        dma_band(5, 5);
        dma_k(1, 1);
        dma_v(0, 0);
        dma_band(6, 0);
        dma_band(7, 1);
    }

    // ---- bias table: entry x holds beta_h[row(X0 - x)], X0 = gtop (row: the
    // clamped distance or its T5 bucket), so that four consecutive registers
    // (descending distance) are one aligned 16-byte read
    const int ntbl = (gtop + 2 * BQ + 3) & ~3;
    if constexpr (HAS_BIAS) {
        const bf16_t* bias = (const bf16_t*)a.bias;
        for (int x = tid; x < ntbl; x += NT)
            *(float*)(smem + OFF_TBL + 4 * x) = bf2f(bias[bias_row(gtop - x, a.bias_kind, a.bias_clamp) * a.H + h]);
        block_sync<63>();
    }
    // bias of position block beta: registers 4q..4q+3 hold distances dtop - 32 beta - 8q - 4hf - t
    const uint32_t tbl_lane = lds0 + OFF_TBL + 4 * (gtop - dtop + 4 * hf) + 128 * S0;

    // ---- LDS read addresses
    const int pr = pi_row(l32);
    uint32_t kaddr[4], baddr[4], vaddr[2];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        kaddr[kc] = (uint32_t)(pr * 128 + (((2 * kc + hf) ^ ((pr >> 1) & 7)) << 4));
        baddr[kc] = (uint32_t)(l32 * 128 + (((2 * kc + hf) ^ ((l32 >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) vaddr[kc] = (uint32_t)(l32 * 64 + (((2 * kc + hf) ^ ((l32 >> 2) & 3)) << 4));
    // ring: key slot p of query ii at float (p + 4 ii) mod 64 of its row; the
    // other parity (slot + 32) is address ^ 128
    const uint32_t ring_row = lds0 + OFF_RING + (uint32_t)(wave * WQ + l32) * RROW;
    uint32_t waddr[16], raddr[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int p = (l32 - (WQ - 1) + acc_row(r, hf)) & 63;    // key slot of band row acc_row(r) in block 0
        waddr[r] = ring_row + (uint32_t)(((p + 4 * l32) & 63) << 2);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int kofs = 16 * (g >> 1) + 8 * hf + 4 * (g & 1);  // keys of registers 4g..4g+3
        raddr[g] = ring_row + (uint32_t)(((kofs + 4 * l32) & 63) << 2);
    }

    auto ring_write = [&](const f32x16& g, uint32_t flip) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) lds_st(waddr[r] ^ flip, g[r]);
    };
    auto ring_read = [&](uint32_t flip) __attribute__((always_inline)) {
        f32x16 acc;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 t4 = lds_ld<f32x4>(raddr[g] ^ flip);
            acc[4 * g] = t4[0]; acc[4 * g + 1] = t4[1]; acc[4 * g + 2] = t4[2]; acc[4 * g + 3] = t4[3];
        }
        return acc;
    };
    auto content = [&](f32x16 acc, int slot) __attribute__((always_inline)) {
        const uint32_t base = lds0 + OFF_K + slot * TILE;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) acc = mfma32(as_bf16x8(lds_ld<u32x4>(base + kaddr[kc])), quB[kc], acc);
        return acc;
    };
    auto pos_init = [&](int beta) __attribute__((always_inline)) {
        f32x16 g;
        if constexpr (HAS_BIAS) {
            const uint32_t t = tbl_lane + (uint32_t)(128 * beta);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 t4 = lds_ld<f32x4>(t + 32 * q);
                g[4 * q] = t4[0]; g[4 * q + 1] = t4[1]; g[4 * q + 2] = t4[2]; g[4 * q + 3] = t4[3];
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) g[r] = 0.f;
        }
        return g;
    };
    // position block beta (< 3) of the prologue, from band block beta + 3 - wave
    auto pos_pro = [&](int beta) __attribute__((always_inline)) {
        const uint32_t base = lds0 + (uint32_t)band0_at(beta + 3 - wave);
        bf16x8 band[4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) band[kc] = as_bf16x8(lds_ld<u32x4>(base + baddr[kc]));
        f32x16 g = pos_init(beta);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) g = mfma32(band[kc], qvB[kc], g);
        return g;
    };

    // ---- softmax state and O^T accumulators (d_head on rows, queries on columns)
    f32x16 o[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // visible-key limit of this lane relative to a local step: key
    // 32 (S0 + s) + c_r + 8 hf is visible when c_r <= lim - 32 s
    const int lim0 = a.mlen + iq - 8 * hf - BKY * S0;
    const int mask_from = a.mlen + iw - BKY * S0;

    // mask, row maximum and lazy rescale of the scores of step s (before their
    // exponentials are taken): the exponentials use the running maximum, which
    // moves (rescaling the running sums) only when some row's maximum grew by
    // more than 2^8
    auto prepare = [&](f32x16& sc, int s) __attribute__((always_inline)) {
        // causal mask: only the last steps of a wave reach past its first query
        if (BKY * s + BKY - 1 > mask_from) {
            const int lim = lim0 - BKY * s;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
                if (c > lim) sc[r] = -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
#pragma unroll
        for (int r = 4; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sc[r], sc[r + 1]));
        mx = halves_max(mx);
        if (__any(mx > m_run + RESCALE_TH)) {
            const float mnew = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f((m_run - mnew) * LOG2E);
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
            m_run = mnew;
        }
    };

    // band slot that wave w reads at a step with s % 6 == i: block s + 6 - w
    uint32_t bslot[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) bslot[i] = lds0 + OFF_B + (uint32_t)(((i + 6 - wave) % 6) * TILE);

    // one step (s % 6 == IDX, so that every LDS slot is a constant): softmax
    // and P.V of the prepared scores `cur` of step s; the content product of
    // step s+1 and position block s+3 run on the matrix cores meanwhile; ends
    // with the scores `nxt` of step s+1 prepared
    auto step = [&](auto idx_c, int s, f32x16& cur, f32x16& nxt) __attribute__((always_inline)) {
        constexpr int IDX = decltype(idx_c)::value;
        constexpr uint32_t FLIP = ((IDX + 1) & 1) << 7;       // parity of step s+1 and block s+3
        dma_k(s + 3, IDX % 3);
        dma_band(s + 8, (IDX + 2) % 6);
        dma_v(s + 2, (IDX + 2) % 3);
        if (s < wsteps) {
            // all LDS operands of the step first
            f32x16 acc = ring_read(FLIP);
            const uint32_t kbase = lds0 + OFF_K + ((IDX + 1) % 3) * TILE;
            const uint32_t bbase = bslot[IDX];
            const uint32_t vbase = lds0 + OFF_V + (IDX % 3) * TILE;
            u32x4 kop[4], bop[4], vop[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                kop[kc] = lds_ld<u32x4>(kbase + kaddr[kc]);
                bop[kc] = lds_ld<u32x4>(bbase + baddr[kc]);
            }
            f32x16 g = pos_init(s + 3);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) vop[2 * t + kc] = lds_ld<u32x4>(vbase + vaddr[kc] + 2048 * t);
            // (the scheduler keeps the reads ahead of the products, so that their
            // latencies overlap instead of adding up)
            __builtin_amdgcn_sched_barrier(0);
            // the wave issues its products and softmax at raised priority, so
            // that a second wave on the SIMD does not delay the matrix burst
            __builtin_amdgcn_s_setprio(1);
            // content product of step s+1 on top of its position terms, and block s+3
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                acc = mfma32(as_bf16x8(kop[kc]), quB[kc], acc);
                g = mfma32(as_bf16x8(bop[kc]), qvB[kc], g);
            }
            // softmax weights of step s
            const float mb = m_run * LOG2E;
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(cur[r], LOG2E, -mb));
            bf16x8 pb[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[kc][e] = (__bf16)p[8 * kc + e];
            // the row sum uses the same rounded weights as P.V
            typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
            const bf16x2v one = {(__bf16)1.0f, (__bf16)1.0f};
            float psum = 0.f;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const bf16x2v pp = {pb[kc][e], pb[kc][e + 1]};
                    psum = __builtin_amdgcn_fdot2_f32_bf16(pp, one, psum, false);
                }
            l_run += psum;
            // the products and the softmax arithmetic interleaved: one MFMA,
            // then vector instructions while it runs
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            ring_write(g, FLIP);               // block s+3 replaces block s+1, read above
            // O^T += V^T P^T
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) o[t] = mfma32(as_bf16x8(vop[2 * t + kc]), pb[kc], o[t]);
            nxt = acc;
            if (s + 1 < wsteps) prepare(nxt, s + 1);
        }
        // the loads the next step reads have landed (this wave's part), and
        // this wave no longer reads the slots the next step refills
        wait_vmcnt<INFLIGHT>();
        if (s + 1 == vtail) fix_v_tail((IDX + 1) % 3);
        block_sync<63>();
    };

    if (nsteps > 0) {
        // ---- prologue compute: blocks 0 and 1, then the scores of step 0, then block 2
        block_sync<6>();                       // queries, u, v, band blocks 0..4
        fold_uv();
        ring_write(pos_pro(0), 0u);
        ring_write(pos_pro(1), 128u);
        block_sync<4>();                       // K(0), band block 5
        f32x16 s0 = content(ring_read(0u), 0), s1;
        ring_write(pos_pro(2), 0u);            // block 2 replaces block 0, read above
        if (wsteps > 0) prepare(s0, 0);
        wait_vmcnt<1>();                       // all but band block 7
        if (vtail == 0) fix_v_tail(0);
        block_sync<63>();
        dma_k(2, 2);                           // into the slots band blocks 1 and 0 held
        dma_v(1, 1);

        // steps in groups of six (slot indices are compile-time constants)
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using I4 = std::integral_constant<int, 4>;
        using I5 = std::integral_constant<int, 5>;
        for (int s = 0;;) {
            step(I0{}, s, s0, s1);
            if (++s >= nsteps) break;
            step(I1{}, s, s1, s0);
            if (++s >= nsteps) break;
            step(I2{}, s, s0, s1);
            if (++s >= nsteps) break;
            step(I3{}, s, s1, s0);
            if (++s >= nsteps) break;
            step(I4{}, s, s0, s1);
            if (++s >= nsteps) break;
            step(I5{}, s, s1, s0);
            if (++s >= nsteps) break;
        }
    }
    wait_vmcnt<0>();   // no load into LDS outlives the workgroup

    // ---- epilogue: o / l, heads concatenated. The wave stages its 32 x 64
    // outputs in its own ring (padded rows of 64 bf16), then writes each query's
    // 128-byte row segment with 16-byte stores.
    const float l_tot = halves_sum(l_run);
    if (nsplit > 1) {
        // partial result of this split: O (unnormalised, [query][d_head] fp32),
        // then (running maximum, sum) per query
        if (iw >= a.qlen) return;
        const int64_t prow = ((int64_t)sp * nbh + bh) * a.qlen + iq;
        if (qok) {
            float* po = (float*)a.part + prow * DH;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    *(f32x4*)(po + 32 * t + 8 * gq + 4 * hf) =
                        (f32x4){o[t][4 * gq], o[t][4 * gq + 1], o[t][4 * gq + 2], o[t][4 * gq + 3]};
            if (hf == 0)
                *(float2*)((float*)a.part + (int64_t)a.split_max * nbh * a.qlen * DH + 2 * prow) =
                    make_float2(m_run, l_tot);
        }
        return;
    }
    if (wsteps == 0) return;
    const float inv = 1.f / l_tot;
    constexpr int OP = DH * 2 + 16;                // staged row: 64 bf16 + padding
    static_assert(WQ * OP <= WQ * RROW, "staging fits in the ring");
    const uint32_t obuf = lds0 + OFF_RING + (uint32_t)(wave * WQ * RROW);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d = 32 * t + 8 * gq + 4 * hf;
            const float v0 = o[t][4 * gq] * inv, v1 = o[t][4 * gq + 1] * inv;
            const float v2 = o[t][4 * gq + 2] * inv, v3 = o[t][4 * gq + 3] * inv;
            *(__attribute__((address_space(3))) u32x2*)(size_t)(obuf + l32 * OP + d * 2) =
                (u32x2){pack2bf(v0, v1), pack2bf(v2, v3)};
        }
    // lane -> 16-byte chunk (lane % 8) of queries lane / 8 + 8 k
    const int ch = lane & 7;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int qi = (lane >> 3) + 8 * k;
        const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)(size_t)(obuf + qi * OP + ch * 16);
        if (iw + qi < a.qlen)
            *(u32x4*)((bf16_t*)a.out + ((int64_t)b * a.qlen + iw + qi) * ((int64_t)a.H * DH) + (int64_t)h * DH + ch * 8) = w;
    }
}

// Merge of the key splits: for query i of head h, with split partials
// (O_s, m_s, l_s), out = sum_s e^(m_s - M) O_s / sum_s e^(m_s - M) l_s,
// M = max_s m_s (an empty split has m_s = -inf, l_s = 0, O_s = 0). The grid
// covers the queries from i_first on (the tiles that were split: the split
// count grows with the tile index); a thread produces 4 consecutive outputs of
// one query. The splits are read in groups of MG (the launch's largest split
// count rounded up to 4, 8 or 16) with all loads of a group in flight
// together, and the running maximum moves between groups. Workgroups of one
// wave spread the few thousand threads over every compute unit.
constexpr int MWG = 64;

template <int MG>
__global__ void __launch_bounds__(MWG) attn_merge_kernel(AttnArgs a, int i_first) {
    const int nq = a.qlen - i_first;
    const int64_t nrow = (int64_t)a.B * a.H * nq;
    const int64_t idx = (int64_t)__builtin_amdgcn_workgroup_id_x() * MWG + __builtin_amdgcn_workitem_id_x();
    if (idx >= nrow * 16) return;
    const int c = (int)(idx & 15);
    const int64_t bh = (idx >> 4) / nq;
    const int i = i_first + (int)((idx >> 4) - bh * nq);
    const int ns = tile_splits(tile_steps(i / BQ, a.qlen, a.mlen), a.split_steps, a.split_max);
    if (ns <= 1) return;                            // written by the attention kernel
    const int64_t row = bh * a.qlen + i, plane = (int64_t)a.B * a.H * a.qlen;
    const f32x4* po = (const f32x4*)a.part + row * (DH / 4) + c;
    const float2* pml = (const float2*)((const float*)a.part + (int64_t)a.split_max * plane * DH) + row;
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ns; s0 += MG) {
        float2 ml[MG];
        f32x4 v[MG];
#pragma unroll
        for (int k = 0; k < MG; ++k) {
            const int sp = min(s0 + k, ns - 1);
            ml[k] = pml[sp * plane];
            v[k] = po[sp * plane * (DH / 4)];
        }
        float mg = M;
#pragma unroll
        for (int k = 0; k < MG; ++k)
            if (s0 + k < ns) mg = fmaxf(mg, ml[k].x);
        // mg is finite: every query sees a key in some split
        const float mb = mg * LOG2E;
        const float alpha = __builtin_amdgcn_exp2f(fmaf(M, LOG2E, -mb));   // 0 while M = -inf
        L *= alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= alpha;
#pragma unroll
        for (int k = 0; k < MG; ++k) {
            const float wgt = s0 + k < ns ? __builtin_amdgcn_exp2f(fmaf(ml[k].x, LOG2E, -mb)) : 0.f;
            L = fmaf(wgt, ml[k].y, L);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, v[k][e], acc[e]);
        }
        M = mg;
    }
    const float inv = 1.f / L;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    *(u32x2*)((bf16_t*)a.out + (b * a.qlen + i) * ((int64_t)a.H * DH) + h * DH + 4 * c) =
        (u32x2){pack2bf(acc[0] * inv, acc[1] * inv), pack2bf(acc[2] * inv, acc[3] * inv)};
}

template <bool HAS_BIAS, bool RING>
hipError_t launch_bf16(const AttnArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const int nqt = (a.qlen + BQ - 1) / BQ;
    if (a.split_steps < 0 || a.split_max < 1 || a.split_max > kMaxAttnSplits || (a.split_steps > 0 && !a.part))
        return hipErrorInvalidValue;
    int64_t grid = 0;
    int qt_first = nqt;                            // first split tile
    for (int qt = nqt - 1; qt >= 0; --qt) {
        const int n = tile_splits(tile_steps(qt, a.qlen, a.mlen), a.split_steps, a.split_max);
        grid += (int64_t)a.B * a.H * n;
        if (n > 1) qt_first = qt;
    }
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    int lds = OFF_TBL;
    if (HAS_BIAS) {
        const int gtop_max = a.mlen + (nqt - 1) * BQ + BQ - 1;
        lds += 4 * ((gtop_max + 2 * BQ + 3) & ~3);
    }
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    // the LDS limit is raised to the whole 160 KB once per process (a
    // function-local static is initialised exactly once, also under
    // concurrent launches)
    static const hipError_t attr = hipFuncSetAttribute((const void*)attn_bf16_kernel<HAS_BIAS, RING>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    (void)hipGetLastError();   // drop a stale error of an earlier runtime call
    if (qt_first == nqt) {
        hipExtLaunchKernelGGL(attn_bf16_kernel<HAS_BIAS, RING>, dim3((unsigned)grid), dim3(NT), (uint32_t)lds, s, ev0, ev1, 0u, a);
        return hipGetLastError();
    }
    // the events bracket both kernels
    hipExtLaunchKernelGGL(attn_bf16_kernel<HAS_BIAS, RING>, dim3((unsigned)grid), dim3(NT), (uint32_t)lds, s, ev0,
                          (hipEvent_t) nullptr, 0u, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int i_first = qt_first * BQ;
    const int64_t threads = (int64_t)a.B * a.H * (a.qlen - i_first) * 16;
    const auto merge = a.split_max <= 4   ? attn_merge_kernel<4>
                       : a.split_max <= 8 ? attn_merge_kernel<8>
                                          : attn_merge_kernel<16>;
    hipExtLaunchKernelGGL(merge, dim3((unsigned)((threads + MWG - 1) / MWG)), dim3(MWG), 0u, s, (hipEvent_t) nullptr,
                          ev1, 0u, a, i_first);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (a.kv_rows > 0)
        return a.bias ? launch_bf16<true, true>(a, s, ev0, ev1) : launch_bf16<false, true>(a, s, ev0, ev1);
    return a.bias ? launch_bf16<true, false>(a, s, ev0, ev1) : launch_bf16<false, false>(a, s, ev0, ev1);
}

SplitPlan attn_bf16_split_plan(int64_t B, int64_t H, int64_t qlen, int64_t mlen, int forced) {
    if (forced == 1) return {0, 1};
    if (forced > 1) return {1, forced};
    // Split only when the query tiles leave compute units idle (a split's
    // partial writes and the merge cost more than a second resident workgroup
    // per compute unit gains). The chosen step count T is the smallest (at
    // least four steps, so that a split outweighs its fixed cost) whose
    // workgroups still fit one per compute unit; tiles with more than T steps
    // are split.
    constexpr int64_t kSlots = kCUs;
    const int64_t nbh = B * H, nqt = (qlen + BQ - 1) / BQ;
    if (nbh * nqt >= kSlots) return {0, 1};
    const int tmax = tile_steps((int)nqt - 1, (int)qlen, (int)mlen);
    if (tmax < 8) return {0, 1};
    int64_t total = 0;
    for (int qt = 0; qt < nqt; ++qt) total += nbh * tile_steps(qt, (int)qlen, (int)mlen);
    for (int T = (int)(total / kSlots > 4 ? total / kSlots : 4); T < tmax; ++T) {
        int64_t w = 0;
        int mx = 1;
        for (int qt = 0; qt < nqt; ++qt) {
            const int n = tile_splits(tile_steps(qt, (int)qlen, (int)mlen), T, kMaxAttnSplits);
            w += nbh * n;
            mx = n > mx ? n : mx;
        }
        if (w <= kSlots) return mx > 1 ? SplitPlan{T, mx} : SplitPlan{0, 1};
    }
    return {0, 1};
}

size_t attn_bf16_part_bytes_bound(int64_t B, int64_t H, int64_t qlen, int forced) {
    // the library's plan splits only when the query tiles leave compute units
    // idle, and its workgroups (B*H per split of a tile) then fit the 256
    // units: no tile takes more than 256 / (B*H) splits, whatever the memory
    // length; a forced count caps every tile at that count
    const int64_t nbh = B * H, nqt = (qlen + BQ - 1) / BQ;
    int64_t smax = 0;
    if (forced > 1) smax = forced;
    else if (forced == 0 && nbh * nqt < kCUs) smax = kCUs / nbh < kMaxAttnSplits ? kCUs / nbh : kMaxAttnSplits;
    return smax > 1 ? (size_t)smax * (size_t)(nbh * qlen) * (DH + 2) * sizeof(float) : 0;
}

size_t attn_bf16_part_bytes(int64_t B, int64_t H, int64_t qlen, const SplitPlan& p) {
    return p.steps > 0 ? (size_t)p.max * (size_t)(B * H * qlen) * (DH + 2) * sizeof(float) : 0;
}

}  // namespace xl
