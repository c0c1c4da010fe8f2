// attn.hip -- fused Transformer-XL relative attention forward on MFMA, fp32
// operands (the tiny configuration, d_head 8; v_mfma_f32_32x32x2_f32).
//
// For one head, query i (segment position, absolute position mlen+i) and key
// j over [memory ; segment] (qidao123.com thread-401555 §3; felixzhao.cn
// article 118 §2.3.2; 2kiu.com/news/5253360 §2.2, §4.3):
//   s(i,j) = qu_i.k_j + qv_i.r[min(delta, n_rel-1)] (+ beta_h[min(delta, bc)])
//   with qu = scale*(q+u), qv = scale*(q+v), delta = mlen + i - j,
//   masked to -inf for j > mlen + i (2kiu.com §4.2), softmax over j, o = P.V.
//
// Work decomposition: one workgroup = (batch, head, NW*32 queries); a wave
// owns 32 queries; keys stream in steps of 32. Workgroups are issued
// longest-first (query tiles near the end of the segment see more keys).
//
// MFMA layout: every product is computed transposed (keys / distances on the
// MFMA rows, queries on the columns), so a lane owns one query and the
// softmax reductions stay inside the lane plus one swap of the half-waves.
//
// Relative shift: the position term of query i and key j depends on delta
// only. A "block" is the 32x32 product of a wave's 32 queries with 32
// consecutive band rows of r (descending distance). Block beta holds, for
// query ii of the wave, the position terms of keys 32*beta - 31 + ii ..
// 32*beta + ii. Blocks are written into a per-wave LDS ring indexed by
// absolute key (j mod 64, each row rotated against bank conflicts); step s
// reads its 32 keys from the ring (blocks s and s+1) as the initial value of
// the content product's accumulator, so the MFMA sums the four terms.
// Software pipeline: during step s a wave issues the content product of step
// s+1 and the position block for step s+2's window (block s+3), which the
// MFMA unit runs while the VALU does the softmax of step s. Each band row is
// multiplied once
// per query: the position product costs what the content product costs, and
// the L x L position matrix is never formed.
//
// Data movement: K (row-major) tiles are staged two steps ahead and V^T tiles
// one step ahead through two LDS buffers each (one barrier per step); band
// rows of r go from L2 straight into the MFMA operand registers one block
// ahead; qu/qv stay in registers.
#include "xl_common.hpp"
#include <hip/hip_ext.h>
#include "xl_internal.hpp"

namespace xl {
namespace {

constexpr int NW = 4;            // waves per workgroup
constexpr int WQ = 32;           // queries per wave
constexpr int BKY = 32;          // keys per step
constexpr int RING = 64;         // key slots per query in the ring (floats, 256 B per row)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_TH = 5.5451774444795623f;   // 8 ln 2: rescale only when the max grows by 2^8

template <int DH>
struct AttnLds {
    static constexpr int KROW = DH * 4 + 16;      // padded key row
    static constexpr int KTILE = BKY * KROW;
    static constexpr int VROW = BKY * 4 + 8;      // padded row of V^T
    static constexpr int VTILE = DH * VROW;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = 2 * KTILE;
    static constexpr int OFF_RING = ((OFF_V + 2 * VTILE) + 255) / 256 * 256;
    static constexpr int TOTAL = OFF_RING + NW * WQ * RING * 4;
};

// Lanes l and l^32 exchange a value; the two results of the swap hold one
// value of each half in every lane.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DH, bool HAS_BIAS>
__global__ void __launch_bounds__(NW * 64) attn_kernel(AttnArgs a) {
    using L = AttnLds<DH>;
    using T = float;
    constexpr int NT = NW * 64;
    constexpr int BQ = NW * WQ;
    constexpr int EPC = 4;                            // elements per 16-byte chunk
    constexpr int NKC = DH / 2;                       // MFMA k-steps over d_head
    static_assert(NKC >= 1 && DH <= 32, "d_head");
    extern __shared__ __attribute__((aligned(256))) char smem[];

    const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: per-wave values live in SGPRs
    const int l32 = lane & 31, hf = lane >> 5;

    // ---- work item: all heads' last query tiles first
    // (integer division runs on the vector unit; readfirstlane returns the
    // wave-uniform results to scalar registers so that branches on them are
    // scalar branches)
    const int nbh = a.B * a.H;
    const int nqt = (a.qlen + BQ - 1) / BQ;
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int qt = __builtin_amdgcn_readfirstlane(nqt - 1 - wg / nbh);
    const int bh = __builtin_amdgcn_readfirstlane(wg % nbh);
    const int h = __builtin_amdgcn_readfirstlane(bh % a.H);
    const int b = __builtin_amdgcn_readfirstlane(bh / a.H);
    const int i0 = qt * BQ;
    const int iw = i0 + wave * WQ;                     // first query of this wave
    const int qend = min(i0 + BQ, a.qlen);
    const int kend = a.mlen + qend;                    // keys [0, kend) are visible to some query
    const int nsteps = __builtin_amdgcn_readfirstlane((kend + BKY - 1) / BKY);
    const int wlast = iw < a.qlen ? a.mlen + min(iw + WQ, a.qlen) - 1 : -1;
    const int wsteps = __builtin_amdgcn_readfirstlane(wlast >= 0 ? wlast / BKY + 1 : 0);   // steps with a visible key for this wave

    const T* kbase = (const T*)a.k + (int64_t)bh * a.klen * DH;
    const T* vtbase = (const T*)a.vt + (int64_t)bh * DH * a.ldv;
    const T* rbase = (const T*)a.r + (int64_t)h * a.r_rows * DH;

    // ---- query operands (MFMA B operand): lane owns query iw + l32
    const int iq = iw + l32;
    const bool qok = iq < a.qlen;
    float quB[NKC], qvB[NKC];
    {
        const int64_t row = ((int64_t)bh * a.qlen + (qok ? iq : a.qlen - 1)) * DH;
        const T* qrow = (const T*)a.q + row;
        const T* ub = (const T*)a.u + h * DH;
        const T* vbias = (const T*)a.v + h * DH;
        // the biases fold into the query operands: scale*(q+u), scale*(q+v)
        for (int kc = 0; kc < NKC; ++kc) {
            const float qe = qrow[2 * kc + hf];
            quB[kc] = a.scale * (qe + ub[2 * kc + hf]);
            qvB[kc] = a.scale * (qe + vbias[2 * kc + hf]);
        }
    }

    // ---- band operand (MFMA A operand of the position product)
    // block beta covers distances dtop - 32*beta - c, c = 0..31 (descending)
    const int dtop = a.mlen + iw + WQ - 1;
    float band[NKC];
    auto load_band = [&](int beta) {
        int d = dtop - BKY * beta - l32;
        d = max(0, min(d, a.n_rel - 1));
        const T* row = rbase + (int64_t)d * DH;
        for (int kc = 0; kc < NKC; ++kc) band[kc] = row[2 * kc + hf];
    };
    auto pos_product = [&](int beta) {
        f32x16 g;
        if constexpr (HAS_BIAS) {
            const T* bias = (const T*)a.bias;
            const int dblk = dtop - BKY * beta;
            for (int r = 0; r < 16; ++r) {
                const int d = max(0, dblk - acc_row(r, hf));
                g[r] = bias[bias_row(d, a.bias_kind, a.bias_clamp) * a.H + h];
            }
        } else {
            for (int r = 0; r < 16; ++r) g[r] = 0.f;
        }
        for (int kc = 0; kc < NKC; ++kc) g = mfma32(band[kc], qvB[kc], g);
        return g;
    };

    // ---- ring addresses. Logical slot p of query row ii lives at float
    // (p + 4 ii) mod 64 of a 256-byte row: groups of 4 consecutive slots stay
    // contiguous and aligned, the writes of one register (32 consecutive
    // slots over the lanes) and the 16-byte reads of one group (8 rows) hit
    // distinct banks, and moving a slot by 32 (the other parity of a block or
    // a step) is address ^ 128.
    const uint32_t ring_row = (uint32_t)L::OFF_RING + (uint32_t)(wave * WQ + l32) * (RING * 4);
    uint32_t waddr[16];          // block of even index: register r -> byte address of its key slot
    for (int r = 0; r < 16; ++r) {
        const int p = (l32 - (WQ - 1) + acc_row(r, hf)) & (RING - 1);
        waddr[r] = ring_row + (uint32_t)(((p + 4 * l32) & (RING - 1)) << 2);
    }
    uint32_t rq[4];              // even step: 16-byte index of the 4 groups of 4 consecutive keys
    for (int g = 0; g < 4; ++g) rq[g] = (ring_row >> 4) + (uint32_t)((((8 * g + 4 * hf) + 4 * l32) & (RING - 1)) >> 2);
    auto ring_write = [&](const f32x16& g, int parity) {
        const uint32_t flip = (uint32_t)parity << 7;
        for (int r = 0; r < 16; ++r) *(float*)(smem + (waddr[r] ^ flip)) = g[r];
    };
    auto ring_read = [&](int parity) {
        const uint32_t flip = (uint32_t)parity << 3;   // 128 bytes in 16-byte units
        const f32x4* base = (const f32x4*)smem;
        f32x16 acc;
        for (int g = 0; g < 4; ++g) {
            const f32x4 t4 = base[rq[g] ^ flip];
            acc[4 * g] = t4[0]; acc[4 * g + 1] = t4[1]; acc[4 * g + 2] = t4[2]; acc[4 * g + 3] = t4[3];
        }
        return acc;
    };
    // content product of a step (its K tile in LDS buffer kbuf) on top of its position terms
    auto content = [&](f32x16 acc, int kbuf) {
        const char* kt = smem + L::OFF_K + kbuf * L::KTILE + l32 * L::KROW;
        for (int kc = 0; kc < NKC; ++kc) acc = mfma32(*(const float*)(kt + (2 * kc + hf) * 4), quB[kc], acc);
        return acc;
    };

    // ---- K / V^T tile staging (global -> registers -> LDS). K of step s is
    // needed one step early (the content product runs a step ahead), so K
    // tiles are staged two steps ahead and V^T tiles one step ahead.
    constexpr int KCPR = DH * (int)sizeof(T) / 16;     // 16-byte chunks per key row
    constexpr int KCH = BKY * KCPR;                    // chunks per K tile
    constexpr int VCPR = BKY * (int)sizeof(T) / 16;    // chunks per V^T row
    constexpr int VCH = DH * VCPR;
    constexpr int KPT = (KCH + NT - 1) / NT, VPT = (VCH + NT - 1) / NT;
    u32x4 kreg[KPT], vreg[VPT];
    auto load_k = [&](int s) {
        const int j0 = s * BKY;
        for (int t = 0; t < KPT; ++t) {
            const int c = tid + t * NT;
            if (KCH % NT == 0 || c < KCH) {
                const int jr = c / KCPR, cc = c - jr * KCPR;
                const int j = min(j0 + jr, a.klen - 1);        // rows past the end are masked keys
                kreg[t] = *(const u32x4*)(kbase + (int64_t)j * DH + cc * EPC);
            }
        }
    };
    auto store_k = [&](int buf) {
        for (int t = 0; t < KPT; ++t) {
            const int c = tid + t * NT;
            if (KCH % NT == 0 || c < KCH) {
                const int jr = c / KCPR, cc = c - jr * KCPR;
                *(u32x4*)(smem + L::OFF_K + buf * L::KTILE + jr * L::KROW + cc * 16) = kreg[t];
            }
        }
    };
    auto load_v = [&](int s) {
        const int j0 = s * BKY;
        const bool tail = j0 + BKY > a.klen;
        for (int t = 0; t < VPT; ++t) {
            const int c = tid + t * NT;
            if (VCH % NT == 0 || c < VCH) {
                const int d = c / VCPR, cc = c - d * VCPR;
                const int j = j0 + cc * EPC;
                const T* src = vtbase + (int64_t)d * a.ldv + j;
                if (!tail) {
                    vreg[t] = *(const u32x4*)src;
                } else {
                    // the last tile: values of keys >= klen are zero (their weight is 0)
                    T tmp[EPC];
                    for (int e = 0; e < EPC; ++e) tmp[e] = (j + e < a.klen) ? src[e] : (T)0;
                    vreg[t] = __builtin_bit_cast(u32x4, tmp);
                }
            }
        }
    };
    auto store_v = [&](int buf) {
        for (int t = 0; t < VPT; ++t) {
            const int c = tid + t * NT;
            if (VCH % NT == 0 || c < VCH) {
                const int d = c / VCPR, cc = c - d * VCPR;
                char* dst = smem + L::OFF_V + buf * L::VTILE + d * L::VROW + cc * 16;
                *(u32x2*)dst = (u32x2){vreg[t][0], vreg[t][1]};
                *(u32x2*)(dst + 8) = (u32x2){vreg[t][2], vreg[t][3]};
            }
        }
    };

    // ---- running softmax state and output accumulators (O^T: d on rows)
    constexpr int NDT = (DH + 31) / 32;
    f32x16 o[NDT];
    for (int t = 0; t < NDT; ++t)
        for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // prologue: K of steps 0 and 1, V of step 0; blocks 0..2; content of step 0
    load_k(0);
    store_k(0);
    if (nsteps > 1) {
        load_k(1);
        store_k(1);
    }
    load_v(0);
    store_v(0);
    f32x16 scur;
    if (wsteps > 0) {
        load_band(0);
        ring_write(pos_product(0), 0);
        load_band(1);
        ring_write(pos_product(1), 1);
        if (wsteps > 1) load_band(2);
    }
    __syncthreads();
    if (wsteps > 0) {
        scur = content(ring_read(0), 0);
        if (wsteps > 1) {
            ring_write(pos_product(2), 0);     // block 2 replaces block 0, already read
            if (wsteps > 2) load_band(3);
        }
    }
    __syncthreads();

    for (int s = 0; s < nsteps; ++s) {
        const int j0 = s * BKY;
        const int par = s & 1;
        if (s + 2 < nsteps) load_k(s + 2);
        if (s + 1 < nsteps) load_v(s + 1);
        if (s < wsteps) {
            // the next step's scores: its position terms (blocks s+1, s+2) and content product
            f32x16 snext, gnext;
            const bool have_next = s + 1 < wsteps;
            const bool want_block = s + 2 < wsteps;          // block s+3, read at step s+1
            if (have_next) snext = content(ring_read(par ^ 1), par ^ 1);
            if (want_block) {
                gnext = pos_product(s + 3);
                if (s + 3 < wsteps) load_band(s + 4);
            }
            // causal mask of this step: key j0 + jj is hidden from query iw + l32 when j > mlen + i
            if (j0 + BKY - 1 > a.mlen + iw) {
                const int lim = a.mlen + iw + l32 - j0;
                for (int r = 0; r < 16; ++r)
                    if (acc_row(r, hf) > lim) scur[r] = -INFINITY;
            }
            // online softmax with lazy rescaling: the exponentials are taken
            // against the running maximum, which moves (rescaling the running
            // sums) only when some row's maximum grew by more than 2^8
            float mx = fmaxf(fmaxf(scur[0], scur[1]), fmaxf(scur[2], scur[3]));
            for (int r = 4; r < 16; r += 2) mx = fmaxf(mx, fmaxf(scur[r], scur[r + 1]));
            mx = halves_max(mx);
            if (__any(mx > m_run + RESCALE_TH)) {
                const float mnew = fmaxf(m_run, mx);
                const float alpha = __builtin_amdgcn_exp2f((m_run - mnew) * LOG2E);
                l_run *= alpha;
                for (int t = 0; t < NDT; ++t)
                    for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
                m_run = mnew;
            }
            const float mb = m_run * LOG2E;
            float p[16];
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(scur[r], LOG2E, -mb));
            if (want_block) ring_write(gnext, par ^ 1);      // block s+3 replaces block s+1, already read
            // O^T += V^T P^T
            const char* vt = smem + L::OFF_V + par * L::VTILE;
            {
                float psum = 0.f;
                for (int r = 0; r < 16; ++r) psum += p[r];
                l_run += psum;
                const bool drow = l32 < DH;
                const float* vrow = (const float*)(vt + (drow ? l32 : 0) * L::VROW);
                for (int r = 0; r < 16; ++r) {
                    const float va = drow ? vrow[acc_row(r, hf)] : 0.f;
                    o[0] = mfma32(va, p[r], o[0]);
                }
            }
            if (have_next) scur = snext;
        }
        if (s + 2 < nsteps) store_k(par);          // K of step s+2 replaces K of step s
        if (s + 1 < nsteps) store_v(par ^ 1);      // V of step s+1 replaces V of step s-1
        __syncthreads();
    }

    // ---- epilogue: o / l, heads concatenated
    const float l_tot = halves_sum(l_run);
    if (!qok || wsteps == 0) return;
    const float inv = 1.f / l_tot;
    T* orow = (T*)a.out + ((int64_t)b * a.qlen + iq) * ((int64_t)a.H * DH) + (int64_t)h * DH;
    for (int t = 0; t < NDT; ++t)
        for (int gq = 0; gq < 4; ++gq) {
            const int d = 32 * t + 8 * gq + 4 * hf;
            if (d >= DH) continue;
            const float v0 = o[t][4 * gq] * inv, v1 = o[t][4 * gq + 1] * inv;
            const float v2 = o[t][4 * gq + 2] * inv, v3 = o[t][4 * gq + 3] * inv;
            *(f32x4*)(orow + d) = (f32x4){v0, v1, v2, v3};
        }
}

template <int DH, bool HAS_BIAS>
hipError_t launch_t(const AttnArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    using L = AttnLds<DH>;
    // the LDS limit is raised once per process (thread-safe: a function-local static)
    static const hipError_t attr = hipFuncSetAttribute((const void*)attn_kernel<DH, HAS_BIAS>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::TOTAL);
    if (attr != hipSuccess) return attr;
    constexpr int BQ = NW * WQ;
    const int nqt = (a.qlen + BQ - 1) / BQ;
    const int64_t grid = (int64_t)a.B * a.H * nqt;
    if (grid <= 0) return hipSuccess;
    (void)hipGetLastError();   // drop a stale error of an earlier runtime call
    hipExtLaunchKernelGGL((attn_kernel<DH, HAS_BIAS>), dim3((unsigned)grid), dim3(NW * 64), L::TOTAL, s, ev0, ev1, 0u,
                          a);
    return hipGetLastError();
}

template <int DH>
hipError_t launch_dt(const AttnArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    return a.bias ? launch_t<DH, true>(a, s, ev0, ev1) : launch_t<DH, false>(a, s, ev0, ev1);
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, bool bf16, int dh, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (bf16 && dh == 64) return launch_attn_bf16(a, s, ev0, ev1);
    if (!bf16 && dh == 8) return launch_dt<8>(a, s, ev0, ev1);
    return hipErrorInvalidValue;
}

}  // namespace xl
