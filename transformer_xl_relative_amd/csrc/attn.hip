// attn.hip -- fused Transformer-XL relative attention forward on MFMA.
//
// For one head, query i (segment position, absolute position mlen+i) and key
// j over [memory ; segment] (qidao123.com thread-401555 §3; felixzhao.cn
// article 118 §2.3.2; 2kiu.com/news/5253360 §2.2, §4.3):
//   s(i,j) = qu_i.k_j + qv_i.r[min(delta, n_rel-1)] (+ beta_h[min(delta, bc)])
//   with qu = scale*(q+u), qv = scale*(q+v), delta = mlen + i - j,
//   masked to -inf for j > mlen + i (2kiu.com §4.2), softmax over j, o = P.V.
//
// Work decomposition: one workgroup = (batch, head, 128 queries); 4 waves of
// 32 queries; keys stream in steps of 32.
//
// MFMA layout: every product is computed transposed (keys / distances on the
// MFMA rows, queries on the columns), so a lane owns one query and the
// softmax reductions stay inside the lane (plus one swap between the two
// half-waves).
//
// Relative shift: the position term of query i and key j only depends on
// delta. Each step a wave multiplies its 32 queries by the 32 band rows of
// the distances that enter its window (one 32x32 MFMA block), and writes the
// result into a per-wave LDS ring indexed by absolute key (j mod 64). Reading
// the ring at the step's keys is then an aligned, contiguous LDS read, and it
// initialises the accumulator of the content product, so the four terms are
// summed by the MFMA itself. Every band row is multiplied once per query: the
// position product costs the same as the content product, and the L x L
// position matrix is never formed.
//
// Data movement: K (row-major) and V^T tiles are staged through two LDS
// stages (one barrier per step); band rows of r go straight from L2 into the
// MFMA operand registers one step ahead; qu/qv stay in registers.
#include "xl_common.hpp"
#include "xl_internal.hpp"

namespace xl {
namespace {

constexpr int NW = 4;            // waves per workgroup
constexpr int WQ = 32;           // queries per wave
constexpr int BQ = NW * WQ;      // queries per workgroup
constexpr int BKY = 32;          // keys per step
constexpr int RING = 64;         // key slots per query in the ring
constexpr int RSTR = 68;         // floats per query row of the ring (4 pad)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_TH = 5.5451774444795623f;   // 8 * ln 2: rescale only when the max grows by 2^8

template <typename T, int DH>
struct AttnLds {
    static constexpr int KROW = DH * (int)sizeof(T) + 16;
    static constexpr int KTILE = BKY * KROW;
    static constexpr int VROW = BKY * (int)sizeof(T) + 8;
    static constexpr int VTILE = DH * VROW;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = 2 * KTILE;
    static constexpr int OFF_RING = ((OFF_V + 2 * VTILE) + 15) / 16 * 16;
    static constexpr int TOTAL = OFF_RING + NW * WQ * RSTR * 4;
};

template <typename T, int DH>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs a) {
    using L = AttnLds<T, DH>;
    constexpr bool BF = Elem<T>::kBf16;
    constexpr int EPC = 16 / (int)sizeof(T);          // elements per 16-byte chunk
    constexpr int NKC = BF ? DH / 16 : DH / 2;        // MFMA k-steps over d_head
    static_assert(NKC >= 1, "d_head too small");
    using OpT = typename std::conditional<BF, bf16x8, float>::type;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

    // ---- workgroup -> (batch, head, query tile); the longest tiles go first
    const int nqt = (a.qlen + BQ - 1) / BQ;
    const int bh = blockIdx.x / nqt;
    const int qt = nqt - 1 - (int)(blockIdx.x - bh * nqt);
    const int b = bh / a.H, h = bh - b * a.H;
    const int i0 = qt * BQ;
    const int iw = i0 + wave * WQ;                     // first query of this wave
    const int qend = min(i0 + BQ, a.qlen);
    const int kend = a.mlen + qend;                    // keys [0, kend) are visible to someone
    const int nsteps = (kend + BKY - 1) / BKY;
    const int wlast = iw < a.qlen ? a.mlen + min(iw + WQ, a.qlen) - 1 : -1;
    const int wsteps = wlast >= 0 ? wlast / BKY + 1 : 0;   // steps with a visible key for this wave

    const T* kbase = (const T*)a.k + (int64_t)bh * a.klen * DH;
    const T* vtbase = (const T*)a.vt + (int64_t)bh * DH * a.ldv;
    const T* rbase = (const T*)a.r + (int64_t)h * a.r_rows * DH;
    const bool has_bias = a.bias != nullptr;
    const T* bias = (const T*)a.bias;

    // ---- query operands (MFMA B operand): lane owns query iw + l32
    const int iq = iw + l32;
    const bool qok = iq < a.qlen;
    OpT quB[NKC], qvB[NKC];
    {
        const T* qu = (const T*)a.qu + ((int64_t)bh * a.qlen + (qok ? iq : 0)) * DH;
        const T* qv = (const T*)a.qv + ((int64_t)bh * a.qlen + (qok ? iq : 0)) * DH;
        for (int kc = 0; kc < NKC; ++kc) {
            if constexpr (BF) {
                const int off = 16 * kc + 8 * hf;
                quB[kc] = qok ? as_bf16x8(*(const u32x4*)(qu + off)) : as_bf16x8((u32x4){0, 0, 0, 0});
                qvB[kc] = qok ? as_bf16x8(*(const u32x4*)(qv + off)) : as_bf16x8((u32x4){0, 0, 0, 0});
            } else {
                const int off = 2 * kc + hf;
                quB[kc] = qok ? Elem<T>::to_f(qu[off]) : 0.f;
                qvB[kc] = qok ? Elem<T>::to_f(qv[off]) : 0.f;
            }
        }
    }

    // ---- band operand (MFMA A operand of the position product)
    // block beta covers distances dtop - 32*beta - c, c = 0..31 (descending)
    const int dtop = a.mlen + iw + WQ - 1;
    OpT band[NKC];
    auto load_band = [&](int beta) {
        int d = dtop - BKY * beta - l32;
        d = d < 0 ? 0 : (d >= a.n_rel ? a.n_rel - 1 : d);
        const T* row = rbase + (int64_t)d * DH;
        for (int kc = 0; kc < NKC; ++kc) {
            if constexpr (BF) band[kc] = as_bf16x8(*(const u32x4*)(row + 16 * kc + 8 * hf));
            else band[kc] = Elem<T>::to_f(row[2 * kc + hf]);
        }
    };

    float* ring = (float*)(smem + L::OFF_RING) + (wave * WQ + l32) * RSTR;   // this lane's query row
    // position block -> ring: register r <-> slot c = acc_row(r, hf) <-> key
    // j = l32 - (WQ-1) + 32*beta + c (absolute), stored at j mod 64
    auto pos_block = [&](int beta) {
        f32x16 g;
        if (has_bias) {
            const int dblk = dtop - BKY * beta;
            for (int r = 0; r < 16; ++r) {
                int d = dblk - acc_row(r, hf);
                d = d < 0 ? 0 : (d > a.bias_clamp ? a.bias_clamp : d);
                g[r] = Elem<T>::to_f(bias[(int64_t)(d + a.bias_clamp) * a.H + h]);
            }
        } else {
            for (int r = 0; r < 16; ++r) g[r] = 0.f;
        }
        for (int kc = 0; kc < NKC; ++kc) g = mfma32(band[kc], qvB[kc], g);
        const int jb = l32 - (WQ - 1) + BKY * beta;
        for (int r = 0; r < 16; ++r) ring[(jb + acc_row(r, hf)) & (RING - 1)] = g[r];
    };

    // ---- K / V^T tile staging (global -> registers -> LDS)
    constexpr int KCPR = DH * (int)sizeof(T) / 16;     // 16-byte chunks per key row
    constexpr int KCH = BKY * KCPR;                    // chunks per K tile
    constexpr int VCPR = BKY * (int)sizeof(T) / 16;    // chunks per V^T row
    constexpr int VCH = DH * VCPR;
    static_assert(KCH <= 256 && VCH <= 256, "tile larger than one chunk per thread");
    u32x4 kreg = {0, 0, 0, 0}, vreg = {0, 0, 0, 0};
    auto stage_load = [&](int s) {
        const int j0 = s * BKY;
        if (tid < KCH) {
            const int jr = tid / KCPR, c = tid - jr * KCPR;
            const int j = j0 + jr;
            kreg = j < a.klen ? *(const u32x4*)(kbase + (int64_t)j * DH + c * EPC) : (u32x4){0, 0, 0, 0};
        }
        if (tid < VCH) {
            const int d = tid / VCPR, c = tid - d * VCPR;
            const int j = j0 + c * EPC;
            const T* src = vtbase + (int64_t)d * a.ldv + j;
            if (j + EPC <= a.klen) {
                vreg = *(const u32x4*)src;
            } else {
                T tmp[EPC];
                for (int e = 0; e < EPC; ++e) tmp[e] = (j + e < a.klen) ? src[e] : (T)0;
                vreg = __builtin_bit_cast(u32x4, tmp);
            }
        }
    };
    auto stage_store = [&](int buf) {
        if (tid < KCH) {
            const int jr = tid / KCPR, c = tid - jr * KCPR;
            *(u32x4*)(smem + L::OFF_K + buf * L::KTILE + jr * L::KROW + c * 16) = kreg;
        }
        if (tid < VCH) {
            const int d = tid / VCPR, c = tid - d * VCPR;
            char* dst = smem + L::OFF_V + buf * L::VTILE + d * L::VROW + c * 16;
            *(u32x2*)dst = (u32x2){vreg[0], vreg[1]};
            *(u32x2*)(dst + 8) = (u32x2){vreg[2], vreg[3]};
        }
    };

    // ---- running softmax state and output accumulators (O^T: d on rows)
    constexpr int NDT = (DH + 31) / 32;
    f32x16 o[NDT];
    for (int t = 0; t < NDT; ++t)
        for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    stage_load(0);
    stage_store(0);
    if (wsteps > 0) {
        load_band(0);
        pos_block(0);
        load_band(1);
    }
    __syncthreads();

    for (int s = 0; s < nsteps; ++s) {
        const int j0 = s * BKY;
        const bool more = s + 1 < nsteps;
        if (more) stage_load(s + 1);
        if (s < wsteps) {
            // position block for the distances entering at this step
            pos_block(s + 1);
            if (s + 1 < wsteps) load_band(s + 2);
            // relative-shifted position term of this step's keys -> accumulator
            f32x16 sacc;
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 t4 = *(const f32x4*)(ring + ((j0 + 8 * gq + 4 * hf) & (RING - 1)));
                sacc[4 * gq] = t4[0]; sacc[4 * gq + 1] = t4[1]; sacc[4 * gq + 2] = t4[2]; sacc[4 * gq + 3] = t4[3];
            }
            // content term
            const char* kt = smem + L::OFF_K + (s & 1) * L::KTILE + l32 * L::KROW;
            for (int kc = 0; kc < NKC; ++kc) {
                OpT ka;
                if constexpr (BF) ka = as_bf16x8(*(const u32x4*)(kt + (2 * kc + hf) * 16));
                else ka = *(const float*)(kt + (2 * kc + hf) * 4);
                sacc = mfma32(ka, quB[kc], sacc);
            }
            // causal mask: key j0 + jj is hidden from query iw + l32 when j > mlen + i
            if (j0 + BKY - 1 > a.mlen + iw) {
                const int lim = a.mlen + iw + l32 - j0;
                for (int r = 0; r < 16; ++r)
                    if (acc_row(r, hf) > lim) sacc[r] = -INFINITY;
            }
            // online softmax with lazy rescaling
            float mx = sacc[0];
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
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
            float psum = 0.f;
            for (int r = 0; r < 16; ++r) {
                p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], LOG2E, -mb));
                psum += p[r];
            }
            l_run += psum;
            // O^T += V^T P^T
            const char* vt = smem + L::OFF_V + (s & 1) * L::VTILE;
            if constexpr (BF) {
                bf16x8 pb[2];
                for (int kc = 0; kc < 2; ++kc)
                    for (int e = 0; e < 8; ++e) pb[kc][e] = (__bf16)p[8 * kc + e];
                for (int t = 0; t < NDT; ++t) {
                    const char* vrow = vt + (32 * t + l32) * L::VROW;
                    for (int kc = 0; kc < 2; ++kc) {
                        const u32x2 lo = *(const u32x2*)(vrow + (16 * kc + 4 * hf) * 2);
                        const u32x2 hi = *(const u32x2*)(vrow + (16 * kc + 8 + 4 * hf) * 2);
                        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
                        o[t] = mfma32(as_bf16x8(w), pb[kc], o[t]);
                    }
                }
            } else {
                const bool drow = l32 < DH;
                const float* vrow = (const float*)(vt + (drow ? l32 : 0) * L::VROW);
                for (int r = 0; r < 16; ++r) {
                    const float va = drow ? vrow[acc_row(r, hf)] : 0.f;
                    o[0] = mfma32(va, p[r], o[0]);
                }
            }
        }
        if (more) stage_store((s + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: o / l, heads concatenated
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!qok || wsteps == 0) return;
    const float inv = 1.f / l_tot;
    T* orow = (T*)a.out + ((int64_t)b * a.qlen + iq) * ((int64_t)a.H * DH) + (int64_t)h * DH;
    for (int t = 0; t < NDT; ++t)
        for (int gq = 0; gq < 4; ++gq) {
            const int d = 32 * t + 8 * gq + 4 * hf;
            if (d >= DH) continue;
            const float v0 = o[t][4 * gq] * inv, v1 = o[t][4 * gq + 1] * inv;
            const float v2 = o[t][4 * gq + 2] * inv, v3 = o[t][4 * gq + 3] * inv;
            if constexpr (BF) *(u32x2*)(orow + d) = (u32x2){pack2bf(v0, v1), pack2bf(v2, v3)};
            else *(f32x4*)(orow + d) = (f32x4){v0, v1, v2, v3};
        }
}

template <typename T, int DH>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
    using L = AttnLds<T, DH>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)attn_kernel<T, DH>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::TOTAL);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int nqt = (a.qlen + BQ - 1) / BQ;
    const int64_t grid = (int64_t)a.B * a.H * nqt;
    if (grid <= 0) return hipSuccess;
    (void)hipGetLastError();   // drop a stale error of an earlier runtime call
    hipLaunchKernelGGL((attn_kernel<T, DH>), dim3((unsigned)grid), dim3(256), L::TOTAL, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, bool bf16, int dh, hipStream_t s) {
    if (bf16 && dh == 64) return launch_t<bf16_t, 64>(a, s);
    if (!bf16 && dh == 8) return launch_t<float, 8>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace xl
