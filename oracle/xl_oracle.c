/*
 * xl_oracle.c -- plain fp64 CPU oracle for the Transformer-XL relative
 * multi-head attention forward over [cached memory ; current segment].
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header, table or helper with the GPU
 * library.
 *
 * Every quantity is computed in double precision, with no blocking, fusion or
 * reordering beyond the definitions cited at each function. In particular the
 * relative score is evaluated as four explicit dot products per (query, key)
 * pair, and the relative embedding of each distance is looked up directly (no
 * relative-shift trick).
 *
 * Sources (pages, by title/host and section):
 *  [P1] 2kiu.com/news/5253360, TransformerXL relative-position tutorial:
 *       §2.2 (four-term score), §2.4 (distance clamp), §3.1 (module code:
 *       bias-free projections, o_proj), §4.2 (mask after the sum), §4.3
 *       (queries from the segment, keys over memory+segment).
 *  [P2] qidao123.com thread-401555, Transformer-XL cross-window RPE:
 *       §2 (sinusoidal R_delta and the worked example R_{-2}, d=4),
 *       §3 (A_rel = Q_i.K_j + Q_i.R_{i-j} + u.K_j + v.R_{i-j}).
 *  [P3] intelliparadigm.com 2238855, "Transformer-XL架构解析":
 *       §1.1 (cached states as extra keys/values, FIFO cache),
 *       §2.1 (memory first in the concatenation; the whole sum is scaled).
 *  [P4] jsqmd.com 1364567, "Transformer偏置型相对位置编码":
 *       §2.2 (softmax(QK^T/sqrt(d) + B), B_ij = b_{i-j}), §3.1-§3.4 (table
 *       [2k+1, H], index clamp(i-j+k, 0, 2k), added after scaling).
 *  [P5] felixzhao.cn article 118, "Transformer-XL 和相对位置编码":
 *       §2.3.1 (h~ = [SG(mem) o h], Q from the segment, K/V from h~),
 *       §2.3.2 (R_{d,2k} = sin(d / 10000^{2k/d_model}), R_{d,2k+1} = cos(...);
 *       separate W_{k,R}; global u, v).
 *
 * Readings where the pages are silent or disagree (each is also listed in the
 * design notes): the 1/sqrt(d_head) scale multiplies the whole four-term sum
 * [P3 §2.1]; sin/cos are interleaved (even = sin, odd = cos) [P2 §2, P5
 * §2.3.2]; the frequency exponent uses d_model [P5 §2.3.2]; distances are
 * clamped to [-C, C] inclusive [P1 §2.4]; query i (0-based in the segment)
 * sits at absolute position mlen+i and key j at position j, so
 * delta = mlen+i-j and the causal mask hides j > mlen+i; masked pairs get
 * probability exactly 0 (their score is never formed, which equals masking
 * after the sum with -inf); the scalar bias is added after scaling.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_ARG 1
#define ORC_NO_MEM 2
#define ORC_RANGE 3

static int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

/*
 * T5-style bucket of a relative distance [P4 §4.2]: the boundaries
 * 1, 2, 4, ..., 1024 on a log scale and one more bucket for larger
 * distances, 12 buckets: bucket i (i < 11) holds the distances up to
 * boundary i that the previous boundaries do not hold, bucket 11 everything
 * above 1024. Negative distances (only masked pairs have them here) share
 * bucket 0.
 */
static const int64_t T5_BOUNDS[11] = {1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024};
enum { T5_BUCKETS = 12 };

int64_t orc_t5_bucket(int64_t delta) {
    if (delta < 0) return 0;
    for (int i = 0; i < 11; ++i)
        if (delta <= T5_BOUNDS[i]) return i;
    return T5_BUCKETS - 1;
}

/* row of the scalar bias table for a distance: kind 0 the clamped distance
 * [P4 §3.1], kind 1 its T5 bucket [P4 §4.2] */
static int64_t bias_row(int64_t delta, int64_t bias_kind, int64_t bias_clamp) {
    return bias_kind == 1 ? orc_t5_bucket(delta) : clamp64(delta, -bias_clamp, bias_clamp) + bias_clamp;
}

/* One sinusoid row R_delta of width d_model [P2 §2; P5 §2.3.2]:
 * R[2t] = sin(delta * base^(-2t/d_model)), R[2t+1] = cos(same angle). */
static void sinusoid_row(double delta, int64_t d_model, double base, double* out) {
    for (int64_t t = 0; t < d_model / 2; ++t) {
        double angle = delta / pow(base, (2.0 * (double)t) / (double)d_model);
        out[2 * t] = sin(angle);
        out[2 * t + 1] = cos(angle);
    }
}

/* Rows n = 0..n_rows-1 of the relative embedding for distance delta0+n,
 * the distance clamped to [-clamp_len, clamp_len] when clamp_len >= 0
 * [P1 §2.4]. out: [n_rows, d_model]. */
int orc_relpos_embed(int64_t delta0, int64_t n_rows, int64_t d_model, int64_t clamp_len,
                     double base, double* out) {
    if (!out || n_rows < 0 || d_model <= 0 || (d_model & 1) || !(base > 0.0)) return ORC_BAD_ARG;
    for (int64_t n = 0; n < n_rows; ++n) {
        int64_t delta = delta0 + n;
        if (clamp_len >= 0) delta = clamp64(delta, -clamp_len, clamp_len);
        sinusoid_row((double)delta, d_model, base, out + n * d_model);
    }
    return ORC_OK;
}

/* y[m, n] = sum_k x[m, k] * W[n, k]: a bias-free linear layer with the
 * weight stored [out, in] [P1 §3.1: nn.Linear(..., bias=False)]. */
int orc_linear(const double* x, int64_t M, int64_t K, const double* W, int64_t N, double* y) {
    if ((M && (!x || !y)) || (N && K && !W) || M < 0 || K < 0 || N < 0) return ORC_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += x[m * K + k] * W[n * K + k];
            y[m * N + n] = s;
        }
    }
    return ORC_OK;
}

static double dot(const double* a, const double* b, int64_t n) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/*
 * Relative attention core on head-major projections.
 *   q [B, H, qlen, dh]; k, v [B, H, klen, dh]
 *   rtab [H, n_rtab, dh]: projected relative embedding, row n is distance
 *       rtab_delta0 + n (after clamping).
 *   u, vb [H, dh]: global content / position biases [P1 §2.3; P5 §2.3.2].
 *   beta [2*bias_clamp+1, H] (bias_kind 0) or [12, H] (bias_kind 1, T5
 *       buckets) or NULL: scalar bias table [P4 §3.1, §4.2]; bias_clamp < 0
 *       switches the bias off.
 *   qpos [qlen], kpos [klen]: absolute positions, or NULL for the default
 *       qpos[i] = klen - qlen + i, kpos[j] = j (memory first [P3 §2.1]).
 * For every pair with kpos[j] <= qpos[i] (causal), with
 * delta = qpos[i] - kpos[j] and dc = delta clamped to [-C, C]:
 *   a = q_i.k_j, b = q_i.r_dc, c = u.k_j, d = vb.r_dc      [P2 §3; P5 §2.3.2]
 *   l_ij = scale*(a+b+c+d) + beta[row(delta), h]   [P3 §2.1; P4 §3.4]
 *   with row(delta) = clamp(delta,-bc,bc)+bc, or the T5 bucket of delta
 * then p_i = softmax_j(l_i) over the visible keys and o_i = sum_j p_ij v_j.
 * Output o [B, qlen, H*dh] (heads concatenated, [P1 §3.1]).
 * Optional: terms [4, B, H, qlen, klen] (a, b, c, d; 0 where masked),
 *           probs [B, H, qlen, klen] (0 where masked).
 */
int orc_rel_attn_core(int64_t B, int64_t H, int64_t dh, int64_t qlen, int64_t klen,
                      const int64_t* qpos, const int64_t* kpos,
                      int64_t clamp_len, int64_t bias_clamp, int64_t bias_kind, double scale,
                      const double* q, const double* k, const double* v,
                      const double* rtab, int64_t rtab_delta0, int64_t n_rtab,
                      const double* u, const double* vb, const double* beta,
                      double* o, double* terms, double* probs) {
    if (B < 0 || H <= 0 || dh <= 0 || qlen < 0 || klen < qlen) return ORC_BAD_ARG;
    if (!q || !k || !v || !rtab || !u || !vb || !o) return ORC_BAD_ARG;
    if (bias_clamp >= 0 && !beta) return ORC_BAD_ARG;
    if (bias_kind != 0 && bias_kind != 1) return ORC_BAD_ARG;
    const int64_t mlen = klen - qlen;
    int status = ORC_OK;
#pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t hh = 0; hh < H; ++hh)
            for (int64_t i = 0; i < qlen; ++i) {
                const double* qi = q + ((b * H + hh) * qlen + i) * dh;
                const double* uh = u + hh * dh;
                const double* vh = vb + hh * dh;
                double* logit = (double*)malloc(sizeof(double) * (size_t)(klen ? klen : 1));
                unsigned char* vis = (unsigned char*)malloc((size_t)(klen ? klen : 1));
                if (!logit || !vis) {
                    free(logit); free(vis);
#pragma omp atomic write
                    status = ORC_NO_MEM;
                    continue;
                }
                const int64_t pi = qpos ? qpos[i] : mlen + i;
                double mx = -INFINITY;
                for (int64_t j = 0; j < klen; ++j) {
                    const int64_t pj = kpos ? kpos[j] : j;
                    vis[j] = (unsigned char)(pj <= pi);   /* causal mask [P1 §4.2] */
                    if (!vis[j]) continue;
                    const int64_t delta = pi - pj;
                    const int64_t dc = clamp_len >= 0 ? clamp64(delta, -clamp_len, clamp_len) : delta;
                    const int64_t row = dc - rtab_delta0;
                    if (row < 0 || row >= n_rtab) {
#pragma omp atomic write
                        status = ORC_RANGE;
                        vis[j] = 0;
                        continue;
                    }
                    const double* kj = k + ((b * H + hh) * klen + j) * dh;
                    const double* rj = rtab + (hh * n_rtab + row) * dh;
                    const double ta = dot(qi, kj, dh);
                    const double tb = dot(qi, rj, dh);
                    const double tc = dot(uh, kj, dh);
                    const double td = dot(vh, rj, dh);
                    double l = scale * (ta + tb + tc + td);
                    if (bias_clamp >= 0) l += beta[bias_row(delta, bias_kind, bias_clamp) * H + hh];
                    logit[j] = l;
                    if (l > mx) mx = l;
                    if (terms) {
                        const int64_t plane = B * H * qlen * klen;
                        const int64_t at = ((b * H + hh) * qlen + i) * klen + j;
                        terms[at] = ta; terms[plane + at] = tb;
                        terms[2 * plane + at] = tc; terms[3 * plane + at] = td;
                    }
                }
                /* softmax with the maximum subtracted, then P.V */
                double den = 0.0;
                for (int64_t j = 0; j < klen; ++j)
                    if (vis[j]) { logit[j] = exp(logit[j] - mx); den += logit[j]; }
                double* oi = o + (b * qlen + i) * (H * dh) + hh * dh;
                for (int64_t d = 0; d < dh; ++d) oi[d] = 0.0;
                for (int64_t j = 0; j < klen; ++j) {
                    const int64_t at = ((b * H + hh) * qlen + i) * klen + j;
                    if (!vis[j]) {
                        if (probs) probs[at] = 0.0;
                        if (terms) {
                            const int64_t plane = B * H * qlen * klen;
                            terms[at] = terms[plane + at] = terms[2 * plane + at] = terms[3 * plane + at] = 0.0;
                        }
                        continue;
                    }
                    const double p = logit[j] / den;
                    if (probs) probs[at] = p;
                    const double* vj = v + ((b * H + hh) * klen + j) * dh;
                    for (int64_t d = 0; d < dh; ++d) oi[d] += p * vj[d];
                }
                free(logit); free(vis);
            }
    return status;
}

/*
 * Gradients of the attention core (default positions: query i at mlen+i,
 * key j at j) for an upstream gradient dout [B, qlen, H*dh] of o. With the
 * logits l_ij = scale*(q_i.k_j + q_i.r + u.k_j + v.r) + beta (as the forward)
 * and P = softmax_j(l), per (b, h, i):
 *   dP_ij = dout_i . v_j,  D_i = sum_j P_ij dP_ij,  dS_ij = P_ij (dP_ij - D_i)
 *   dq_i  = scale sum_j dS_ij (k_j + r_ij)     dk_j += scale dS_ij (q_i + u)
 *   dv_j += P_ij dout_i                        dr_row += scale dS_ij (q_i + v)
 *   du   += scale sum_j dS_ij k_j              dvb  += scale sum_j dS_ij r_ij
 *   dbeta[brow, h] += dS_ij
 * where r_ij is the table row of the clamped distance (memory gets no other
 * gradient path here: the memory rows of k and v receive theirs like any key).
 * The chain rule of the softmax and of the four dot products, written out per
 * pair. Outputs are overwritten: dq [B,H,qlen,dh], dk, dv [B,H,klen,dh],
 * drtab [H, n_rtab, dh], du, dvb [H, dh], dbeta as beta (or NULL).
 */
int orc_rel_attn_core_bwd(int64_t B, int64_t H, int64_t dh, int64_t qlen, int64_t klen, int64_t clamp_len,
                          int64_t bias_clamp, int64_t bias_kind, double scale, const double* q, const double* k,
                          const double* v, const double* rtab, int64_t n_rtab, const double* u, const double* vb,
                          const double* beta, const double* dout, double* dq, double* dk, double* dv, double* drtab,
                          double* du, double* dvb, double* dbeta) {
    if (B < 0 || H <= 0 || dh <= 0 || qlen < 0 || klen < qlen || n_rtab <= 0) return ORC_BAD_ARG;
    if (!q || !k || !v || !rtab || !u || !vb || !dout || !dq || !dk || !dv || !drtab || !du || !dvb)
        return ORC_BAD_ARG;
    if (bias_clamp >= 0 && (!beta || !dbeta)) return ORC_BAD_ARG;
    if (bias_kind != 0 && bias_kind != 1) return ORC_BAD_ARG;
    const int64_t mlen = klen - qlen;
    const int64_t n_beta = bias_kind == 1 ? 12 : 2 * bias_clamp + 1;
    memset(dq, 0, sizeof(double) * (size_t)(B * H * qlen * dh));
    memset(dk, 0, sizeof(double) * (size_t)(B * H * klen * dh));
    memset(dv, 0, sizeof(double) * (size_t)(B * H * klen * dh));
    memset(drtab, 0, sizeof(double) * (size_t)(H * n_rtab * dh));
    memset(du, 0, sizeof(double) * (size_t)(H * dh));
    memset(dvb, 0, sizeof(double) * (size_t)(H * dh));
    if (bias_clamp >= 0) memset(dbeta, 0, sizeof(double) * (size_t)(n_beta * H));
    int status = ORC_OK;
    /* heads are independent; everything a head accumulates belongs to it */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t hh = 0; hh < H; ++hh) {
        double* P = (double*)malloc(sizeof(double) * (size_t)(klen ? klen : 1));
        double* dS = (double*)malloc(sizeof(double) * (size_t)(klen ? klen : 1));
        int64_t* rrow = (int64_t*)malloc(sizeof(int64_t) * (size_t)(klen ? klen : 1));
        if (!P || !dS || !rrow) {
            free(P); free(dS); free(rrow);
#pragma omp atomic write
            status = ORC_NO_MEM;
            continue;
        }
        const double* uh = u + hh * dh;
        const double* vh = vb + hh * dh;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t i = 0; i < qlen; ++i) {
                const double* qi = q + ((b * H + hh) * qlen + i) * dh;
                const double* gi = dout + (b * qlen + i) * (H * dh) + hh * dh;
                const int64_t nv = mlen + i + 1;   /* visible keys j <= mlen + i */
                double mx = -INFINITY;
                for (int64_t j = 0; j < nv; ++j) {
                    const int64_t delta = mlen + i - j;
                    const int64_t dc = clamp_len >= 0 ? clamp64(delta, -clamp_len, clamp_len) : delta;
                    if (dc >= n_rtab) {
#pragma omp atomic write
                        status = ORC_RANGE;
                        rrow[j] = n_rtab - 1;
                    } else {
                        rrow[j] = dc;
                    }
                    const double* kj = k + ((b * H + hh) * klen + j) * dh;
                    const double* rj = rtab + (hh * n_rtab + rrow[j]) * dh;
                    double l = scale * (dot(qi, kj, dh) + dot(qi, rj, dh) + dot(uh, kj, dh) + dot(vh, rj, dh));
                    if (bias_clamp >= 0) l += beta[bias_row(delta, bias_kind, bias_clamp) * H + hh];
                    P[j] = l;
                    if (l > mx) mx = l;
                }
                double den = 0.0;
                for (int64_t j = 0; j < nv; ++j) { P[j] = exp(P[j] - mx); den += P[j]; }
                double Di = 0.0;
                for (int64_t j = 0; j < nv; ++j) {
                    P[j] /= den;
                    dS[j] = dot(gi, v + ((b * H + hh) * klen + j) * dh, dh);   /* dP_ij for now */
                    Di += P[j] * dS[j];
                }
                double* dqi = dq + ((b * H + hh) * qlen + i) * dh;
                for (int64_t j = 0; j < nv; ++j) {
                    dS[j] = P[j] * (dS[j] - Di);
                    const double* kj = k + ((b * H + hh) * klen + j) * dh;
                    const double* rj = rtab + (hh * n_rtab + rrow[j]) * dh;
                    double* dkj = dk + ((b * H + hh) * klen + j) * dh;
                    double* dvj = dv + ((b * H + hh) * klen + j) * dh;
                    double* drj = drtab + (hh * n_rtab + rrow[j]) * dh;
                    for (int64_t d = 0; d < dh; ++d) {
                        dqi[d] += scale * dS[j] * (kj[d] + rj[d]);
                        dkj[d] += scale * dS[j] * (qi[d] + uh[d]);
                        dvj[d] += P[j] * gi[d];
                        drj[d] += scale * dS[j] * (qi[d] + vh[d]);
                        du[hh * dh + d] += scale * dS[j] * kj[d];
                        dvb[hh * dh + d] += scale * dS[j] * rj[d];
                    }
                    if (bias_clamp >= 0) dbeta[bias_row(mlen + i - j, bias_kind, bias_clamp) * H + hh] += dS[j];
                }
            }
        free(P); free(dS); free(rrow);
    }
    return status;
}

/*
 * Full layer forward [P5 §2.3.1-§2.3.2; P1 §3.1]:
 *   x~ = [mem ; h] per batch (memory rows first)
 *   q = h W_q^T, k = x~ W_k^T, v = x~ W_v^T   (weights [H*dh, D])
 *   r_dc = R_dc W_r^T for each clamped distance dc in use
 *   o = core(q, k, v, r, u, vb, beta), out = o W_o^T  (W_o [D, H*dh])
 * h [B, qlen, D]; mem [B, mlen, D] (may be NULL when mlen == 0);
 * out [B, qlen, D]. qpos/kpos/terms/probs as for the core.
 */
int orc_rel_attn_fwd(int64_t B, int64_t D, int64_t H, int64_t dh, int64_t qlen, int64_t mlen,
                     int64_t clamp_len, int64_t bias_clamp, int64_t bias_kind, double scale, double base,
                     const int64_t* qpos, const int64_t* kpos,
                     const double* h, const double* mem,
                     const double* w_q, const double* w_k, const double* w_v,
                     const double* w_r, const double* w_o,
                     const double* u, const double* vb, const double* beta,
                     double* out, double* terms, double* probs) {
    if (B < 0 || D <= 0 || (D & 1) || H <= 0 || dh <= 0 || qlen < 0 || mlen < 0) return ORC_BAD_ARG;
    if (!h || (mlen > 0 && !mem) || !w_q || !w_k || !w_v || !w_r || !w_o || !u || !vb || !out)
        return ORC_BAD_ARG;
    const int64_t klen = mlen + qlen, HD = H * dh;
    int status = ORC_OK;

    /* range of clamped distances over the visible pairs */
    int64_t dmin = INT64_MAX, dmax = INT64_MIN;
    for (int64_t i = 0; i < qlen; ++i)
        for (int64_t j = 0; j < klen; ++j) {
            const int64_t pi = qpos ? qpos[i] : mlen + i, pj = kpos ? kpos[j] : j;
            if (pj > pi) continue;
            int64_t dc = pi - pj;
            if (clamp_len >= 0) dc = clamp64(dc, -clamp_len, clamp_len);
            if (dc < dmin) dmin = dc;
            if (dc > dmax) dmax = dc;
        }
    if (dmin > dmax) { dmin = 0; dmax = 0; }
    const int64_t n_r = dmax - dmin + 1;

    double* xt = (double*)calloc((size_t)(B * klen * D + 1), sizeof(double));
    double* qp = (double*)malloc(sizeof(double) * (size_t)(B * qlen * HD + 1));
    double* kp = (double*)malloc(sizeof(double) * (size_t)(B * klen * HD + 1));
    double* vp = (double*)malloc(sizeof(double) * (size_t)(B * klen * HD + 1));
    double* R = (double*)malloc(sizeof(double) * (size_t)(n_r * D));
    double* rp = (double*)malloc(sizeof(double) * (size_t)(n_r * HD));
    double* qh = (double*)malloc(sizeof(double) * (size_t)(B * qlen * HD + 1));
    double* kh = (double*)malloc(sizeof(double) * (size_t)(B * klen * HD + 1));
    double* vh = (double*)malloc(sizeof(double) * (size_t)(B * klen * HD + 1));
    double* rh = (double*)malloc(sizeof(double) * (size_t)(n_r * HD));
    double* o = (double*)malloc(sizeof(double) * (size_t)(B * qlen * HD + 1));
    if (!xt || !qp || !kp || !vp || !R || !rp || !qh || !kh || !vh || !rh || !o) { status = ORC_NO_MEM; goto done; }

    for (int64_t b = 0; b < B; ++b) {
        if (mlen) memcpy(xt + b * klen * D, mem + b * mlen * D, sizeof(double) * (size_t)(mlen * D));
        if (qlen) memcpy(xt + (b * klen + mlen) * D, h + b * qlen * D, sizeof(double) * (size_t)(qlen * D));
    }
    orc_linear(h, B * qlen, D, w_q, HD, qp);
    orc_linear(xt, B * klen, D, w_k, HD, kp);
    orc_linear(xt, B * klen, D, w_v, HD, vp);
    for (int64_t n = 0; n < n_r; ++n) sinusoid_row((double)(dmin + n), D, base, R + n * D);
    orc_linear(R, n_r, D, w_r, HD, rp);

    /* split heads: [rows, H*dh] -> [B, H, rows, dh] */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t hh = 0; hh < H; ++hh) {
            for (int64_t i = 0; i < qlen; ++i)
                memcpy(qh + ((b * H + hh) * qlen + i) * dh, qp + (b * qlen + i) * HD + hh * dh, sizeof(double) * (size_t)dh);
            for (int64_t j = 0; j < klen; ++j) {
                memcpy(kh + ((b * H + hh) * klen + j) * dh, kp + (b * klen + j) * HD + hh * dh, sizeof(double) * (size_t)dh);
                memcpy(vh + ((b * H + hh) * klen + j) * dh, vp + (b * klen + j) * HD + hh * dh, sizeof(double) * (size_t)dh);
            }
        }
    for (int64_t hh = 0; hh < H; ++hh)
        for (int64_t n = 0; n < n_r; ++n)
            memcpy(rh + (hh * n_r + n) * dh, rp + n * HD + hh * dh, sizeof(double) * (size_t)dh);

    status = orc_rel_attn_core(B, H, dh, qlen, klen, qpos, kpos, clamp_len, bias_clamp, bias_kind, scale,
                               qh, kh, vh, rh, dmin, n_r, u, vb, beta, o, terms, probs);
    if (status == ORC_OK) orc_linear(o, B * qlen, HD, w_o, D, out);
done:
    free(xt); free(qp); free(kp); free(vp); free(R); free(rp);
    free(qh); free(kh); free(vh); free(rh); free(o);
    return status;
}

/*
 * FIFO memory update [P3 §1.1; P5 §2.3.1]: the new memory is the last
 * min(mem_len + qlen, mlen_max) rows of [mem ; h] for each batch element;
 * the newest states push out the oldest. It is a copy (stop-gradient: the
 * memory never aliases the layer input).
 * mem [B, mem_len, D], h [B, qlen, D], new_mem [B, new_len, D].
 * Returns new_len through *new_len.
 */
int orc_fifo_update(int64_t B, int64_t D, int64_t mlen_max, int64_t mem_len, const double* mem,
                    int64_t qlen, const double* h, double* new_mem, int64_t* new_len) {
    if (B < 0 || D <= 0 || mlen_max < 0 || mem_len < 0 || mem_len > mlen_max || qlen < 0 || !new_len)
        return ORC_BAD_ARG;
    const int64_t total = mem_len + qlen;
    const int64_t keep = total < mlen_max ? total : mlen_max;
    const int64_t first = total - keep;   /* index into [mem ; h] of the first kept row */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t r = 0; r < keep; ++r) {
            const int64_t src = first + r;
            const double* s = src < mem_len ? mem + (b * mem_len + src) * D : h + (b * qlen + (src - mem_len)) * D;
            memcpy(new_mem + (b * keep + r) * D, s, sizeof(double) * (size_t)D);
        }
    *new_len = keep;
    return ORC_OK;
}

/*
 * Layer normalisation of each row of x [rows, D]: the row's mean and
 * (population) variance, then y = (x - mean) / sqrt(var + eps) * gamma + beta
 * elementwise. The pre-LN decoder layer normalises the attention input this
 * way [P1 §3.4: the input of the attention module is layer-normalised]; the
 * epsilon is a parameter (the pages name 1e-5 as the usual value [P3 §4.2]).
 * gamma and beta [D] may be NULL (1 and 0).
 */
int orc_layer_norm(int64_t rows, int64_t D, const double* x, const double* gamma, const double* beta, double eps,
                   double* y) {
    if (rows < 0 || D <= 0 || (rows && (!x || !y)) || !(eps >= 0.0)) return ORC_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * D;
        double mean = 0.0;
        for (int64_t k = 0; k < D; ++k) mean += xr[k];
        mean /= (double)D;
        double var = 0.0;
        for (int64_t k = 0; k < D; ++k) var += (xr[k] - mean) * (xr[k] - mean);
        var /= (double)D;
        const double inv = 1.0 / sqrt(var + eps);
        for (int64_t k = 0; k < D; ++k)
            y[r * D + k] = (xr[k] - mean) * inv * (gamma ? gamma[k] : 1.0) + (beta ? beta[k] : 0.0);
    }
    return ORC_OK;
}

/* Number of OpenMP threads the oracle's parallel loops use (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
#endif
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
