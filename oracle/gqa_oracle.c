/*
 * gqa_oracle.c -- CPU oracle for masked grouped-query softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, fp64 definition the
 * GPU path is checked against. Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load it; the product path never does. It shares no
 * code with the HIP library.
 *
 * What it computes (the plain definition, not the chunked algorithm):
 *   logits   l[t,s] = sum_h q[b,k,g,t,h] * k[b,k,s,h]          (no scale: q
 *            arrives pre-multiplied by H^-1/2 -- danielwatson6.github.io/fa,
 *            "What is wrong with naive attention?", the attn_naive listing)
 *   softmax  over the visible s of row t, with the maximum subtracted first
 *            (same page, "Chunked attention": softmax(l) = softmax(l + c))
 *   output   O[t,:] = sum_s P[t,s] * v[s,:];  lse[t] = m + ln(sum exp(l - m))
 *   visible  (no segment ids || q_seg[b,t] == kv_seg[b,s])
 *            && (s < prefix || (causal rule && window rule))
 *            -- segment equality per the SegmentIds section of the fjformer
 *            Pallas flash-attention page; causal masking as in apple/axlearn
 *            PR 845 (lazy causal mask), in one of two alignments:
 *              causal = 1 (top-left):   s <= t
 *              causal = 2 (end-aligned): s <= t + (S - T), the last query
 *              seeing every key, as new queries appended to a context do
 *              (danielwatson6.github.io/fa, "Quick digression: what about
 *              inference?");
 *            window rule (wl < 0 || s >= t - wl) && (wr < 0 || s <= t + wr):
 *            a local window (a band of diagonals; wl = wr = -1 leaves it
 *            out); prefix: keys s < prefix are visible to every query
 *            (a prefix-LM; prefix = 0 leaves it out). The pages run splash
 *            attention's block-mask processing only with a FullMask; the band
 *            and the prefix are the readings used for its non-full cases (see
 *            the tests' pins).
 *            A test-only explicit mask M[b,t,s] may replace that rule.
 *   A row with no visible key gives O = 0 and lse = -inf (a convention: the
 *   pages are silent on it; parity unpinned).
 *
 * Backward (the pages give no backward math; standard calculus of softmax):
 *   dP[t,s] = dO[t,:].v[s,:];  D[t] = sum_s P[t,s] dP[t,s];
 *   dS[t,s] = P[t,s] (dP[t,s] - D[t])
 *   dQ[t,:] = sum_s dS[t,s] k[s,:]
 *   dK[s,:] = sum_{g,t} dS[g,t,s] q[g,t,:];  dV[s,:] = sum_{g,t} P[g,t,s] dO[g,t,:]
 *   Gradients are with respect to the pre-scaled q as passed.
 *
 * Inputs are bf16 bit patterns (uint16); each is widened exactly to the
 * accumulation type acc_t. All sums run in acc_t, in index order. OpenMP
 * splits independent output rows across threads; it does not change any row's
 * arithmetic. acc_t is double (the parity reference, libgqa_oracle.so); built
 * with -DORACLE_ACC_FLOAT it is float (libgqa_oracle_f32.so, the same
 * definition in single precision, used only as a timed CPU baseline and
 * checked against the double build). Results are returned as double either
 * way.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef ORACLE_ACC_FLOAT
typedef float acc_t;
#define ACC_EXP expf
#define ACC_LOG logf
#else
typedef double acc_t;
#define ACC_EXP exp
#define ACC_LOG log
#endif

static acc_t bf(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (acc_t)f;
}

typedef struct {
    const uint16_t *q, *k, *v, *dout;
    const int32_t *q_seg, *kv_seg;
    const uint8_t *mask; /* [B, T, S] or NULL */
    int64_t B, K, G, T, S, H;
    int causal;     /* 0 none, 1 top-left, 2 end-aligned */
    int64_t wl, wr; /* local window sides, -1 = unbounded */
    int64_t prefix; /* keys s < prefix visible to every query */
} problem;

static int is_visible(const problem *p, int64_t b, int64_t t, int64_t s) {
    if (p->mask) return p->mask[(b * p->T + t) * p->S + s] != 0;
    if (p->q_seg && p->q_seg[b * p->T + t] != p->kv_seg[b * p->S + s]) return 0;
    if (s < p->prefix) return 1;
    if (p->causal == 1 && s > t) return 0;
    if (p->causal == 2 && s > t + (p->S - p->T)) return 0;
    if (p->wl >= 0 && s < t - p->wl) return 0;
    if (p->wr >= 0 && s > t + p->wr) return 0;
    return 1;
}

static const uint16_t *q_row(const problem *p, const uint16_t *base, int64_t b, int64_t k, int64_t g, int64_t t) {
    return base + (((b * p->K + k) * p->G + g) * p->T + t) * p->H;
}

static const uint16_t *kv_row(const problem *p, const uint16_t *base, int64_t b, int64_t k, int64_t s) {
    return base + ((b * p->K + k) * p->S + s) * p->H;
}

static acc_t dot_bf(const uint16_t *x, const uint16_t *y, int64_t H) {
    acc_t acc = 0.0;
    for (int64_t h = 0; h < H; h++) acc += bf(x[h]) * bf(y[h]);
    return acc;
}

/* Row statistics of query row (b,k,g,t): max logit m and Z = sum exp(l - m)
 * over visible keys; logits written to l[] (S entries, masked ones unused).
 * Returns the number of visible keys. */
static int64_t row_softmax_stats(const problem *p, int64_t b, int64_t k, int64_t g, int64_t t,
                                 acc_t *l, acc_t *m_out, acc_t *z_out) {
    const uint16_t *qr = q_row(p, p->q, b, k, g, t);
    int64_t nvis = 0;
    acc_t m = -INFINITY;
    for (int64_t s = 0; s < p->S; s++) {
        if (!is_visible(p, b, t, s)) continue;
        l[s] = dot_bf(qr, kv_row(p, p->k, b, k, s), p->H);
        if (l[s] > m) m = l[s];
        nvis++;
    }
    acc_t z = 0.0;
    for (int64_t s = 0; s < p->S; s++)
        if (is_visible(p, b, t, s)) z += ACC_EXP(l[s] - m);
    *m_out = m;
    *z_out = z;
    return nvis;
}

/* Forward for selected query rows. rows[i] is a flat index into [B,K,G,T];
 * rows == NULL means every row in order. o_out: [n, H]; lse_out: [n] (may be NULL). */
int oracle_fwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const int32_t *q_seg, const int32_t *kv_seg, const uint8_t *mask,
                    int64_t B, int64_t K, int64_t G, int64_t T, int64_t S, int64_t H, int causal,
                    int64_t wl, int64_t wr, int64_t prefix,
                    int64_t n_rows, const int64_t *rows, double *o_out, double *lse_out) {
    if (!q || !k || !v || !o_out || B < 1 || K < 1 || G < 1 || T < 1 || S < 1 || H < 1) return 1;
    if ((q_seg == NULL) != (kv_seg == NULL)) return 2;
    if (causal < 0 || causal > 2 || prefix < 0) return 5;
    problem p = {q, k, v, NULL, q_seg, kv_seg, mask, B, K, G, T, S, H, causal, wl, wr, prefix};
    int64_t total = B * K * G * T;
    if (!rows) n_rows = total;
    int err = 0;
#pragma omp parallel
    {
        acc_t *l = (acc_t *)malloc(sizeof(acc_t) * (size_t)(S + H));
        acc_t *oacc = l ? l + S : NULL; /* the row's output accumulators */
        if (!l) {
#pragma omp atomic write
            err = 3;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_rows; i++) {
            if (!l) continue;
            int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= total) {
#pragma omp atomic write
                err = 4;
                continue;
            }
            int64_t t = r % T, g = (r / T) % G, kk = (r / (T * G)) % K, b = r / (T * G * K);
            acc_t m, z;
            double *o = o_out + i * H;
            int64_t nvis = row_softmax_stats(&p, b, kk, g, t, l, &m, &z);
            for (int64_t h = 0; h < H; h++) oacc[h] = 0.0;
            if (nvis == 0) {
                for (int64_t h = 0; h < H; h++) o[h] = 0.0;
                if (lse_out) lse_out[i] = -INFINITY;
                continue;
            }
            for (int64_t s = 0; s < S; s++) {
                if (!is_visible(&p, b, t, s)) continue;
                acc_t w = ACC_EXP(l[s] - m) / z;
                const uint16_t *vr = kv_row(&p, v, b, kk, s);
                for (int64_t h = 0; h < H; h++) oacc[h] += w * bf(vr[h]);
            }
            for (int64_t h = 0; h < H; h++) o[h] = (double)oacc[h];
            if (lse_out) lse_out[i] = (double)(m + ACC_LOG(z));
        }
        free(l);
    }
    return err;
}

/* Per-row statistics needed by the backward for every query row of one
 * (b, kv-head) unit: m, Z and D = sum_s P dP.  Arrays of length G*T. */
static void unit_row_stats(const problem *p, int64_t b, int64_t k, acc_t *m_arr, acc_t *z_arr,
                           acc_t *d_arr, int *err) {
#pragma omp parallel
    {
        acc_t *l = (acc_t *)malloc(sizeof(acc_t) * (size_t)p->S);
        if (!l) {
#pragma omp atomic write
            *err = 3;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < p->G * p->T; r++) {
            if (!l) continue;
            int64_t g = r / p->T, t = r % p->T;
            acc_t m, z;
            int64_t nvis = row_softmax_stats(p, b, k, g, t, l, &m, &z);
            m_arr[r] = m;
            z_arr[r] = z;
            acc_t d = 0.0;
            if (nvis > 0) {
                const uint16_t *dor = q_row(p, p->dout, b, k, g, t);
                for (int64_t s = 0; s < p->S; s++) {
                    if (!is_visible(p, b, t, s)) continue;
                    acc_t w = ACC_EXP(l[s] - m) / z;
                    d += w * dot_bf(dor, kv_row(p, p->v, b, k, s), p->H);
                }
            }
            d_arr[r] = d;
        }
        free(l);
    }
}

/* Backward for selected rows.
 * qrows: flat indices into [B,K,G,T] -> dq_out [n_q, H]
 * kvrows: flat indices into [B,K,S]  -> dk_out, dv_out [n_kv, H]
 * NULL row lists mean every row. d_out (optional, [n_q]) receives D of the qrows. */
int oracle_bwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                    const int32_t *q_seg, const int32_t *kv_seg, const uint8_t *mask,
                    int64_t B, int64_t K, int64_t G, int64_t T, int64_t S, int64_t H, int causal,
                    int64_t wl, int64_t wr, int64_t prefix,
                    int64_t n_q, const int64_t *qrows, double *dq_out, double *d_out,
                    int64_t n_kv, const int64_t *kvrows, double *dk_out, double *dv_out) {
    if (!q || !k || !v || !dout || B < 1 || K < 1 || G < 1 || T < 1 || S < 1 || H < 1) return 1;
    if ((q_seg == NULL) != (kv_seg == NULL)) return 2;
    if (causal < 0 || causal > 2 || prefix < 0) return 5;
    problem p = {q, k, v, dout, q_seg, kv_seg, mask, B, K, G, T, S, H, causal, wl, wr, prefix};
    int64_t nq_total = B * K * G * T, nkv_total = B * K * S;
    if (!qrows) n_q = nq_total;
    if (!kvrows) n_kv = nkv_total;
    int err = 0;
    /* Which (b,k) units are referenced. */
    uint8_t *need = (uint8_t *)calloc((size_t)(B * K), 1);
    if (!need) return 3;
    for (int64_t i = 0; i < n_q; i++) {
        int64_t r = qrows ? qrows[i] : i;
        if (r < 0 || r >= nq_total) { free(need); return 4; }
        need[r / (G * T)] = 1;
    }
    for (int64_t i = 0; i < n_kv; i++) {
        int64_t r = kvrows ? kvrows[i] : i;
        if (r < 0 || r >= nkv_total) { free(need); return 4; }
        need[r / S] = 1;
    }
    size_t gt = (size_t)(G * T);
    acc_t *m_all = (acc_t *)malloc(sizeof(acc_t) * gt * (size_t)(B * K));
    acc_t *z_all = (acc_t *)malloc(sizeof(acc_t) * gt * (size_t)(B * K));
    acc_t *d_all = (acc_t *)malloc(sizeof(acc_t) * gt * (size_t)(B * K));
    if (!m_all || !z_all || !d_all) { free(need); free(m_all); free(z_all); free(d_all); return 3; }
    for (int64_t u = 0; u < B * K; u++)
        if (need[u]) unit_row_stats(&p, u / K, u % K, m_all + u * gt, z_all + u * gt, d_all + u * gt, &err);

    /* dQ rows */
    if (dq_out) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_q; i++) {
            int64_t r = qrows ? qrows[i] : i;
            int64_t t = r % T, g = (r / T) % G, kk = (r / (T * G)) % K, b = r / (T * G * K);
            int64_t u = b * K + kk;
            acc_t m = m_all[u * gt + g * T + t], z = z_all[u * gt + g * T + t];
            acc_t dd = d_all[u * gt + g * T + t];
            double *dq = dq_out + i * H;
            for (int64_t h = 0; h < H; h++) dq[h] = 0.0;
            if (d_out) d_out[i] = (double)dd;
            if (z == 0.0) continue;
            const uint16_t *qr = q_row(&p, q, b, kk, g, t);
            const uint16_t *dor = q_row(&p, dout, b, kk, g, t);
            for (int64_t s = 0; s < S; s++) {
                if (!is_visible(&p, b, t, s)) continue;
                const uint16_t *kr = kv_row(&p, k, b, kk, s);
                acc_t w = ACC_EXP(dot_bf(qr, kr, H) - m) / z;
                acc_t dp = dot_bf(dor, kv_row(&p, v, b, kk, s), H);
                acc_t ds = w * (dp - dd);
                for (int64_t h = 0; h < H; h++) dq[h] += (double)(ds * bf(kr[h]));
            }
        }
    }
    /* dK, dV rows */
    if (dk_out || dv_out) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_kv; i++) {
            int64_t r = kvrows ? kvrows[i] : i;
            int64_t s = r % S, kk = (r / S) % K, b = r / (S * K);
            int64_t u = b * K + kk;
            double *dk = dk_out ? dk_out + i * H : NULL;
            double *dv = dv_out ? dv_out + i * H : NULL;
            for (int64_t h = 0; h < H; h++) {
                if (dk) dk[h] = 0.0;
                if (dv) dv[h] = 0.0;
            }
            const uint16_t *kr = kv_row(&p, k, b, kk, s);
            const uint16_t *vr = kv_row(&p, v, b, kk, s);
            for (int64_t g = 0; g < G; g++) {
                for (int64_t t = 0; t < T; t++) {
                    if (!is_visible(&p, b, t, s)) continue;
                    acc_t z = z_all[u * gt + g * T + t];
                    if (z == 0.0) continue;
                    acc_t m = m_all[u * gt + g * T + t];
                    acc_t dd = d_all[u * gt + g * T + t];
                    const uint16_t *qr = q_row(&p, q, b, kk, g, t);
                    const uint16_t *dor = q_row(&p, dout, b, kk, g, t);
                    acc_t w = ACC_EXP(dot_bf(qr, kr, H) - m) / z;
                    acc_t dp = dot_bf(dor, vr, H);
                    acc_t ds = w * (dp - dd);
                    for (int64_t h = 0; h < H; h++) {
                        if (dk) dk[h] += (double)(ds * bf(qr[h]));
                        if (dv) dv[h] += (double)(w * bf(dor[h]));
                    }
                }
            }
        }
    }
    free(need);
    free(m_all);
    free(z_all);
    free(d_all);
    return err;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
