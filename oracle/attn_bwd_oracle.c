/*
 * Attention-backward oracle -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow, obviously correct CPU computation, in IEEE double
 * precision, of the gradients of exact attention.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load this library;
 * the product path never links it, and no source is shared with the GPU
 * kernels.
 *
 * What it computes.  The forward pass is O = softmax(S) V with
 * S = scale * Q K^T + mask (page "FlashAttention (DE)", systems-analysis.info,
 * section "Problematik der Standard-Attention").  Given the gradient dO of a
 * loss with respect to O, the gradients with respect to Q, K and V follow by
 * the chain rule through that definition, one query row i at a time (P_i is
 * the probability row, materialised in full as in the forward oracle):
 *
 *   dV_j  += P_ij dO_i                      (O_i = sum_j P_ij V_j)
 *   dP_ij  = <dO_i, V_j>
 *   dS_ij  = P_ij (dP_ij - sum_k P_ik dP_ik)   (Jacobian of the softmax row)
 *   dQ_i   = scale * sum_j dS_ij K_j
 *   dK_j  += scale * dS_ij Q_i
 *
 * Masked keys have P_ij = 0 and therefore contribute nothing; a row that
 * sees no key has no gradient.  With grouped-query heads, the gradient of a
 * key/value head sums the contributions of every query head that reads it.
 * The pages say the backward pass recomputes attention from the stored
 * statistics instead of storing P (page "Flash Attention", 21medien.de, key
 * techniques, recomputation); this oracle simply recomputes P from Q and K.
 *
 * Conventions shared with the forward oracle (listed in the design notes):
 * bottom-right causal mask (key j visible to query i iff j <= i + Nk - Nq),
 * query head h reads key/value head floor(h / (Hq / Hkv)), and inputs arrive
 * as bfloat16 bit patterns (decoded exactly) or as doubles.
 *
 * Build: compiled into the same liboracle.so as attn_oracle.c.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { BW_BF16 = 0, BW_F64 = 2 };

static double bw_load(const void* base, int dtype, int64_t idx) {
    if (dtype == BW_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double*)base)[idx];
}

typedef struct {
    const void *q, *k, *v, *dout;
    int dtype;
    int64_t B, Hq, Hkv, Nq, Nk, d;
    int causal;
    double scale;
} bw_problem_t;

static int bw_check(const bw_problem_t* p) {
    if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Nq < 0 || p->Nk < 0 || p->d <= 0) return -1;
    if (p->Hq % p->Hkv != 0) return -1;
    if (p->dtype != BW_BF16 && p->dtype != BW_F64) return -1;
    return 0;
}

/* Scratch for one query row. */
typedef struct {
    double *qrow, *dorow, *prow, *dprow;
} bw_row_t;

static int bw_row_alloc(bw_row_t* r, int64_t d, int64_t Nk) {
    size_t nd = (size_t)(d > 0 ? d : 1), nk = (size_t)(Nk > 0 ? Nk : 1);
    r->qrow = (double*)malloc(sizeof(double) * nd);
    r->dorow = (double*)malloc(sizeof(double) * nd);
    r->prow = (double*)malloc(sizeof(double) * nk);
    r->dprow = (double*)malloc(sizeof(double) * nk);
    return (r->qrow && r->dorow && r->prow && r->dprow) ? 0 : -1;
}

static void bw_row_free(bw_row_t* r) {
    free(r->qrow); free(r->dorow); free(r->prow); free(r->dprow);
}

/*
 * For query row i of head (b, h): P_i (prow), dP_i (dprow), then dS_i in
 * place of dprow.  Returns 0, or 1 when the row sees no key (then dS = 0).
 */
static int bw_row(const bw_problem_t* p, int64_t b, int64_t h, int64_t i, bw_row_t* r) {
    const int64_t d = p->d, Nk = p->Nk;
    const int64_t kvh = h / (p->Hq / p->Hkv);
    const int64_t qoff = ((b * p->Hq + h) * p->Nq + i) * d;
    for (int64_t t = 0; t < d; ++t) {
        r->qrow[t] = bw_load(p->q, p->dtype, qoff + t);
        r->dorow[t] = bw_load(p->dout, p->dtype, qoff + t);
    }
    /* scores, masked keys at -inf */
    double M = -INFINITY;
    for (int64_t j = 0; j < Nk; ++j) {
        if (p->causal && j > i + (Nk - p->Nq)) { r->prow[j] = -INFINITY; continue; }
        const int64_t koff = ((b * p->Hkv + kvh) * Nk + j) * d;
        double dot = 0.0;
        for (int64_t t = 0; t < d; ++t) dot += r->qrow[t] * bw_load(p->k, p->dtype, koff + t);
        r->prow[j] = p->scale * dot;
        if (r->prow[j] > M) M = r->prow[j];
    }
    if (M == -INFINITY) {
        for (int64_t j = 0; j < Nk; ++j) { r->prow[j] = 0.0; r->dprow[j] = 0.0; }
        return 1;
    }
    /* the softmax row */
    double L = 0.0;
    for (int64_t j = 0; j < Nk; ++j) { r->prow[j] = exp(r->prow[j] - M); L += r->prow[j]; }
    for (int64_t j = 0; j < Nk; ++j) r->prow[j] /= L;
    /* dP_ij = <dO_i, V_j> for the keys the row sees */
    for (int64_t j = 0; j < Nk; ++j) {
        if (r->prow[j] == 0.0) { r->dprow[j] = 0.0; continue; }
        const int64_t voff = ((b * p->Hkv + kvh) * Nk + j) * d;
        double dot = 0.0;
        for (int64_t t = 0; t < d; ++t) dot += r->dorow[t] * bw_load(p->v, p->dtype, voff + t);
        r->dprow[j] = dot;
    }
    /* softmax Jacobian: dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik) */
    double Dsum = 0.0;
    for (int64_t j = 0; j < Nk; ++j) Dsum += r->prow[j] * r->dprow[j];
    for (int64_t j = 0; j < Nk; ++j) r->dprow[j] = r->prow[j] * (r->dprow[j] - Dsum);
    return 0;
}

/*
 * Full gradients: dq [B,Hq,Nq,d], dk and dv [B,Hkv,Nk,d], all doubles, all
 * overwritten.  Parallel over (batch, key/value head): one thread owns the
 * dk and dv rows of its head and the dq rows of the query heads reading it.
 * Returns 0, or -1 on invalid sizes or allocation failure.
 */
int oracle_attention_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                         int causal, double scale, double* dq, double* dk, double* dv) {
    bw_problem_t p = {q, k, v, dout, dtype, B, Hq, Hkv, Nq, Nk, d, causal, scale};
    if (bw_check(&p) != 0) return -1;
    memset(dq, 0, sizeof(double) * (size_t)(B * Hq * Nq * d));
    memset(dk, 0, sizeof(double) * (size_t)(B * Hkv * Nk * d));
    memset(dv, 0, sizeof(double) * (size_t)(B * Hkv * Nk * d));
    const int64_t G = Hq / Hkv;
    int failed = 0;
#pragma omp parallel
    {
        bw_row_t r;
        if (bw_row_alloc(&r, d, Nk) != 0) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bk = 0; bk < B * Hkv; ++bk) {
                const int64_t b = bk / Hkv, kvh = bk % Hkv;
                for (int64_t h = kvh * G; h < (kvh + 1) * G; ++h)
                    for (int64_t i = 0; i < Nq; ++i) {
                        if (bw_row(&p, b, h, i, &r) != 0) continue;
                        double* dqi = dq + ((b * Hq + h) * Nq + i) * d;
                        for (int64_t j = 0; j < Nk; ++j) {
                            const double ds = r.dprow[j], pj = r.prow[j];
                            if (pj == 0.0) continue;
                            const int64_t koff = ((b * Hkv + kvh) * Nk + j) * d;
                            for (int64_t t = 0; t < d; ++t) {
                                dqi[t] += scale * ds * bw_load(k, dtype, koff + t);
                                dk[koff + t] += scale * ds * r.qrow[t];
                                dv[koff + t] += pj * r.dorow[t];
                            }
                        }
                    }
            }
        }
        bw_row_free(&r);
    }
    return failed ? -1 : 0;
}

/*
 * dQ of the listed query rows only (flat index (b*Hq + h)*Nq + i), n x d
 * doubles in the order of `rows`.  Row-local, so it scales to any size.
 */
int oracle_bwd_dq_rows(const void* q, const void* k, const void* v, const void* dout, int dtype,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                       int causal, double scale, const int64_t* rows, int64_t n_rows, double* dq) {
    bw_problem_t p = {q, k, v, dout, dtype, B, Hq, Hkv, Nq, Nk, d, causal, scale};
    if (bw_check(&p) != 0 || n_rows < 0) return -1;
    const int64_t total = B * Hq * Nq;
    for (int64_t x = 0; x < n_rows; ++x)
        if (rows[x] < 0 || rows[x] >= total) return -1;
    int failed = 0;
#pragma omp parallel
    {
        bw_row_t r;
        if (bw_row_alloc(&r, d, Nk) != 0) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t x = 0; x < n_rows; ++x) {
                const int64_t row = rows[x];
                const int64_t i = row % Nq, h = (row / Nq) % Hq, b = row / (Nq * Hq);
                const int64_t kvh = h / (Hq / Hkv);
                double* out = dq + x * d;
                for (int64_t t = 0; t < d; ++t) out[t] = 0.0;
                if (bw_row(&p, b, h, i, &r) != 0) continue;
                for (int64_t j = 0; j < Nk; ++j) {
                    if (r.prow[j] == 0.0) continue;
                    const int64_t koff = ((b * Hkv + kvh) * Nk + j) * d;
                    for (int64_t t = 0; t < d; ++t) out[t] += scale * r.dprow[j] * bw_load(k, dtype, koff + t);
                }
            }
        }
        bw_row_free(&r);
    }
    return failed ? -1 : 0;
}
