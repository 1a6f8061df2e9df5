/*
 * Exact-attention oracle -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow, obviously correct CPU implementation of scaled-dot-product
 * attention in IEEE double precision.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library; the product
 * path (the HIP library) never links it, and this file shares no source with
 * the GPU kernels.
 *
 * What it computes (page "FlashAttention (DE)", systems-analysis.info,
 * section "Problematik der Standard-Attention", the attention formula):
 *
 *     O = softmax(scale * Q K^T + mask) V,   scale = 1/sqrt(d) by convention,
 *
 * one query row at a time: the row of scores S and the row of probabilities
 * P are materialised in full (Nk doubles each), exactly as the "standard"
 * attention those pages describe, and the per-row log-sum-exp
 * LSE = max_j s_j + ln sum_j exp(s_j - max_j s_j) is returned next to O.
 *
 * Readings of points the pages leave open (each is listed in the design
 * notes of the repository):
 *   - causal masking is aligned to the bottom-right corner: key j is visible
 *     to query i iff j <= i + (Nk - Nq); for Nq == Nk that is j <= i;
 *   - a row that sees no key has O = 0 and LSE = -inf;
 *   - grouped-query heads: query head h reads key/value head
 *     floor(h / (Hq / Hkv)) (page "Flash Attention", 21medien.de, list of
 *     key techniques: multi-query / grouped-query attention; page
 *     "FlashAttention 4" on centron.de, compatibility section: several
 *     query heads share one key/value projection);
 *   - inputs arrive as the exact bytes the GPU receives: bfloat16 bit
 *     patterns (upper half of an IEEE binary32), OCP FP8 E4M3 codes with a
 *     per-tensor scale, or doubles (hand-made cases).  Each element is
 *     decoded to double exactly, by this file's own decoders.
 *
 * The tiled variant (oracle_attn_tiled) follows page "FlashAttention (DE)",
 * section "Online-Softmax-Berechnung": a running maximum and a running sum of
 * exponentials per query row, updated block by block, give the exact result
 * without the full row.  It is used only to pin the recurrence against the
 * naive definition in the test suite.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math: IEEE semantics).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_E4M3 = 1, ORACLE_F64 = 2 };

/* bfloat16 is the upper 16 bits of an IEEE-754 binary32; widening puts the
 * 16 bits back on top of 16 zero bits, which is exact. */
double oracle_bf16_to_f64(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 flavour: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals when the exponent field is 0, no
 * infinities, and S.1111.111 is NaN.  Largest finite magnitude 448. */
double oracle_e4m3_to_f64(uint8_t c) {
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - 7);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

static double load_elem(const void* base, int dtype, int64_t idx, double descale) {
    switch (dtype) {
        case ORACLE_BF16: return oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
        case ORACLE_E4M3: return oracle_e4m3_to_f64(((const uint8_t*)base)[idx]) * descale;
        default: return ((const double*)base)[idx];
    }
}

typedef struct {
    const void *q, *k, *v;
    int dtype;
    double dq, dk, dv;
    int64_t B, Hq, Hkv, Nq, Nk, d;
    int causal;
    double scale;
} problem_t;

/* Key j is visible to query i (bottom-right aligned causal mask). */
static int visible(const problem_t* p, int64_t i, int64_t j) {
    return !p->causal || j <= i + (p->Nk - p->Nq);
}

/* The row of scores s_j = scale * <q_i, k_j> for every key j, -inf where the
 * mask hides the key.  qrow receives the decoded query row. */
static void score_row(const problem_t* p, int64_t b, int64_t h, int64_t i,
                      double* qrow, double* s) {
    int64_t kvh = h / (p->Hq / p->Hkv);
    int64_t qoff = ((b * p->Hq + h) * p->Nq + i) * p->d;
    for (int64_t t = 0; t < p->d; ++t) qrow[t] = load_elem(p->q, p->dtype, qoff + t, p->dq);
    for (int64_t j = 0; j < p->Nk; ++j) {
        if (!visible(p, i, j)) { s[j] = -INFINITY; continue; }
        int64_t koff = ((b * p->Hkv + kvh) * p->Nk + j) * p->d;
        double dot = 0.0;
        for (int64_t t = 0; t < p->d; ++t) dot += qrow[t] * load_elem(p->k, p->dtype, koff + t, p->dk);
        s[j] = p->scale * dot;
    }
}

/* Naive attention for one row: materialise S and P, then O = P V. */
static void naive_row(const problem_t* p, int64_t r, double* qrow, double* s,
                      double* o, double* lse) {
    int64_t i = r % p->Nq;
    int64_t h = (r / p->Nq) % p->Hq;
    int64_t b = r / (p->Nq * p->Hq);
    int64_t kvh = h / (p->Hq / p->Hkv);
    score_row(p, b, h, i, qrow, s);
    double M = -INFINITY;
    for (int64_t j = 0; j < p->Nk; ++j) if (s[j] > M) M = s[j];
    if (M == -INFINITY) {           /* no visible key */
        for (int64_t t = 0; t < p->d; ++t) o[t] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double L = 0.0;
    for (int64_t j = 0; j < p->Nk; ++j) { s[j] = exp(s[j] - M); L += s[j]; }  /* s now holds p_j */
    for (int64_t j = 0; j < p->Nk; ++j) s[j] /= L;                          /* s now holds P_j */
    for (int64_t t = 0; t < p->d; ++t) o[t] = 0.0;
    for (int64_t j = 0; j < p->Nk; ++j) {
        if (s[j] == 0.0) continue;
        int64_t voff = ((b * p->Hkv + kvh) * p->Nk + j) * p->d;
        for (int64_t t = 0; t < p->d; ++t) o[t] += s[j] * load_elem(p->v, p->dtype, voff + t, p->dv);
    }
    *lse = M + log(L);
}

/* Online-softmax recurrence over key blocks of Bc keys, for one row. */
static void tiled_row(const problem_t* p, int64_t r, int64_t Bc, double* qrow,
                      double* s, double* o, double* lse) {
    int64_t i = r % p->Nq;
    int64_t h = (r / p->Nq) % p->Hq;
    int64_t b = r / (p->Nq * p->Hq);
    int64_t kvh = h / (p->Hq / p->Hkv);
    score_row(p, b, h, i, qrow, s);   /* scores of all keys; only read block by block below */
    double m = -INFINITY, l = 0.0;
    for (int64_t t = 0; t < p->d; ++t) o[t] = 0.0;
    for (int64_t j0 = 0; j0 < p->Nk; j0 += Bc) {
        int64_t j1 = j0 + Bc < p->Nk ? j0 + Bc : p->Nk;
        double mb = -INFINITY;
        for (int64_t j = j0; j < j1; ++j) if (s[j] > mb) mb = s[j];
        double mnew = m > mb ? m : mb;
        if (mnew == -INFINITY) continue;              /* nothing visible yet */
        double alpha = exp(m - mnew);                 /* 0 when m == -inf */
        l *= alpha;
        for (int64_t t = 0; t < p->d; ++t) o[t] *= alpha;
        for (int64_t j = j0; j < j1; ++j) {
            double e = exp(s[j] - mnew);
            if (e == 0.0) continue;
            l += e;
            int64_t voff = ((b * p->Hkv + kvh) * p->Nk + j) * p->d;
            for (int64_t t = 0; t < p->d; ++t) o[t] += e * load_elem(p->v, p->dtype, voff + t, p->dv);
        }
        m = mnew;
    }
    if (l == 0.0) {
        for (int64_t t = 0; t < p->d; ++t) o[t] = 0.0;
        *lse = -INFINITY;
        return;
    }
    for (int64_t t = 0; t < p->d; ++t) o[t] /= l;
    *lse = m + log(l);
}

static int check_problem(const problem_t* p) {
    if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Nq < 0 || p->Nk < 0 || p->d <= 0) return -1;
    if (p->Hq % p->Hkv != 0) return -1;
    if (p->dtype < ORACLE_BF16 || p->dtype > ORACLE_F64) return -1;
    return 0;
}

/*
 * Attention over the rows listed in `rows` (flat index r = (b*Hq + h)*Nq + i),
 * or over every row when rows == NULL.  o receives n x d doubles and lse n
 * doubles, in the order of `rows` (or row-major [B,Hq,Nq] when rows == NULL).
 * block_keys == 0 selects the naive, row-materialising definition; a positive
 * value selects the tiled online-softmax recurrence with that block size.
 * descale points at {dq, dk, dv} for E4M3 inputs and is ignored otherwise.
 * Returns 0, or -1 on invalid sizes.
 */
int oracle_attention(const void* q, const void* k, const void* v, int dtype,
                     const double* descale, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                     const int64_t* rows, int64_t n_rows, int64_t block_keys,
                     double* o, double* lse) {
    problem_t p = {q, k, v, dtype, 1.0, 1.0, 1.0, B, Hq, Hkv, Nq, Nk, d, causal, scale};
    if (check_problem(&p) != 0 || block_keys < 0) return -1;
    if (dtype == ORACLE_E4M3) {
        if (!descale) return -1;
        p.dq = descale[0]; p.dk = descale[1]; p.dv = descale[2];
    }
    int64_t total = B * Hq * Nq;
    int64_t n = rows ? n_rows : total;
    if (rows)
        for (int64_t x = 0; x < n; ++x)
            if (rows[x] < 0 || rows[x] >= total) return -1;
    int failed = 0;
#pragma omp parallel
    {
        double* qrow = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!qrow || !s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t x = 0; x < n; ++x) {
                int64_t r = rows ? rows[x] : x;
                if (block_keys == 0)
                    naive_row(&p, r, qrow, s, o + x * d, lse + x);
                else
                    tiled_row(&p, r, block_keys, qrow, s, o + x * d, lse + x);
            }
        }
        free(qrow);
        free(s);
    }
    return failed ? -1 : 0;
}

/*
 * The probability row P[i, :] (Nk doubles) of query row r, as materialised by
 * the naive definition; masked keys get exactly 0.  Returns 0, -1 on invalid
 * input, 1 when the row sees no key (p is then all zeros).
 */
int oracle_probs_row(const void* q, const void* k, const void* v, int dtype,
                     const double* descale, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                     int64_t r, double* prow) {
    problem_t p = {q, k, v, dtype, 1.0, 1.0, 1.0, B, Hq, Hkv, Nq, Nk, d, causal, scale};
    if (check_problem(&p) != 0 || r < 0 || r >= B * Hq * Nq) return -1;
    if (dtype == ORACLE_E4M3) {
        if (!descale) return -1;
        p.dq = descale[0]; p.dk = descale[1]; p.dv = descale[2];
    }
    int64_t i = r % Nq, h = (r / Nq) % Hq, b = r / (Nq * Hq);
    double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
    if (!qrow) return -1;
    score_row(&p, b, h, i, qrow, prow);
    free(qrow);
    double M = -INFINITY;
    for (int64_t j = 0; j < Nk; ++j) if (prow[j] > M) M = prow[j];
    if (M == -INFINITY) {
        for (int64_t j = 0; j < Nk; ++j) prow[j] = 0.0;
        return 1;
    }
    double L = 0.0;
    for (int64_t j = 0; j < Nk; ++j) { prow[j] = exp(prow[j] - M); L += prow[j]; }
    for (int64_t j = 0; j < Nk; ++j) prow[j] /= L;
    return 0;
}

/* Element-wise decoders exposed for the codec pins. */
void oracle_decode(const void* src, int dtype, double descale, int64_t n, double* dst) {
    for (int64_t x = 0; x < n; ++x) dst[x] = load_elem(src, dtype, x, descale);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
