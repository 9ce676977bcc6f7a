/*
 * TEST INFRASTRUCTURE ONLY.  fp64 reference for joint multi-stream attention.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this library.  It shares no source with the HIP path.
 *
 * What it computes.  The everytik.com translation of NVIDIA's "FLUX 3 Image Klein in
 * TensorRT LLM VisualGen" article (section 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理)
 * says the text, noisy-target and optional reference-image streams are processed apart
 * and combined only through one joint attention; its section 量化注意力与稀疏注意力 names
 * that attention as the dominant cost at 2048x2048 but prints no formula.  The plainest
 * reading, used here, is unmasked scaled-dot-product softmax attention over the packed
 * sequence:
 *
 *   for one batch b, head h and query row i
 *     s_j  = scale * sum_c q[i][c] * k[j][c]        for every key j in 0..N-1
 *     m    = max_j s_j
 *     w_j  = exp(s_j - m)
 *     l    = sum_j w_j
 *     o[c] = (sum_j w_j * v[j][c]) / l
 *     lse  = m + ln(l)
 *
 * Two plain passes per row in double precision; no tiling, no online softmax.
 * Inputs are token-major (the layout of the concatenated streams): queries [B, Nq, H, D],
 * keys and values [B, N, H, D] (Nq == N for self-attention), given either as bf16 bit
 * patterns (widened exactly to double) or as doubles.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F64 = 0, ORACLE_BF16 = 1 };

/* bf16 is the top half of an IEEE binary32; widening to double is exact. */
static double load_elem(const void *base, int kind, int64_t idx) {
    if (kind == ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double *)base)[idx];
}

/* One query row of one (b, h): writes o[0..D-1] and *lse_out.  s has room for N doubles. */
static void attend_row(const void *q, const void *k, const void *v, int kind,
                       int64_t Nq, int64_t N, int64_t H, int64_t D, double scale,
                       int64_t b, int64_t h, int64_t i,
                       double *qrow, double *s, double *o, double *lse_out) {
    const int64_t row_stride = H * D;             /* between consecutive tokens */
    const int64_t base_bh = b * N * row_stride + h * D;
    const int64_t q_at = (b * Nq + i) * row_stride + h * D;

    for (int64_t c = 0; c < D; ++c)
        qrow[c] = load_elem(q, kind, q_at + c);

    /* pass 1: logits and their maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
        double dot = 0.0;
        const int64_t kj = base_bh + j * row_stride;
        for (int64_t c = 0; c < D; ++c)
            dot += qrow[c] * load_elem(k, kind, kj + c);
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }

    /* pass 2: weights, their sum, and the weighted sum of values */
    double l = 0.0;
    for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        const double w = exp(s[j] - m);
        l += w;
        const int64_t vj = base_bh + j * row_stride;
        for (int64_t c = 0; c < D; ++c)
            o[c] += w * load_elem(v, kind, vj + c);
    }
    for (int64_t c = 0; c < D; ++c) o[c] /= l;
    *lse_out = m + log(l);
}

/*
 * Selected rows.  sel holds n_sel triples (b, h, i) with i < Nq; out is [n_sel, D],
 * lse is [n_sel].  Returns 0 on success, 1 on a bad argument, 2 when scratch memory
 * is unavailable.
 */
int oracle_attention_rows(const void *q, const void *k, const void *v, int kind,
                          int64_t B, int64_t Nq, int64_t N, int64_t H, int64_t D,
                          double scale, const int64_t *sel, int64_t n_sel, double *out,
                          double *lse, int n_threads) {
    if (!q || !k || !v || !sel || !out || !lse) return 1;
    if (B <= 0 || Nq <= 0 || N <= 0 || H <= 0 || D <= 0 || n_sel < 0) return 1;
    if (kind != ORACLE_F64 && kind != ORACLE_BF16) return 1;
    for (int64_t r = 0; r < n_sel; ++r) {
        const int64_t b = sel[3 * r], h = sel[3 * r + 1], i = sel[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Nq) return 1;
    }
    if (n_threads < 1) n_threads = 1;

    int failed = 0;
#pragma omp parallel num_threads(n_threads)
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *qrow = (double *)malloc((size_t)D * sizeof(double));
        if (!s || !qrow) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_sel; ++r) {
            if (!s || !qrow) continue;
            attend_row(q, k, v, kind, Nq, N, H, D, scale, sel[3 * r], sel[3 * r + 1],
                       sel[3 * r + 2], qrow, s, out + r * D, lse + r);
        }
        free(s);
        free(qrow);
    }
    return failed ? 2 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
