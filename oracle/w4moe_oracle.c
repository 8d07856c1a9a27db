/*
 * Plain CPU oracle of the W4A16 SwiGLU Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE, NOT THE PRODUCT. Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load or run this. It shares no code, header, table or helper with the HIP
 * path, and the HIP path never calls it.
 *
 * What it computes is the textbook sparsely-gated MoE layer with SwiGLU experts whose weights are
 * signed INT4 codes (or INT8 codes, the pages' repack taking the bit width as a parameter) with one
 * bf16 scale per group of consecutive values of the reduction dimension:
 *   - "The Pivot to Real Hardware: Diagnosing Throughput and Building the INT4 MoE Benchmark for
 *     Kimi K2.6", Step 1 (Understanding the Weight Format): eight 4-bit codes to each 32-bit word in
 *     the logical GPTQ layout; w1 holds the gate and the up projection side by side; w2 is the down
 *     projection; one scale for every 32 consecutive values of the reduction dimension.
 *   - same page, Input Knowledge Required, item 1 and "The Weight-Streaming Threshold", Input
 *     Knowledge Required (Mixture-of-Experts architecture): 384 experts, top-8 routing, SwiGLU MLP.
 * Readings taken where the pages are silent (each one is listed with its reason in the design notes):
 *   code c of a word is the signed value c - 8 (offset binary); value t of a word (t = 0..7) sits in
 *   bits 4t..4t+3; words pack 8 consecutive rows of the reduction dimension (with 8-bit codes: value
 *   c - 128, value t = 0..3 in bits 8t..8t+7, 4 rows per word); scales group the
 *   reduction dimension (hidden for w1, intermediate for w2); no zero points; w1 columns [0, N) are
 *   the gate and [N, 2N) the up projection; act = SiLU(gate) * up with SiLU(z) = z / (1 + e^-z);
 *   the routing weight multiplies each expert's output in the combine.
 * Activation order (the repack's `perm` argument, same page, Step 2: The Repack Pipeline, empty
 * for K2.6): GPTQ then records the group of every reduction row (its g_idx) instead of grouping
 * consecutive rows; row r of an expert matrix is dequantised with the scale row g_idx[r]. The
 * oracle takes that index as given and needs no permutation.
 *
 * Precision: dequantisation in fp32 (q * s is exact in fp32), every sum and the activation in fp64,
 * no intermediate rounding. The align routine is integer-exact.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t E, K, N, topk, group, bits;
} w4o_dims;

static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Signed code of element (r, c) of a matrix stored as int32 words [R*bits/32][cols] (bits 4 or 8). */
int w4o_code(const int32_t *wq, int32_t cols, int32_t bits, int32_t r, int32_t c) {
    const int32_t per = 32 / bits;
    uint32_t word = (uint32_t)wq[(size_t)(r / per) * (size_t)cols + (size_t)c];
    const uint32_t mask = (1u << bits) - 1u;
    return (int)((word >> (bits * (r % per))) & mask) - (int)(1u << (bits - 1));
}

/* Dequantised weight (r, c) with the scales of row srow: fp32(code) * fp32(scale) (exact in fp32:
 * an 8-bit code times an 8-bit-mantissa scale needs at most 16 significant bits). */
float w4o_dequant_row(const int32_t *wq, const uint16_t *sc, int32_t cols, int32_t bits, int32_t srow, int32_t r,
                      int32_t c) {
    float s = bf16_to_f32(sc[(size_t)srow * (size_t)cols + (size_t)c]);
    return (float)w4o_code(wq, cols, bits, r, c) * s;
}

/* Dequantised weight (r, c) of consecutive groups: the scale row is r / group. */
float w4o_dequant(const int32_t *wq, const uint16_t *sc, int32_t cols, int32_t bits, int32_t group, int32_t r,
                  int32_t c) {
    return w4o_dequant_row(wq, sc, cols, bits, r / group, r, c);
}

/* Scale row of reduction row r: its recorded group (activation order) or r / group. */
static int32_t group_of(const int32_t *gidx, int32_t group, int32_t r) { return gidx ? gidx[r] : r / group; }

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * One routed (token, expert) pair: y = down(SiLU(gate(x)) * up(x)), all in fp64.
 * g1 [K] and g2 [N] are the group indices of the reduction rows of w1 and w2 (activation order), or
 * NULL for consecutive groups. h is scratch of 2N doubles, y receives K doubles.
 */
void w4o_expert_ffn(const w4o_dims *d, const uint16_t *xrow, const int32_t *w1, const uint16_t *s1,
                    const int32_t *w2, const uint16_t *s2, const int32_t *g1, const int32_t *g2, double *h,
                    double *y) {
    const int32_t K = d->K, N = d->N, C1 = 2 * d->N, g = d->group, b = d->bits;
    for (int32_t c = 0; c < C1; ++c) h[c] = 0.0;
    /* h[c] = sum_r x[r] * W1[r][c] */
    for (int32_t r = 0; r < K; ++r) {
        const double xr = (double)bf16_to_f32(xrow[r]);
        const int32_t sr = group_of(g1, g, r);
        for (int32_t c = 0; c < C1; ++c) h[c] += xr * (double)w4o_dequant_row(w1, s1, C1, b, sr, r, c);
    }
    /* a[n] = SiLU(h[n]) * h[N + n], kept in h[0..N) */
    for (int32_t n = 0; n < N; ++n) h[n] = silu(h[n]) * h[N + n];
    /* y[c] = sum_n a[n] * W2[n][c] */
    for (int32_t c = 0; c < K; ++c) y[c] = 0.0;
    for (int32_t n = 0; n < N; ++n) {
        const double an = h[n];
        const int32_t sr = group_of(g2, g, n);
        for (int32_t c = 0; c < K; ++c) y[c] += an * (double)w4o_dequant_row(w2, s2, K, b, sr, n, c);
    }
}

/* 1 when every entry of gidx [R] names one of the R / group scale rows. */
static int groups_valid(const int32_t *gidx, int32_t R, int32_t group) {
    if (!gidx) return 1;
    for (int32_t r = 0; r < R; ++r)
        if (gidx[r] < 0 || gidx[r] >= R / group) return 0;
    return 1;
}

/*
 * Layer output for the token rows listed in `rows` (all M tokens when rows == NULL, n_rows = M):
 *   out[i][c] = sum_j topk_w[m][j] * expert_{ids[m][j]}(x[m])[c]   with m = rows[i], j in order.
 * Expert weights come as per-expert pointer arrays (NULL for experts that are not needed); g1 and g2
 * are per-expert group indices of activation-ordered weights (the arrays, or an entry, NULL for
 * consecutive groups).
 * Returns 0, or -1 (bad dims), -2 (id outside [0, E)), -3 (routed expert without weights),
 * -4 (out of memory), -6 (a group index outside [0, R / group)).
 */
int w4o_moe_forward(const w4o_dims *d, int32_t M, const uint16_t *x, const int32_t *ids, const float *topk_w,
                    const int32_t *const *w1, const uint16_t *const *s1, const int32_t *const *w2,
                    const uint16_t *const *s2, const int32_t *const *g1, const int32_t *const *g2, int32_t n_rows,
                    const int32_t *rows, double *out, int32_t nthreads) {
    if (d->E <= 0 || d->K <= 0 || d->N <= 0 || d->topk <= 0 || d->group <= 0 || (d->bits != 4 && d->bits != 8) ||
        d->K % 8 || d->N % 8 || d->K % d->group || d->N % d->group || M < 0 || n_rows < 0)
        return -1;
    const int32_t K = d->K, k = d->topk;
    for (int32_t i = 0; i < n_rows; ++i) {
        const int32_t m = rows ? rows[i] : i;
        if (m < 0 || m >= M) return -1;
        for (int32_t j = 0; j < k; ++j) {
            const int32_t e = ids[(size_t)m * k + j];
            if (e < 0 || e >= d->E) return -2;
            if (!w1[e] || !s1[e] || !w2[e] || !s2[e]) return -3;
            if (!groups_valid(g1 ? g1[e] : NULL, d->K, d->group) || !groups_valid(g2 ? g2[e] : NULL, d->N, d->group))
                return -6;
        }
    }
    const size_t npairs = (size_t)n_rows * (size_t)k;
    double *ys = (double *)malloc(npairs * (size_t)K * sizeof(double));
    if (!ys && npairs) return -4;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *h = (double *)malloc((size_t)2 * d->N * sizeof(double));
        if (!h) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long long pr = 0; pr < (long long)npairs; ++pr) {
            if (!h) continue;
            const int32_t i = (int32_t)(pr / k), j = (int32_t)(pr % k);
            const int32_t m = rows ? rows[i] : i;
            const int32_t e = ids[(size_t)m * k + j];
            w4o_expert_ffn(d, x + (size_t)m * K, w1[e], s1[e], w2[e], s2[e], g1 ? g1[e] : NULL, g2 ? g2[e] : NULL, h,
                           ys + (size_t)pr * K);
        }
        free(h);
    }
    if (failed) {
        free(ys);
        return -4;
    }
    /* combine in slot order */
    for (int32_t i = 0; i < n_rows; ++i) {
        const int32_t m = rows ? rows[i] : i;
        double *o = out + (size_t)i * K;
        for (int32_t c = 0; c < K; ++c) o[c] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            const double wj = (double)topk_w[(size_t)m * k + j];
            const double *y = ys + ((size_t)i * k + j) * K;
            for (int32_t c = 0; c < K; ++c) o[c] += wj * y[c];
        }
    }
    free(ys);
    return 0;
}

/*
 * Token-to-expert alignment of the T = M * topk flat routing entries (flat id f = m * topk + j):
 *   counts[e]      = number of f with ids[f] == e
 *   offsets[0] = 0, offsets[e + 1] = offsets[e] + B * ceil(counts[e] / B)
 *   sorted_ids[offsets[e] + r] = the r-th smallest f with ids[f] == e (r < counts[e]);
 *                               the rest of [offsets[e], offsets[e + 1]) holds the sentinel T
 *   block_expert[b] = e for every block b of B rows in [offsets[e], offsets[e + 1])
 *   active         = the experts with counts > 0, ascending; *n_active their number
 * Returns offsets[E] (the padded row count), or -1 (bad arguments), -2 (id outside [0, E)),
 * -5 (an output capacity is too small).
 */
int32_t w4o_moe_align(int32_t T, int32_t E, int32_t B, const int32_t *flat_ids, int32_t *counts, int32_t *offsets,
                      int32_t *sorted_ids, int32_t sorted_cap, int32_t *block_expert, int32_t block_cap,
                      int32_t *active, int32_t *n_active) {
    if (T < 0 || E <= 0 || B <= 0) return -1;
    for (int32_t f = 0; f < T; ++f)
        if (flat_ids[f] < 0 || flat_ids[f] >= E) return -2;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int32_t f = 0; f < T; ++f) counts[flat_ids[f]] += 1;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + B * ((counts[e] + B - 1) / B);
    const int32_t P = offsets[E];
    if (P > sorted_cap || P / B > block_cap) return -5;
    for (int32_t p = 0; p < P; ++p) sorted_ids[p] = T;
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!fill) return -1;
    for (int32_t f = 0; f < T; ++f) {
        const int32_t e = flat_ids[f];
        sorted_ids[offsets[e] + fill[e]] = f;
        fill[e] += 1;
    }
    free(fill);
    for (int32_t e = 0; e < E; ++e)
        for (int32_t b = offsets[e] / B; b < offsets[e + 1] / B; ++b) block_expert[b] = e;
    int32_t na = 0;
    for (int32_t e = 0; e < E; ++e)
        if (counts[e] > 0) active[na++] = e;
    *n_active = na;
    return P;
}
