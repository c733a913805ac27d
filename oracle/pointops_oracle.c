/*
 * pointops oracle: the plain CPU definition of dense, batched float32
 * point-cloud neighbour search (farthest point sampling, k nearest neighbours,
 * first-K Ball Query).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU library never calls it and
 * shares no code with it: this file includes none of the GPU sources and they
 * include nothing from here.
 *
 * Every function is written straight from the definitions on two pages:
 *   [P1] "mps-pointops" project page (PyPI, version 0.5.0):
 *        section "The operators in equations" (the shared squared distance,
 *        "Farthest point sampling", "k nearest neighbors",
 *        "Ball Query: first K within a radius"), section "How the kernels
 *        work" (FMA contraction off, sum ((dx^2 + dy^2) + dz^2)) and section
 *        "Contracts" (start index, repeat-0 rule, k <= N).
 *   [P2] "Numerical contracts" page, section "Selection and output"
 *        (r32 = fl32(r), R2 = fl32(r32 * r32), strict s32 < R2, exact ties to
 *        the smaller index, zero distance can be a real match).
 *
 * Arithmetic: float32 for the selections (the pages fix it), each
 * operation rounded to nearest-even, no fused multiply-add, denormals kept.
 * The Ball Query backward, whose precision the pages leave open, is float64.
 * The nearest-point selection of the Chamfer distance is here too; its
 * reductions and gradients are float64 numpy code in oracle/__init__.py. Build with -O2 -ffp-contract=off and
 * never with -ffast-math; the preprocessor checks below refuse builds that
 * would evaluate in a wider type or with fast-math.
 *
 * Parity pins (what fixes this code other than itself) live in the test suite:
 * the pages' worked example, exact integer/dyadic brute force in float64,
 * exact-rational per-step rounding of s32, the bisection closed form of FPS on
 * a line, invariants, and for the backward central differences of the
 * quadratic loss. Non-finite inputs are outside the contract and their results
 * are "parity unpinned".
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs every float expression evaluated in float32 (FLT_EVAL_METHOD == 0)"
#endif
#ifdef __FAST_MATH__
#error "the oracle must not be built with -ffast-math"
#endif
#ifdef __FP_FAST_FMAF
#error "the oracle must be built without a fused float multiply-add (no -mfma / -march=native)"
#endif

enum {
    PCO_OK = 0,
    PCO_INVALID_ARGUMENT = 1,
    PCO_OUT_OF_MEMORY = 5,
};

/* Squared distance s32(a, b) = ((dx*dx + dy*dy) + dz*dz), dx = fl32(a.x - b.x).
 * [P1] "The operators in equations": s_ij = sum over d of (q_id - x_jd)^2;
 * [P1] "How the kernels work": that sum is taken as ((dx^2 + dy^2) + dz^2)
 * without contraction. Each line below is one rounded float32 operation. */
float pco_s32(const float *a, const float *b)
{
    float dx = a[0] - b[0];
    float dy = a[1] - b[1];
    float dz = a[2] - b[2];
    float sx = dx * dx;
    float sy = dy * dy;
    float sz = dz * dz;
    float sxy = sx + sy;
    return sxy + sz;
}

/* Dense Ball Query threshold R2 = fl32(r32 * r32), r32 = fl32(r).
 * [P1] "Ball Query: first K within a radius"; [P2] "Selection and output".
 * The argument already is r32 (the caller rounds its radius to float32). */
float pco_ball_query_r2(float r32)
{
    float r2 = r32 * r32;
    return r2;
}

/* Farthest point sampling, one cloud at a time.
 * [P1] "Farthest point sampling": c_0 = start_idx;
 *   m_j^(t) = min over u <= t of s(x_j, x_{c_u});
 *   c_{t+1} = the smallest j whose m_j^(t) equals the largest m^(t).
 * [P1] "Contracts": once every point is taken the remaining slots repeat
 * index 0 (this falls out of the rule: every m is then 0 and the smallest
 * index wins). Out: (B, M) int64. */
int pco_fps(const float *xyz, int64_t B, int64_t N, int64_t M, int64_t start_idx,
            int64_t *out)
{
    if (B < 0 || N < 0 || M < 0)
        return PCO_INVALID_ARGUMENT;
    if (B == 0 || M == 0)
        return PCO_OK;
    if (N == 0 || start_idx < 0 || start_idx >= N)
        return PCO_INVALID_ARGUMENT;
    float *m = (float *)malloc((size_t)N * sizeof(float));
    if (!m)
        return PCO_OUT_OF_MEMORY;
    for (int64_t b = 0; b < B; ++b) {
        const float *x = xyz + (size_t)b * (size_t)N * 3;
        int64_t *o = out + (size_t)b * (size_t)M;
        for (int64_t j = 0; j < N; ++j)
            m[j] = INFINITY;               /* min over an empty set of centres */
        int64_t c = start_idx;
        o[0] = c;
        for (int64_t t = 1; t < M; ++t) {
            /* fold centre c_{t-1} into every point's running minimum */
            for (int64_t j = 0; j < N; ++j) {
                float s = pco_s32(x + 3 * j, x + 3 * c);
                if (s < m[j])
                    m[j] = s;
            }
            /* farthest point: the first (smallest) index holding the maximum */
            int64_t best = 0;
            for (int64_t j = 1; j < N; ++j)
                if (m[j] > m[best])
                    best = j;
            c = best;
            o[t] = c;
        }
    }
    free(m);
    return PCO_OK;
}

typedef struct {
    float s;
    int64_t j;
} pco_pair;

/* Order by squared distance, then by reference index.
 * [P1] "k nearest neighbors": pi = argsort over j of (s_bij, j). */
static int pco_pair_cmp(const void *pa, const void *pb)
{
    const pco_pair *a = (const pco_pair *)pa;
    const pco_pair *b = (const pco_pair *)pb;
    if (a->s < b->s)
        return -1;
    if (a->s > b->s)
        return 1;
    if (a->j < b->j)
        return -1;
    if (a->j > b->j)
        return 1;
    return 0;
}

/* k nearest neighbours of the query rows [row_begin, row_end) of the flattened
 * (B*Q) query set. [P1] "k nearest neighbors": sort every reference by
 * (s, j), keep the first k, return D = sqrt(s) (IEEE sqrtf, correctly
 * rounded) and I = j. [P1] "Contracts": k <= N is required.
 * Out: dist (B, Q, k) float32, idx (B, Q, k) int64, rows outside the range
 * untouched. */
int pco_knn_rows(const float *query, const float *ref, int64_t B, int64_t Q, int64_t P,
                 int64_t k, float *out_dist, int64_t *out_idx, int64_t row_begin,
                 int64_t row_end)
{
    if (B < 0 || Q < 0 || P < 0 || k < 1 || k > P)
        return PCO_INVALID_ARGUMENT;
    if (row_begin < 0 || row_end > B * Q || row_begin > row_end)
        return PCO_INVALID_ARGUMENT;
    if (row_begin == row_end)
        return PCO_OK;
    pco_pair *all = (pco_pair *)malloc((size_t)P * sizeof(pco_pair));
    if (!all)
        return PCO_OUT_OF_MEMORY;
    for (int64_t row = row_begin; row < row_end; ++row) {
        int64_t b = row / Q;
        const float *q = query + (size_t)row * 3;
        const float *x = ref + (size_t)b * (size_t)P * 3;
        for (int64_t j = 0; j < P; ++j) {
            all[j].s = pco_s32(q, x + 3 * j);
            all[j].j = j;
        }
        qsort(all, (size_t)P, sizeof(pco_pair), pco_pair_cmp);
        for (int64_t n = 0; n < k; ++n) {
            out_dist[(size_t)row * k + n] = sqrtf(all[n].s);
            out_idx[(size_t)row * k + n] = all[n].j;
        }
    }
    free(all);
    return PCO_OK;
}

int pco_knn(const float *query, const float *ref, int64_t B, int64_t Q, int64_t P, int64_t k,
            float *out_dist, int64_t *out_idx)
{
    return pco_knn_rows(query, ref, B, Q, P, k, out_dist, out_idx, 0, B * Q);
}

/* Nearest reference of the query rows [row_begin, row_end), squared distance
 * kept: [P1] "k nearest neighbors" with k = 1 (the first reference in the
 * (s, j) order, i.e. the smallest j reaching the minimum s32), which is the
 * nearest-point selection of [P1]'s Chamfer distance (roadmap, "Phase 4":
 * a(i) = the nearest point of the other cloud). Cloud b uses only its first
 * p_len[b] references (all P when p_len is NULL); a row with none gets
 * (s, j) = (0, -1).
 * Out: s (B, Q) float32, idx (B, Q) int64, rows outside the range untouched. */
int pco_nearest_rows(const float *query, const float *ref, int64_t B, int64_t Q, int64_t P,
                     const int64_t *p_len, float *out_s, int64_t *out_idx, int64_t row_begin,
                     int64_t row_end)
{
    if (B < 0 || Q < 0 || P < 0)
        return PCO_INVALID_ARGUMENT;
    if (row_begin < 0 || row_end > B * Q || row_begin > row_end)
        return PCO_INVALID_ARGUMENT;
    for (int64_t row = row_begin; row < row_end; ++row) {
        int64_t b = row / Q;
        int64_t n = p_len ? p_len[b] : P;
        if (n < 0 || n > P)
            return PCO_INVALID_ARGUMENT;
        const float *q = query + (size_t)row * 3;
        const float *x = ref + (size_t)b * (size_t)P * 3;
        float best = 0.0f;
        int64_t arg = -1;
        for (int64_t j = 0; j < n; ++j) {
            float d = pco_s32(q, x + 3 * j);
            if (arg < 0 || d < best) {  /* strict: an equal distance keeps the smaller j */
                best = d;
                arg = j;
            }
        }
        out_s[row] = best;
        out_idx[row] = arg;
    }
    return PCO_OK;
}

/* First-K Ball Query of the query rows [row_begin, row_end).
 * [P1] "Ball Query: first K within a radius" and [P2] "Selection and output":
 * J = the references with s32 < R2 in input order; slot n < min(K, |J|) holds
 * (J[n], s of J[n]); the other slots hold (-1, 0). The scan stops once K
 * references are taken, which does not change the result.
 * Out: dist2 (B, Q, K) float32, idx (B, Q, K) int64. */
int pco_ball_query_rows(const float *query, const float *ref, int64_t B, int64_t Q, int64_t P,
                        float radius, int64_t K, float *out_dist2, int64_t *out_idx,
                        int64_t row_begin, int64_t row_end)
{
    if (B < 0 || Q < 0 || P < 0 || K < 1)
        return PCO_INVALID_ARGUMENT;
    if (!(radius > 0.0f) || isinf(radius))
        return PCO_INVALID_ARGUMENT;
    if (row_begin < 0 || row_end > B * Q || row_begin > row_end)
        return PCO_INVALID_ARGUMENT;
    float r2 = pco_ball_query_r2(radius);
    for (int64_t row = row_begin; row < row_end; ++row) {
        int64_t b = row / Q;
        const float *q = query + (size_t)row * 3;
        const float *x = ref + (size_t)b * (size_t)P * 3;
        float *d = out_dist2 + (size_t)row * K;
        int64_t *o = out_idx + (size_t)row * K;
        int64_t count = 0;
        for (int64_t j = 0; j < P && count < K; ++j) {
            float s = pco_s32(q, x + 3 * j);
            if (s < r2) {
                d[count] = s;
                o[count] = j;
                ++count;
            }
        }
        for (; count < K; ++count) {
            d[count] = 0.0f;
            o[count] = -1;
        }
    }
    return PCO_OK;
}

int pco_ball_query(const float *query, const float *ref, int64_t B, int64_t Q, int64_t P,
                   float radius, int64_t K, float *out_dist2, int64_t *out_idx)
{
    return pco_ball_query_rows(query, ref, B, Q, P, radius, K, out_dist2, out_idx, 0, B * Q);
}

/* Ball Query backward, in float64.
 * [P1] "Ball Query: first K within a radius", the two gradient formulas, and
 * [P2] "Differentiation": with G = dL/dS for the selected pairs,
 *   dL/dq_i = 2 * sum over k with I_ik >= 0 of G_ik (q_i - x_{I_ik}),
 *   dL/dx_j = 2 * sum over (i, k) with I_ik = j of G_ik (x_j - q_i).
 * Padding slots (I < 0) contribute nothing. Each output also gets the sum of
 * the absolute values of its terms (abs_q, abs_x), from which a caller bounds
 * the rounding error of a float32 evaluation. All outputs are overwritten.
 * Any of grad_q/abs_q or grad_x/abs_x may be NULL to skip that side. */
int pco_ball_query_backward(const float *query, const float *ref, const int64_t *idx,
                            const float *grad, int64_t B, int64_t Q, int64_t P, int64_t K,
                            double *grad_q, double *grad_x, double *abs_q, double *abs_x)
{
    if (B < 0 || Q < 0 || P < 0 || K < 1)
        return PCO_INVALID_ARGUMENT;
    if (grad_q) memset(grad_q, 0, sizeof(double) * (size_t)(B * Q * 3));
    if (abs_q) memset(abs_q, 0, sizeof(double) * (size_t)(B * Q * 3));
    if (grad_x) memset(grad_x, 0, sizeof(double) * (size_t)(B * P * 3));
    if (abs_x) memset(abs_x, 0, sizeof(double) * (size_t)(B * P * 3));
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < Q; ++i) {
            const int64_t row = b * Q + i;
            const float *q = query + (size_t)row * 3;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = idx[(size_t)row * K + k];
                if (j < 0)
                    continue;
                if (j >= P)
                    return PCO_INVALID_ARGUMENT;
                const double g = (double)grad[(size_t)row * K + k];
                const float *x = ref + ((size_t)b * P + (size_t)j) * 3;
                for (int d = 0; d < 3; ++d) {
                    const double t = 2.0 * g * ((double)q[d] - (double)x[d]);
                    if (grad_q) grad_q[(size_t)row * 3 + d] += t;
                    if (abs_q) abs_q[(size_t)row * 3 + d] += fabs(t);
                    if (grad_x) grad_x[((size_t)b * P + (size_t)j) * 3 + d] -= t;
                    if (abs_x) abs_x[((size_t)b * P + (size_t)j) * 3 + d] += fabs(t);
                }
            }
        }
    }
    return PCO_OK;
}
