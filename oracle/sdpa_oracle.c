/*
 * CPU oracle for the materialised-probability scaled-dot-product attention
 * forward: returns the output O, the full probability map P and the row
 * log-sum-exp LSE, in float64.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the checker, not the product: only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or constant with the HIP library.
 *
 * What it computes (the plain definition, one query row at a time, no
 * blocking, no fusion, no online rescaling):
 *
 *   s_j   = scale * sum_d q[d] * k_{h'}[j][d]        j = 0 .. Skv-1
 *   s_j   = -inf  where a causal or boolean (False) mask removes key j;
 *                 s_j += mask[i][j] for an additive mask. Causal removes
 *                 j > i + c: c = 0 top-left (is_causal 1), c = Skv - Sq
 *                 bottom-right (is_causal 2: the last query row keeps every
 *                 key, rows i < Sq - Skv keep none)
 *   m     = max_j s_j
 *   dead row (m == -inf):  P[i][:] = 0, O[i][:] = 0, LSE[i] = -inf
 *   else:  LSE = m + log(sum_j exp(s_j - m)),  P_j = exp(s_j - LSE),
 *          O[i][:] = sum_j P_j * v_{h'}[j][:]
 *   with h' = h / (Hq / Hkv) (contiguous groups of query heads share a KV head)
 *
 * Passages followed:
 *  - FlagOS-OP pull request "feat: add sdpa_math operator (Ascend Triton +
 *    P800 exact-P/A1)", Overview: the math backend returns (out, attn_probs);
 *    Implementation: a fully-masked row gives P = O = 0, a head count that
 *    does not divide is an error, causal and an explicit mask are exclusive;
 *    Intentional divergences: a boolean mask removes keys with -inf;
 *    "P800 exact-P fast path" update: P = exp(scale * QK^T - LSE) with the
 *    row-wise LSE.
 *  - cudnn-frontend pull request "[SDPA] SM80 fwd: TemplateParams kernels,
 *    plan-time compile, sym_int THD extents", merge-log notes: a dead row
 *    reports LSE = -inf and O = 0; LSE is float32 laid out (B, H, S);
 *    bottom-right causal is the alignment of chunked prefill (a chunk of
 *    queries against a longer key cache).
 *
 * Inputs are contiguous float64 arrays (the caller upcasts the exact
 * dtype-rounded values the GPU receives):
 *   q [B,Hq,Sq,D], k [B,Hkv,Skv,D], v [B,Hkv,Skv,Dv]
 *   mask: NULL, or uint8 (bool kind) / float64 (additive kind) addressed with
 *         mask_strides[4] in elements over the logical [B,Hq,Sq,Skv] index
 *         (a stride of 0 broadcasts that dimension)
 * Outputs (contiguous float64): out [B,Hq,Sq,Dv], probs [B,Hq,Sq,Skv],
 *   lse [B,Hq,Sq].
 * Returns 0 on success, 1 when Hq is not a multiple of Hkv, 2 when causal is
 * combined with a mask, 3 for a bad mask kind, 4 for a bad is_causal, 5 for
 * a bad dropout probability or rule.
 *
 * oracle_sdpa_bwd (at the end of this file) is the backward of the same
 * definition: dq, dk, dv from dL/dO and dL/dP by the plain chain rule.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MASK_NONE 0
#define ORACLE_MASK_BOOL 1
#define ORACLE_MASK_ADD 2

int oracle_sdpa_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Dropout (FlagOS-OP page, Implementation section: the explicit and the
 * random dropout rule; Intentional divergences: with dropout_p > 0 the
 * output is the product of the dropped probabilities with V). keep is a
 * uint8 keep-mask over [B,Hq,Sq,Skv] addressed with keep_strides (NULL: no
 * dropout), drop_p the dropout probability, keep_rule 0 or 1:
 *   rule 0 (explicit mask): P_out = keep * P,         O = (keep * P) V / (1 - p)
 *   rule 1 (random):        P_out = keep * P / (1-p), O = P_out V
 * LSE is that of the undropped softmax.
 */
int oracle_sdpa_fwd(const double* q, const double* k, const double* v,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                    int64_t D, int64_t Dv,
                    int mask_kind, const void* mask, const int64_t* mask_strides,
                    int is_causal, double scale,
                    const uint8_t* keep, const int64_t* keep_strides, double drop_p, int keep_rule,
                    double* out, double* probs, double* lse)
{
    if (keep && (!(drop_p >= 0.0 && drop_p < 1.0) || (keep_rule != 0 && keep_rule != 1)))
        return 5;
    if (Hkv <= 0 || Hq % Hkv != 0)
        return 1;
    if (is_causal < 0 || is_causal > 2)
        return 4;
    const int64_t coff = is_causal == 2 ? Skv - Sq : 0;
    if (is_causal && mask_kind != ORACLE_MASK_NONE)
        return 2;
    if (mask_kind != ORACLE_MASK_NONE && mask_kind != ORACLE_MASK_BOOL &&
        mask_kind != ORACLE_MASK_ADD)
        return 3;

    const int64_t group = Hq / Hkv;
    const int64_t nrows = B * Hq * Sq;

#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t row = 0; row < nrows; ++row) {
        const int64_t i = row % Sq;
        const int64_t h = (row / Sq) % Hq;
        const int64_t b = row / (Sq * Hq);
        const int64_t hk = h / group;

        const double* qi = q + row * D;
        const double* kh = k + (b * Hkv + hk) * Skv * D;
        const double* vh = v + (b * Hkv + hk) * Skv * Dv;
        double* p = probs + row * Skv; /* holds the scores until normalised */
        double* o = out + row * Dv;

        /* scores, masking, running maximum */
        double m = -INFINITY;
        for (int64_t j = 0; j < Skv; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dot += qi[d] * kh[j * D + d];
            double s = scale * dot;
            if (is_causal && j > i + coff) {
                s = -INFINITY;
            } else if (mask_kind != ORACLE_MASK_NONE) {
                const int64_t off = b * mask_strides[0] + h * mask_strides[1] +
                                    i * mask_strides[2] + j * mask_strides[3];
                if (mask_kind == ORACLE_MASK_BOOL) {
                    if (((const uint8_t*)mask)[off] == 0)
                        s = -INFINITY;
                } else {
                    s += ((const double*)mask)[off];
                }
            }
            p[j] = s;
            if (s > m)
                m = s;
        }

        if (m == -INFINITY) { /* every key removed (or no keys at all) */
            for (int64_t j = 0; j < Skv; ++j)
                p[j] = 0.0;
            for (int64_t d = 0; d < Dv; ++d)
                o[d] = 0.0;
            lse[row] = -INFINITY;
            continue;
        }

        double l = 0.0;
        for (int64_t j = 0; j < Skv; ++j)
            l += exp(p[j] - m);
        const double L = m + log(l);
        lse[row] = L;

        for (int64_t j = 0; j < Skv; ++j)
            p[j] = exp(p[j] - L);

        double oscale = 1.0;
        if (keep) { /* drop the removed probabilities, then the rule's scaling */
            const double inv = 1.0 / (1.0 - drop_p);
            for (int64_t j = 0; j < Skv; ++j) {
                const int64_t off = b * keep_strides[0] + h * keep_strides[1] +
                                    i * keep_strides[2] + j * keep_strides[3];
                if (keep[off] == 0)
                    p[j] = 0.0;
                else if (keep_rule == 1)
                    p[j] *= inv;
            }
            if (keep_rule == 0)
                oscale = inv;
        }

        for (int64_t d = 0; d < Dv; ++d) {
            double acc = 0.0;
            for (int64_t j = 0; j < Skv; ++j)
                acc += p[j] * vh[j * Dv + d];
            o[d] = acc * oscale;
        }
    }
    return 0;
}

/*
 * Backward of the same forward: gradients of a scalar loss with respect to
 * q, k, v, given its gradients with respect to both outputs the math backend
 * returns, dout = dL/dO and dprobs = dL/dP (NULL: no gradient reaches P).
 * This is the two-output (dout + dprobs) gradient of the FlagOS-OP page's
 * Implementation section (its autograd.Function) and of its "P800 fused
 * backward" update (the softmax Jacobian taken from the probability map,
 * query/key gradients reduced back to the key/value heads). Plain chain
 * rule, in float64, one query row at a time:
 *
 *   P_i    recomputed exactly as in oracle_sdpa_fwd (0 on removed keys and
 *          on dead rows, which therefore receive no gradient)
 *   dP_ij  = sum_d dout[i][d] * v_{h'}[j][d] + dprobs[i][j]
 *   Dsum_i = sum_j P_ij * dP_ij
 *   dS_ij  = P_ij * (dP_ij - Dsum_i)          (softmax Jacobian)
 *   dq[i][d]      = scale * sum_j dS_ij * k_{h'}[j][d]
 *   dk_{h'}[j][d] += scale * dS_ij * q[i][d]  (summed over the query heads
 *   dv_{h'}[j][d] += P_ij * dout[i][d]         of the group and their rows)
 *
 * Same argument conventions as oracle_sdpa_fwd; dout is [B,Hq,Sq,Dv],
 * dprobs [B,Hq,Sq,Skv] (or NULL); outputs dq [B,Hq,Sq,D], dk [B,Hkv,Skv,D],
 * dv [B,Hkv,Skv,Dv], contiguous float64. Same return codes.
 */
int oracle_sdpa_bwd(const double* q, const double* k, const double* v,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                    int64_t D, int64_t Dv,
                    int mask_kind, const void* mask, const int64_t* mask_strides,
                    int is_causal, double scale,
                    const double* dout, const double* dprobs,
                    double* dq, double* dk, double* dv)
{
    if (Hkv <= 0 || Hq % Hkv != 0)
        return 1;
    if (is_causal < 0 || is_causal > 2)
        return 4;
    const int64_t coff = is_causal == 2 ? Skv - Sq : 0;
    if (is_causal && mask_kind != ORACLE_MASK_NONE)
        return 2;
    if (mask_kind != ORACLE_MASK_NONE && mask_kind != ORACLE_MASK_BOOL &&
        mask_kind != ORACLE_MASK_ADD)
        return 3;

    const int64_t group = Hq / Hkv;

    /* one (batch, kv head) per iteration: it owns its dk and dv slices */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bk = 0; bk < B * Hkv; ++bk) {
        const int64_t b = bk / Hkv;
        const int64_t hk = bk % Hkv;
        const double* kh = k + (b * Hkv + hk) * Skv * D;
        const double* vh = v + (b * Hkv + hk) * Skv * Dv;
        double* dkh = dk + (b * Hkv + hk) * Skv * D;
        double* dvh = dv + (b * Hkv + hk) * Skv * Dv;
        for (int64_t x = 0; x < Skv * D; ++x)
            dkh[x] = 0.0;
        for (int64_t x = 0; x < Skv * Dv; ++x)
            dvh[x] = 0.0;
        double* p = (double*)malloc((size_t)(Skv > 0 ? Skv : 1) * sizeof(double));
        double* dp = (double*)malloc((size_t)(Skv > 0 ? Skv : 1) * sizeof(double));

        for (int64_t h = hk * group; h < (hk + 1) * group; ++h) {
            for (int64_t i = 0; i < Sq; ++i) {
                const int64_t row = (b * Hq + h) * Sq + i;
                const double* qi = q + row * D;
                const double* doi = dout + row * Dv;
                double* dqi = dq + row * D;
                for (int64_t d = 0; d < D; ++d)
                    dqi[d] = 0.0;

                /* the forward's probabilities of this row */
                double m = -INFINITY;
                for (int64_t j = 0; j < Skv; ++j) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        dot += qi[d] * kh[j * D + d];
                    double s = scale * dot;
                    if (is_causal && j > i + coff) {
                        s = -INFINITY;
                    } else if (mask_kind != ORACLE_MASK_NONE) {
                        const int64_t off = b * mask_strides[0] + h * mask_strides[1] +
                                            i * mask_strides[2] + j * mask_strides[3];
                        if (mask_kind == ORACLE_MASK_BOOL) {
                            if (((const uint8_t*)mask)[off] == 0)
                                s = -INFINITY;
                        } else {
                            s += ((const double*)mask)[off];
                        }
                    }
                    p[j] = s;
                    if (s > m)
                        m = s;
                }
                if (m == -INFINITY)
                    continue; /* dead row: P = 0, no gradient flows */
                double l = 0.0;
                for (int64_t j = 0; j < Skv; ++j)
                    l += exp(p[j] - m);
                const double L = m + log(l);
                for (int64_t j = 0; j < Skv; ++j)
                    p[j] = exp(p[j] - L);

                /* gradient reaching the probabilities, and its row dot with P */
                double dsum = 0.0;
                for (int64_t j = 0; j < Skv; ++j) {
                    double acc = 0.0;
                    for (int64_t d = 0; d < Dv; ++d)
                        acc += doi[d] * vh[j * Dv + d];
                    if (dprobs)
                        acc += dprobs[row * Skv + j];
                    dp[j] = acc;
                    dsum += p[j] * acc;
                }

                for (int64_t j = 0; j < Skv; ++j) {
                    const double ds = p[j] * (dp[j] - dsum);
                    for (int64_t d = 0; d < D; ++d) {
                        dqi[d] += scale * ds * kh[j * D + d];
                        dkh[j * D + d] += scale * ds * qi[d];
                    }
                    for (int64_t d = 0; d < Dv; ++d)
                        dvh[j * Dv + d] += p[j] * doi[d];
                }
            }
        }
        free(p);
        free(dp);
    }
    return 0;
}
