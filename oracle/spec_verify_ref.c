/*
 * spec_verify_ref.c -- fp64 CPU oracle for the batched verify-and-sample step
 * of speculative decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity reference for the HIP
 * library.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it.  It shares no code, header, table or constant
 * with the GPU path, and nothing on the product path may call it.
 *
 * It is deliberately plain: every sum is sequential in index order, in
 * double precision, with libm's exp(); no blocking, fusion or reordering.
 * OpenMP parallelism is over independent sequences only and does not change
 * any result.
 *
 * Sources (page title, then the section / equation used):
 *   [FI] "Fast Inference from Transformers via Speculative Decoding"
 *        (paper summary page): "Standardized Sampling", "Speculative
 *        Sampling: The Core Algorithm" (Algorithm 1, Phases 1-4), "Why This
 *        Procedure Preserves the Target Distribution" (Appendix A.1).
 *   [TM] "Speculative Decoding: Two Models, One Output": "The algorithm".
 *   [PB] "Speculative Decoding Paper Breakdown: Lossless Draft-and-Verify
 *        Acceleration for Autoregressive Transformers": section 3, "The
 *        Algorithm at Position i", and "Reference Implementation".
 *   [ST] "The exact decoding shortcut that burns compute when guesses miss":
 *        the correction_distribution snippet (zero-residual fallback).
 *   [FI] "Computing alpha from p and q: The DLK Divergence" (Theorem 3.5,
 *        Corollary 3.6) and "Expected Number of Generated Tokens" (alpha
 *        as the expectation of beta): the acceptance-rate telemetry.
 *   [FI] "Ablation Studies and Robustness Checks" (Appendix A.5) and "How
 *        This Work Changes the Landscape": a lenience l in [0, 1] multiplies
 *        q(x) before it is compared with p(x), and no token is then sampled
 *        with probability above p(x)/l.
 *
 * Readings where the pages leave a step open (each one is also listed in the
 * design notes of the repository):
 *   - temperature divides the target logits only; draft probabilities are
 *     used exactly as given, never renormalised;
 *   - uniforms[b][i] (i < gamma) drives the acceptance test at position i,
 *     uniforms[b][gamma] drives the single residual-or-bonus draw;
 *   - the draw is an inverse CDF: the smallest k whose running sum exceeds
 *     u * total (strict), falling back to the largest positive-weight index;
 *   - a draft probability q <= 0 means "accept" ([PB] Reference
 *     Implementation treats q_x <= 0 that way);
 *   - the residual is replaced by the target row when its mass is <= 1e-15
 *     ([ST] correction_distribution);
 *   - greedy (argmax) mode: the draft is a point mass at x_i, a draft is
 *     accepted iff it equals the first index attaining the row maximum of
 *     the raw target logits, and the emitted token is that argmax ([FI]
 *     "Standardized Sampling", argmax case);
 *   - a draft token outside [0, V) marks the whole sequence invalid:
 *     n_accepted = -1 and every output token = -1;
 *   - lenience l (the pages give only the acceptance side): accept iff
 *     u <= min(1, p / (l q)), and after a rejection draw from
 *     norm(max(0, p - l q)), the residual of the same comparison (the same
 *     [ST] fallback to p when its mass is <= 1e-15); l = 1 is the exact
 *     method, l = 0 accepts every draft.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_FP32 0
#define REF_BF16 1
#define REF_SAMPLE 0
#define REF_GREEDY 1

/* Relative distance of a uniform to a decision boundary inside which the
 * GPU path is exempt from bit-exact agreement: 1e-6 around an acceptance
 * threshold, 1e-9 around an inverse-CDF boundary.  The CDF window is
 * tighter because a draw over V ~ 1e5 tokens has ~V boundaries, so a 1e-6
 * window would cover percent-level fractions of all draws. */
#define REF_NEAR_REL 1e-6
#define REF_NEAR_REL_CDF 1e-9
/* Residual mass at or below which the target row is used instead ([ST]). */
#define REF_RESID_EPS 1e-15

typedef struct {
    double*  p_tok;       /* [B][gamma]   p_i(x_i) for every tested position, NaN otherwise   */
    double*  q_tok;       /* [B][gamma]   q_i(x_i) for every tested position, NaN otherwise   */
    double*  thr;         /* [B][gamma]   min(1, p/q) (1 if q <= 0) for tested positions      */
    double*  resid_mass;  /* [B]          sum_v max(0, p_n - q_n) when a residual is drawn    */
    double*  row_max;     /* [B][gamma+1] max_v z for every row the walk normalised, else NaN */
    double*  row_sum;     /* [B][gamma+1] sum_v exp((z - max)/T) for those rows, else NaN     */
    int32_t* flag_pos;    /* [B]          position of the first near-boundary decision, -1    */
    int32_t* n_decisions; /* [B]          acceptance tests run + 1 final draw                 */
    int32_t* n_flags;     /* [B]          near-boundary decisions taken                        */
    double*  beta;        /* [B][gamma]   sum_v min(p_i, q_i) for EVERY position (sample mode) */
    double*  alpha;       /* [gamma]      mean over the batch of beta[.][i]                    */
    double*  p_out;       /* [B]          p_n(t), t the token drawn at position n (the bonus token
                                          when n = gamma), sample mode; NaN otherwise              */
} ref_aux_t;

/* Exact promotion of one input element to double: fp32 directly, bf16 by
 * placing its 16 bits in the high half of an fp32 word. */
static double load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == REF_FP32) return (double)((const float*)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Temperature softmax of one row ([FI] "Standardized Sampling": divide the
 * logits by T, then softmax).  Max-subtracted form; -inf logits give 0.
 * Writes p[0..V), returns the row max and the sum of exponentials. */
static void softmax_row(const void* z, int dtype, int64_t off, int V, double T,
                        double* p, double* out_max, double* out_sum)
{
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double x = load_elem(z, dtype, off + v);
        if (x > m) m = x;
    }
    double s = 0.0;
    for (int v = 0; v < V; ++v) {
        double e = exp((load_elem(z, dtype, off + v) - m) / T);
        p[v] = e;
        s += e;
    }
    for (int v = 0; v < V; ++v) p[v] = p[v] / s;
    *out_max = m;
    *out_sum = s;
}

/* First index attaining the maximum of the raw row ([FI] "Standardized
 * Sampling", argmax case: a point mass at the mode). */
static int argmax_row(const void* z, int dtype, int64_t off, int V)
{
    int best = 0;
    double bv = load_elem(z, dtype, off);
    for (int v = 1; v < V; ++v) {
        double x = load_elem(z, dtype, off + v);
        if (x > bv) { bv = x; best = v; }
    }
    return best;
}

static int near_boundary(double u, double b, double rel)
{
    return fabs(u - b) <= rel * b;
}

/* Inverse-CDF draw from an unnormalised weight row: the smallest k with
 * C_k > u * C_total, where C_k = w_0 + ... + w_k summed in index order.
 * If no such k exists (u * total >= total) the largest k with w_k > 0.
 * Sets *flagged when u lies within REF_NEAR_REL_CDF (relative) of either
 * normalised boundary C_{k-1}/C_total or C_k/C_total of the chosen k. */
static int icdf_draw(const double* w, int V, double u, int* flagged)
{
    double total = 0.0;
    for (int v = 0; v < V; ++v) total += w[v];
    double target = u * total;
    double c = 0.0, lo = 0.0, hi = 0.0;
    int k = -1;
    for (int v = 0; v < V; ++v) {
        double prev = c;
        c += w[v];
        if (c > target) { k = v; lo = prev; hi = c; break; }
    }
    if (k < 0) {
        for (int v = V - 1; v >= 0; --v)
            if (w[v] > 0.0) { k = v; break; }
        lo = hi = total;
    }
    if (flagged) {
        *flagged = 0;
        if (total > 0.0 &&
            (near_boundary(u, lo / total, REF_NEAR_REL_CDF) ||
             near_boundary(u, hi / total, REF_NEAR_REL_CDF)))
            *flagged = 1;
    }
    return k;
}

/* One sequence in sample mode: [FI] Algorithm 1 Phases 3 and 4, with the
 * acceptance rule of [PB] section 3 (accept iff u <= min(1, p/q)) and the
 * correction distribution of [FI] Phase 4 / [ST]. */
static void verify_sample_one(int b, int gamma, int V,
                              const void* zl, int zd, const void* qp, int qd,
                              const int32_t* x, const float* u, double T, double l,
                              int32_t* n_out, int32_t* tok_out,
                              const ref_aux_t* aux, double* p, double* w)
{
    const int G1 = gamma + 1;
    int first_flag = -1, n_dec = 0, n_flag = 0;
    double rmax, rsum;

    int n = gamma;
    for (int i = 0; i < gamma; ++i) {
        /* Phase 2 output p_i, needed only while every earlier draft passed. */
        softmax_row(zl, zd, ((int64_t)b * G1 + i) * V, V, T, p, &rmax, &rsum);
        if (aux && aux->row_max) aux->row_max[(int64_t)b * G1 + i] = rmax;
        if (aux && aux->row_sum) aux->row_sum[(int64_t)b * G1 + i] = rsum;

        /* Phase 3: accept x_i with probability min(1, p_i(x_i)/q_i(x_i)). */
        double P = p[x[i]];
        double Q = load_elem(qp, qd, ((int64_t)b * gamma + i) * V + x[i]);
        double lQ = l * Q; /* lenience scales q before the comparison (l = 1: exact) */
        double thr = (Q <= 0.0) ? 1.0 : fmin(1.0, P / lQ);
        double ui = (double)u[i];
        ++n_dec;
        if (near_boundary(ui, thr, REF_NEAR_REL)) { ++n_flag; if (first_flag < 0) first_flag = i; }
        if (aux && aux->p_tok) aux->p_tok[(int64_t)b * gamma + i] = P;
        if (aux && aux->q_tok) aux->q_tok[(int64_t)b * gamma + i] = Q;
        if (aux && aux->thr) aux->thr[(int64_t)b * gamma + i] = thr;
        if (!(ui <= thr)) { n = i; break; } /* stop at the first rejection */
    }

    for (int i = 0; i < n; ++i) tok_out[i] = x[i];

    int t, fl = 0;
    double ug = (double)u[gamma];
    if (n < gamma) {
        /* Phase 4, rejection at position n: p holds p_n already.  Sample from
         * norm(max(0, p_n - l q_n)); if that mass is <= 1e-15 use p_n ([ST]). */
        double Z = 0.0;
        for (int v = 0; v < V; ++v) {
            double r = p[v] - l * load_elem(qp, qd, ((int64_t)b * gamma + n) * V + v);
            w[v] = r > 0.0 ? r : 0.0;
            Z += w[v];
        }
        if (aux && aux->resid_mass) aux->resid_mass[b] = Z;
        int zflag = fabs(Z - REF_RESID_EPS) <= REF_NEAR_REL * REF_RESID_EPS;
        t = icdf_draw(Z > REF_RESID_EPS ? w : p, V, ug, &fl);
        fl = fl || zflag;
    } else {
        /* Phase 4, every draft accepted: bonus token from p_{gamma+1}. */
        softmax_row(zl, zd, ((int64_t)b * G1 + gamma) * V, V, T, p, &rmax, &rsum);
        if (aux && aux->row_max) aux->row_max[(int64_t)b * G1 + gamma] = rmax;
        if (aux && aux->row_sum) aux->row_sum[(int64_t)b * G1 + gamma] = rsum;
        t = icdf_draw(p, V, ug, &fl);
    }
    ++n_dec;
    if (fl) { ++n_flag; if (first_flag < 0) first_flag = n; }

    tok_out[n] = t;
    for (int i = n + 1; i <= gamma; ++i) tok_out[i] = -1;
    *n_out = n;
    /* p still holds p_n, the row the token was drawn for */
    if (aux && aux->p_out) aux->p_out[b] = p[t];
    if (aux && aux->flag_pos) aux->flag_pos[b] = first_flag;
    if (aux && aux->n_decisions) aux->n_decisions[b] = n_dec;
    if (aux && aux->n_flags) aux->n_flags[b] = n_flag;
}

/* One sequence in greedy mode ([FI] "Standardized Sampling": with argmax
 * standardisation p_i and q_i are point masses, so a draft survives iff it
 * equals the target argmax and the correction is that argmax). */
static void verify_greedy_one(int b, int gamma, int V, const void* zl, int zd,
                              const int32_t* x, int32_t* n_out, int32_t* tok_out,
                              const ref_aux_t* aux)
{
    const int G1 = gamma + 1;
    int n = gamma, t = -1;
    for (int i = 0; i < gamma; ++i) {
        int a = argmax_row(zl, zd, ((int64_t)b * G1 + i) * V, V);
        if (x[i] != a) { n = i; t = a; break; }
    }
    if (n == gamma) t = argmax_row(zl, zd, ((int64_t)b * G1 + gamma) * V, V);
    for (int i = 0; i < n; ++i) tok_out[i] = x[i];
    tok_out[n] = t;
    for (int i = n + 1; i <= gamma; ++i) tok_out[i] = -1;
    *n_out = n;
    if (aux && aux->flag_pos) aux->flag_pos[b] = -1;
    if (aux && aux->n_decisions) aux->n_decisions[b] = (n < gamma) ? n + 1 : gamma;
    if (aux && aux->n_flags) aux->n_flags[b] = 0;
}

/* Acceptance rate of one position: beta = sum_v min(p(v), q(v)) with p the
 * temperature softmax of the target row and q the draft row as given
 * ([FI] Theorem 3.5: the probability that the draft token is accepted,
 * 1 - DLK(p, q)).  Sequential sum in index order. */
static double accept_rate_row(const void* zl, int zd, int64_t zoff, const void* qp, int qd,
                              int64_t qoff, int V, double T, double* p)
{
    double m, s;
    softmax_row(zl, zd, zoff, V, T, p, &m, &s);
    double beta = 0.0;
    for (int v = 0; v < V; ++v) {
        double q = load_elem(qp, qd, qoff + v);
        beta += p[v] < q ? p[v] : q;
    }
    return beta;
}

static void fill_nan(double* a, int64_t count)
{
    if (!a) return;
    for (int64_t i = 0; i < count; ++i) a[i] = NAN;
}

/* Returns 0 on success, a negative value for arguments outside the domain. */
int spec_verify_ref(int batch, int gamma, int vocab,
                    const void* target_logits, int logits_dtype,
                    const void* draft_probs, int probs_dtype,
                    const int32_t* draft_tokens, const float* uniforms,
                    float temperature, float lenience, int mode,
                    int32_t* n_accepted, int32_t* out_tokens,
                    const ref_aux_t* aux, int n_threads)
{
    if (batch < 1) return -2;
    if (gamma < 1 || gamma > 63) return -3;
    if (vocab < 1) return -4;
    if (mode != REF_SAMPLE && mode != REF_GREEDY) return -7;
    if (logits_dtype != REF_FP32 && logits_dtype != REF_BF16) return -6;
    if (!target_logits || !draft_tokens || !n_accepted || !out_tokens) return -1;
    if (mode == REF_SAMPLE) {
        if (!draft_probs || !uniforms) return -1;
        if (probs_dtype != REF_FP32 && probs_dtype != REF_BF16) return -6;
        if (!(temperature > 0.0f) || !isfinite(temperature)) return -5;
        if (!(lenience >= 0.0f && lenience <= 1.0f)) return -12;
    }

    const int64_t B = batch, G = gamma, G1 = gamma + 1;
    if (aux) {
        fill_nan(aux->p_tok, B * G);
        fill_nan(aux->q_tok, B * G);
        fill_nan(aux->thr, B * G);
        fill_nan(aux->resid_mass, B);
        fill_nan(aux->row_max, B * G1);
        fill_nan(aux->row_sum, B * G1);
        fill_nan(aux->beta, B * G);
        fill_nan(aux->alpha, G);
        fill_nan(aux->p_out, B);
    }

#ifdef _OPENMP
    int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#else
    int nt = 1;
    (void)n_threads;
#endif
    int bad_alloc = 0;

#pragma omp parallel num_threads(nt)
    {
        double* p = NULL;
        double* w = NULL;
        if (mode == REF_SAMPLE) {
            p = (double*)malloc(sizeof(double) * (size_t)vocab);
            w = (double*)malloc(sizeof(double) * (size_t)vocab);
            if (!p || !w) {
#pragma omp atomic write
                bad_alloc = 1;
            }
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            const int32_t* x = draft_tokens + b * G;
            int32_t* tok = out_tokens + b * G1;
            int valid = 1;
            for (int i = 0; i < gamma; ++i)
                if (x[i] < 0 || x[i] >= vocab) valid = 0;
            if (!valid) {
                n_accepted[b] = -1;
                for (int i = 0; i <= gamma; ++i) tok[i] = -1;
                if (aux && aux->flag_pos) aux->flag_pos[b] = -1;
                if (aux && aux->n_decisions) aux->n_decisions[b] = 0;
                if (aux && aux->n_flags) aux->n_flags[b] = 0;
                continue;
            }
            if (mode == REF_GREEDY) {
                verify_greedy_one((int)b, gamma, vocab, target_logits, logits_dtype,
                                  x, &n_accepted[b], tok, aux);
            } else if (p && w) {
                verify_sample_one((int)b, gamma, vocab, target_logits, logits_dtype,
                                  draft_probs, probs_dtype, x, uniforms + b * G1,
                                  (double)temperature, (double)lenience, &n_accepted[b], tok, aux, p, w);
            }
        }
        free(p);
        free(w);
    }
    if (bad_alloc) return -10;

    /* Telemetry: beta for every position of every sequence (not only the
     * ones the walk reached), then alpha_i = (1/B) sum_b beta[b][i] summed
     * in order of b. */
    if (mode == REF_SAMPLE && aux && (aux->beta || aux->alpha)) {
        double* beta = aux->beta ? aux->beta : (double*)malloc(sizeof(double) * (size_t)(B * G));
        if (!beta) return -10;
#pragma omp parallel num_threads(nt)
        {
            double* p = (double*)malloc(sizeof(double) * (size_t)vocab);
            if (!p) {
#pragma omp atomic write
                bad_alloc = 1;
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t bi = 0; bi < B * G; ++bi) {
                if (!p) continue;
                const int64_t b = bi / G, i = bi % G;
                beta[bi] = accept_rate_row(target_logits, logits_dtype, (b * G1 + i) * vocab,
                                           draft_probs, probs_dtype, (b * G + i) * vocab, vocab,
                                           (double)temperature, p);
            }
            free(p);
        }
        if (aux->alpha && !bad_alloc) {
            for (int64_t i = 0; i < G; ++i) {
                double a = 0.0;
                for (int64_t b = 0; b < B; ++b) a += beta[b * G + i];
                aux->alpha[i] = a / (double)B;
            }
        }
        if (!aux->beta) free(beta);
    }
    return bad_alloc ? -10 : 0;
}

/* ---- single-step entry points used by the oracle's own pin tests ------- */

int ref_softmax_row(const void* z, int dtype, int vocab, float temperature, double* p)
{
    double m, s;
    if (vocab < 1 || !z || !p || !(temperature > 0.0f)) return -1;
    softmax_row(z, dtype, 0, vocab, (double)temperature, p, &m, &s);
    return 0;
}

int ref_icdf(const double* w, int vocab, double u, int* flagged)
{
    if (vocab < 1 || !w) return -1;
    return icdf_draw(w, vocab, u, flagged);
}

int ref_argmax_row(const void* z, int dtype, int vocab)
{
    if (vocab < 1 || !z) return -1;
    return argmax_row(z, dtype, 0, vocab);
}

/* ---- top-k / nucleus standardisation ([FI] "Standardized Sampling") ----
 *
 * Top-k: keep the k largest probabilities, zero the rest, renormalise.
 * Nucleus: sort the probabilities in decreasing order and keep the shortest
 * prefix whose cumulative probability reaches top_p, zero the rest,
 * renormalise.  The output is the row of logits with every dropped entry set
 * to -inf, so that the temperature softmax of the output is exactly the
 * standardised distribution.  Readings: ties in value are ordered by
 * increasing index (so top-k keeps exactly min(k, V) entries); the nucleus
 * prefix includes the entry at which the running sum (fp64, in sorted order,
 * p_v = exp((z_v - max)/T) / S with S summed in index order) first reaches
 * top_p; if rounding keeps it below top_p to the end, every entry is kept,
 * and top_p = 1 keeps every entry (the whole distribution: only rounding
 * could make a running sum reach 1 before the last positive entry).
 * flag (nucleus only): 1 when top_p lies within 1e-9 (relative) of the
 * running sum just before or at the boundary entry -- a decision that
 * another summation order may take differently. */

typedef struct {
    double z;
    int v;
} ref_kv_t;

static int kv_desc(const void* a, const void* b)
{
    const ref_kv_t* x = (const ref_kv_t*)a;
    const ref_kv_t* y = (const ref_kv_t*)b;
    if (x->z > y->z) return -1;
    if (x->z < y->z) return 1;
    return x->v < y->v ? -1 : (x->v > y->v ? 1 : 0);
}

static void store_elem(void* base, int dtype, int64_t idx, const void* src)
{
    if (dtype == REF_FP32) ((float*)base)[idx] = ((const float*)src)[idx];
    else ((uint16_t*)base)[idx] = ((const uint16_t*)src)[idx];
}

static void store_neg_inf(void* base, int dtype, int64_t idx)
{
    if (dtype == REF_FP32) ((float*)base)[idx] = -INFINITY;
    else ((uint16_t*)base)[idx] = 0xff80u;
}

#define REF_TOPK 0
#define REF_TOPP 1

int ref_standardize(int rows, int vocab, const void* z, int dtype, int method, int k, float top_p,
                    float temperature, void* out, int32_t* kept, int32_t* flag)
{
    if (rows < 1 || vocab < 1 || !z || !out) return -1;
    if (dtype != REF_FP32 && dtype != REF_BF16) return -6;
    if (method == REF_TOPK && k < 1) return -13;
    if (method == REF_TOPP && !(top_p > 0.0f && top_p <= 1.0f)) return -13;
    if (method == REF_TOPP && (!(temperature > 0.0f) || !isfinite(temperature))) return -5;
    if (method != REF_TOPK && method != REF_TOPP) return -13;
    int bad = 0;
#pragma omp parallel
    {
        ref_kv_t* kv = (ref_kv_t*)malloc(sizeof(ref_kv_t) * (size_t)vocab);
        char* keep = (char*)malloc((size_t)vocab);
        if (!kv || !keep) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < rows; ++r) {
            if (!kv || !keep) continue;
            const int64_t off = (int64_t)r * vocab;
            for (int v = 0; v < vocab; ++v) {
                kv[v].z = load_elem(z, dtype, off + v);
                kv[v].v = v;
            }
            qsort(kv, (size_t)vocab, sizeof(ref_kv_t), kv_desc);
            memset(keep, 0, (size_t)vocab);
            int nk = 0, fl = 0;
            if (method == REF_TOPK) {
                nk = k < vocab ? k : vocab;
            } else if (top_p >= 1.0f) {
                nk = vocab;
            } else {
                const double m = kv[0].z;
                double s = 0.0;
                for (int v = 0; v < vocab; ++v) s += exp((load_elem(z, dtype, off + v) - m) / (double)temperature);
                double c = 0.0, prev = 0.0;
                nk = vocab;
                for (int j = 0; j < vocab; ++j) {
                    prev = c;
                    c += exp((kv[j].z - m) / (double)temperature) / s;
                    if (c >= (double)top_p) { nk = j + 1; break; }
                }
                if (near_boundary((double)top_p, prev, 1e-9) || near_boundary((double)top_p, c, 1e-9)) fl = 1;
            }
            for (int j = 0; j < nk; ++j) keep[kv[j].v] = 1;
            for (int v = 0; v < vocab; ++v) {
                if (keep[v]) store_elem(out, dtype, off + v, z);
                else store_neg_inf(out, dtype, off + v);
            }
            if (kept) kept[r] = nk;
            if (flag) flag[r] = fl;
        }
        free(kv);
        free(keep);
    }
    return bad ? -10 : 0;
}
