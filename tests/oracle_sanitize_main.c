/* Memory and undefined-behaviour check of the fp64 oracle (test side only).
 *
 * Built by tests/test_oracle_sanitizers.py with gcc's AddressSanitizer and
 * UndefinedBehaviorSanitizer into a standalone program that includes the
 * oracle's source, then run on the CPU.  It calls every entry point of the
 * oracle over seeded random shapes and inputs with the awkward cases in them
 * (vocabularies of 1, 2 and 3 entries, gamma up to 63, -inf logits, zero
 * draft probabilities, out-of-range draft tokens, uniforms of 0 and 1,
 * lenience 0 and 1, top-k with k above V, nucleus at 1), every output and
 * auxiliary array allocated to its exact size so that any access past an end
 * is caught.  Any sanitizer report ends the program with a non-zero status.
 * The results themselves are checked elsewhere; here only that the calls
 * succeed or refuse their arguments as documented.
 */
#include "../oracle/spec_verify_ref.c"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void)
{
    /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

static double uniform01(void) { return (double)(next_u64() >> 11) * 0x1p-53; }

static int below(int n) { return (int)(next_u64() % (uint64_t)n); }

static uint16_t to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* An array of count elements of dtype (fp32 or bf16), exactly sized. */
static void* alloc_elems(int dtype, int64_t count)
{
    return malloc((size_t)count * (dtype == REF_BF16 ? 2 : 4));
}

static void put(void* base, int dtype, int64_t i, float v)
{
    if (dtype == REF_BF16) ((uint16_t*)base)[i] = to_bf16(v);
    else ((float*)base)[i] = v;
}

static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(3);
    }
    return p;
}

static int run_verify(int B, int gamma, int V, int zd, int qd, float T, float lenience, int mode, int threads,
                      int with_aux, int with_tele)
{
    const int G1 = gamma + 1;
    void* z = alloc_elems(zd, (int64_t)B * G1 * V);
    void* q = alloc_elems(qd, (int64_t)B * gamma * V);
    int32_t* x = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)B * gamma);
    float* u = (float*)xmalloc(sizeof(float) * (size_t)B * G1);
    for (int64_t i = 0; i < (int64_t)B * G1 * V; ++i) {
        const int pick = below(40);
        float v = (float)(3.0 * (uniform01() * 2.0 - 1.0) * 3.0);
        if (pick == 0) v = -INFINITY;
        put(z, zd, i, v);
    }
    /* keep one finite logit per row */
    for (int64_t r = 0; r < (int64_t)B * G1; ++r) put(z, zd, r * V + below(V), 1.0f);
    for (int64_t r = 0; r < (int64_t)B * gamma; ++r) {
        double s = 0.0;
        double* w = (double*)xmalloc(sizeof(double) * (size_t)V);
        for (int v = 0; v < V; ++v) {
            w[v] = below(10) == 0 ? 0.0 : uniform01();
            s += w[v];
        }
        for (int v = 0; v < V; ++v) put(q, qd, r * V + v, s > 0.0 ? (float)(w[v] / s) : 0.0f);
        free(w);
    }
    for (int64_t i = 0; i < (int64_t)B * gamma; ++i) {
        const int pick = below(50);
        x[i] = pick == 0 ? -1 : pick == 1 ? V : below(V);
    }
    for (int64_t i = 0; i < (int64_t)B * G1; ++i) {
        const int pick = below(30);
        u[i] = pick == 0 ? 0.0f : pick == 1 ? 1.0f : (float)uniform01();
    }
    int32_t* n = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)B);
    int32_t* out = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)B * G1);
    ref_aux_t aux;
    memset(&aux, 0, sizeof(aux));
    if (with_aux) {
        aux.p_tok = (double*)xmalloc(sizeof(double) * (size_t)B * gamma);
        aux.q_tok = (double*)xmalloc(sizeof(double) * (size_t)B * gamma);
        aux.thr = (double*)xmalloc(sizeof(double) * (size_t)B * gamma);
        aux.resid_mass = (double*)xmalloc(sizeof(double) * (size_t)B);
        aux.row_max = (double*)xmalloc(sizeof(double) * (size_t)B * G1);
        aux.row_sum = (double*)xmalloc(sizeof(double) * (size_t)B * G1);
        aux.flag_pos = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)B);
        aux.n_decisions = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)B);
        aux.n_flags = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)B);
        aux.p_out = (double*)xmalloc(sizeof(double) * (size_t)B);
    }
    if (with_tele) {
        aux.beta = (double*)xmalloc(sizeof(double) * (size_t)B * gamma);
        aux.alpha = (double*)xmalloc(sizeof(double) * (size_t)gamma);
    }
    const int rc = spec_verify_ref(B, gamma, V, z, zd, mode == REF_SAMPLE ? q : NULL, qd, x,
                                   mode == REF_SAMPLE ? u : NULL, T, lenience, mode, n, out,
                                   (with_aux || with_tele) ? &aux : NULL, threads);
    int bad = rc != 0;
    for (int b = 0; b < B && !bad; ++b) bad = n[b] < -1 || n[b] > gamma;
    free(z);
    free(q);
    free(x);
    free(u);
    free(n);
    free(out);
    free(aux.p_tok);
    free(aux.q_tok);
    free(aux.thr);
    free(aux.resid_mass);
    free(aux.row_max);
    free(aux.row_sum);
    free(aux.flag_pos);
    free(aux.n_decisions);
    free(aux.n_flags);
    free(aux.beta);
    free(aux.alpha);
    free(aux.p_out);
    if (bad) fprintf(stderr, "spec_verify_ref: rc %d on B=%d gamma=%d V=%d\n", rc, B, gamma, V);
    return bad;
}

static int run_standardize(int rows, int V, int dtype, int method, int k, float top_p, float T)
{
    void* z = alloc_elems(dtype, (int64_t)rows * V);
    void* out = alloc_elems(dtype, (int64_t)rows * V);
    int32_t* kept = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)rows);
    int32_t* flag = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)rows);
    for (int64_t i = 0; i < (int64_t)rows * V; ++i) {
        const int pick = below(20);
        /* ties and -inf on purpose */
        put(z, dtype, i, pick == 0 ? -INFINITY : pick < 4 ? 0.5f : (float)(uniform01() * 6.0 - 3.0));
    }
    const int rc = ref_standardize(rows, V, z, dtype, method, k, top_p, T, out, kept, flag);
    const int expect_ok = method == REF_TOPK ? k >= 1 : (top_p > 0.0f && top_p <= 1.0f);
    int bad = expect_ok ? rc != 0 : rc == 0;
    for (int r = 0; r < rows && !bad && rc == 0; ++r) bad = kept[r] < 1 || kept[r] > V;
    free(z);
    free(out);
    free(kept);
    free(flag);
    if (bad) fprintf(stderr, "ref_standardize: rc %d on rows=%d V=%d method=%d k=%d p=%g\n", rc, rows, V, method, k,
                     (double)top_p);
    return bad;
}

int main(void)
{
    static const int vocabs[] = {1, 2, 3, 7, 16, 100, 513, 3000};
    static const float temps[] = {0.5f, 1.0f, 1.7f};
    static const float lens[] = {1.0f, 0.5f, 0.0f};
    int failures = 0;
    for (int trial = 0; trial < 60; ++trial) {
        const int V = vocabs[below(8)];
        const int gamma = trial == 0 ? 63 : 1 + below(8);
        const int B = 1 + below(6);
        const int zd = below(2) ? REF_BF16 : REF_FP32;
        const int qd = below(2) ? REF_BF16 : REF_FP32;
        const int mode = below(4) == 0 ? REF_GREEDY : REF_SAMPLE;
        failures += run_verify(B, gamma, V, zd, qd, temps[below(3)], lens[below(3)], mode, 1 + below(4),
                               below(4) != 0, mode == REF_SAMPLE && below(2));
    }
    for (int trial = 0; trial < 30; ++trial) {
        const int V = vocabs[below(8)];
        const int dtype = below(2) ? REF_BF16 : REF_FP32;
        const int ks[] = {0, 1, V / 2 + 1, V, V + 5};
        const float ps[] = {0.1f, 0.9f, 1.0f, 0.0f};
        if (below(2)) failures += run_standardize(1 + below(4), V, dtype, REF_TOPK, ks[below(5)], 1.0f, 1.0f);
        else failures += run_standardize(1 + below(4), V, dtype, REF_TOPP, 0, ps[below(4)], temps[below(3)]);
    }
    /* the single-row helpers */
    for (int trial = 0; trial < 20; ++trial) {
        const int V = vocabs[below(8)];
        float* z = (float*)xmalloc(sizeof(float) * (size_t)V);
        double* p = (double*)xmalloc(sizeof(double) * (size_t)V);
        for (int v = 0; v < V; ++v) z[v] = below(10) == 0 ? -INFINITY : (float)(uniform01() * 4.0);
        z[below(V)] = 2.0f;
        int flagged = 0;
        failures += ref_softmax_row(z, REF_FP32, V, 1.0f, p) != 0;
        const int t = ref_icdf(p, V, uniform01(), &flagged);
        failures += t < 0 || t >= V;
        const int a = ref_argmax_row(z, REF_FP32, V);
        failures += a < 0 || a >= V;
        free(z);
        free(p);
    }
    if (failures) fprintf(stderr, "%d failed calls\n", failures);
    printf("oracle sanitizer run: %d failed calls\n", failures);
    return failures ? 1 : 0;
}
