/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) verify-and-sample library
 * for speculative decoding.
 *
 * The operation ("Fast Inference from Transformers via Speculative
 * Decoding", paper summary page, "Speculative Sampling: The Core
 * Algorithm", Algorithm 1 Phases 3 and 4; "Speculative Decoding Paper
 * Breakdown: Lossless Draft-and-Verify Acceleration for Autoregressive
 * Transformers", section 3 "The Algorithm at Position i"; "Speculative
 * Decoding: Two Models, One Output", "The algorithm"):
 *
 *   for each sequence b, positions i = 0 .. gamma-1 in order:
 *     p_i = softmax(target_logits[b][i] / T)           ("Standardized Sampling")
 *     accept x_i iff u_i <= min(1, p_i(x_i) / q_i(x_i))  (q_i(x_i) <= 0: accept)
 *     stop at the first rejection; n = number accepted (0 .. gamma)
 *   if n < gamma: t ~ norm(max(0, p_n - q_n)), or t ~ p_n when that residual
 *                 mass is <= 1e-15 ("The exact decoding shortcut that burns
 *                 compute when guesses miss", correction_distribution)
 *   if n == gamma: bonus token t ~ p_gamma
 *   emit x_0 .. x_{n-1}, t   (between 1 and gamma+1 tokens)
 *
 * Draws use the caller's uniforms: u_i = uniforms[b][i] for the acceptance
 * test at position i, u_gamma = uniforms[b][gamma] for the one final draw,
 * by inverse CDF (the smallest k whose running weight sum exceeds
 * u * total).  In greedy mode every distribution is the point mass at the
 * first index attaining the row maximum of the raw logits ("Standardized
 * Sampling", argmax case): a draft survives iff it equals that argmax and
 * the emitted token is the argmax of the row where the walk stopped.
 *
 * Every tensor argument is a DEVICE pointer on the current HIP device,
 * row-major and contiguous, owned by the caller.  The library never
 * allocates, frees or synchronises; a call only enqueues kernels on
 * `stream` (a hipStream_t; NULL = the default stream) and returns.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  SV_BF16 data are raw bfloat16 bit patterns (uint16). */
#define SV_FP32 0
#define SV_BF16 1

/* Modes. */
#define SV_SAMPLE 0 /* temperature sampling, exact rejection rule            */
#define SV_GREEDY 1 /* argmax standardisation; T, draft_probs, uniforms unused */

/* Largest supported gamma: the gamma + 1 rows of a sequence are the bits of
 * a 64-bit word (the reject mask uses bits 0 .. gamma-1 and keeps bit 63 for
 * an invalid draft token). */
#define SV_MAX_GAMMA 63

/* Status codes returned synchronously by every entry point. */
#define SV_OK 0
#define SV_ERR_NULL_POINTER -1  /* a required pointer is NULL                        */
#define SV_ERR_BATCH -2         /* batch < 1                                         */
#define SV_ERR_GAMMA -3         /* gamma < 1 or gamma > SV_MAX_GAMMA                 */
#define SV_ERR_VOCAB -4         /* vocab < 1                                         */
#define SV_ERR_TEMPERATURE -5   /* sample mode with temperature <= 0 or not finite  */
#define SV_ERR_DTYPE -6         /* dtype tag is neither SV_FP32 nor SV_BF16          */
#define SV_ERR_MODE -7          /* mode is neither SV_SAMPLE nor SV_GREEDY           */
#define SV_ERR_WORKSPACE -8     /* workspace NULL or smaller than sv_workspace_bytes */
#define SV_ERR_ALIGNMENT -9     /* a pointer is not aligned to its element size, or
                                   the workspace is not 256-byte aligned             */
#define SV_ERR_TOO_LARGE -10    /* the problem exceeds the launch-grid limits, or
                                   batch > 67 108 861 in sample mode               */
#define SV_ERR_LAUNCH -11       /* the HIP runtime rejected a kernel launch          */
#define SV_ERR_LENIENCE -12     /* sample mode with lenience outside [0, 1]          */
#define SV_ERR_STANDARDIZE -13  /* unknown method, k < 1, or top_p outside (0, 1]    */
#define SV_ERR_SCRATCH -14      /* spec_verify_noalloc: sv_workspace_bytes() of the
                                   shape exceeds SV_NOALLOC_SCRATCH_BYTES            */

/* Size of the static per-GPU scratch array of spec_verify_noalloc. */
#define SV_NOALLOC_SCRATCH_BYTES (8u << 20)

/* Standardisation methods (sv_standardize). */
#define SV_TOPK 0
#define SV_TOPP 1

/* Optional outputs for tests and telemetry (every pointer may be NULL;
 * all are device pointers).  Values for positions the walk did not reach
 * are NaN. */
typedef struct {
    double* p_tok;      /* [B][gamma]   p_i(x_i) for every tested position i       */
    double* q_tok;      /* [B][gamma]   q_i(x_i) for every tested position i       */
    double* resid_mass; /* [B]          sum_v max(0, p_n - q_n) when n < gamma     */
    float*  row_max;    /* [B][gamma+1] max_v z of each row the walk normalised
                                        (sample) or examined (greedy)            */
    double* row_sum;    /* [B][gamma+1] sum_v exp((z - row_max) / T), sample mode */
    double* p_out;      /* [B]          p_n(t): the target probability, at T, of the
                                        token t drawn at position n (the bonus
                                        token when n = gamma), sample mode      */
    /* hipEvent_t handles recorded on `stream`: before the first launch,
     * after the first launch (the row stage, which in sample mode also
     * streams most of the draw), and after the last launch.  Any may be
     * NULL.  For V <= 512 without telemetry the call is a single launch (one
     * wave per sequence), and ev_mid is recorded after it, like ev_end. */
    void* ev_begin;
    void* ev_mid;
    void* ev_end;
    /* Acceptance-rate telemetry, sample mode only ("Fast Inference from
     * Transformers via Speculative Decoding", paper summary page,
     * "Computing alpha from p and q: The DLK Divergence", Theorem 3.5: the
     * probability that the draft at position i is accepted is
     * beta_i = sum_v min(p_i(v), q_i(v)) = 1 - DLK(p_i, q_i); alpha is its
     * expectation, "Expected Number of Generated Tokens").  Computed for
     * EVERY position i < gamma of every sequence, reached by the walk or not
     * (valid draft tokens or not), with q used as given.  Either pointer
     * non-NULL makes the call stream every target row and every draft row:
     * the early exit after a rejection is switched off, and a second sweep
     * over target rows 0..gamma-1 and the draft rows follows the row stage.
     * The verification results are the same as without telemetry.  Ignored
     * in greedy mode. */
    double* beta;       /* [B][gamma]   beta of position i of sequence b        */
    double* alpha;      /* [gamma]      mean over the batch of beta[.][i]       */
    /* hipEvent_t recorded after the telemetry sweep (before the last launch)
     * when the sweep runs; may be NULL. */
    void* ev_tele;
    /* Device counter (may be NULL): incremented once for every sequence
     * whose outputs were withheld because a bounded device-side wait for
     * another workgroup's partial result ran out (n_accepted[b] = -2, every
     * token -1; see spec_verify).  The caller zeroes it. */
    uint32_t* error_count;
    /* Tests of that failure path only; leave both 0.  withhold_partial =
     * k + 1 makes the workgroup of the first chunk of every row at position
     * k withhold its partial row statistics (sample mode, vocab > 512), and
     * wait_polls > 0 bounds the merge's wait for a partial to that many
     * polls, so that the wait runs out and the sequences are reported as
     * failed while every kernel still completes normally. */
    int32_t withhold_partial;
    int32_t wait_polls;
    /* Test of the draw's fallback only; leave 0.  help_polls > 0 bounds the
     * wait of the first launch's draw helpers for their sequence to that
     * many polls (sample mode, vocab > 512, no telemetry); a helper whose
     * wait runs out leaves its draw chunk to the last launch.  The results
     * are the same for any value. */
    int32_t help_polls;
} sv_extras_t;

/* sizeof(sv_extras_t) as this library was built: a binding that mirrors
 * the struct checks its own size against it before passing one. */
size_t sv_extras_bytes(void);

/* Workspace size in bytes for a problem shape (any mode). */
size_t sv_workspace_bytes(int batch, int gamma, int vocab);

/* Zero-fills `bytes` bytes of a workspace on `stream` with a kernel.  A
 * workspace must be zero-filled once before its first use; every call of
 * spec_verify that returns SV_OK leaves it zero-filled again when the
 * stream has finished the call, for any later problem shape.  After
 * SV_ERR_LAUNCH, zero-fill it again.  Returns SV_OK or SV_ERR_*. */
int sv_workspace_init(void* workspace, size_t bytes, void* stream);

/*
 * spec_verify -- the batched verify-and-sample step.
 *
 *   batch, gamma, vocab   B >= 1, 1 <= gamma <= SV_MAX_GAMMA, V >= 1
 *   target_logits         [B][gamma+1][V], logits_dtype; finite values or -inf,
 *                         every row with a finite maximum
 *   draft_probs           [B][gamma][V], probs_dtype; q >= 0, used as given
 *                         (not renormalised).  Unused (may be NULL) in greedy mode
 *   draft_tokens          [B][gamma] int32.  A token outside [0, V) makes the
 *                         whole sequence invalid: n_accepted[b] = -1 and
 *                         out_tokens[b][*] = -1
 *   uniforms              [B][gamma+1] fp32 in (0, 1).  Unused (may be NULL) in
 *                         greedy mode
 *   temperature           T > 0, finite, in sample mode; ignored in greedy mode
 *   mode                  SV_SAMPLE or SV_GREEDY
 *   n_accepted            [B] int32 out: accepted drafts n in [0, gamma]; -1 for
 *                         an invalid draft token; -2 if a bounded device-side
 *                         wait for another workgroup's partial row statistics
 *                         ran out (never expected: the wait covers stores that
 *                         were issued before the count that started it; the
 *                         sequence's tokens are then all -1 and
 *                         extras->error_count, if given, counts it)
 *   out_tokens            [B][gamma+1] int32 out: x_0..x_{n-1}, t, then -1
 *   workspace             device buffer of >= sv_workspace_bytes(B, gamma, V)
 *                         bytes, 256-byte aligned, zero-filled before first use
 *                         (sv_workspace_init); calls that overlap on the same
 *                         workspace race.  (Always checked; the single-launch
 *                         path for V <= 512 does not touch it.)
 *   extras                optional outputs / timing events, or NULL
 *   stream                hipStream_t to enqueue on
 *
 * Returns SV_OK after enqueueing, or a negative SV_ERR_* code without
 * touching any buffer.  Results are valid once the stream reaches them.
 */
int spec_verify(int batch, int gamma, int vocab,
                const void* target_logits, int logits_dtype,
                const void* draft_probs, int probs_dtype,
                const int32_t* draft_tokens, const float* uniforms,
                float temperature, int mode,
                int32_t* n_accepted, int32_t* out_tokens,
                void* workspace, size_t workspace_bytes,
                const sv_extras_t* extras, void* stream);

/*
 * spec_verify_lenient -- spec_verify with a lenience l in [0, 1] ("Fast
 * Inference from Transformers via Speculative Decoding", summary page,
 * "Ablation Studies and Robustness Checks", Appendix A.5: l multiplies
 * q(x) before it is compared with p(x), for a higher acceptance rate at the
 * price of exactness; "How This Work Changes the Landscape": no token is
 * then sampled with probability above p(x)/l).  A draft is accepted iff
 * u_i <= min(1, p_i(x_i) / (l q_i(x_i))) (q <= 0 accepts); after a rejection
 * the correction is drawn from norm(max(0, p_n - l q_n)), with the same
 * fallback to p_n at residual mass <= 1e-15 (the pages give only the
 * acceptance side; this residual is the same comparison's).  l = 1 is
 * exactly spec_verify; l = 0 accepts every draft.  resid_mass reports the
 * lenient residual's mass.  Every other argument as for spec_verify; greedy
 * mode ignores l.  Returns SV_ERR_LENIENCE for l outside [0, 1] (NaN
 * included) in sample mode.
 */
int spec_verify_lenient(int batch, int gamma, int vocab,
                        const void* target_logits, int logits_dtype,
                        const void* draft_probs, int probs_dtype,
                        const int32_t* draft_tokens, const float* uniforms,
                        float temperature, float lenience, int mode,
                        int32_t* n_accepted, int32_t* out_tokens,
                        void* workspace, size_t workspace_bytes,
                        const sv_extras_t* extras, void* stream);

/*
 * spec_verify_noalloc -- spec_verify_lenient without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * allocates nothing: its workspace is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES (8 MiB) in the library, one per GPU, held until
 * the process ends.  The first call on a device looks up the array's
 * address and zero-fills it with a kernel on `stream`; every completed call
 * leaves it zero again.  Every call on one GPU shares that GPU's array:
 * calls that overlap on the same GPU (other streams, other threads) race,
 * and after SV_ERR_LAUNCH the array must be considered dirty (later calls
 * may give wrong results).  Returns SV_ERR_SCRATCH, without launching
 * anything, when sv_workspace_bytes(batch, gamma, vocab) exceeds the array
 * (batch up to 1231 at gamma 8 and vocab 152 064 fits, and up to 475 at
 * gamma 16 and vocab 256 000).  Every other argument, the results and the status codes as for
 * spec_verify_lenient.
 */
int spec_verify_noalloc(int batch, int gamma, int vocab,
                        const void* target_logits, int logits_dtype,
                        const void* draft_probs, int probs_dtype,
                        const int32_t* draft_tokens, const float* uniforms,
                        float temperature, float lenience, int mode,
                        int32_t* n_accepted, int32_t* out_tokens,
                        const sv_extras_t* extras, void* stream);

/*
 * sv_standardize -- top-k or nucleus (top-p) standardisation of rows of
 * target logits ("Fast Inference from Transformers via Speculative
 * Decoding", summary page, "Standardized Sampling": top-k keeps the k
 * largest probabilities, nucleus sorts them and keeps those up to the point
 * where the running sum reaches top_p, and both renormalise; the verify step
 * then compares these standardised distributions).  For each of `rows` rows
 * of `vocab` logits, writes the row to logits_out with every dropped entry
 * set to -inf, so that softmax(out / T) is exactly the standardised
 * distribution and spec_verify can take logits_out as its target_logits.
 *
 *   rows, vocab    R >= 1 rows of V >= 1 entries, contiguous, row-major
 *   logits         [R][V] device, dtype SV_FP32 or SV_BF16; finite or -inf
 *   method         SV_TOPK (k >= 1; k >= V keeps the row) or SV_TOPP
 *                  (0 < top_p <= 1, temperature T > 0 finite: the nucleus is
 *                  taken on softmax(z / T))
 *   logits_out     [R][V] device, same dtype; may equal logits (in place)
 *   stream         hipStream_t
 *
 * Ties in value are ordered by index: top-k keeps exactly min(k, V)
 * entries, and the nucleus keeps the shortest prefix of the order (value
 * decreasing, index increasing) whose probability reaches top_p (every
 * entry if rounding keeps the running sum below top_p; top_p = 1 keeps
 * every entry).  -0 and +0 are
 * equal values.  The draft side standardises its own q before sampling
 * (the caller's q is used as given).  Returns SV_OK after enqueueing, or
 * SV_ERR_* without touching any buffer.
 */
int sv_standardize(int rows, int vocab, const void* logits, int dtype, int method, int k, float top_p,
                   float temperature, void* logits_out, void* stream);

/* Static description of a status code (never NULL). */
const char* sv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
