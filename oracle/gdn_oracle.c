/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * of the package entry file and the benchmark's CPU-baseline leg may load this
 * library.  It shares no code, header, table or helper with the HIP path.
 *
 * What it computes (per sequence s and head h, independently):
 *
 *   The state M is head_dim x head_dim, stored [value][key]: row i is a value
 *   channel, column j a key channel ("ggml attention kernels" model card,
 *   huggingface.co/marcsun13/ggml-gated-delta-net, the contract notes under
 *   "Shapes, in torch order", second bullet).  For each token t of the call:
 *
 *     alpha = exp(g_t)                 g is a log-domain gate that the op
 *                                      exponentiates itself (same card, the
 *                                      paragraph after the contract bullets)
 *     M     = alpha * M                gating: scale the whole summary down
 *                                      ("Gated Delta Net on AMD: why ROCm
 *                                      stumbles on hybrid-attention LLMs",
 *                                      velstech.net, section "What Gated Delta
 *                                      Net is, in plain language", Gating)
 *     u     = M k_t                    what the decayed state holds under k_t
 *     delta = beta_t (v_t - u)         delta rule: overwrite that part rather
 *     M     = M + delta k_t^T          than append (same section, Delta rule)
 *     out_t = (1/sqrt(head_dim)) M q_t readout after the write; the op applies
 *                                      the 1/sqrt(head_dim) scaling itself
 *                                      (model card, paragraph after bullets)
 *
 *   Shapes follow the card's "Shapes, in torch order" table: q, k, v and out
 *   are (n_seqs, n_tokens, n_heads, head_dim); g and beta are
 *   (n_seqs, n_tokens, n_heads); the state is (n_seqs, n_heads, d, d).
 *   q and k carry one head per value head (first contract bullet), so head h
 *   of q/k pairs with head h of v.
 *
 *   Reading taken where the pages leave the order open: the retrieval u is
 *   taken from the already-decayed state, and the readout comes after the
 *   token's own write.  Under that reading beta = 1 and a unit key make the
 *   write an exact overwrite for any gate, which the pins check.
 *
 * Two forms are provided:
 *   oracle_gdn_recurrent -- the token recurrence above, written out plainly.
 *   oracle_gdn_chunked   -- the same result reorganised into chunks of C
 *                           tokens: the chunked kernel that the velstech
 *                           page (section "Why this bites AMD users
 *                           specifically") says llama.cpp lacks on ROCm,
 *                           which runs the recurrence in parallel blocks.
 *                           Used only to check the first form and to give
 *                           stage-by-stage values.
 *
 * Inputs q, k, v, g, beta are fp32 storage (bf16 inputs arrive already widened
 * to fp32, which is exact); every operation here is fp64.  The initial state is
 * fp64 so that a carried state is passed on without rounding.
 *
 * ORACLE_MUTANT (a compile-time number, 0 and absent in every normal build)
 * plants one plausible mistake in the token recurrence, so that a test can show
 * each of them is caught by the pins: 1 readout before the token's write,
 * 2 no 1/sqrt(head_dim), 3 the state read transposed, 4 the gate applied after
 * the retrieval, 5 the delta's sign flipped, 6 beta dropped from the delta.
 */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static long idx_tok(long s, long t, long h, long j, long T, long H, long d)
{
    return ((s * T + t) * H + h) * d + j;
}

static long idx_gate(long s, long t, long h, long T, long H)
{
    return (s * T + t) * H + h;
}

static long idx_state(long s, long h, long i, long j, long H, long d)
{
    return ((s * H + h) * d + i) * d + j;
}

/* Optional transforms of raw inputs, applied in fp64 before the step (the
 * steps that precede the op in a model layer, done inside it on request):
 *   ORACLE_L2NORM_QK  q_t <- q_t / sqrt(|q_t|^2 + ORACLE_L2_EPS), same for k_t
 *   ORACLE_RAW_GATES  g_t <- -softplus(g_t) = -log(1 + exp(g_t)),
 *                     beta_t <- sigmoid(beta_t) = 1 / (1 + exp(-beta_t))
 * The epsilon keeps an all-zero row at zero instead of dividing by zero. */
#define ORACLE_L2NORM_QK 1
#define ORACLE_RAW_GATES 2
#define ORACLE_L2_EPS 1e-6

/* x <- x / sqrt(|x|^2 + eps) */
static void l2_normalize(double *x, long d)
{
    double ss = 0.0;
    for (long j = 0; j < d; ++j)
        ss += x[j] * x[j];
    const double r = 1.0 / sqrt(ss + ORACLE_L2_EPS);
    for (long j = 0; j < d; ++j)
        x[j] *= r;
}

/* log(1 + exp(x)) without overflow: max(x, 0) + log1p(exp(-|x|)) */
static double softplus(double x)
{
    return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* out_t = scale * M q_t for one (seq, head) and token t. */
static void readout(const double *M, const double *qt, double *out, double scale, long s,
                    long t, long h, long T, long H, long d)
{
    for (long i = 0; i < d; ++i) {
        double acc = 0.0;
        for (long j = 0; j < d; ++j)
            acc += M[i * d + j] * qt[j];
        out[idx_tok(s, t, h, i, T, H, d)] = scale * acc;
    }
}

/* Token-sequential recurrence for one (seq, head).  M is d*d doubles, u is 3*d
 * doubles of scratch. */
static void recur_one(const float *q, const float *k, const float *v,
                      const float *g, const float *beta, double *out,
                      double *M, double *u, long s, long h, long T, long H,
                      long d, int flags)
{
    const double scale = ORACLE_MUTANT == 2 ? 1.0 : 1.0 / sqrt((double)d);
    double *kt = u + d, *qt = u + 2 * d;
    for (long t = 0; t < T; ++t) {
        for (long j = 0; j < d; ++j) {
            kt[j] = (double)k[idx_tok(s, t, h, j, T, H, d)];
            qt[j] = (double)q[idx_tok(s, t, h, j, T, H, d)];
        }
        const float *vt = v + idx_tok(s, t, h, 0, T, H, d);
        double gt = (double)g[idx_gate(s, t, h, T, H)];
        double b = (double)beta[idx_gate(s, t, h, T, H)];
        if (flags & ORACLE_L2NORM_QK) {
            l2_normalize(kt, d);
            l2_normalize(qt, d);
        }
        if (flags & ORACLE_RAW_GATES) {
            gt = -softplus(gt);
            b = 1.0 / (1.0 + exp(-b));
        }
        const double alpha = exp(gt);

        if (ORACLE_MUTANT != 4)
            for (long i = 0; i < d * d; ++i)
                M[i] *= alpha;
        for (long i = 0; i < d; ++i) {
            double acc = 0.0;
            for (long j = 0; j < d; ++j)
                acc += (ORACLE_MUTANT == 3 ? M[j * d + i] : M[i * d + j]) * kt[j];
            u[i] = acc;
        }
        if (ORACLE_MUTANT == 4)
            for (long i = 0; i < d * d; ++i)
                M[i] *= alpha;
        if (ORACLE_MUTANT == 1)
            readout(M, qt, out, scale, s, t, h, T, H, d);
        for (long i = 0; i < d; ++i) {
            double delta = b * ((double)vt[i] - u[i]);
            if (ORACLE_MUTANT == 5)
                delta = -delta;
            if (ORACLE_MUTANT == 6)
                delta = (double)vt[i] - u[i];
            for (long j = 0; j < d; ++j)
                M[i * d + j] += delta * kt[j];
        }
        if (ORACLE_MUTANT != 1)
            readout(M, qt, out, scale, s, t, h, T, H, d);
    }
}

static void set_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* out: (S, T, H, d) fp64.  state_out: (S, H, d, d) fp64.  state_in may be NULL
 * for a zero initial state.  flags: ORACLE_L2NORM_QK | ORACLE_RAW_GATES or 0.
 * Returns 0, or -1 on allocation failure or unknown flags. */
int oracle_gdn_recurrent(const float *q, const float *k, const float *v,
                         const float *g, const float *beta,
                         const double *state_in, double *out,
                         double *state_out, long S, long T, long H, long d,
                         int flags, int n_threads)
{
    if (flags & ~(ORACLE_L2NORM_QK | ORACLE_RAW_GATES))
        return -1;
    int failed = 0;
    set_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long sh = 0; sh < S * H; ++sh) {
        const long s = sh / H, h = sh % H;
        double *M = state_out + idx_state(s, h, 0, 0, H, d);
        double *u = (double *)malloc(sizeof(double) * (size_t)(3 * d));
        if (!u) {
            failed = 1;
            continue;
        }
        if (state_in)
            memcpy(M, state_in + idx_state(s, h, 0, 0, H, d),
                   sizeof(double) * (size_t)(d * d));
        else
            memset(M, 0, sizeof(double) * (size_t)(d * d));
        recur_one(q, k, v, g, beta, out, M, u, s, h, T, H, d, flags);
        free(u);
    }
    return failed ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * Chunked form.  For a chunk of n <= C tokens starting from state M_n, with
 * local inclusive gate sums gam_r = g_0 + ... + g_r (r counted inside the
 * chunk):
 *   A[r][s] = beta_r exp(gam_r - gam_s) (k_r . k_s)       for s < r, else 0
 *   T       = (I + A)^{-1}                                (forward substitution)
 *   W       = T diag(beta exp(gam)) K,   U = T diag(beta) V
 *   Delta   = U - W M_n^T                  (row r = the delta vector of token r)
 *   P[r][s] = exp(gam_r - gam_s) (q_r . k_s)               for s <= r, else 0
 *   O       = scale (diag(exp(gam)) Q M_n^T + P Delta)
 *   M_{n+1} = exp(gam_last) M_n + sum_s exp(gam_last - gam_s) Delta_s k_s^T
 * Only differences gam_r - gam_s with s <= r are exponentiated, so nothing
 * overflows however strong the decay.
 * ------------------------------------------------------------------------- */

struct chunk_scratch {
    double *gam, *A, *T, *W, *U, *Delta, *P, *Mnew;
};

static int scratch_alloc(struct chunk_scratch *w, long C, long d)
{
    w->gam = malloc(sizeof(double) * (size_t)C);
    w->A = malloc(sizeof(double) * (size_t)(C * C));
    w->T = malloc(sizeof(double) * (size_t)(C * C));
    w->W = malloc(sizeof(double) * (size_t)(C * d));
    w->U = malloc(sizeof(double) * (size_t)(C * d));
    w->Delta = malloc(sizeof(double) * (size_t)(C * d));
    w->P = malloc(sizeof(double) * (size_t)(C * C));
    w->Mnew = malloc(sizeof(double) * (size_t)(d * d));
    return (w->gam && w->A && w->T && w->W && w->U && w->Delta && w->P &&
            w->Mnew)
               ? 0
               : -1;
}

static void scratch_free(struct chunk_scratch *w)
{
    free(w->gam);
    free(w->A);
    free(w->T);
    free(w->W);
    free(w->U);
    free(w->Delta);
    free(w->P);
    free(w->Mnew);
}

static double dot_f(const float *a, const float *b, long d)
{
    double acc = 0.0;
    for (long j = 0; j < d; ++j)
        acc += (double)a[j] * (double)b[j];
    return acc;
}

/* One chunk [t0, t0+n) of one (seq, head).  M (d x d) is updated in place;
 * out rows are written.  All matrices are row-major with the chunk-local
 * token index first. */
static void chunk_one(const float *q, const float *k, const float *v,
                      const float *g, const float *beta, double *out,
                      double *M, struct chunk_scratch *w, long s, long h,
                      long t0, long n, long T, long H, long d)
{
    const double scale = 1.0 / sqrt((double)d);
#define KROW(r) (k + idx_tok(s, t0 + (r), h, 0, T, H, d))
#define QROW(r) (q + idx_tok(s, t0 + (r), h, 0, T, H, d))
#define VROW(r) (v + idx_tok(s, t0 + (r), h, 0, T, H, d))
#define BETA(r) ((double)beta[idx_gate(s, t0 + (r), h, T, H)])

    double run = 0.0;
    for (long r = 0; r < n; ++r) {
        run += (double)g[idx_gate(s, t0 + r, h, T, H)];
        w->gam[r] = run;
    }
    const double gl = w->gam[n - 1];

    for (long r = 0; r < n; ++r)
        for (long c = 0; c < n; ++c)
            w->A[r * n + c] =
                (c < r) ? BETA(r) * exp(w->gam[r] - w->gam[c]) *
                              dot_f(KROW(r), KROW(c), d)
                        : 0.0;

    /* T = (I + A)^{-1}: row r of (I + A) T = I gives
     * T[r][c] = [r == c] - sum_{s < r} A[r][s] T[s][c]. */
    for (long r = 0; r < n; ++r)
        for (long c = 0; c < n; ++c) {
            double acc = (r == c) ? 1.0 : 0.0;
            for (long x = 0; x < r; ++x)
                acc -= w->A[r * n + x] * w->T[x * n + c];
            w->T[r * n + c] = acc;
        }

    for (long r = 0; r < n; ++r)
        for (long j = 0; j < d; ++j) {
            double aw = 0.0, au = 0.0;
            for (long x = 0; x < n; ++x) {
                aw += w->T[r * n + x] * BETA(x) * exp(w->gam[x]) *
                      (double)KROW(x)[j];
                au += w->T[r * n + x] * BETA(x) * (double)VROW(x)[j];
            }
            w->W[r * d + j] = aw;
            w->U[r * d + j] = au;
        }

    for (long r = 0; r < n; ++r)
        for (long i = 0; i < d; ++i) {
            double acc = 0.0;
            for (long j = 0; j < d; ++j)
                acc += w->W[r * d + j] * M[i * d + j];
            w->Delta[r * d + i] = w->U[r * d + i] - acc;
        }

    for (long r = 0; r < n; ++r)
        for (long c = 0; c < n; ++c)
            w->P[r * n + c] =
                (c <= r) ? exp(w->gam[r] - w->gam[c]) *
                               dot_f(QROW(r), KROW(c), d)
                         : 0.0;

    for (long r = 0; r < n; ++r)
        for (long i = 0; i < d; ++i) {
            double inter = 0.0, intra = 0.0;
            for (long j = 0; j < d; ++j)
                inter += (double)QROW(r)[j] * M[i * d + j];
            for (long c = 0; c < n; ++c)
                intra += w->P[r * n + c] * w->Delta[c * d + i];
            out[idx_tok(s, t0 + r, h, i, T, H, d)] =
                scale * (exp(w->gam[r]) * inter + intra);
        }

    for (long i = 0; i < d; ++i)
        for (long j = 0; j < d; ++j) {
            double acc = 0.0;
            for (long c = 0; c < n; ++c)
                acc += exp(gl - w->gam[c]) * w->Delta[c * d + i] *
                       (double)KROW(c)[j];
            w->Mnew[i * d + j] = exp(gl) * M[i * d + j] + acc;
        }
    memcpy(M, w->Mnew, sizeof(double) * (size_t)(d * d));
#undef KROW
#undef QROW
#undef VROW
#undef BETA
}

int oracle_gdn_chunked(const float *q, const float *k, const float *v,
                       const float *g, const float *beta,
                       const double *state_in, double *out, double *state_out,
                       long S, long T, long H, long d, long C, int n_threads)
{
    int failed = 0;
    if (C < 1)
        return -2;
    set_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long sh = 0; sh < S * H; ++sh) {
        const long s = sh / H, h = sh % H;
        double *M = state_out + idx_state(s, h, 0, 0, H, d);
        struct chunk_scratch w;
        memset(&w, 0, sizeof(w));
        if (scratch_alloc(&w, C, d)) {
            scratch_free(&w);
            failed = 1;
            continue;
        }
        if (state_in)
            memcpy(M, state_in + idx_state(s, h, 0, 0, H, d),
                   sizeof(double) * (size_t)(d * d));
        else
            memset(M, 0, sizeof(double) * (size_t)(d * d));
        for (long t0 = 0; t0 < T; t0 += C) {
            const long n = (T - t0 < C) ? (T - t0) : C;
            chunk_one(q, k, v, g, beta, out, M, &w, s, h, t0, n, T, H, d);
        }
        scratch_free(&w);
    }
    return failed ? -1 : 0;
}

/* Stage values of one chunk of a single-sequence, single-head problem (inputs
 * shaped (1, n, 1, d), the chunk being all n tokens), starting from state M
 * (d x d, updated in place to the state after the chunk).  Any output pointer
 * may be NULL.  Shapes: gam n; A, T, P n x n; W, U, Delta n x d; out n x d. */
int oracle_gdn_chunk_stages(const float *q, const float *k, const float *v,
                            const float *g, const float *beta, double *M,
                            long n, long d, double *gam, double *A, double *Tm,
                            double *P, double *W, double *U, double *Delta,
                            double *out)
{
    struct chunk_scratch w;
    memset(&w, 0, sizeof(w));
    double *o = (double *)malloc(sizeof(double) * (size_t)(n * d));
    if (!o || scratch_alloc(&w, n, d)) {
        free(o);
        scratch_free(&w);
        return -1;
    }
    chunk_one(q, k, v, g, beta, o, M, &w, 0, 0, 0, n, n, 1, d);
#define COPY(dst, src, cnt)                                                    \
    do {                                                                       \
        if (dst)                                                               \
            memcpy(dst, src, sizeof(double) * (size_t)(cnt));                  \
    } while (0)
    COPY(gam, w.gam, n);
    COPY(A, w.A, n * n);
    COPY(Tm, w.T, n * n);
    COPY(P, w.P, n * n);
    COPY(W, w.W, n * d);
    COPY(U, w.U, n * d);
    COPY(Delta, w.Delta, n * d);
    COPY(out, o, n * d);
#undef COPY
    scratch_free(&w);
    free(o);
    return 0;
}
