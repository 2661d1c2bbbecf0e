/*
 * ssd_oracle.c -- plain, slow, fp64 CPU oracle for the chunked linear recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the HIP library.
 *
 * Source of the method: the page "分块推理：解锁循环模型并行计算，实现长序列高效处理"
 * (chunked inference for recurrent models), cited below as [分块推理 §n].
 *
 *   [分块推理 §2]   the recurrence h_t = A_t h_{t-1} + B_t x_t,  y_t = C_t h_t,
 *                   and the chunk partition L = C * Q.
 *   [分块推理 §2.1] intra-chunk output by_intra(c) and local end state b_intra(c),
 *                   both computed from a zero initial state.
 *   [分块推理 §2.2] global state b(c) = b_intra(c) + (product of A_t over the chunk) b(c-1),
 *                   correction by_inter(c) = diag(L) C(c) b(c-1),  y(c) = by_intra + by_inter.
 *
 * Readings taken where the page is silent (each is listed in the design notes):
 *   - A_t is a per-(token, head) scalar a_t = exp(dt_t * A_h) (Mamba-2 diagonal form).
 *   - The state of one head is a P x N matrix; "B_t x_t" is the outer product
 *     x_t (P) (x) B_t (N); "C_t h_t" contracts over N.
 *   - The input term carries no dt factor: dt only enters through a_t.
 *   - A skip term D_h x_t is added to y_t; D may be absent (treated as 0).
 *   - Head h reads B/C group g = h / (H / G).
 *   - The product "from (c-1)Q to cQ" is taken over the tokens of chunk c, and diag(L)
 *     holds L_i = product of a_r from the chunk start up to and including token i.
 *   - The last chunk may be shorter than Q.
 *
 * Everything is double precision.  Decay products are formed by multiplying the a_t
 * themselves, so a_t = 0 is handled exactly.  Threads split the independent
 * (batch, head) pairs; each pair is computed by exactly the same sequential code.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t batch, L, H, P, N, G, Q;
    const double *x, *dt, *A, *B, *C, *D, *init;
    double *y, *final_state;
    /* chunked-only outputs (any may be NULL) */
    double *logcum, *b_intra, *b_in, *by_intra, *by_inter;
    int nthreads, tid;
    int mode; /* 0 = sequential recurrence, 1 = chunked decomposition */
} job_t;

#define IX_X(b, t, h, p)  ((((b) * j->L + (t)) * j->H + (h)) * j->P + (p))
#define IX_DT(b, t, h)    (((b) * j->L + (t)) * j->H + (h))
#define IX_BC(b, t, g, n) ((((b) * j->L + (t)) * j->G + (g)) * j->N + (n))
#define IX_S(b, h)        (((b) * j->H + (h)) * j->P * j->N)

/* ---------------------------------------------------------------------------------
 * Sequential recurrence [分块推理 §2], token by token, for one (batch, head) pair.
 *   a_t = exp(dt_t A_h);  S <- a_t S + x_t (x) B_t;  y_t = S C_t + D_h x_t.
 * This is the plain definition the chunked method must reproduce exactly.
 * ------------------------------------------------------------------------------- */
static void seq_one(const job_t *j, int64_t b, int64_t h, double *S)
{
    const int64_t P = j->P, N = j->N, g = h / (j->H / j->G);
    const double Dh = j->D ? j->D[h] : 0.0;
    if (j->init) memcpy(S, j->init + IX_S(b, h), sizeof(double) * P * N);
    else memset(S, 0, sizeof(double) * P * N);
    for (int64_t t = 0; t < j->L; ++t) {
        const double a = exp(j->dt[IX_DT(b, t, h)] * j->A[h]);
        const double *xt = j->x + IX_X(b, t, h, 0);
        const double *Bt = j->B + IX_BC(b, t, g, 0);
        const double *Ct = j->C + IX_BC(b, t, g, 0);
        double *yt = j->y + IX_X(b, t, h, 0);
        for (int64_t p = 0; p < P; ++p) {
            double *Sp = S + p * N;
            for (int64_t n = 0; n < N; ++n) Sp[n] = a * Sp[n] + xt[p] * Bt[n];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += Sp[n] * Ct[n];
            yt[p] = acc + Dh * xt[p];
        }
    }
    if (j->final_state) memcpy(j->final_state + IX_S(b, h), S, sizeof(double) * P * N);
}

/* ---------------------------------------------------------------------------------
 * Chunked decomposition [分块推理 §2.1-§2.2] for one (batch, head) pair, in the page's
 * order: (1) every chunk's intra part from a zero state, (2) the sequential pass of
 * global states b(c), (3) the by_inter correction and y(c) = by_intra(c) + by_inter(c).
 * Chunk c covers tokens [cQ, min(cQ+Q, L)).
 * ------------------------------------------------------------------------------- */
static void chunked_one(const job_t *j, int64_t b, int64_t h, double *S, double *bprev,
                        double *by_i, double *bint)
{
    const int64_t P = j->P, N = j->N, Q = j->Q, L = j->L, H = j->H;
    const int64_t g = h / (j->H / j->G), nc = (L + Q - 1) / Q, PN = P * N;
    const double Dh = j->D ? j->D[h] : 0.0;

    /* step (1) [分块推理 §2.1]: for each chunk, run the recurrence from a zero state over
     * the chunk's own tokens only.  The outputs are by_intra(c) (per token) and the local
     * end state b_intra(c).  by_i holds by_intra for all L tokens, bint holds b_intra for
     * all chunks. */
    for (int64_t c = 0; c < nc; ++c) {
        const int64_t t0 = c * Q, t1 = (t0 + Q < L) ? t0 + Q : L;
        memset(S, 0, sizeof(double) * PN);
        for (int64_t t = t0; t < t1; ++t) {
            const double a = exp(j->dt[IX_DT(b, t, h)] * j->A[h]);
            const double *xt = j->x + IX_X(b, t, h, 0);
            const double *Bt = j->B + IX_BC(b, t, g, 0);
            const double *Ct = j->C + IX_BC(b, t, g, 0);
            for (int64_t p = 0; p < P; ++p) {
                double *Sp = S + p * N;
                for (int64_t n = 0; n < N; ++n) Sp[n] = a * Sp[n] + xt[p] * Bt[n];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += Sp[n] * Ct[n];
                by_i[t * P + p] = acc;
            }
        }
        memcpy(bint + c * PN, S, sizeof(double) * PN);
        if (j->b_intra) memcpy(j->b_intra + ((b * nc + c) * H + h) * PN, S, sizeof(double) * PN);
        /* The log of diag(L): sum of dt_r A_h from the chunk start to token i inclusive. */
        if (j->logcum) {
            double s = 0.0;
            for (int64_t t = t0; t < t1; ++t) {
                s += j->dt[IX_DT(b, t, h)] * j->A[h];
                j->logcum[((b * H + h) * nc + c) * Q + (t - t0)] = s;
            }
        }
    }

    /* step (2) [分块推理 §2.2]: b(c) = b_intra(c) + (prod of a_t over chunk c) * b(c-1),
     * starting from b(-1) = the initial state (zero when absent).  bint[c] is overwritten
     * with b(c-1), the state that enters chunk c. */
    if (j->init) memcpy(bprev, j->init + IX_S(b, h), sizeof(double) * PN);
    else memset(bprev, 0, sizeof(double) * PN);
    for (int64_t c = 0; c < nc; ++c) {
        const int64_t t0 = c * Q, t1 = (t0 + Q < L) ? t0 + Q : L;
        double prod = 1.0;
        for (int64_t t = t0; t < t1; ++t) prod *= exp(j->dt[IX_DT(b, t, h)] * j->A[h]);
        double *bc = bint + c * PN;
        for (int64_t e = 0; e < PN; ++e) {
            const double next = bc[e] + prod * bprev[e];
            bc[e] = bprev[e];     /* state entering chunk c */
            bprev[e] = next;      /* b(c) */
        }
        if (j->b_in) memcpy(j->b_in + ((b * nc + c) * H + h) * PN, bc, sizeof(double) * PN);
    }
    if (j->final_state) memcpy(j->final_state + IX_S(b, h), bprev, sizeof(double) * PN);

    /* step (3) [分块推理 §2.2]: by_inter_i = L_i (b(c-1) C_i) with L_i the product of a_r
     * from the chunk start to token i inclusive; y = by_intra + by_inter (+ D x). */
    for (int64_t c = 0; c < nc; ++c) {
        const int64_t t0 = c * Q, t1 = (t0 + Q < L) ? t0 + Q : L;
        const double *bc = bint + c * PN;
        double Li = 1.0;
        for (int64_t t = t0; t < t1; ++t) {
            Li *= exp(j->dt[IX_DT(b, t, h)] * j->A[h]);
            const double *Ct = j->C + IX_BC(b, t, g, 0);
            const double *xt = j->x + IX_X(b, t, h, 0);
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += bc[p * N + n] * Ct[n];
                const double inter = Li * acc;
                const double intra = by_i[t * P + p];
                if (j->by_intra) j->by_intra[IX_X(b, t, h, p)] = intra;
                if (j->by_inter) j->by_inter[IX_X(b, t, h, p)] = inter;
                j->y[IX_X(b, t, h, p)] = intra + inter + Dh * xt[p];
            }
        }
    }
}

static void *worker(void *arg)
{
    const job_t *j = (const job_t *)arg;
    const int64_t PN = j->P * j->N;
    const int64_t nc = j->mode ? (j->L + j->Q - 1) / j->Q : 0;
    double *S = (double *)malloc(sizeof(double) * PN);
    double *bprev = (double *)malloc(sizeof(double) * PN);
    double *by_i = j->mode ? (double *)malloc(sizeof(double) * (j->L > 0 ? j->L : 1) * j->P) : NULL;
    double *bint = j->mode ? (double *)malloc(sizeof(double) * (nc > 0 ? nc : 1) * PN) : NULL;
    if (!S || !bprev || (j->mode && (!by_i || !bint))) {
        free(S); free(bprev); free(by_i); free(bint);
        return (void *)1;
    }
    for (int64_t k = j->tid; k < j->batch * j->H; k += j->nthreads) {
        const int64_t b = k / j->H, h = k % j->H;
        if (j->mode == 0) seq_one(j, b, h, S);
        else chunked_one(j, b, h, S, bprev, by_i, bint);
    }
    free(S); free(bprev); free(by_i); free(bint);
    return NULL;
}

static int run_jobs(job_t *proto)
{
    if (proto->batch < 0 || proto->L < 0 || proto->H <= 0 || proto->P <= 0 || proto->N <= 0 ||
        proto->G <= 0 || proto->H % proto->G != 0 || (proto->mode && proto->Q <= 0))
        return 1;
    int nt = proto->nthreads > 0 ? proto->nthreads : 1;
    const int64_t pairs = proto->batch * proto->H;
    if (pairs < nt) nt = pairs > 0 ? (int)pairs : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nt);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * nt);
    if (!th || !jobs) { free(th); free(jobs); return 2; }
    int rc = 0;
    for (int i = 0; i < nt; ++i) {
        jobs[i] = *proto;
        jobs[i].nthreads = nt;
        jobs[i].tid = i;
        if (pthread_create(&th[i], NULL, worker, &jobs[i]) != 0) { nt = i; rc = 3; break; }
    }
    for (int i = 0; i < nt; ++i) {
        void *ret = NULL;
        pthread_join(th[i], &ret);
        if (ret) rc = 2;
    }
    free(th); free(jobs);
    return rc;
}

/* Sequential recurrence over all (batch, head) pairs.  Layouts (row-major):
 *   x, y [batch, L, H, P];  dt [batch, L, H];  A, D [H];  B, C [batch, L, G, N];
 *   init, final_state [batch, H, P, N].  D, init and final_state may be NULL.
 * Returns 0 on success, non-zero on a bad shape or an allocation failure. */
int oracle_seq(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
               const double *x, const double *dt, const double *A, const double *B,
               const double *C, const double *D, const double *init,
               double *y, double *final_state, int nthreads)
{
    job_t j;
    memset(&j, 0, sizeof(j));
    j.batch = batch; j.L = L; j.H = H; j.P = P; j.N = N; j.G = G; j.Q = 0;
    j.x = x; j.dt = dt; j.A = A; j.B = B; j.C = C; j.D = D; j.init = init;
    j.y = y; j.final_state = final_state; j.nthreads = nthreads; j.mode = 0;
    return run_jobs(&j);
}

/* Chunked decomposition with its intermediates (nc = ceil(L / Q)):
 *   logcum   [batch, H, nc, Q]      sum of dt*A from the chunk start, inclusive (log of diag(L))
 *   b_intra  [batch, nc, H, P, N]   local end state of each chunk from a zero state
 *   b_in     [batch, nc, H, P, N]   global state entering each chunk, b(c-1)
 *   by_intra, by_inter [batch, L, H, P]
 * Any of these may be NULL; y is required.  Entries of logcum past a short last chunk
 * are left untouched. */
int oracle_chunked(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                   int64_t Q, const double *x, const double *dt, const double *A,
                   const double *B, const double *C, const double *D, const double *init,
                   double *y, double *final_state, double *logcum, double *b_intra,
                   double *b_in, double *by_intra, double *by_inter, int nthreads)
{
    job_t j;
    memset(&j, 0, sizeof(j));
    j.batch = batch; j.L = L; j.H = H; j.P = P; j.N = N; j.G = G; j.Q = Q;
    j.x = x; j.dt = dt; j.A = A; j.B = B; j.C = C; j.D = D; j.init = init;
    j.y = y; j.final_state = final_state;
    j.logcum = logcum; j.b_intra = b_intra; j.b_in = b_in;
    j.by_intra = by_intra; j.by_inter = by_inter;
    j.nthreads = nthreads; j.mode = 1;
    return run_jobs(&j);
}

/* Round each double to the nearest bfloat16 value (8 significant bits, exponent range of
 * IEEE binary32), ties to even, and return it as a double.  Used to model values the
 * library stores in bfloat16 (the residual stream between stacked layers).
 * Written from the format's definition: a finite nonzero v = m * 2^e with 0.5 <= |m| < 1
 * keeps 8 significant bits, so it is a multiple of 2^(e-8); below the smallest normal
 * (2^-126) the spacing stays at the subnormal step 2^-133.  Results above the largest
 * finite bfloat16 become infinities. */
void oracle_round_bf16(const double *in, double *out, int64_t n)
{
    const double max_bf16 = ldexp(255.0, 120);  /* (2 - 2^-7) * 2^127 */
    for (int64_t i = 0; i < n; ++i) {
        const double v = in[i];
        if (v == 0.0 || isnan(v) || isinf(v)) { out[i] = v; continue; }
        int e;
        frexp(v, &e);
        int step = e - 8;
        if (step < -133) step = -133;
        const double q = nearbyint(ldexp(v, -step));   /* default mode: ties to even */
        const double r = ldexp(q, step);
        if (fabs(r) > max_bf16) out[i] = v > 0 ? INFINITY : -INFINITY;
        else out[i] = r;
    }
}
