/*
 * CPU oracle for NSA selection-attention forward, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg
 * do.  It shares no code, header or constant with the GPU library.
 *
 * What it computes is the plain definition of the operation described in the
 * wave issue "[wave] NSA: selection attention forward kernel":
 *   - section Operation: Q [B,M,H,D], K [B,N,G,D], V [B,N,G,D],
 *     block_indices [B,M,G,T]  ->  O_slc [B,M,H,D], LSE_slc [B,H,M];
 *   - section Algorithm: for a query m, each selected block t contributes the
 *     tokens [t*bs, (t+1)*bs); scores are q.k, causally masked, and one
 *     softmax runs over all selected blocks (section Requirements: "online
 *     softmax across all T blocks" is, in exact arithmetic, the softmax over
 *     the union of the selected keys);
 *   - section Requirements: heads of one GQA group share the group's index row;
 *     causal masking inside the gathered blocks; LSE is returned.
 *
 * Readings taken where the page is silent (each is listed with its reason in
 * the design notes of the repository):
 *   - head h belongs to group g = h / (H/G) (contiguous groups);
 *   - key n is visible to query m iff n <= m, and n < N;
 *   - an index entry t counts iff t >= 0 and t*bs < N; negative entries are
 *     padding; repeated entries select the same block once (set union);
 *   - softmax scale is 1/sqrt(D); LSE is the natural log of the sum of
 *     exp(score) over the visible selected keys;
 *   - a query with no visible selected key gets O = 0 and LSE = -inf.
 *
 * Arithmetic: fp16 inputs are decoded exactly into fp64 (IEEE 754 binary16:
 * 1 sign bit, 5 exponent bits with bias 15, 10 fraction bits); all sums and
 * the two-pass softmax run in fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Exact decode of an IEEE 754 binary16 bit pattern. */
double nsa_oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 / 2^10 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Exact decode of a bfloat16 bit pattern (the upper half of an IEEE 754
   binary32: 1 sign bit, 8 exponent bits with bias 127, 7 fraction bits). */
double nsa_oracle_bf16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);                /* subnormal: f * 2^-126 / 2^7 */
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/2^7) * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* All 2^16 decoded values of each element type, filled once. */
static double g_half[65536];
static double g_bf16[65536];
static pthread_once_t g_half_once = PTHREAD_ONCE_INIT;
static void fill_half_table(void) {
    for (int i = 0; i < 65536; ++i) {
        g_half[i] = nsa_oracle_half_to_double((uint16_t)i);
        g_bf16[i] = nsa_oracle_bf16_to_double((uint16_t)i);
    }
}

typedef struct {
    const uint16_t *Q, *K, *V;
    const int32_t *idx;
    int64_t B, M, N, H, G, D, bs, T;
    const int64_t *units;
    int64_t n_units;
    double *O, *LSE;
    int thread_id, n_threads;
    int64_t dup_units;   /* units whose valid entries repeat a block */
    int error;
    const double *tab;   /* decode table of the element type (fp16 or bf16) */
    int64_t left, right; /* window of the attention without index rows */
} job_t;

typedef struct {
    unsigned char *mark;  /* [NB] selected-block flags            */
    int64_t *keys;        /* [N] visible selected keys, ascending */
    double *score;        /* [gs * N] scores, head-major          */
    double *qd, *kd;      /* [gs * D], [D] decoded rows           */
    double *mu, *z;       /* [gs] per-head max and normaliser     */
} scratch_t;

/* Returns the number of visible selected keys (w->keys[0 .. nk-1]). */
static int64_t one_unit(job_t *j, int64_t u, scratch_t *w) {
    const int64_t b = j->units[3 * u], m = j->units[3 * u + 1], g = j->units[3 * u + 2];
    const int64_t N = j->N, M = j->M, H = j->H, G = j->G, D = j->D, bs = j->bs, T = j->T;
    const int64_t gs = H / G;
    const int64_t NB = (N + bs - 1) / bs;
    const double scale = 1.0 / sqrt((double)D);

    int64_t nk = 0;
    if (j->idx) {
        /* Selected-block set (union over the row). */
        memset(w->mark, 0, (size_t)NB);
        const int32_t *row = j->idx + ((b * M + m) * G + g) * T;
        int dup = 0;
        for (int64_t i = 0; i < T; ++i) {
            int64_t t = row[i];
            if (t < 0 || t >= NB) continue;
            if (w->mark[t]) dup = 1;
            w->mark[t] = 1;
        }
        if (dup) j->dup_units++;

        /* Visible selected keys, ascending. */
        for (int64_t t = 0; t < NB; ++t) {
            if (!w->mark[t]) continue;
            for (int64_t n = t * bs; n < (t + 1) * bs && n < N; ++n)
                if (n <= m) w->keys[nk++] = n;
        }
    } else {
        /* Attention without index rows: every key n < N with
           m - left <= n <= m + right (a negative bound is unbounded);
           (left, right) = (-1, 0) is dense causal attention. */
        const int64_t lo = j->left < 0 ? 0 : m - j->left;
        const int64_t hi = j->right < 0 ? N - 1 : m + j->right;
        for (int64_t n = lo < 0 ? 0 : lo; n <= hi && n < N; ++n) w->keys[nk++] = n;
    }

    /* Head h = g*gs + i of query m, decoded. */
    for (int64_t i = 0; i < gs; ++i) {
        const uint16_t *q = j->Q + ((b * M + m) * H + g * gs + i) * D;
        for (int64_t d = 0; d < D; ++d) w->qd[i * D + d] = j->tab[q[d]];
    }

    /* Pass 1: scores s = scale * q.k for every head and key, and their maxima. */
    for (int64_t i = 0; i < gs; ++i) w->mu[i] = -INFINITY;
    for (int64_t s = 0; s < nk; ++s) {
        const uint16_t *k = j->K + ((b * N + w->keys[s]) * G + g) * D;
        for (int64_t d = 0; d < D; ++d) w->kd[d] = j->tab[k[d]];
        for (int64_t i = 0; i < gs; ++i) {
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d) acc += w->qd[i * D + d] * w->kd[d];
            const double sc = scale * acc;
            w->score[i * N + s] = sc;
            if (sc > w->mu[i]) w->mu[i] = sc;
        }
    }

    /* Pass 2: normaliser z = sum exp(s - mu) and O = sum exp(s - mu) v / z. */
    for (int64_t i = 0; i < gs; ++i) {
        w->z[i] = 0.0;
        double *o = j->O + (u * gs + i) * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    }
    for (int64_t s = 0; s < nk; ++s) {
        const uint16_t *v = j->V + ((b * N + w->keys[s]) * G + g) * D;
        for (int64_t d = 0; d < D; ++d) w->kd[d] = j->tab[v[d]];
        for (int64_t i = 0; i < gs; ++i) {
            const double e = exp(w->score[i * N + s] - w->mu[i]);
            double *o = j->O + (u * gs + i) * D;
            w->z[i] += e;
            for (int64_t d = 0; d < D; ++d) o[d] += e * w->kd[d];
        }
    }
    for (int64_t i = 0; i < gs; ++i) {
        double *o = j->O + (u * gs + i) * D;
        if (nk == 0) {                      /* nothing visible: O = 0, LSE = -inf */
            j->LSE[u * gs + i] = -INFINITY;
            continue;
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= w->z[i];
        j->LSE[u * gs + i] = w->mu[i] + log(w->z[i]);
    }
    return nk;
}

static void *worker(void *arg) {
    job_t *j = (job_t *)arg;
    const int64_t NB = (j->N + j->bs - 1) / j->bs;
    const int64_t gs = j->H / j->G;
    scratch_t w;
    w.mark = (unsigned char *)malloc((size_t)NB);
    w.keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)j->N);
    w.score = (double *)malloc(sizeof(double) * (size_t)(gs * j->N));
    w.qd = (double *)malloc(sizeof(double) * (size_t)(gs * j->D));
    w.kd = (double *)malloc(sizeof(double) * (size_t)j->D);
    w.mu = (double *)malloc(sizeof(double) * (size_t)gs);
    w.z = (double *)malloc(sizeof(double) * (size_t)gs);
    if (!w.mark || !w.keys || !w.score || !w.qd || !w.kd || !w.mu || !w.z) {
        j->error = 1;
    } else {
        for (int64_t u = j->thread_id; u < j->n_units; u += j->n_threads) one_unit(j, u, &w);
    }
    free(w.mark);
    free(w.keys);
    free(w.score);
    free(w.qd);
    free(w.kd);
    free(w.mu);
    free(w.z);
    return NULL;
}

/*
 * Oracle over a list of units.
 *   units  : int64 [n_units, 3] rows (b, m, g); each must be in range.
 *   O      : fp64 [n_units, H/G, D]   (output; heads g*gs .. g*gs+gs-1)
 *   LSE    : fp64 [n_units, H/G]      (output)
 *   n_dup  : optional; receives the number of units whose row repeats a
 *            valid block (outside the operation's contract; union is used).
 *   n_threads <= 0 uses every online host core.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
static int run_units(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                     const int32_t *block_indices, int64_t B, int64_t M, int64_t N,
                     int64_t H, int64_t G, int64_t D, int64_t block_size, int64_t T,
                     const int64_t *units, int64_t n_units, double *O, double *LSE,
                     int64_t *n_dup, int elem, int64_t left, int64_t right, int n_threads) {
    if (elem != 0 && elem != 1) return -1;
    if (!Q || !K || !V || !units || !O || !LSE) return -1;
    if (B < 1 || M < 1 || N < 1 || H < 1 || G < 1 || D < 1 || block_size < 1 || T < 1) return -1;
    if (H % G) return -1;
    for (int64_t u = 0; u < n_units; ++u) {
        if (units[3 * u] < 0 || units[3 * u] >= B || units[3 * u + 1] < 0 ||
            units[3 * u + 1] >= M || units[3 * u + 2] < 0 || units[3 * u + 2] >= G)
            return -1;
    }
    pthread_once(&g_half_once, fill_half_table);
    if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1) n_threads = 1;
    if (n_units < n_threads) n_threads = n_units > 0 ? (int)n_units : 1;

    job_t *jobs = (job_t *)calloc((size_t)n_threads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    int rc = 0;
    for (int i = 0; i < n_threads; ++i) {
        job_t *j = &jobs[i];
        j->Q = Q; j->K = K; j->V = V; j->idx = block_indices;
        j->B = B; j->M = M; j->N = N; j->H = H; j->G = G; j->D = D;
        j->bs = block_size; j->T = T;
        j->units = units; j->n_units = n_units; j->O = O; j->LSE = LSE;
        j->thread_id = i; j->n_threads = n_threads;
        j->tab = elem ? g_bf16 : g_half;
        j->left = left; j->right = right;
    }
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &jobs[i]) != 0) {
            rc = -1;
            break;
        }
        started++;
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    int64_t dups = 0;
    for (int i = 0; i < started; ++i) {
        if (jobs[i].error) rc = -1;
        dups += jobs[i].dup_units;
    }
    if (started < n_threads) rc = -1;
    if (n_dup) *n_dup = dups;
    free(jobs);
    free(th);
    return rc;
}

int nsa_oracle_units(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                     const int32_t *block_indices, int64_t B, int64_t M, int64_t N,
                     int64_t H, int64_t G, int64_t D, int64_t block_size, int64_t T,
                     const int64_t *units, int64_t n_units, double *O, double *LSE,
                     int64_t *n_dup, int n_threads) {
    if (!block_indices) return -1;
    return run_units(Q, K, V, block_indices, B, M, N, H, G, D, block_size, T, units, n_units, O, LSE, n_dup, 0,
                     -1, 0, n_threads);
}

/* As nsa_oracle_units for Q, K, V of element type elem: 0 = fp16, 1 = bf16. */
int nsa_oracle_units_t(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                       const int32_t *block_indices, int64_t B, int64_t M, int64_t N,
                       int64_t H, int64_t G, int64_t D, int64_t block_size, int64_t T,
                       const int64_t *units, int64_t n_units, double *O, double *LSE,
                       int64_t *n_dup, int elem, int n_threads) {
    if (!block_indices) return -1;
    return run_units(Q, K, V, block_indices, B, M, N, H, G, D, block_size, T, units, n_units, O, LSE, n_dup,
                     elem, -1, 0, n_threads);
}

/*
 * Dense causal attention over a list of units: the same two-pass fp64
 * computation with every key n <= m (n < N) visible -- the selection with all
 * causal blocks selected, without an index array.  Arguments and outputs as
 * for nsa_oracle_units.
 */
int nsa_oracle_dense_units(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B, int64_t M,
                           int64_t N, int64_t H, int64_t G, int64_t D, const int64_t *units, int64_t n_units,
                           double *O, double *LSE, int n_threads) {
    return run_units(Q, K, V, NULL, B, M, N, H, G, D, 1, 1, units, n_units, O, LSE, NULL, 0, -1, 0, n_threads);
}

/*
 * Sliding-window attention (the FlyDSL pull request "[Kernel][MI350] Add 8
 * wave GQA sliding-window attention kernel", section What it does: query i
 * attends to keys [i - LEFT, i + RIGHT]): every key n < N with
 * m - left <= n <= m + right, a negative bound meaning unbounded on that side.
 * (left, right) = (-1, 0) is dense causal attention.  elem: 0 = fp16,
 * 1 = bf16.  A query whose window holds no key gets O = 0, LSE = -inf.
 */
int nsa_oracle_window_units(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B, int64_t M,
                            int64_t N, int64_t H, int64_t G, int64_t D, int64_t left, int64_t right,
                            const int64_t *units, int64_t n_units, double *O, double *LSE, int elem,
                            int n_threads) {
    return run_units(Q, K, V, NULL, B, M, N, H, G, D, 1, 1, units, n_units, O, LSE, NULL, elem, left, right,
                     n_threads);
}

/*
 * Streaming comparison of a computed forward result with the oracle, unit by
 * unit, keeping no fp64 copy of the outputs (the plain definition above is
 * evaluated for each unit into a per-thread buffer and compared at once).
 *
 *   Og  : 16-bit patterns [B, M, H, D] of the output to check (elem 0 = fp16,
 *         1 = bf16), decoded exactly;
 *   Lg  : fp32 [B, H, M] log-sum-exp to check;
 *   units u0 .. u1-1 of the linear order u = (b*M + m)*G + g;
 *   idx NULL with (left, right) compares against the attention without index
 *   rows (keys m - left .. m + right, negative = unbounded; (-1, 0) = dense
 *   causal).
 *
 * stats (double[8]) receives:
 *   [0] max |O - O_ref| over every element of the units (an empty row's
 *       O_ref is 0);
 *   [1] max |LSE - LSE_ref| over the rows whose LSE_ref is finite;
 *   [2] rows with a non-finite O element, a non-finite LSE where LSE_ref is
 *       finite, or an LSE other than -inf where the row is empty (LSE_ref =
 *       -inf);
 *   [3] the unit (linear index) holding the largest O error, [4] the one
 *       holding the largest LSE error (the smallest such unit; -1 while
 *       every error is 0);
 *   [5] units compared; [6] units whose row repeats a valid block;
 *   [7] rows whose LSE_ref is -inf.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
typedef struct {
    job_t base;
    const uint16_t *Og;
    const float *Lg;
    int64_t u0, u1;
    double max_o, max_l;
    int64_t worst_o, worst_l, bad, empty, count;
} cjob_t;

static void *cworker(void *arg) {
    cjob_t *c = (cjob_t *)arg;
    job_t *J = &c->base;
    const int64_t NB = (J->N + J->bs - 1) / J->bs;
    const int64_t gs = J->H / J->G, D = J->D, M = J->M, G = J->G, H = J->H;
    scratch_t w;
    double *O = (double *)malloc(sizeof(double) * (size_t)(gs * D));
    double *L = (double *)malloc(sizeof(double) * (size_t)gs);
    w.mark = (unsigned char *)malloc((size_t)NB);
    w.keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)J->N);
    w.score = (double *)malloc(sizeof(double) * (size_t)(gs * J->N));
    w.qd = (double *)malloc(sizeof(double) * (size_t)(gs * D));
    w.kd = (double *)malloc(sizeof(double) * (size_t)D);
    w.mu = (double *)malloc(sizeof(double) * (size_t)gs);
    w.z = (double *)malloc(sizeof(double) * (size_t)gs);
    c->max_o = 0.0;
    c->max_l = 0.0;
    c->worst_o = -1;
    c->worst_l = -1;
    if (!O || !L || !w.mark || !w.keys || !w.score || !w.qd || !w.kd || !w.mu || !w.z) {
        J->error = 1;
    } else {
        job_t fj = *J;
        fj.O = O;
        fj.LSE = L;
        for (int64_t u = c->u0 + J->thread_id; u < c->u1; u += J->n_threads) {
            const int64_t g = u % G, m = (u / G) % M, b = u / (G * M);
            int64_t one[3] = {b, m, g};
            fj.units = one;
            one_unit(&fj, 0, &w);
            for (int64_t i = 0; i < gs; ++i) {
                const int64_t h = g * gs + i;
                const uint16_t *og = c->Og + ((b * M + m) * H + h) * D;
                int bad = 0;
                for (int64_t d = 0; d < D; ++d) {
                    const double x = J->tab[og[d]];
                    if (!isfinite(x)) {
                        bad = 1;
                        continue;
                    }
                    const double e = fabs(x - O[i * D + d]);
                    if (e > c->max_o) {
                        c->max_o = e;
                        c->worst_o = u;
                    }
                }
                const double lg = (double)c->Lg[(b * H + h) * M + m];
                if (isfinite(L[i])) {
                    if (!isfinite(lg)) {
                        bad = 1;
                    } else {
                        const double e = fabs(lg - L[i]);
                        if (e > c->max_l) {
                            c->max_l = e;
                            c->worst_l = u;
                        }
                    }
                } else {
                    c->empty++;
                    if (!(isinf(lg) && lg < 0)) bad = 1;
                }
                c->bad += bad;
            }
            c->count++;
        }
        J->dup_units = fj.dup_units;
    }
    free(O); free(L);
    free(w.mark); free(w.keys); free(w.score); free(w.qd); free(w.kd); free(w.mu); free(w.z);
    return NULL;
}

int nsa_oracle_compare(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const int32_t *block_indices,
                       int64_t B, int64_t M, int64_t N, int64_t H, int64_t G, int64_t D, int64_t block_size,
                       int64_t T, int64_t left, int64_t right, const uint16_t *Og, const float *Lg, int64_t u0,
                       int64_t u1, int elem, int n_threads, double *stats) {
    if (elem != 0 && elem != 1) return -1;
    if (!Q || !K || !V || !Og || !Lg || !stats) return -1;
    if (B < 1 || M < 1 || N < 1 || H < 1 || G < 1 || D < 1 || block_size < 1 || T < 1) return -1;
    if (H % G) return -1;
    if (u0 < 0 || u1 < u0 || u1 > B * M * G) return -1;
    pthread_once(&g_half_once, fill_half_table);
    if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1) n_threads = 1;
    if (u1 - u0 < n_threads) n_threads = u1 > u0 ? (int)(u1 - u0) : 1;
    cjob_t *jobs = (cjob_t *)calloc((size_t)n_threads, sizeof(cjob_t));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int i = 0; i < n_threads; ++i) {
        job_t *J = &jobs[i].base;
        J->Q = Q; J->K = K; J->V = V; J->idx = block_indices;
        J->B = B; J->M = M; J->N = N; J->H = H; J->G = G; J->D = D;
        J->bs = block_indices ? block_size : 1;
        J->T = block_indices ? T : 1;
        J->thread_id = i; J->n_threads = n_threads;
        J->tab = elem ? g_bf16 : g_half;
        J->left = left; J->right = right;
        jobs[i].Og = Og; jobs[i].Lg = Lg; jobs[i].u0 = u0; jobs[i].u1 = u1;
    }
    int rc = 0, started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&th[i], NULL, cworker, &jobs[i]) != 0) {
            rc = -1;
            break;
        }
        started++;
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    if (started < n_threads) rc = -1;
    double mo = 0.0, ml = 0.0;
    int64_t wo = -1, wl = -1, bad = 0, dup = 0, empty = 0, count = 0;
    for (int i = 0; i < started; ++i) {
        const cjob_t *c = &jobs[i];
        if (c->base.error) rc = -1;
        /* Largest error; among equal ones the smallest unit. */
        if (c->worst_o >= 0 && (c->max_o > mo || (c->max_o == mo && (wo < 0 || c->worst_o < wo)))) {
            mo = c->max_o;
            wo = c->worst_o;
        }
        if (c->worst_l >= 0 && (c->max_l > ml || (c->max_l == ml && (wl < 0 || c->worst_l < wl)))) {
            ml = c->max_l;
            wl = c->worst_l;
        }
        bad += c->bad;
        dup += c->base.dup_units;
        empty += c->empty;
        count += c->count;
    }
    stats[0] = mo;
    stats[1] = ml;
    stats[2] = (double)bad;
    stats[3] = (double)wo;
    stats[4] = (double)wl;
    stats[5] = (double)count;
    stats[6] = (double)dup;
    stats[7] = (double)empty;
    free(jobs);
    free(th);
    return rc;
}

/*
 * Backward of the same operation, in fp64 (the reason the forward returns LSE:
 * wave issue "[wave] NSA: selection attention forward kernel", section
 * Requirements).  For a unit (b, m, g), head h of the group, with the visible
 * selected keys n, scores s_n = q.k_n / sqrt(D), probabilities P_n and the
 * upstream gradient dO_h:
 *   dP_n = dO_h . v_n,   Delta_h = sum_n P_n dP_n  (= dO_h . O_h),
 *   dS_n = P_n (dP_n - Delta_h),
 *   dQ_h = sum_n dS_n k_n / sqrt(D),
 *   dK_n += dS_n q_h / sqrt(D),   dV_n += P_n dO_h   (summed over every unit
 *   and head that sees key n).
 * These are the derivatives of softmax attention (chain rule through the
 * softmax: dS = P * (dP - rowsum(P * dP))).
 *
 * kblocks: optional (b, g, t) triples; when given, dK/dV are accumulated only
 * for the keys of those blocks, into dK/dV laid out [n_kblocks, bs, D];
 * otherwise into [B, N, G, D].  dK/dV are accumulated (the caller zeroes
 * them); dQ [n_units, H/G, D] is written.  Threads keep private partial sums
 * that are added in thread order at the end.
 */
typedef struct {
    job_t base;
    const uint16_t *dO;
    const int64_t *kblocks;
    int64_t n_kblocks;
    double *dQ;
    double *dK, *dV;     /* this thread's partial sums */
    double *mQ;          /* optional: sums of squared term magnitudes of dQ */
    double *mK, *mV;     /* this thread's partial sums of squared term magnitudes */
    int64_t kv_elems;
} bjob_t;

/* Position of key n of (b, g) in the dK/dV arrays, or -1 if filtered out. */
static int64_t kv_pos(const bjob_t *j, int64_t b, int64_t g, int64_t n) {
    const job_t *J = &j->base;
    if (!j->kblocks) return ((b * J->N + n) * J->G + g) * J->D;
    const int64_t t = n / J->bs;
    for (int64_t i = 0; i < j->n_kblocks; ++i)
        if (j->kblocks[3 * i] == b && j->kblocks[3 * i + 1] == g && j->kblocks[3 * i + 2] == t)
            return (i * J->bs + (n - t * J->bs)) * J->D;
    return -1;
}

static void *bworker(void *arg) {
    bjob_t *j = (bjob_t *)arg;
    job_t *J = &j->base;
    const int64_t NB = (J->N + J->bs - 1) / J->bs;
    const int64_t gs = J->H / J->G, D = J->D;
    scratch_t w;
    double *fwdO = (double *)malloc(sizeof(double) * (size_t)(gs * D));
    double *fwdL = (double *)malloc(sizeof(double) * (size_t)gs);
    double *dOd = (double *)malloc(sizeof(double) * (size_t)(gs * D));
    double *dP = (double *)malloc(sizeof(double) * (size_t)(gs * J->N));
    double *delta = (double *)malloc(sizeof(double) * (size_t)gs);
    double *adelta = (double *)malloc(sizeof(double) * (size_t)gs);
    w.mark = (unsigned char *)malloc((size_t)NB);
    w.keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)J->N);
    w.score = (double *)malloc(sizeof(double) * (size_t)(gs * J->N));
    w.qd = (double *)malloc(sizeof(double) * (size_t)(gs * D));
    w.kd = (double *)malloc(sizeof(double) * (size_t)D);
    w.mu = (double *)malloc(sizeof(double) * (size_t)gs);
    w.z = (double *)malloc(sizeof(double) * (size_t)gs);
    if (!fwdO || !fwdL || !dOd || !dP || !delta || !adelta || !w.mark || !w.keys || !w.score || !w.qd || !w.kd || !w.mu || !w.z) {
        J->error = 1;
    } else {
        const double scale = 1.0 / sqrt((double)D);
        /* The forward pass of each unit is recomputed by one_unit into a
           private O/LSE slot; the job's outputs are redirected there. */
        job_t fj = *J;
        fj.O = fwdO;
        fj.LSE = fwdL;
        for (int64_t u = J->thread_id; u < J->n_units; u += J->n_threads) {
            const int64_t b = J->units[3 * u], m = J->units[3 * u + 1], g = J->units[3 * u + 2];
            int64_t one[3] = {b, m, g};
            fj.units = one;
            /* Forward of the unit: scaled scores in w.score, visible keys in
               w.keys, decoded queries in w.qd, O and LSE in fwdO / fwdL. */
            const int64_t nk = one_unit(&fj, 0, &w);
            for (int64_t i = 0; i < gs; ++i) {
                const uint16_t *src = j->dO + ((b * J->M + m) * J->H + g * gs + i) * D;
                for (int64_t d = 0; d < D; ++d) dOd[i * D + d] = J->tab[src[d]];
            }
            /* dP and Delta. P_n = exp(s_n - LSE). */
            for (int64_t i = 0; i < gs; ++i) {
                delta[i] = 0.0;
                adelta[i] = 0.0;
                for (int64_t d = 0; d < D; ++d) adelta[i] += fabs(dOd[i * D + d] * fwdO[i * D + d]);
            }
            for (int64_t s = 0; s < nk; ++s) {
                const uint16_t *v = J->V + ((b * J->N + w.keys[s]) * J->G + g) * D;
                for (int64_t d = 0; d < D; ++d) w.kd[d] = J->tab[v[d]];
                for (int64_t i = 0; i < gs; ++i) {
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d) acc += dOd[i * D + d] * w.kd[d];
                    dP[i * J->N + s] = acc;
                    delta[i] += exp(w.score[i * J->N + s] - fwdL[i]) * acc;
                }
            }
            double *dq = j->dQ + u * gs * D;
            double *mq = j->mQ ? j->mQ + u * gs * D : NULL;
            for (int64_t e = 0; e < gs * D; ++e) dq[e] = 0.0;
            if (mq)
                for (int64_t e = 0; e < gs * D; ++e) mq[e] = 0.0;
            for (int64_t s = 0; s < nk; ++s) {
                const int64_t n = w.keys[s];
                const uint16_t *k = J->K + ((b * J->N + n) * J->G + g) * D;
                for (int64_t d = 0; d < D; ++d) w.kd[d] = J->tab[k[d]];
                const int64_t pos = kv_pos(j, b, g, n);
                for (int64_t i = 0; i < gs; ++i) {
                    const double P = exp(w.score[i * J->N + s] - fwdL[i]);
                    const double dS = P * (dP[i * J->N + s] - delta[i]);
                    /* Size of dS before the cancellation of its two parts,
                       with Delta taken as sum_d |dO_d O_d| (which also bounds
                       the error of a Delta formed from a rounded O): the
                       scale of the rounding errors a term can carry. */
                    const double dSm = P * (fabs(dP[i * J->N + s]) + adelta[i]);
                    for (int64_t d = 0; d < D; ++d) dq[i * D + d] += dS * w.kd[d] * scale;
                    if (mq)
                        for (int64_t d = 0; d < D; ++d) {
                            const double t = dSm * w.kd[d] * scale;
                            mq[i * D + d] += t * t;
                        }
                    if (pos >= 0) {
                        for (int64_t d = 0; d < D; ++d) {
                            j->dK[pos + d] += dS * w.qd[i * D + d] * scale;
                            j->dV[pos + d] += P * dOd[i * D + d];
                        }
                        if (j->mK)
                            for (int64_t d = 0; d < D; ++d) {
                                const double tk = dSm * w.qd[i * D + d] * scale, tv = P * dOd[i * D + d];
                                j->mK[pos + d] += tk * tk;
                                j->mV[pos + d] += tv * tv;
                            }
                    }
                }
            }
        }
    }
    free(fwdO); free(fwdL); free(dOd); free(dP); free(delta); free(adelta);
    free(w.mark); free(w.keys); free(w.score); free(w.qd); free(w.kd); free(w.mu); free(w.z);
    return NULL;
}

/*
 * mQ, mK, mV (optional, all or none): for every gradient element, the square
 * root of the sum of the squared magnitudes of its terms, with dS taken as
 * P (|dP| + sum_d |dO_d O_d|): the scale of the rounding error a kernel that
 * rounds P, dS and O to a short format accumulates in that element.  Laid out as dQ, dK,
 * dV; mK and mV are accumulated like dK and dV (as sums of squares) and the
 * square root is taken at the end.
 */
int nsa_oracle_bwd_units(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const int32_t *block_indices,
                         const uint16_t *dO, int64_t B, int64_t M, int64_t N, int64_t H, int64_t G, int64_t D,
                         int64_t block_size, int64_t T, const int64_t *units, int64_t n_units,
                         const int64_t *kblocks, int64_t n_kblocks, double *dQ, double *dK, double *dV,
                         double *mQ, double *mK, double *mV, int n_threads) {
    if (!Q || !K || !V || !dO || !units || !dQ || !dK || !dV) return -1;
    if ((mQ != NULL) != (mK != NULL) || (mK != NULL) != (mV != NULL)) return -1;
    if (B < 1 || M < 1 || N < 1 || H < 1 || G < 1 || D < 1 || block_size < 1 || T < 1) return -1;
    if (H % G) return -1;
    for (int64_t u = 0; u < n_units; ++u) {
        if (units[3 * u] < 0 || units[3 * u] >= B || units[3 * u + 1] < 0 || units[3 * u + 1] >= M ||
            units[3 * u + 2] < 0 || units[3 * u + 2] >= G)
            return -1;
    }
    pthread_once(&g_half_once, fill_half_table);
    if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1) n_threads = 1;
    if (n_units < n_threads) n_threads = n_units > 0 ? (int)n_units : 1;
    const int64_t kv_elems = kblocks ? n_kblocks * block_size * D : B * N * G * D;
    bjob_t *jobs = (bjob_t *)calloc((size_t)n_threads, sizeof(bjob_t));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    int rc = 0;
    for (int i = 0; i < n_threads; ++i) {
        bjob_t *j = &jobs[i];
        job_t *J = &j->base;
        J->Q = Q; J->K = K; J->V = V; J->idx = block_indices;
        J->B = B; J->M = M; J->N = N; J->H = H; J->G = G; J->D = D;
        J->bs = block_size; J->T = T;
        J->units = units; J->n_units = n_units;
        J->thread_id = i; J->n_threads = n_threads;
        J->tab = g_half;
        J->left = -1; J->right = 0;
        j->dO = dO; j->kblocks = kblocks; j->n_kblocks = n_kblocks; j->dQ = dQ; j->kv_elems = kv_elems;
        j->mQ = mQ;
        j->dK = (double *)calloc((size_t)kv_elems, sizeof(double));
        j->dV = (double *)calloc((size_t)kv_elems, sizeof(double));
        if (!j->dK || !j->dV) rc = -1;
        if (mK) {
            j->mK = (double *)calloc((size_t)kv_elems, sizeof(double));
            j->mV = (double *)calloc((size_t)kv_elems, sizeof(double));
            if (!j->mK || !j->mV) rc = -1;
        }
    }
    int started = 0;
    if (rc == 0) {
        for (int i = 0; i < n_threads; ++i) {
            if (pthread_create(&th[i], NULL, bworker, &jobs[i]) != 0) {
                rc = -1;
                break;
            }
            started++;
        }
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < started; ++i) {
        if (jobs[i].base.error) rc = -1;
        for (int64_t e = 0; rc == 0 && e < kv_elems; ++e) {
            dK[e] += jobs[i].dK[e];
            dV[e] += jobs[i].dV[e];
        }
        if (mK)
            for (int64_t e = 0; rc == 0 && e < kv_elems; ++e) {
                mK[e] += jobs[i].mK[e];
                mV[e] += jobs[i].mV[e];
            }
    }
    if (mK && rc == 0) {
        for (int64_t e = 0; e < kv_elems; ++e) {
            mK[e] = sqrt(mK[e]);
            mV[e] = sqrt(mV[e]);
        }
        for (int64_t e = 0; e < n_units * (H / G) * D; ++e) mQ[e] = sqrt(mQ[e]);
    }
    for (int i = 0; i < n_threads; ++i) {
        free(jobs[i].dK);
        free(jobs[i].dV);
        free(jobs[i].mK);
        free(jobs[i].mV);
    }
    free(jobs);
    free(th);
    return rc;
}

/*
 * Top-k block selection: the step that produces block_indices (wave issue
 * "[wave] NSA: selection attention forward kernel", section Depends on, names
 * a top-k kernel; the pages give no algorithm for it).  Plain reading: for
 * every row (b, m, g) of scores [B, M, G, NB] (one importance score per key
 * block), the candidates are the blocks a query may select, t = 0 .. min(m/bs,
 * NB - 1); the T candidates with the highest scores are chosen, ordered by
 * score descending and, among equal scores, by block index ascending (a NaN
 * score counts as -inf; -0 equals +0).  The row is written in ascending block
 * order and padded with -1 (fewer than T candidates: all of them).
 */
typedef struct {
    double key;
    int64_t t;
} cand_t;

static int cand_cmp(const void *a, const void *b) {
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

static int i64_cmp(const void *a, const void *b) {
    const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* One row: the T best of candidates 0 .. nc-1 into o[0 .. T-1]. */
static void select_row(const float *row, int64_t nc, int64_t T, cand_t *c, int64_t *sel, int32_t *o) {
    for (int64_t t = 0; t < nc; ++t) {
        const double v = (double)row[t];
        c[t].key = isnan(v) ? -INFINITY : v;   /* -0.0 == +0.0 under > and < */
        c[t].t = t;
    }
    qsort(c, (size_t)nc, sizeof(cand_t), cand_cmp);
    const int64_t k = nc < T ? nc : T;
    for (int64_t i = 0; i < k; ++i) sel[i] = c[i].t;
    qsort(sel, (size_t)k, sizeof(int64_t), i64_cmp);
    for (int64_t i = 0; i < T; ++i) o[i] = i < k ? (int32_t)sel[i] : -1;
}

int nsa_oracle_topk(const float *scores, int64_t B, int64_t M, int64_t G, int64_t NB, int64_t block_size,
                    int64_t T, int32_t *out) {
    if (!scores || !out || B < 1 || M < 1 || G < 1 || NB < 1 || block_size < 1 || T < 1) return -1;
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)NB);
    int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)NB);
    if (!c || !sel) {
        free(c);
        free(sel);
        return -1;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t g = 0; g < G; ++g) {
                const int64_t last = (m / block_size < NB - 1) ? m / block_size : NB - 1;
                select_row(scores + ((b * M + m) * G + g) * NB, last + 1, T, c, sel,
                           out + ((b * M + m) * G + g) * T);
            }
    free(c);
    free(sel);
    return 0;
}

/* The same selection for R explicit rows: scores [R, NB], query positions
   ms [R], output [R, T]. */
int nsa_oracle_topk_rows(const float *scores, const int64_t *ms, int64_t R, int64_t NB, int64_t block_size,
                         int64_t T, int32_t *out) {
    if (!scores || !ms || !out || R < 0 || NB < 1 || block_size < 1 || T < 1) return -1;
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)NB);
    int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)NB);
    if (!c || !sel) {
        free(c);
        free(sel);
        return -1;
    }
    for (int64_t r = 0; r < R; ++r) {
        if (ms[r] < 0) {
            free(c);
            free(sel);
            return -1;
        }
        const int64_t last = (ms[r] / block_size < NB - 1) ? ms[r] / block_size : NB - 1;
        select_row(scores + r * NB, last + 1, T, c, sel, out + r * T);
    }
    free(c);
    free(sel);
    return 0;
}
