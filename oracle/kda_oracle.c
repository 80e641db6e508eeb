/*
 * kda_oracle.c -- float64 CPU oracle for the Kimi Delta Attention (KDA) forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent reference that the
 * GPU path is checked against.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load it.  It shares no code, header, table
 * or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes is the plain definition of the method, token by token, in
 * float64, with no chunking, blocking or reordering:
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t,          alpha_t = exp(g'_t)  (one decay per key channel)
 *
 * Sources (web pages; cited by title and section):
 *   [ENG]   "flash-linear-attention KDA 内核工程实践：门控模式、safe_gate 数值稳定性
 *            与 chunk intra/inter 双路径解析" (dpshk.com news 4765615)
 *   [NOTES] "Reading Notes: Implementation Notes for KDA in FLA"
 *            (mzeromiko.github.io, kimi_linear / kda-fla)
 *   [FKDA]  "FlashKDA gate偏置加載路徑完整解析如何讀取A_log與dt_bias"
 *            (m.czchanglian.com news 37351)
 *
 * Readings taken where the pages leave a step open:
 *   - q/k L2 normalisation is x / sqrt(sum x^2 + 1e-6), per (token, qk head);
 *     the query scale multiplies the normalised q.
 *   - value head hv reads qk head hv / (HV/H) (contiguous groups).
 *   - g, lower_bound and the gate output are natural-log quantities.
 *
 * Parity pins (tests/test_oracle_pins.py): a dense chunk-form evaluation of the
 * [NOTES] forward steps, closed forms for beta = 0 / g = 0 / beta = 1 / beta = 2,
 * T = 1, a hand-worked K = V = 1 case and closed-form gate values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { GATE_PRE = 0, GATE_SOFTPLUS = 1, GATE_LOWER_BOUND = 2 };
enum { BETA_AS_GIVEN = 0, BETA_SIGMOID = 1, BETA_TWO_SIGMOID = 2 };

/* softplus(x) = log(1 + e^x), written so that neither branch overflows. */
static double softplus(double x) {
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/* logistic sigmoid 1 / (1 + e^-x), overflow-free in both directions. */
static double sigmoid(double x) {
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/*
 * Gate activation, natural-log units.  [ENG] §2 gives the two input contracts:
 * pre-gated (g is already the log decay) and in-kernel, where
 *   no lower bound:   g' = -exp(A_log[hv]) * softplus(g + dt_bias)
 *   with lower bound: g' = lower_bound * sigmoid(exp(A_log[hv]) * (g + dt_bias))
 * and, with a lower bound but no A_log, the multiplier exp(A_log) becomes 1.
 * [FKDA] §三 fixes the order for the bounded form: add the bias, multiply by
 * exp(A_log), then scale the sigmoid by the lower bound.
 */
static double gate_activate(int mode, double graw, const double *A_log, const double *dt_bias,
                            int hv, int K, int d, double lower_bound) {
    if (mode == GATE_PRE) return graw;
    double x = graw + (dt_bias ? dt_bias[(size_t)hv * K + d] : 0.0);
    if (mode == GATE_SOFTPLUS) return -exp(A_log[hv]) * softplus(x);
    double a = A_log ? exp(A_log[hv]) : 1.0;
    return lower_bound * sigmoid(a * x);
}

/* beta transform: [ENG] §2.1 -- sigmoid in-kernel, or 2*sigmoid when negative
 * eigenvalues are allowed (beta in [0, 2)). */
static double beta_activate(int mode, double b) {
    if (mode == BETA_SIGMOID) return sigmoid(b);
    if (mode == BETA_TWO_SIGMOID) return 2.0 * sigmoid(b);
    return b;
}

typedef struct {
    int num_seqs;
    const int64_t *seq_starts; /* [num_seqs + 1] offsets on the flattened token axis */
    int H, HV, K, V;
    const double *q, *k, *v, *g, *beta, *A_log, *dt_bias, *h0;
    int gate_mode, qk_l2norm, beta_mode;
    double lower_bound, scale;
    double *o, *ht;
    const unsigned char *unit_mask; /* [num_seqs * HV], NULL = every unit */
    int chunk;                      /* snapshot period (tokens), with states */
    const int64_t *chunk_first;     /* [num_seqs] index of each sequence's first chunk */
    double *states;                 /* [chunks][HV][K][V] state before each chunk, or NULL */
    int next_unit;                  /* work counter, guarded by lock */
    pthread_mutex_t lock;
} oracle_job;

/* Copy one K-vector, L2-normalising it when asked: x / sqrt(sum x^2 + 1e-6). */
static void load_qk(const double *src, int K, int normalise, double mult, double *dst) {
    double inv = 1.0;
    if (normalise) {
        double ss = 0.0;
        for (int d = 0; d < K; ++d) ss += src[d] * src[d];
        inv = 1.0 / sqrt(ss + 1e-6);
    }
    for (int d = 0; d < K; ++d) dst[d] = src[d] * inv * mult;
}

/*
 * One (sequence, value head) unit: the token recurrence of the method.
 * The update is applied in the factored form
 *   S <- Diag(alpha) S;  u = S^T k;  S <- S + beta k (v - u)^T;  o = S^T q
 * which is the same matrix as (I - beta k k^T) Diag(alpha) S + beta k v^T.
 * The state is stored [K][V] (key rows, value columns), as [NOTES] forward
 * step 4 states for the hidden state's memory layout.
 */
static void run_unit(oracle_job *J, int n, int hv, double *S, double *qv, double *kv, double *u) {
    const int H = J->H, HV = J->HV, K = J->K, V = J->V;
    const int h = hv / (HV / H);
    const size_t KV = (size_t)K * V;
    if (J->h0) memcpy(S, J->h0 + ((size_t)n * HV + hv) * KV, KV * sizeof(double));
    else memset(S, 0, KV * sizeof(double));

    for (int64_t t = J->seq_starts[n]; t < J->seq_starts[n + 1]; ++t) {
        const int64_t r = t - J->seq_starts[n];
        if (J->states && r % J->chunk == 0)  /* the state the chunk starting here begins from */
            memcpy(J->states + ((size_t)(J->chunk_first[n] + r / J->chunk) * HV + hv) * KV, S, KV * sizeof(double));
        load_qk(J->q + ((size_t)t * H + h) * K, K, J->qk_l2norm, J->scale, qv);
        load_qk(J->k + ((size_t)t * H + h) * K, K, J->qk_l2norm, 1.0, kv);
        const double *vt = J->v + ((size_t)t * HV + hv) * V;
        const double *gt = J->g + ((size_t)t * HV + hv) * K;
        const double b = beta_activate(J->beta_mode, J->beta[(size_t)t * HV + hv]);

        for (int d = 0; d < K; ++d) {
            double alpha = exp(gate_activate(J->gate_mode, gt[d], J->A_log, J->dt_bias, hv, K, d,
                                             J->lower_bound));
            for (int j = 0; j < V; ++j) S[(size_t)d * V + j] *= alpha;
        }
        for (int j = 0; j < V; ++j) u[j] = 0.0;
        for (int d = 0; d < K; ++d)
            for (int j = 0; j < V; ++j) u[j] += S[(size_t)d * V + j] * kv[d];
        for (int d = 0; d < K; ++d) {
            double c = b * kv[d];
            for (int j = 0; j < V; ++j) S[(size_t)d * V + j] += c * (vt[j] - u[j]);
        }
        double *ot = J->o + ((size_t)t * HV + hv) * V;
        for (int j = 0; j < V; ++j) ot[j] = 0.0;
        for (int d = 0; d < K; ++d)
            for (int j = 0; j < V; ++j) ot[j] += S[(size_t)d * V + j] * qv[d];
    }
    if (J->ht) memcpy(J->ht + ((size_t)n * HV + hv) * KV, S, KV * sizeof(double));
}

static void *worker(void *arg) {
    oracle_job *J = (oracle_job *)arg;
    const int units = J->num_seqs * J->HV;
    double *S = (double *)malloc(sizeof(double) * ((size_t)J->K * J->V + 2 * (size_t)J->K + J->V));
    if (!S) return (void *)1;
    double *qv = S + (size_t)J->K * J->V, *kv = qv + J->K, *u = kv + J->K;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int id = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (id >= units) break;
        if (J->unit_mask && !J->unit_mask[id]) continue;
        run_unit(J, id / J->HV, id % J->HV, S, qv, kv, u);
    }
    free(S);
    return NULL;
}

int kda_oracle_num_threads(int requested) {
    if (requested > 0) return requested;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int run_job(oracle_job *J, int nthreads) {
    pthread_mutex_init(&J->lock, NULL);
    int nt = kda_oracle_num_threads(nthreads);
    if (nt > J->num_seqs * J->HV) nt = J->num_seqs * J->HV > 0 ? J->num_seqs * J->HV : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    int failed = 0;
    for (int i = 0; i < nt; ++i)
        if (pthread_create(&tid[i], NULL, worker, J) != 0) { nt = i; failed = 1; break; }
    for (int i = 0; i < nt; ++i) {
        void *r = NULL;
        pthread_join(tid[i], &r);
        if (r) failed = 1;
    }
    free(tid);
    pthread_mutex_destroy(&J->lock);
    return failed ? -1 : nt;
}

/*
 * Forward pass.  Shapes (row-major, float64):
 *   q, k [Ttot][H][K];  v [Ttot][HV][V];  g [Ttot][HV][K];  beta [Ttot][HV]
 *   A_log [HV] or NULL;  dt_bias [HV*K] or NULL;  h0 [N][HV][K][V] or NULL
 *   o [Ttot][HV][V];  ht [N][HV][K][V] or NULL
 * Sequences are the token ranges [seq_starts[n], seq_starts[n+1]).
 * Units whose unit_mask entry is 0 are skipped (their o rows and ht are left
 * untouched).  Returns the number of threads used, or -1 on bad arguments.
 */
int kda_oracle_fwd(int num_seqs, const int64_t *seq_starts, int H, int HV, int K, int V,
                   const double *q, const double *k, const double *v, const double *g,
                   const double *beta, const double *A_log, const double *dt_bias,
                   int gate_mode, double lower_bound, int qk_l2norm, int beta_mode, double scale,
                   const double *h0, double *o, double *ht, const unsigned char *unit_mask,
                   int nthreads) {
    if (num_seqs < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0) return -1;
    if (gate_mode == GATE_SOFTPLUS && !A_log) return -1;
    oracle_job J = {num_seqs, seq_starts, H, HV, K, V, q, k, v, g, beta, A_log, dt_bias, h0,
                    gate_mode, qk_l2norm, beta_mode, lower_bound, scale, o, ht, unit_mask, 0, NULL, NULL, 0};
    return run_job(&J, nthreads);
}

/*
 * kda_oracle_fwd that also records, for every sequence and value head, the state
 * each chunk starts from: the state after the last token before the chunk (the
 * sequence's initial state for its first chunk).  Chunks start at every sequence
 * start and then every `chunk` tokens; sequence n's chunks are numbered from
 * chunk_first[n].  states: [total chunks][HV][K][V].
 */
int kda_oracle_fwd_states(int num_seqs, const int64_t *seq_starts, int H, int HV, int K, int V,
                          const double *q, const double *k, const double *v, const double *g,
                          const double *beta, const double *A_log, const double *dt_bias,
                          int gate_mode, double lower_bound, int qk_l2norm, int beta_mode, double scale,
                          const double *h0, double *o, double *ht, int chunk, const int64_t *chunk_first,
                          double *states, int nthreads) {
    if (num_seqs < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0) return -1;
    if (gate_mode == GATE_SOFTPLUS && !A_log) return -1;
    if (chunk <= 0 || !chunk_first || !states) return -1;
    oracle_job J = {num_seqs, seq_starts, H, HV, K, V, q, k, v, g, beta, A_log, dt_bias, h0,
                    gate_mode, qk_l2norm, beta_mode, lower_bound, scale, o, ht, NULL, chunk, chunk_first, states, 0};
    return run_job(&J, nthreads);
}

/*
 * Gate activation and chunk-local cumulative sum, natural-log units.
 * [NOTES] forward step 1: within chunk t the cumulative log decay at row r is
 * the sum of the activated gates of rows 1..r of that chunk (inclusive).
 * Chunks start at every sequence start and then every `chunk` tokens.
 *   g [Ttot][HV][K] -> g_act [Ttot][HV][K] (may be NULL), g_cum [Ttot][HV][K]
 */
int kda_oracle_gate_cumsum(int num_seqs, const int64_t *seq_starts, int HV, int K, int chunk,
                           const double *g, const double *A_log, const double *dt_bias,
                           int gate_mode, double lower_bound, double *g_act, double *g_cum) {
    if (chunk <= 0 || (gate_mode == GATE_SOFTPLUS && !A_log)) return -1;
    for (int n = 0; n < num_seqs; ++n)
        for (int hv = 0; hv < HV; ++hv)
            for (int d = 0; d < K; ++d) {
                double run = 0.0;
                for (int64_t t = seq_starts[n]; t < seq_starts[n + 1]; ++t) {
                    if ((t - seq_starts[n]) % chunk == 0) run = 0.0;
                    size_t idx = ((size_t)t * HV + hv) * K + d;
                    double a = gate_activate(gate_mode, g[idx], A_log, dt_bias, hv, K, d, lower_bound);
                    run += a;
                    if (g_act) g_act[idx] = a;
                    g_cum[idx] = run;
                }
            }
    return 0;
}
