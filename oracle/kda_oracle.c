/*
 * kda_oracle.c -- float64 CPU reference for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is
 * checked against.  It is slow on purpose: one token at a time, in float64,
 * with no chunking, no blocking and no reordering beyond the recurrence
 * itself.  Only tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it; the product library never does, and the two share no code.
 *
 * What it computes (fireworks.ai, "Kimi K3 on Fireworks: Fast RL at frontier
 * scale", section on Kimi Delta Attention: a linear attention whose compact
 * per-head recurrent state is updated with channel-wise gating).  The pages
 * give the mechanism only in prose; the recurrence written out here is the
 * gated delta rule with a per-channel decay, taken literally:
 *
 *   per (sequence, head), state S in R^{dk x dv} (row = key channel),
 *   S_0 = init_state (or 0)
 *   for t = 1..T:
 *     a_t     = exp(log_alpha_t)                  (dk channel decays)
 *     P_t     = Diag(a_t) S_{t-1}                 (decay first)
 *     delta_t = v_t - P_t^T k_t                   (prediction error of v_t)
 *     S_t     = P_t + beta_t k_t delta_t^T        (= (I - b k k^T) Diag(a) S + b k v^T)
 *     o_t     = scale * S_t^T q_t                 (output reads the updated state)
 *   final_state = S_T
 *
 * The backward pass is reverse-mode differentiation of exactly those steps,
 * token by token, with the states of each 64-token segment recomputed from a
 * checkpoint taken at the segment start (memory only; the arithmetic is the
 * same as storing every state).
 *
 * Layouts (token-major, sequences packed back to back):
 *   q, k, log_alpha, dq, dk, dlog_alpha : [n_tok][H][dk]
 *   v, out, d_out, dv                    : [n_tok][H][dv]
 *   beta, dbeta                          : [n_tok][H]
 *   states                               : [num_seqs][H][dk][dv]
 *   cu_seqlens                           : [num_seqs + 1], cu[0] = 0
 * Units of work are (sequence, head) pairs; a caller may restrict the run to
 * a list of units, in which case only their outputs are written.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int H, dk, dv, num_seqs;
    const int32_t *cu;
    const double *q, *k, *v, *log_alpha, *beta, *init;
    double scale;
    double *out, *final_state;
    /* backward only */
    const double *d_out, *d_final;
    double *dq, *dk_, *dv_, *dlog_alpha, *dbeta, *d_init;
    /* work list */
    const int32_t *units; /* pairs (seq, head); NULL => all */
    int n_units;
    int next;
    int failed;
    pthread_mutex_t mu;
} kda_job;

#define SEG 64

static int take_unit(kda_job *j) {
    pthread_mutex_lock(&j->mu);
    int u = j->next < j->n_units ? j->next++ : -1;
    pthread_mutex_unlock(&j->mu);
    return u;
}

static void unit_of(const kda_job *j, int u, int *seq, int *head) {
    if (j->units) {
        *seq = j->units[2 * u];
        *head = j->units[2 * u + 1];
    } else {
        *seq = u / j->H;
        *head = u % j->H;
    }
}

/* One token of the forward recurrence: S (in) -> S (out), writes P and delta. */
static void token_step(int dk, int dv, const double *la, const double *kt, const double *vt,
                       double bt, double *S, double *P, double *delta) {
    for (int c = 0; c < dk; ++c) {
        double a = exp(la[c]);
        for (int j = 0; j < dv; ++j) P[c * dv + j] = a * S[c * dv + j];
    }
    for (int j = 0; j < dv; ++j) {
        double pk = 0.0;
        for (int c = 0; c < dk; ++c) pk += P[c * dv + j] * kt[c];
        delta[j] = vt[j] - pk;
    }
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[c * dv + j] = P[c * dv + j] + bt * kt[c] * delta[j];
}

static void fwd_unit(const kda_job *j, int seq, int h) {
    const int H = j->H, dk = j->dk, dv = j->dv;
    const size_t sz = (size_t)dk * dv;
    double *S = malloc(sz * sizeof(double));
    double *P = malloc(sz * sizeof(double));
    double *delta = malloc(dv * sizeof(double));
    const double *S0 = j->init ? j->init + ((size_t)seq * H + h) * sz : NULL;
    for (size_t i = 0; i < sz; ++i) S[i] = S0 ? S0[i] : 0.0;
    for (int t = j->cu[seq]; t < j->cu[seq + 1]; ++t) {
        const size_t rk = ((size_t)t * H + h) * dk, rv = ((size_t)t * H + h) * dv;
        token_step(dk, dv, j->log_alpha + rk, j->k + rk, j->v + rv, j->beta[(size_t)t * H + h], S, P, delta);
        if (j->out) {
            const double *qt = j->q + rk;
            for (int jj = 0; jj < dv; ++jj) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += S[c * dv + jj] * qt[c];
                j->out[rv + jj] = j->scale * acc;
            }
        }
    }
    if (j->final_state) memcpy(j->final_state + ((size_t)seq * H + h) * sz, S, sz * sizeof(double));
    free(S);
    free(P);
    free(delta);
}

/*
 * Reverse-mode through the token steps.  G holds dL/dS_t while walking t
 * downward.  For token t with S_prev = S_{t-1}, P = Diag(a) S_prev,
 * delta = v - P^T k, S_t = P + b k delta^T, o_t = scale S_t^T q_t:
 *   G      += scale q_t dO_t^T
 *   dq_t    = scale S_t dO_t
 *   gk      = G^T k_t,  ddelta = b gk
 *   dv_t    = ddelta,   dbeta_t = gk . delta
 *   dk_t    = b G delta - P ddelta
 *   dP      = G - k_t ddelta^T
 *   dlog_alpha_t[c] = sum_j dP[c,j] P[c,j]
 *   G       = Diag(a) dP                     (becomes dL/dS_{t-1})
 */
static int bwd_unit(const kda_job *j, int seq, int h) {
    const int H = j->H, dk = j->dk, dv = j->dv;
    const size_t sz = (size_t)dk * dv;
    const int t0 = j->cu[seq], t1 = j->cu[seq + 1], len = t1 - t0;
    const int nseg = (len + SEG - 1) / SEG;
    double *ckpt = malloc(((size_t)(nseg > 0 ? nseg : 1)) * sz * sizeof(double));
    double *states = malloc((size_t)(SEG + 1) * sz * sizeof(double)); /* S_{s-1} .. S_{e} of a segment */
    double *P = malloc(sz * sizeof(double));
    double *dP = malloc(sz * sizeof(double));
    double *G = malloc(sz * sizeof(double));
    double *delta = malloc(dv * sizeof(double));
    double *gk = malloc(dv * sizeof(double));
    double *dd = malloc(dv * sizeof(double));
    if (!ckpt || !states || !P || !dP || !G || !delta || !gk || !dd) {
        free(ckpt); free(states); free(P); free(dP); free(G); free(delta); free(gk); free(dd);
        return 1;
    }
    const double *S0 = j->init ? j->init + ((size_t)seq * H + h) * sz : NULL;

    /* forward sweep: checkpoint the state entering each segment */
    double *S = states;
    for (size_t i = 0; i < sz; ++i) S[i] = S0 ? S0[i] : 0.0;
    for (int s = 0; s < nseg; ++s) {
        memcpy(ckpt + (size_t)s * sz, S, sz * sizeof(double));
        const int a = t0 + s * SEG, b = a + SEG < t1 ? a + SEG : t1;
        for (int t = a; t < b; ++t) {
            const size_t rk = ((size_t)t * H + h) * dk, rv = ((size_t)t * H + h) * dv;
            token_step(dk, dv, j->log_alpha + rk, j->k + rk, j->v + rv, j->beta[(size_t)t * H + h], S, P, delta);
        }
    }

    const double *dfin = j->d_final ? j->d_final + ((size_t)seq * H + h) * sz : NULL;
    for (size_t i = 0; i < sz; ++i) G[i] = dfin ? dfin[i] : 0.0;

    for (int s = nseg - 1; s >= 0; --s) {
        const int a = t0 + s * SEG, b = a + SEG < t1 ? a + SEG : t1;
        /* recompute S_{a-1} .. S_{b-1} of this segment into states[0..b-a] */
        memcpy(states, ckpt + (size_t)s * sz, sz * sizeof(double));
        for (int t = a; t < b; ++t) {
            const size_t rk = ((size_t)t * H + h) * dk, rv = ((size_t)t * H + h) * dv;
            double *Sn = states + (size_t)(t - a + 1) * sz;
            memcpy(Sn, states + (size_t)(t - a) * sz, sz * sizeof(double));
            token_step(dk, dv, j->log_alpha + rk, j->k + rk, j->v + rv, j->beta[(size_t)t * H + h], Sn, P, delta);
        }
        for (int t = b - 1; t >= a; --t) {
            const size_t rk = ((size_t)t * H + h) * dk, rv = ((size_t)t * H + h) * dv;
            const double *Sp = states + (size_t)(t - a) * sz;     /* S_{t-1} */
            const double *St = states + (size_t)(t - a + 1) * sz; /* S_t */
            const double *qt = j->q + rk, *kt = j->k + rk, *vt = j->v + rv, *la = j->log_alpha + rk;
            const double *dot = j->d_out + rv;
            const double bt = j->beta[(size_t)t * H + h];
            /* rebuild P and delta of this token */
            for (int c = 0; c < dk; ++c) {
                double al = exp(la[c]);
                for (int jj = 0; jj < dv; ++jj) P[c * dv + jj] = al * Sp[c * dv + jj];
            }
            for (int jj = 0; jj < dv; ++jj) {
                double pk = 0.0;
                for (int c = 0; c < dk; ++c) pk += P[c * dv + jj] * kt[c];
                delta[jj] = vt[jj] - pk;
            }
            /* output */
            for (int c = 0; c < dk; ++c)
                for (int jj = 0; jj < dv; ++jj) G[c * dv + jj] += j->scale * qt[c] * dot[jj];
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int jj = 0; jj < dv; ++jj) acc += St[c * dv + jj] * dot[jj];
                j->dq[rk + c] = j->scale * acc;
            }
            /* state update */
            double dbt = 0.0;
            for (int jj = 0; jj < dv; ++jj) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += G[c * dv + jj] * kt[c];
                gk[jj] = acc;
                dd[jj] = bt * acc;
                j->dv_[rv + jj] = dd[jj];
                dbt += acc * delta[jj];
            }
            j->dbeta[(size_t)t * H + h] = dbt;
            for (int c = 0; c < dk; ++c) {
                double gd = 0.0, pd = 0.0;
                for (int jj = 0; jj < dv; ++jj) {
                    gd += G[c * dv + jj] * delta[jj];
                    pd += P[c * dv + jj] * dd[jj];
                }
                j->dk_[rk + c] = bt * gd - pd;
            }
            for (int c = 0; c < dk; ++c) {
                double al = exp(la[c]);
                double dla = 0.0;
                for (int jj = 0; jj < dv; ++jj) {
                    dP[c * dv + jj] = G[c * dv + jj] - kt[c] * dd[jj];
                    dla += dP[c * dv + jj] * P[c * dv + jj];
                    G[c * dv + jj] = al * dP[c * dv + jj];
                }
                j->dlog_alpha[rk + c] = dla;
            }
        }
    }
    if (j->d_init) memcpy(j->d_init + ((size_t)seq * H + h) * sz, G, sz * sizeof(double));
    free(ckpt); free(states); free(P); free(dP); free(G); free(delta); free(gk); free(dd);
    return 0;
}

static void *worker_fwd(void *arg) {
    kda_job *j = arg;
    int u, seq, h;
    while ((u = take_unit(j)) >= 0) {
        unit_of(j, u, &seq, &h);
        fwd_unit(j, seq, h);
    }
    return NULL;
}

static void *worker_bwd(void *arg) {
    kda_job *j = arg;
    int u, seq, h;
    while ((u = take_unit(j)) >= 0) {
        unit_of(j, u, &seq, &h);
        if (bwd_unit(j, seq, h)) {
            pthread_mutex_lock(&j->mu);
            j->failed = 1;
            pthread_mutex_unlock(&j->mu);
        }
    }
    return NULL;
}

static int run(kda_job *j, void *(*fn)(void *), int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > j->n_units) nthreads = j->n_units > 0 ? j->n_units : 1;
    pthread_mutex_init(&j->mu, NULL);
    pthread_t *th = malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, fn, j) == 0) ++started;
    if (started == 0) fn(j);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&j->mu);
    return j->failed ? 2 : 0;
}

static int check(int H, int dk, int dv, int num_seqs, const int32_t *cu) {
    if (H < 1 || dk < 1 || dv < 1 || num_seqs < 0 || !cu || cu[0] != 0) return 1;
    for (int i = 0; i < num_seqs; ++i)
        if (cu[i + 1] < cu[i]) return 1;
    return 0;
}

/* Forward.  out / final_state may be NULL.  units: n_units (seq, head) pairs or NULL for all. */
int kda_oracle_fwd(int H, int dk, int dv, int num_seqs, const int32_t *cu_seqlens,
                   const double *q, const double *k, const double *v, const double *log_alpha,
                   const double *beta, const double *init_state, double scale,
                   double *out, double *final_state,
                   const int32_t *units, int n_units, int nthreads) {
    if (check(H, dk, dv, num_seqs, cu_seqlens)) return 1;
    kda_job j;
    memset(&j, 0, sizeof j);
    j.H = H; j.dk = dk; j.dv = dv; j.num_seqs = num_seqs; j.cu = cu_seqlens;
    j.q = q; j.k = k; j.v = v; j.log_alpha = log_alpha; j.beta = beta; j.init = init_state;
    j.scale = scale; j.out = out; j.final_state = final_state;
    j.units = units; j.n_units = units ? n_units : num_seqs * H;
    return run(&j, worker_fwd, nthreads);
}

/* Backward.  d_final_state may be NULL (treated as zero); d_init_state may be NULL. */
int kda_oracle_bwd(int H, int dk, int dv, int num_seqs, const int32_t *cu_seqlens,
                   const double *q, const double *k, const double *v, const double *log_alpha,
                   const double *beta, const double *init_state, double scale,
                   const double *d_out, const double *d_final_state,
                   double *dq, double *dk_out, double *dv_out, double *dlog_alpha, double *dbeta,
                   double *d_init_state, const int32_t *units, int n_units, int nthreads) {
    if (check(H, dk, dv, num_seqs, cu_seqlens)) return 1;
    if (!d_out || !dq || !dk_out || !dv_out || !dlog_alpha || !dbeta) return 1;
    kda_job j;
    memset(&j, 0, sizeof j);
    j.H = H; j.dk = dk; j.dv = dv; j.num_seqs = num_seqs; j.cu = cu_seqlens;
    j.q = q; j.k = k; j.v = v; j.log_alpha = log_alpha; j.beta = beta; j.init = init_state;
    j.scale = scale; j.d_out = d_out; j.d_final = d_final_state;
    j.dq = dq; j.dk_ = dk_out; j.dv_ = dv_out; j.dlog_alpha = dlog_alpha; j.dbeta = dbeta; j.d_init = d_init_state;
    j.units = units; j.n_units = units ? n_units : num_seqs * H;
    return run(&j, worker_bwd, nthreads);
}

/*
 * Decode / replay step (same page: KDA keeps a fixed-size decoding state; the
 * section on speculative decoding replays the state-update inputs of the
 * accepted tokens from a committed state instead of keeping a snapshot per
 * candidate).  B sequences with T tokens each, token-major [B][T][H][.];
 * sequence b reads its state from pool slot idx[b] (padding when idx[b] is
 * outside [0, pool_size): outputs 0, no state touched), runs the recurrence
 * over its T tokens writing every o_t, and the state after its first
 * n_commit[b] tokens (clamped to [0, T]; NULL means T) is written to slot
 * idx[b] of pool_out.  pool_out must hold a copy of pool_in on entry; slots
 * with nothing committed keep that copy.
 */
int kda_oracle_decode(int H, int dk, int dv, int B, int T, int pool_size,
                      const double *q, const double *k, const double *v, const double *log_alpha,
                      const double *beta, double scale, const double *pool_in,
                      const int32_t *idx, const int32_t *n_commit, double *out, double *pool_out) {
    if (H < 1 || dk < 1 || dv < 1 || B < 0 || T < 0 || pool_size < 0) return 1;
    if (B > 0 && T > 0 && (!q || !k || !v || !log_alpha || !beta || !out)) return 1;
    if (B > 0 && (!pool_in || !pool_out || !idx)) return 1;
    const size_t sz = (size_t)dk * dv;
    double *S = malloc(sz * sizeof(double));
    double *P = malloc(sz * sizeof(double));
    double *delta = malloc(dv * sizeof(double));
    if (!S || !P || !delta) {
        free(S); free(P); free(delta);
        return 1;
    }
    for (int b = 0; b < B; ++b) {
        const int slot = idx[b];
        const int pad = slot < 0 || slot >= pool_size;
        int n = n_commit ? n_commit[b] : T;
        if (n < 0) n = 0;
        if (n > T) n = T;
        for (int h = 0; h < H; ++h) {
            if (!pad) memcpy(S, pool_in + ((size_t)slot * H + h) * sz, sz * sizeof(double));
            for (int t = 0; t < T; ++t) {
                const size_t tok = (size_t)b * T + t;
                const size_t rk = (tok * H + h) * dk, rv = (tok * H + h) * dv;
                if (pad) {
                    for (int jj = 0; jj < dv; ++jj) out[rv + jj] = 0.0;
                    continue;
                }
                token_step(dk, dv, log_alpha + rk, k + rk, v + rv, beta[tok * H + h], S, P, delta);
                for (int jj = 0; jj < dv; ++jj) {
                    double acc = 0.0;
                    for (int c = 0; c < dk; ++c) acc += S[c * dv + jj] * q[rk + c];
                    out[rv + jj] = scale * acc;
                }
                if (t + 1 == n) memcpy(pool_out + ((size_t)slot * H + h) * sz, S, sz * sizeof(double));
            }
        }
    }
    free(S);
    free(P);
    free(delta);
    return 0;
}
