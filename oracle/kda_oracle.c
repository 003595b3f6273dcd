/*
 * kda_oracle.c -- plain, slow, token-by-token fp64 CPU reference for the
 * Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * kernels behind include/kda.h) never calls it and shares no source with it.
 *
 * What is computed, and where it comes from
 * -----------------------------------------
 * "Kimi K3 technical FAQ" (Runpod guide), question "What is KDA, and why does
 * a serving engineer care?": KDA is the delta-rule linear-attention
 * recurrence with a per-channel forget gate; every layer keeps a recurrent
 * state of shape dk x dv per head.  The same page, question "What does the
 * architecture actually look like?", says the forget gate is channel-wise and
 * the state is fixed-size.  The pages print no formula; the reading used here
 * (recorded with every other reading in the design notes) is
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = dk^(-1/2) S_t^T q_t,      alpha_t = exp(g_t) in (0,1]^dk.
 *
 * The update is evaluated in the algebraically identical rank-1 form
 *     S'  = Diag(alpha_t) S_{t-1}
 *     u_t = beta_t (v_t - S'^T k_t)
 *     S_t = S' + k_t u_t^T
 * which is the product form above with the bracket multiplied out
 * (the test suite checks it against the literal matrix-product form).
 *
 * "Day-0 vLLM support for Kimi K3" (vLLM blog), section "Kimi K3's
 * architecture, and how vLLM serves it": a prefix cache over recurrent state
 * reuses state snapshots taken at block boundaries, with the prefix-match
 * granularity separate from the physical state-block size.  A sequence's
 * first token in a call sits at absolute position s (0 unless given), and a
 * snapshot is the state after every absolute position P in (s, s + L] that is
 * a multiple of the interval, in order of P: with s = 0, snapshot j (1-based)
 * is the state after the sequence's first j*interval tokens.
 *
 * Precision: every quantity is fp64.  Inputs arrive as fp32 arrays holding
 * exactly the values the device path consumes (bf16 and fp32 values are both
 * exact in fp32); states arrive and leave as fp64.
 *
 * Layouts (row-major):
 *   q, k, g : [T_total, H, dk]     v : [T_total, H, dv]     beta : [T_total, H]
 *   states  : [num_seqs, H, dk, dv]   out : [T_total, H, dv]
 *   snapshots : [sum_b floor(L_b/interval), H, dk, dv], sequence b's block
 *   starting at row sum_{b'<b} floor(L_b'/interval).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* One token of the recurrence on one (sequence, head) state, in place.      */
/* S: dk x dv fp64, row i = key channel, column j = value channel.           */
/* u: scratch of dv doubles.  o: dv outputs (may be NULL).                   */
/* ------------------------------------------------------------------------ */
static void kda_token(int dk, int dv, double *S, double *u, const float *qt,
                      const float *kt, const float *vt, const float *gt,
                      double beta_t, double scale, double *o)
{
    int i, j;
    /* S' = Diag(alpha_t) S : channel i of the key side forgets by alpha_i. */
    for (i = 0; i < dk; ++i) {
        double alpha = exp((double)gt[i]);
        for (j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] *= alpha;
    }
    /* u = beta_t (v_t - S'^T k_t) : the delta-rule correction. */
    for (j = 0; j < dv; ++j) {
        double ks = 0.0;
        for (i = 0; i < dk; ++i)
            ks += (double)kt[i] * S[(size_t)i * dv + j];
        u[j] = beta_t * ((double)vt[j] - ks);
    }
    /* S_t = S' + k_t u^T */
    for (i = 0; i < dk; ++i) {
        double ki = (double)kt[i];
        for (j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] += ki * u[j];
    }
    /* o_t = scale * S_t^T q_t */
    if (o) {
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i)
                acc += (double)qt[i] * S[(size_t)i * dv + j];
            o[j] = scale * acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Prefill: packed variable-length sequences.                                */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t num_seqs, H, dk, dv;
    const int64_t *cu;
    const int64_t *start; /* absolute position of each first token, or NULL */
    const float *q, *k, *v, *g, *beta;
    const double *init;
    double scale;
    int64_t interval;
    const int64_t *snap_base;
    double *out, *final_state, *snapshots;
    int64_t next_unit; /* shared work counter */
    pthread_mutex_t lock;
    int failed;
} prefill_job;

static void prefill_unit(prefill_job *J, int64_t unit, double *S, double *u)
{
    const int H = J->H, dk = J->dk, dv = J->dv;
    const int b = (int)(unit / H), h = (int)(unit % H);
    const size_t ssz = (size_t)dk * dv;
    const int64_t t0 = J->cu[b], t1 = J->cu[b + 1];
    const int64_t s0 = J->start ? J->start[b] : 0;
    int64_t t;

    if (J->init)
        memcpy(S, J->init + ((size_t)b * H + h) * ssz, ssz * sizeof(double));
    else
        memset(S, 0, ssz * sizeof(double));

    for (t = t0; t < t1; ++t) {
        const size_t row = (size_t)t * H + h;
        kda_token(dk, dv, S, u, J->q + row * dk, J->k + row * dk,
                  J->v + row * dv, J->g + row * dk, (double)J->beta[row],
                  J->scale, J->out + row * dv);
        /* absolute position reached after token t: s0 + (t - t0 + 1) */
        if (J->interval > 0 && J->snapshots && ((s0 + t - t0 + 1) % J->interval) == 0) {
            int64_t jsnap = (s0 + t - t0 + 1) / J->interval - s0 / J->interval - 1;
            double *dst = J->snapshots +
                          ((size_t)(J->snap_base[b] + jsnap) * H + h) * ssz;
            memcpy(dst, S, ssz * sizeof(double));
        }
    }
    memcpy(J->final_state + ((size_t)b * H + h) * ssz, S, ssz * sizeof(double));
}

static int64_t take_unit(int64_t *counter, pthread_mutex_t *lock)
{
    int64_t u;
    pthread_mutex_lock(lock);
    u = (*counter)++;
    pthread_mutex_unlock(lock);
    return u;
}

static void *prefill_worker(void *arg)
{
    prefill_job *J = (prefill_job *)arg;
    const int64_t units = (int64_t)J->num_seqs * J->H;
    double *S = (double *)malloc((size_t)J->dk * J->dv * sizeof(double));
    double *u = (double *)malloc((size_t)J->dv * sizeof(double));
    if (!S || !u) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
    } else {
        for (;;) {
            int64_t unit = take_unit(&J->next_unit, &J->lock);
            if (unit >= units)
                break;
            prefill_unit(J, unit, S, u);
        }
    }
    free(S);
    free(u);
    return NULL;
}

static int run_pool(void *(*fn)(void *), void *job, int nthreads)
{
    pthread_t *tids;
    int i, started = 0;
    if (nthreads < 1)
        nthreads = 1;
    tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tids)
        return -1;
    for (i = 0; i < nthreads; ++i) {
        if (pthread_create(&tids[i], NULL, fn, job) != 0)
            break;
        ++started;
    }
    if (started == 0) /* no thread could start: do the work here */
        fn(job);
    for (i = 0; i < started; ++i)
        pthread_join(tids[i], NULL);
    free(tids);
    return 0;
}

/*
 * Number of snapshot rows the prefill writes: the multiples of the interval
 * in (s_b, s_b + L_b] summed over the sequences (s_b = 0 when start is NULL).
 */
int64_t kda_oracle_snapshot_count(int32_t num_seqs, const int64_t *cu,
                                  const int64_t *start, int64_t interval)
{
    int64_t n = 0;
    int32_t b;
    if (interval <= 0)
        return 0;
    for (b = 0; b < num_seqs; ++b) {
        const int64_t s0 = start ? start[b] : 0;
        n += (s0 + cu[b + 1] - cu[b]) / interval - s0 / interval;
    }
    return n;
}

/*
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 * initial_state may be NULL (zero state).  snapshots may be NULL only when
 * no snapshot falls due.  scale <= 0 selects dk^(-1/2).
 */
int kda_oracle_prefill(int32_t num_seqs, const int64_t *cu_seqlens,
                       const int64_t *start_pos, int32_t H, int32_t dk,
                       int32_t dv, const float *q, const float *k,
                       const float *v, const float *g, const float *beta,
                       const double *initial_state, double scale,
                       int64_t interval, double *out, double *final_state,
                       double *snapshots, int32_t nthreads)
{
    prefill_job J;
    int64_t *snap_base = NULL;
    int32_t b;
    int rc;

    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens ||
        !final_state || interval < 0)
        return -1;
    for (b = 0; b < num_seqs; ++b)
        if (cu_seqlens[b + 1] < cu_seqlens[b] || (start_pos && start_pos[b] < 0))
            return -1;
    if (!snapshots &&
        kda_oracle_snapshot_count(num_seqs, cu_seqlens, start_pos, interval) > 0)
        return -1;

    snap_base = (int64_t *)malloc(sizeof(int64_t) * ((size_t)num_seqs + 1));
    if (!snap_base)
        return -1;
    snap_base[0] = 0;
    for (b = 0; b < num_seqs; ++b)
        snap_base[b + 1] = snap_base[b] +
            kda_oracle_snapshot_count(1, cu_seqlens + b, start_pos ? start_pos + b : NULL,
                                      interval);

    memset(&J, 0, sizeof(J));
    J.num_seqs = num_seqs;
    J.H = H;
    J.dk = dk;
    J.dv = dv;
    J.cu = cu_seqlens;
    J.start = start_pos;
    J.q = q;
    J.k = k;
    J.v = v;
    J.g = g;
    J.beta = beta;
    J.init = initial_state;
    J.scale = scale > 0.0 ? scale : 1.0 / sqrt((double)dk);
    J.interval = interval;
    J.snap_base = snap_base;
    J.out = out;
    J.final_state = final_state;
    J.snapshots = snapshots;
    J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);

    rc = run_pool(prefill_worker, &J, nthreads);
    pthread_mutex_destroy(&J.lock);
    free(snap_base);
    return (rc != 0 || J.failed) ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Decode: `steps` chained single-token steps for N sequences.               */
/* Inputs are [steps, N, H, d]; state [num_slots, H, dk, dv] fp64 in place;  */
/* slots (nullable = identity) maps sequence n to its state row.             */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t steps, N, H, dk, dv;
    const float *q, *k, *v, *g, *beta;
    double *state;
    const int32_t *slots;
    double scale;
    double *out;
    int64_t next_unit;
    pthread_mutex_t lock;
    int failed;
} decode_job;

static void *decode_worker(void *arg)
{
    decode_job *J = (decode_job *)arg;
    const int64_t units = (int64_t)J->N * J->H;
    const int H = J->H, dk = J->dk, dv = J->dv;
    const size_t ssz = (size_t)dk * dv;
    double *u = (double *)malloc((size_t)dv * sizeof(double));
    if (!u) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
        return NULL;
    }
    for (;;) {
        int64_t unit = take_unit(&J->next_unit, &J->lock);
        int n, h, s;
        double *S;
        if (unit >= units)
            break;
        n = (int)(unit / H);
        h = (int)(unit % H);
        S = J->state + ((size_t)(J->slots ? J->slots[n] : n) * H + h) * ssz;
        for (s = 0; s < J->steps; ++s) {
            const size_t row = ((size_t)s * J->N + n) * H + h;
            kda_token(dk, dv, S, u, J->q + row * dk, J->k + row * dk,
                      J->v + row * dv, J->g + row * dk, (double)J->beta[row],
                      J->scale, J->out + row * dv);
        }
    }
    free(u);
    return NULL;
}

int kda_oracle_decode(int32_t steps, int32_t N, int32_t H, int32_t dk,
                      int32_t dv, const float *q, const float *k,
                      const float *v, const float *g, const float *beta,
                      double *state, const int32_t *slots, double scale,
                      double *out, int32_t nthreads)
{
    decode_job J;
    int rc;
    if (steps < 0 || N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !state || !out)
        return -1;
    memset(&J, 0, sizeof(J));
    J.steps = steps;
    J.N = N;
    J.H = H;
    J.dk = dk;
    J.dv = dv;
    J.q = q;
    J.k = k;
    J.v = v;
    J.g = g;
    J.beta = beta;
    J.state = state;
    J.slots = slots;
    J.scale = scale > 0.0 ? scale : 1.0 / sqrt((double)dk);
    J.out = out;
    pthread_mutex_init(&J.lock, NULL);
    rc = run_pool(decode_worker, &J, nthreads);
    pthread_mutex_destroy(&J.lock);
    return (rc != 0 || J.failed) ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Front end of q and k: short convolution -> Swish -> L2 normalisation.     */
/*                                                                          */
/* "Kimi K3 technical FAQ" (Runpod guide), question "What is KDA, and why    */
/* does a serving engineer care?": queries and keys pass through a short     */
/* convolution, Swish and L2 normalisation before the recurrence.  The page  */
/* gives neither the width nor the exact forms; the reading used here is     */
/*                                                                          */
/*   z_t[c] = sum_{j=0}^{W-1} w[c][j] * x_{t-(W-1)+j}[c]    (c = h*dk + i)   */
/*   a_t[c] = z_t[c] * sigmoid(z_t[c])                      (Swish, beta 1)  */
/*   y_t[h] = a_t[h] / sqrt(|a_t[h]|^2 + eps)      (per token and head)      */
/*                                                                          */
/* a depthwise, causal convolution along each sequence's own tokens (no      */
/* bias): tap W-1 weighs the current token, tap 0 the oldest.  Inputs before */
/* the sequence's first token come from its convolution state (the W-1       */
/* inputs that preceded it, oldest first) or are zero when there is none.    */
/* After the call the state of sequence b holds its last W-1 inputs (taken   */
/* from the state itself where the sequence is shorter than W-1).            */
/*                                                                          */
/* Layouts: x, y [T, H, dk]; w [H*dk, W]; states [num_slots, W-1, H, dk];    */
/* slots (nullable = identity) maps sequence b to its state row.             */
/* ------------------------------------------------------------------------ */
typedef struct {
    const int64_t *cu;
    int32_t H, dk, W;
    size_t C; /* channels per token, H * dk */
    const float *x, *w, *state_in;
} frontend_args;

/* Input of channel ch at token u of sequence b (u may precede the start). */
static double frontend_input(const frontend_args *A, int32_t b, int32_t slot,
                             int64_t u, size_t ch)
{
    const int64_t start = A->cu[b];
    if (u >= start)
        return (double)A->x[(size_t)u * A->C + ch];
    if (!A->state_in)
        return 0.0;
    /* state row r holds the input (W-1) - r tokens before the start */
    return (double)A->state_in[((size_t)slot * (A->W - 1) +
                                (size_t)((A->W - 1) + (u - start))) * A->C + ch];
}

int kda_oracle_qk_frontend(int32_t num_seqs, const int64_t *cu, int32_t H,
                           int32_t dk, int32_t W, const float *x,
                           const float *w, const float *state_in,
                           const int32_t *slots, double eps, double *y,
                           float *state_out)
{
    frontend_args A;
    double *a = NULL;
    float *tail = NULL;
    int32_t b;
    if (num_seqs < 0 || !cu || H <= 0 || dk <= 0 || W < 1 || !w || !(eps > 0.0))
        return -1;
    for (b = 0; b < num_seqs; ++b)
        if (cu[b + 1] < cu[b])
            return -1;
    A.cu = cu;
    A.H = H;
    A.dk = dk;
    A.W = W;
    A.C = (size_t)H * dk;
    A.x = x;
    A.w = w;
    A.state_in = state_in;
    a = (double *)malloc(sizeof(double) * (size_t)dk);
    tail = (float *)malloc(sizeof(float) * (A.C * (size_t)W + 1));
    if (!a || !tail) {
        free(a);
        free(tail);
        return -1;
    }
    for (b = 0; b < num_seqs; ++b) {
        const int32_t slot = slots ? slots[b] : b;
        int64_t t;
        int32_t h, i, j, r;
        for (t = cu[b]; t < cu[b + 1]; ++t) {
            for (h = 0; h < H; ++h) {
                double n2 = 0.0;
                for (i = 0; i < dk; ++i) {
                    const size_t ch = (size_t)h * dk + i;
                    double z = 0.0;
                    for (j = 0; j < W; ++j)
                        z += (double)w[ch * W + j] *
                             frontend_input(&A, b, slot, t - (W - 1) + j, ch);
                    a[i] = z / (1.0 + exp(-z));
                    n2 += a[i] * a[i];
                }
                for (i = 0; i < dk; ++i)
                    y[((size_t)t * H + h) * dk + i] = a[i] / sqrt(n2 + eps);
            }
        }
        /* new state: the last W-1 inputs, gathered before any is written so
           that state_out may be state_in itself */
        if (state_out && W > 1) {
            size_t ch;
            for (r = 0; r < W - 1; ++r)
                for (ch = 0; ch < A.C; ++ch)
                    tail[(size_t)r * A.C + ch] = (float)frontend_input(
                        &A, b, slot, cu[b + 1] - (W - 1) + r, ch);
            memcpy(state_out + (size_t)slot * (W - 1) * A.C, tail,
                   sizeof(float) * A.C * (size_t)(W - 1));
        }
    }
    free(a);
    free(tail);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention Residuals aggregation (block variant), one layer's input.       */
/*                                                                          */
/* "Kimi K3 technical FAQ" (Runpod guide), question "What does the          */
/* architecture actually look like?": each layer can attend over the        */
/* embedding plus the preceding block outputs through a learned             */
/* pseudo-query (blocks of 12 layers, about 8 blocks).  "Day-0 vLLM support */
/* for Kimi K3" (vLLM blog), section "Kimi K3's architecture, and how vLLM  */
/* serves it": the fused kernel computes the logits, the softmax across the */
/* previous layers and the aggregation, and folds in the residual add and   */
/* the output RMSNorm.  The pages give no formula; the reading used here,   */
/* per token t, with sources s_m (m < M), pseudo-query w and residual x:    */
/*                                                                          */
/*   l_m = scale * <w, s_m,t>            p = softmax_m(l)                   */
/*   h_t = sum_m p_m s_m,t + x_t         (x absent: no residual add)        */
/*   y_t = h_t / sqrt(mean_c h_t[c]^2 + eps) * gamma   (gamma absent: 1)    */
/*                                                                          */
/* Layouts: sources [M][T][d] (one array per source, contiguous here);      */
/* x, h, y [T][d]; w, gamma [d].                                            */
/* ------------------------------------------------------------------------ */
int kda_oracle_attnres(int32_t M, int64_t T, int32_t d, const float *src,
                       const float *x, const float *w, const float *gamma,
                       double scale, double eps, double *h, double *y)
{
    double *l;
    int64_t t;
    int32_t m, c;
    if (M < 1 || T < 0 || d < 1 || !src || !w || !h || !y || !(eps > 0.0))
        return -1;
    l = (double *)malloc(sizeof(double) * (size_t)M);
    if (!l)
        return -1;
    for (t = 0; t < T; ++t) {
        double mx, z = 0.0, ms = 0.0, r;
        double *ht = h + (size_t)t * d, *yt = y + (size_t)t * d;
        /* logits of the sources */
        for (m = 0; m < M; ++m) {
            const float *s = src + ((size_t)m * T + t) * d;
            double acc = 0.0;
            for (c = 0; c < d; ++c)
                acc += (double)w[c] * (double)s[c];
            l[m] = scale * acc;
        }
        /* softmax over the sources (shifted by the largest logit) */
        mx = l[0];
        for (m = 1; m < M; ++m)
            if (l[m] > mx)
                mx = l[m];
        for (m = 0; m < M; ++m) {
            l[m] = exp(l[m] - mx);
            z += l[m];
        }
        for (m = 0; m < M; ++m)
            l[m] /= z;
        /* weighted sum of the sources, plus the residual */
        for (c = 0; c < d; ++c) {
            double acc = x ? (double)x[(size_t)t * d + c] : 0.0;
            for (m = 0; m < M; ++m)
                acc += l[m] * (double)src[((size_t)m * T + t) * d + c];
            ht[c] = acc;
            ms += acc * acc;
        }
        /* RMSNorm of the result */
        r = 1.0 / sqrt(ms / d + eps);
        for (c = 0; c < d; ++c)
            yt[c] = ht[c] * r * (gamma ? (double)gamma[c] : 1.0);
    }
    free(l);
    return 0;
}
