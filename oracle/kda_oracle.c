/*
 * kda_oracle.c - plain CPU oracle for the KDA recurrent-state step.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU library never links,
 * includes or calls it, and it shares no code with the GPU library.
 *
 * What is computed.
 *   The pages name the KDA recurrent state as a decode bottleneck of Kimi K3
 *   ("Kimi K3 performance optimization in vLLM", opening paragraph) and say the
 *   decode test used an FP32 SSM cache ("Kimi K3 vLLM optimization: NVIDIA
 *   decode speed-up 1.68x", section "What the upstream tests actually show").
 *   They do not write the update out. This file takes KDA to be the gated delta
 *   rule with per-channel decay. Per head, with the state S a dk x dv matrix
 *   (row i = key channel, column j = value channel), each token applies
 *       S <- Diag(alpha) S                      (decay, one factor per key channel)
 *       S <- S + beta k (v - S^T k)^T            (delta-rule write)
 *       o  = S^T q                               (read-out on the updated state)
 *   Verify and commit follow "ReplaySSM for state reconstruction" (same page as
 *   above, section "Advanced memory and state management"): a speculative
 *   chunk of draft tokens is evaluated without touching the committed state,
 *   and the commit rebuilds the state after the accepted prefix of the chunk.
 *   Rows of a mixed batch are packed contiguously and outputs are written at
 *   each row's offset ("Zero-copy mixed KDA batching", same page).
 *   The optional output gate (per head, over the whole value vector) is
 *       y = o / sqrt(mean_j o_j^2 + eps) * w * sigmoid(gate),
 *   the gating fused at the output that "Hyper Optimizing Kimi K3 in vLLM",
 *   section "Finding time between operators", mentions.
 *
 * Precision. All arithmetic is double. The state is stored as float32 (the
 * FP32 SSM cache) and, when state_fp32 is set, re-rounded to float32 (round to
 * nearest even) after every token, as a GPU that keeps float32 state between
 * tokens does. With state_fp32 == 0 the state stays double inside one call.
 * Outputs are rounded to float32. bf16 inputs widen exactly.
 *
 * Layouts (host arrays, all contiguous):
 *   cache  float [num_slots slots, stride slot_stride][H][dv][dk]: element
 *          (i, j) of head h in slot s is cache[s*slot_stride + (h*dv + j)*dk + i]
 *   q, k   bf16 bits [n_tok][H][dk]; v, gate bf16 bits [n_tok][H][dv]
 *   alpha  float [n_tok][H][dk]; beta float [n_tok][H]; out float [n_tok][H][dv]
 *   replay buffers rk [B][T_max][H][dk] (bf16), rv [B][T_max][H][dv] (bf16),
 *          ralpha [B][T_max][H][dk], rbeta [B][T_max][H]
 *   draft  float [B][T_max][H][dv][dk]
 * Slot and row handling: slot < 0 is padding (nothing read or written);
 * slot >= num_slots sets error bit 1; a row whose token range is decreasing,
 * out of [0, n_tok] or longer than T_max sets bit 2; an accepted length
 * outside [0, T_b] sets bit 4; a checkpoint position outside [0, T_b] (prefill)
 * sets bit 8. A row with an error is skipped entirely.
 *
 * Raw inputs (prologue != 0): q, k, alpha and beta hold the raw projections and
 * the oracle prepares them per (token, head) first, in double:
 *     k <- k / sqrt(sum_i k_i^2 + 1e-12)
 *     q <- q / sqrt(sum_i q_i^2 + 1e-12) / sqrt(dk)
 *     alpha_i <- exp(-softplus(alpha_i)) = exp(-log(1 + exp(alpha_i)))
 *     beta <- sigmoid(beta) = 1 / (1 + exp(-beta))
 * (the normalization and gate activations that precede the recurrence; the
 * fused form of "Hyper Optimizing Kimi K3 in vLLM", section "Finding time
 * between operators"). Replay buffers then hold the raw values.
 *
 * Prefill ("Kimi K3 performance optimization in vLLM", section "Internal KDA
 * prefix checkpoint"): one pass over a row's whole prompt from the slot's
 * state, outputs for every token, the final state written back to the slot,
 * and, in the same pass, the state after the first ckpt_pos[b] tokens exported
 * to a checkpoint buffer [B][H][dv][dk] (ckpt_pos[b] < 0: no export).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_REPLAY 0
#define ORACLE_PER_POSITION 1

#define ERR_SLOT 1
#define ERR_SEQLEN 2
#define ERR_ACCEPTED 4
#define ERR_CKPT 8

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * The recurrence for one (sequence, head) over n tokens.
 *   S      in/out, dk*dv doubles, S[i*dv + j] = row i, column j
 *   q, k   n*dk; v n*dv; alpha n*dk; beta n
 *   o      n*dv or NULL: the read-out after each token
 *   S_tok  n*dk*dv or NULL: the state after each token
 */
void kda_oracle_unit(double *S, int dk, int dv, int n,
                     const double *q, const double *k, const double *v,
                     const double *alpha, const double *beta,
                     int state_fp32, double *o, double *S_tok)
{
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int t = 0; t < n; ++t) {
        const double *qt = q ? q + (size_t)t * dk : NULL;
        const double *kt = k + (size_t)t * dk;
        const double *vt = v + (size_t)t * dv;
        const double *at = alpha + (size_t)t * dk;
        const double bt = beta[t];

        /* decay: S <- Diag(alpha) S scales row i by alpha[i] */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] = at[i] * S[i * dv + j];

        /* what the memory currently returns for key k: u = S^T k */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += S[i * dv + j] * kt[i];
            u[j] = acc;
        }

        /* delta-rule write: S <- S + beta k (v - u)^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] += bt * kt[i] * (vt[j] - u[j]);

        /* read-out on the updated state: o = S^T q */
        if (o) {
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i)
                    acc += S[i * dv + j] * qt[i];
                o[(size_t)t * dv + j] = acc;
            }
        }

        if (state_fp32)
            for (int e = 0; e < dk * dv; ++e)
                S[e] = (double)(float)S[e];
        if (S_tok)
            memcpy(S_tok + (size_t)t * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    }
    free(u);
}

/* Output gate over one head's value vector: y = o / sqrt(mean(o^2) + eps) * w * sigmoid(g). */
void kda_oracle_epilogue(const double *o, int dv, const double *g, const double *w,
                         double eps, double *y)
{
    double ms = 0.0;
    for (int j = 0; j < dv; ++j)
        ms += o[j] * o[j];
    ms /= (double)dv;
    const double inv_rms = 1.0 / sqrt(ms + eps);
    for (int j = 0; j < dv; ++j) {
        const double wj = w ? w[j] : 1.0;
        const double sig = 1.0 / (1.0 + exp(-g[j]));
        y[j] = o[j] * inv_rms * wj * sig;
    }
}

/* Raw projections of one (token, head) to the recurrence's inputs (see the header). */
static void prepare_inputs(double *q, double *k, double *alpha, double *beta, int dk)
{
    double kk = 0.0, qq = 0.0;
    for (int i = 0; i < dk; ++i) {
        kk += k[i] * k[i];
        qq += q[i] * q[i];
    }
    const double kn = 1.0 / sqrt(kk + 1e-12);
    const double qn = 1.0 / sqrt(qq + 1e-12) / sqrt((double)dk);
    for (int i = 0; i < dk; ++i) {
        k[i] *= kn;
        q[i] *= qn;
        alpha[i] = exp(-log1p(exp(alpha[i])));
    }
    *beta = 1.0 / (1.0 + exp(-*beta));
}

/* ---------------------------------------------------------------------------
 * Batch drivers: slot lookup, token ranges, layouts, modes. One work item per
 * (row b, head h); items are independent, so threads only split the list.
 * ------------------------------------------------------------------------- */

enum { KIND_DECODE = 0, KIND_VERIFY = 1, KIND_COMMIT = 2, KIND_PREFILL = 3 };

typedef struct {
    int kind;
    float *cache;
    int64_t num_slots, slot_stride;
    const int32_t *slot_ids, *cu, *accepted;
    int32_t B, T_max, n_tok, H, dk, dv;
    const uint16_t *q, *k, *v, *gate;
    const float *alpha, *beta, *weight;
    double eps;
    float *out;
    int32_t mode, t1_inplace;
    uint16_t *rk, *rv;
    float *ralpha, *rbeta, *draft;
    const int32_t *ckpt_pos;
    float *ckpt;
    int32_t prologue;
    int32_t state_fp32;
} call_t;

typedef struct {
    const call_t *c;
    int tid, nthreads;
    int err;
} worker_t;

static int64_t cache_index(const call_t *c, int64_t slot, int h, int j, int i)
{
    return slot * c->slot_stride + ((int64_t)h * c->dv + j) * c->dk + i;
}

static int run_item(const call_t *c, int b, int h)
{
    const int dk = c->dk, dv = c->dv, H = c->H;
    const int64_t slot = c->slot_ids[b];
    if (slot < 0)
        return 0;
    if (slot >= c->num_slots)
        return ERR_SLOT;

    int64_t row0, Tb;
    if (c->kind == KIND_DECODE) {
        row0 = b;
        Tb = 1;
    } else {
        row0 = c->cu[b];
        Tb = (int64_t)c->cu[b + 1] - row0;
        if (row0 < 0 || Tb < 0 || row0 + Tb > c->n_tok || (c->kind != KIND_PREFILL && Tb > c->T_max))
            return ERR_SEQLEN;
    }
    int64_t ckpt_at = -1;
    if (c->kind == KIND_PREFILL && c->ckpt_pos) {
        ckpt_at = c->ckpt_pos[b];
        if (ckpt_at > Tb)
            return ERR_CKPT;
    }
    int64_t n = Tb;
    if (c->kind == KIND_COMMIT) {
        const int32_t a = c->accepted[b];
        if (a < 0 || a > Tb)
            return ERR_ACCEPTED;
        n = a;
    }
    if (n == 0 && ckpt_at != 0)
        return 0;

    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *q = (double *)malloc(sizeof(double) * (size_t)n * dk);
    double *k = (double *)malloc(sizeof(double) * (size_t)n * dk);
    double *a = (double *)malloc(sizeof(double) * (size_t)n * dk);
    double *v = (double *)malloc(sizeof(double) * (size_t)n * dv);
    double *be = (double *)malloc(sizeof(double) * (size_t)n);
    double *o = (double *)malloc(sizeof(double) * (size_t)n * dv);
    /* a single-token row of a mixed batch, updated in place (t1_inplace) */
    const int inplace_row = c->kind == KIND_VERIFY && Tb == 1 && c->t1_inplace;
    const int per_position = c->kind == KIND_VERIFY && c->mode == ORACLE_PER_POSITION && !inplace_row;
    double *S_tok = per_position ? (double *)malloc(sizeof(double) * (size_t)n * dk * dv) : NULL;

    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[i * dv + j] = (double)c->cache[cache_index(c, slot, h, j, i)];

    for (int64_t t = 0; t < n; ++t) {
        const int64_t r = (row0 + t) * H + h;
        for (int i = 0; i < dk; ++i) {
            q[t * dk + i] = c->q ? bf16_to_double(c->q[r * dk + i]) : 0.0;
            k[t * dk + i] = bf16_to_double(c->k[r * dk + i]);
            a[t * dk + i] = (double)c->alpha[r * dk + i];
        }
        for (int j = 0; j < dv; ++j)
            v[t * dv + j] = bf16_to_double(c->v[r * dv + j]);
        be[t] = (double)c->beta[r];
        if (c->prologue)
            prepare_inputs(q + t * dk, k + t * dk, a + t * dk, &be[t], dk);
    }

    if (c->kind == KIND_PREFILL && ckpt_at >= 0) {
        /* the prompt in two runs, split at the checkpoint: the state carries over unchanged */
        kda_oracle_unit(S, dk, dv, (int)ckpt_at, q, k, v, a, be, c->state_fp32, o, NULL);
        float *dst = c->ckpt + ((int64_t)b * H + h) * (int64_t)dv * dk;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                dst[(int64_t)j * dk + i] = (float)S[i * dv + j];
        kda_oracle_unit(S, dk, dv, (int)(n - ckpt_at), q + ckpt_at * dk, k + ckpt_at * dk, v + ckpt_at * dv,
                        a + ckpt_at * dk, be + ckpt_at, c->state_fp32, o + ckpt_at * dv, NULL);
    } else {
        kda_oracle_unit(S, dk, dv, (int)n, q, k, v, a, be, c->state_fp32,
                        c->kind == KIND_COMMIT ? NULL : o, S_tok);
    }

    if (c->kind != KIND_COMMIT && c->out) {
        double *y = (double *)malloc(sizeof(double) * (size_t)dv);
        double *g = (double *)malloc(sizeof(double) * (size_t)dv);
        double *w = c->weight ? (double *)malloc(sizeof(double) * (size_t)dv) : NULL;
        if (w)
            for (int j = 0; j < dv; ++j)
                w[j] = (double)c->weight[j];
        for (int64_t t = 0; t < n; ++t) {
            const int64_t r = (row0 + t) * H + h;
            const double *ot = o + t * dv;
            if (c->gate) {
                for (int j = 0; j < dv; ++j)
                    g[j] = bf16_to_double(c->gate[r * dv + j]);
                kda_oracle_epilogue(ot, dv, g, w, c->eps, y);
                ot = y;
            }
            for (int j = 0; j < dv; ++j)
                c->out[r * dv + j] = (float)ot[j];
        }
        free(y);
        free(g);
        free(w);
    }

    /* Where the row's state goes: a speculative row in per-position mode writes
     * every draft position; the single-token steps (decode, in-place rows), the
     * commit and the prefill write the slot; a speculative row in replay mode
     * buffers its inputs and leaves the slot alone. */
    const int write_slot = c->kind == KIND_DECODE || c->kind == KIND_COMMIT || c->kind == KIND_PREFILL ||
                           inplace_row;
    if (per_position) {
        for (int64_t t = 0; t < n; ++t) {
            float *dst = c->draft + (((int64_t)b * c->T_max + t) * H + h) * (int64_t)dv * dk;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    dst[(int64_t)j * dk + i] = (float)S_tok[t * dk * dv + i * dv + j];
        }
    } else if (write_slot) {
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                c->cache[cache_index(c, slot, h, j, i)] = (float)S[i * dv + j];
    } else if (c->kind == KIND_VERIFY) {
        /* replay buffer: exact copies of this row's per-token inputs */
        for (int64_t t = 0; t < n; ++t) {
            const int64_t r = (row0 + t) * H + h;
            const int64_t d = ((int64_t)b * c->T_max + t) * H + h;
            memcpy(c->rk + d * dk, c->k + r * dk, sizeof(uint16_t) * dk);
            memcpy(c->ralpha + d * dk, c->alpha + r * dk, sizeof(float) * dk);
            memcpy(c->rv + d * dv, c->v + r * dv, sizeof(uint16_t) * dv);
            c->rbeta[d] = c->beta[r];
        }
    }

    free(S);
    free(q);
    free(k);
    free(a);
    free(v);
    free(be);
    free(o);
    free(S_tok);
    return 0;
}

static void *worker_main(void *arg)
{
    worker_t *w = (worker_t *)arg;
    const call_t *c = w->c;
    const int64_t items = (int64_t)c->B * c->H;
    for (int64_t it = w->tid; it < items; it += w->nthreads)
        w->err |= run_item(c, (int)(it / c->H), (int)(it % c->H));
    return NULL;
}

static int run_call(const call_t *c, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    worker_t *ws = (worker_t *)calloc((size_t)nthreads, sizeof(worker_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int t = 0; t < nthreads; ++t) {
        ws[t].c = c;
        ws[t].tid = t;
        ws[t].nthreads = nthreads;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker_main, &ws[t]) != 0)
            break;
        started = t;
    }
    /* items of threads that failed to start run here, in order */
    for (int t = started + 1; t < nthreads; ++t)
        worker_main(&ws[t]);
    worker_main(&ws[0]);
    int err = ws[0].err;
    for (int t = 1; t <= started; ++t) {
        pthread_join(th[t], NULL);
        err |= ws[t].err;
    }
    for (int t = started + 1; t < nthreads; ++t)
        err |= ws[t].err;
    free(ws);
    free(th);
    return err;
}

static int dims_ok(int32_t B, int32_t H, int32_t dk, int32_t dv, int64_t num_slots,
                   int64_t slot_stride)
{
    return B >= 0 && H > 0 && dk > 0 && dv > 0 && num_slots >= 0 &&
           slot_stride >= (int64_t)H * dk * dv;
}

/* One token per row (row b reads token b); the state is updated in place. */
int kda_oracle_decode(float *cache, int64_t num_slots, int64_t slot_stride,
                      const int32_t *slot_ids, int32_t B, int32_t H, int32_t dk, int32_t dv,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const float *alpha, const float *beta, float *out,
                      const uint16_t *gate, const float *weight, double eps,
                      int32_t prologue, int32_t state_fp32, int32_t nthreads)
{
    if (!dims_ok(B, H, dk, dv, num_slots, slot_stride))
        return -1;
    if (B == 0)
        return 0;
    if (!cache || !slot_ids || !q || !k || !v || !alpha || !beta || !out)
        return -1;
    call_t c;
    memset(&c, 0, sizeof c);
    c.kind = KIND_DECODE;
    c.cache = cache;
    c.num_slots = num_slots;
    c.slot_stride = slot_stride;
    c.slot_ids = slot_ids;
    c.B = B;
    c.T_max = 1;
    c.n_tok = B;
    c.H = H;
    c.dk = dk;
    c.dv = dv;
    c.q = q;
    c.k = k;
    c.v = v;
    c.alpha = alpha;
    c.beta = beta;
    c.out = out;
    c.gate = gate;
    c.weight = weight;
    c.eps = eps;
    c.prologue = prologue;
    c.state_fp32 = state_fp32;
    return run_call(&c, nthreads);
}

/*
 * A packed chunk of rows; row b owns tokens [cu[b], cu[b+1]). Outputs are
 * written for every token. The committed slot is not written, except for rows
 * of one token when t1_inplace is set (the non-speculative members of a mixed
 * batch), which are updated in place. mode ORACLE_REPLAY copies each row's
 * per-token inputs to the replay buffers; ORACLE_PER_POSITION writes the state
 * after each token to draft.
 */
int kda_oracle_verify(float *cache, int64_t num_slots, int64_t slot_stride,
                      const int32_t *slot_ids, const int32_t *cu_seqlens,
                      int32_t B, int32_t T_max, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const float *alpha, const float *beta, float *out,
                      const uint16_t *gate, const float *weight, double eps,
                      int32_t mode, int32_t t1_inplace,
                      uint16_t *rk, uint16_t *rv, float *ralpha, float *rbeta, float *draft,
                      int32_t prologue, int32_t state_fp32, int32_t nthreads)
{
    if (!dims_ok(B, H, dk, dv, num_slots, slot_stride) || T_max < 1 || n_tok < 0)
        return -1;
    if (mode != ORACLE_REPLAY && mode != ORACLE_PER_POSITION)
        return -1;
    if (B == 0)
        return 0;
    if (!cache || !slot_ids || !cu_seqlens || !q || !k || !v || !alpha || !beta || !out)
        return -1;
    if (mode == ORACLE_REPLAY && (!rk || !rv || !ralpha || !rbeta))
        return -1;
    if (mode == ORACLE_PER_POSITION && !draft)
        return -1;
    call_t c;
    memset(&c, 0, sizeof c);
    c.kind = KIND_VERIFY;
    c.cache = cache;
    c.num_slots = num_slots;
    c.slot_stride = slot_stride;
    c.slot_ids = slot_ids;
    c.cu = cu_seqlens;
    c.B = B;
    c.T_max = T_max;
    c.n_tok = n_tok;
    c.H = H;
    c.dk = dk;
    c.dv = dv;
    c.q = q;
    c.k = k;
    c.v = v;
    c.alpha = alpha;
    c.beta = beta;
    c.out = out;
    c.gate = gate;
    c.weight = weight;
    c.eps = eps;
    c.mode = mode;
    c.t1_inplace = t1_inplace;
    c.rk = rk;
    c.rv = rv;
    c.ralpha = ralpha;
    c.rbeta = rbeta;
    c.draft = draft;
    c.prologue = prologue;
    c.state_fp32 = state_fp32;
    return run_call(&c, nthreads);
}

/*
 * Commit: slot of row b <- the state after the first accepted_len[b] tokens of
 * the row's chunk, starting from the slot's committed state. This is the
 * definition both GPU commit modes must reach; the oracle reads the original
 * packed inputs (k, v, alpha, beta) rather than any buffer.
 */
int kda_oracle_commit(float *cache, int64_t num_slots, int64_t slot_stride,
                      const int32_t *slot_ids, const int32_t *cu_seqlens,
                      const int32_t *accepted_len,
                      int32_t B, int32_t T_max, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                      const uint16_t *k, const uint16_t *v, const float *alpha, const float *beta,
                      int32_t prologue, int32_t state_fp32, int32_t nthreads)
{
    if (!dims_ok(B, H, dk, dv, num_slots, slot_stride) || T_max < 1 || n_tok < 0)
        return -1;
    if (B == 0)
        return 0;
    if (!cache || !slot_ids || !cu_seqlens || !accepted_len || !k || !v || !alpha || !beta)
        return -1;
    call_t c;
    memset(&c, 0, sizeof c);
    c.kind = KIND_COMMIT;
    c.cache = cache;
    c.num_slots = num_slots;
    c.slot_stride = slot_stride;
    c.slot_ids = slot_ids;
    c.cu = cu_seqlens;
    c.accepted = accepted_len;
    c.B = B;
    c.T_max = T_max;
    c.n_tok = n_tok;
    c.H = H;
    c.dk = dk;
    c.dv = dv;
    c.k = k;
    c.v = v;
    c.alpha = alpha;
    c.beta = beta;
    c.prologue = prologue;
    c.state_fp32 = state_fp32;
    return run_call(&c, nthreads);
}

/*
 * Prefill: row b runs its whole prompt [cu[b], cu[b+1]) from the slot's state;
 * outputs for every token; the final state goes back to the slot; the state
 * after the first ckpt_pos[b] tokens (0 = the state before the prompt) is
 * exported to ckpt [B][H][dv][dk] in the same pass. ckpt_pos may be NULL.
 */
int kda_oracle_prefill(float *cache, int64_t num_slots, int64_t slot_stride,
                       const int32_t *slot_ids, const int32_t *cu_seqlens,
                       int32_t B, int32_t n_tok, int32_t H, int32_t dk, int32_t dv,
                       const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const float *alpha, const float *beta, float *out,
                       const int32_t *ckpt_pos, float *ckpt,
                       int32_t prologue, int32_t state_fp32, int32_t nthreads)
{
    if (!dims_ok(B, H, dk, dv, num_slots, slot_stride) || n_tok < 0)
        return -1;
    if (B == 0)
        return 0;
    if (!cache || !slot_ids || !cu_seqlens || !q || !k || !v || !alpha || !beta || !out)
        return -1;
    if (ckpt_pos && !ckpt)
        return -1;
    call_t c;
    memset(&c, 0, sizeof c);
    c.kind = KIND_PREFILL;
    c.cache = cache;
    c.num_slots = num_slots;
    c.slot_stride = slot_stride;
    c.slot_ids = slot_ids;
    c.cu = cu_seqlens;
    c.B = B;
    c.T_max = n_tok;
    c.n_tok = n_tok;
    c.H = H;
    c.dk = dk;
    c.dv = dv;
    c.q = q;
    c.k = k;
    c.v = v;
    c.alpha = alpha;
    c.beta = beta;
    c.out = out;
    c.ckpt_pos = ckpt_pos;
    c.ckpt = ckpt;
    c.prologue = prologue;
    c.state_fp32 = state_fp32;
    return run_call(&c, nthreads);
}
