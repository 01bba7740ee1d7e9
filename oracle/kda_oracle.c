/*
 * kda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of the Kimi Delta
 * Attention (KDA) recurrence in double precision.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load this library; the
 * product path (the HIP library under gated_delta_rule_54_amd/) never does,
 * and the two share no code, header, table or helper.
 *
 * Pages cited (each by title and section):
 *   [XT] xutianle.me, "Kimi Linear：用 KDA 重写长上下文注意力"
 *   [XD] xiudou.site, "Kimi Delta Attention：把遗忘门做到每个通道"
 *   [DS] docsaid.org, "Kimi Linear" (逐通道的遺忘)
 *
 * What is computed, per (sequence, head) chain, token by token:
 *   1. q^ = q / sqrt(sum q^2 + eps), k^ likewise (eps = 1e-6), when
 *      qk_l2norm is set.  [XT §6.2 "L2Norm 稳定 key 与 query"; XD, the
 *      preprocessing list before the recurrence]  The pages give no eps; 1e-6
 *      under the square root is this project's reading.
 *   2. alpha = exp(g), one factor per key channel.  [XT §3: alpha_t is a
 *      d_k-vector; the operator receives it in log space]
 *   3. S~ = Diag(alpha) S : every ROW c of the d_k x d_v state is scaled by
 *      alpha_c.  [XT §3, decay step; DS §"KDA：把衰減拆到每個通道", the state
 *      is d_k x d_v and the matrices multiply on the left; its two-channel
 *      table (8,6) -> (8,0.6) fixes that rows are key channels]
 *   4. u = beta (v - S~^T k^)           [XT §2/§3, the error-correcting form]
 *   5. S = S~ + k^ u^T                  [XT §3, boxed KDA update]
 *   6. o = scale * S^T q^, with the UPDATED state.  [XT §1: o_t = S_t^T q_t]
 * The decode oracle applies the same single-token step to a saved state;
 * [XT §5] names the recurrent form S_(t-1) + current token -> S_t + output.
 * The backward oracle (kda_oracle_bwd_f64) is the reverse-mode derivative of
 * the same token steps; its derivation is written above the function.
 *
 * Parity pins: every function here is pinned by tests under tests/ that do
 * not re-type these formulas (worked example, GDN / delta-rule / linear
 * attention special cases, brute-force transition products, the gradient
 * identity, invariances; for the backward: central differences of the
 * forward, the frozen-state and linear-attention closed forms, Euler's
 * identity).  No function is "parity unpinned".
 *
 * Data layout (all row-major, last index fastest):
 *   q, k  [B, T, H, dk]    v [B, T, H, dv]     g [B, T, H, dk] (fp32)
 *   beta  [B, T, H] (fp32) states [N, H, dk, dv] (fp32 in, fp64 out)
 *   o     [B, T, H, dv] (fp64 out)
 * q, k, v are fp32 (in_dtype 0) or bf16 bit patterns (in_dtype 1); a bf16
 * value is widened exactly (its 16 bits become the top half of an fp32).
 * Varlen: B = 1 and sequence n covers tokens cu_seqlens[n] .. cu_seqlens[n+1]-1.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EPS 1e-6

/* Widen one stored input element to double.  bf16 -> fp32 is exact (the
 * 16 bits are the high half of the fp32 pattern); fp32 -> fp64 is exact. */
static double load_in(const void* base, int dtype, int64_t idx) {
    if (dtype == 0) return (double)((const float*)base)[idx];
    uint16_t h = ((const uint16_t*)base)[idx];
    uint32_t w = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

typedef struct {
    /* problem */
    int64_t batch, seqlen, num_seqs, heads, dk, dv;
    int in_dtype, qk_l2norm;
    double scale;
    int64_t ckpt_every;
    const void *q, *k, *v;
    const float *g, *beta, *init_state;
    const int32_t* cu_seqlens;
    double *o, *final_state, *ckpt;
    /* decode mode: steps > 0 means [steps, N, H, d] inputs, one token per step */
    int64_t steps;
    /* backward mode (bwd != 0): upstream gradients in, input gradients out */
    int bwd;
    const void* d_o;
    const float* dfinal;
    double *grad_q, *grad_k, *grad_v, *grad_g, *grad_beta, *grad_init;
    /* work split */
    int64_t next_chain; /* guarded by mu */
    pthread_mutex_t mu;
} job_t;

/* One token of the recurrence on state S (dk x dv, row-major).  qrow/krow/vrow
 * are element offsets of this token's q, k, v vectors; grow of g; bidx of beta;
 * orow is where o goes (fp64). */
static void token_step(const job_t* J, double* S, double* qh, double* kh,
                       double* u, int64_t qrow, int64_t vrow, int64_t grow,
                       int64_t bidx, int64_t orow) {
    const int64_t dk = J->dk, dv = J->dv;
    /* step 1: read q, k, optionally L2-normalise */
    double qq = 0.0, kk = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
        qh[c] = load_in(J->q, J->in_dtype, qrow + c);
        kh[c] = load_in(J->k, J->in_dtype, qrow + c);
        qq += qh[c] * qh[c];
        kk += kh[c] * kh[c];
    }
    if (J->qk_l2norm) {
        double rq = 1.0 / sqrt(qq + ORACLE_EPS), rk = 1.0 / sqrt(kk + ORACLE_EPS);
        for (int64_t c = 0; c < dk; ++c) { qh[c] *= rq; kh[c] *= rk; }
    }
    /* steps 2-3: per-channel decay of the state's rows */
    for (int64_t c = 0; c < dk; ++c) {
        double a = exp((double)J->g[grow + c]);
        double* row = S + c * dv;
        for (int64_t j = 0; j < dv; ++j) row[j] *= a;
    }
    /* step 4: u = beta * (v - S~^T k^) */
    const double b = (double)J->beta[bidx];
    for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < dk; ++c) acc += S[c * dv + j] * kh[c];
        u[j] = b * (load_in(J->v, J->in_dtype, vrow + j) - acc);
    }
    /* step 5: S = S~ + k^ u^T */
    for (int64_t c = 0; c < dk; ++c) {
        double* row = S + c * dv;
        for (int64_t j = 0; j < dv; ++j) row[j] += kh[c] * u[j];
    }
    /* step 6: o = scale * S^T q^ (post-update state) */
    for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < dk; ++c) acc += S[c * dv + j] * qh[c];
        J->o[orow + j] = J->scale * acc;
    }
}

/* Run one (sequence, head) chain of the prefill problem. */
static void run_fwd_chain(const job_t* J, int64_t n, int64_t h, double* S,
                          double* qh, double* kh, double* u) {
    const int64_t H = J->heads, dk = J->dk, dv = J->dv, sz = dk * dv;
    /* token range of this sequence in the [B, T] token grid */
    int64_t tok0, len;
    if (J->cu_seqlens) {
        tok0 = J->cu_seqlens[n];
        len = (int64_t)J->cu_seqlens[n + 1] - tok0;
    } else {
        tok0 = n * J->seqlen;
        len = J->seqlen;
    }
    const int64_t sidx = (n * H + h) * sz;
    for (int64_t i = 0; i < sz; ++i)
        S[i] = J->init_state ? (double)J->init_state[sidx + i] : 0.0;
    const int64_t nck = (J->ckpt_every > 0) ? J->seqlen / J->ckpt_every : 0;
    for (int64_t t = 0; t < len; ++t) {
        const int64_t tok = tok0 + t;
        token_step(J, S, qh, kh, u, (tok * H + h) * dk, (tok * H + h) * dv,
                   (tok * H + h) * dk, tok * H + h, (tok * H + h) * dv);
        if (J->ckpt && J->ckpt_every > 0 && (t + 1) % J->ckpt_every == 0) {
            const int64_t j = (t + 1) / J->ckpt_every - 1;
            double* dst = J->ckpt + (((n * nck) + j) * H + h) * sz;
            memcpy(dst, S, (size_t)sz * sizeof(double));
        }
    }
    if (J->final_state) memcpy(J->final_state + sidx, S, (size_t)sz * sizeof(double));
}

/* Run one (sequence, head) chain of the decode problem: steps tokens, each
 * from its own [N, H, d] slab. */
static void run_decode_chain(const job_t* J, int64_t n, int64_t h, double* S,
                             double* qh, double* kh, double* u) {
    const int64_t N = J->num_seqs, H = J->heads, dk = J->dk, dv = J->dv, sz = dk * dv;
    const int64_t sidx = (n * H + h) * sz;
    for (int64_t i = 0; i < sz; ++i)
        S[i] = J->init_state ? (double)J->init_state[sidx + i] : 0.0;
    for (int64_t s = 0; s < J->steps; ++s) {
        const int64_t row = (s * N + n) * H + h;
        token_step(J, S, qh, kh, u, row * dk, row * dv, row * dk, row, row * dv);
    }
    if (J->final_state) memcpy(J->final_state + sidx, S, (size_t)sz * sizeof(double));
}

/* ---------------------------------------------------------------------------
 * Backward (gradient) oracle.
 *
 * [XT §5] has training run the chunkwise form of the same recurrence and
 * gives no gradient algorithm.  The gradient itself has a plain definition:
 * the vector-Jacobian product of steps 1-6 above with the upstream gradients
 * do_t (of every output) and dS_T (of the final state).  It is formed here by
 * reverse-mode differentiation of the token recurrence, last token first.
 * With dS = dL/dS_t (everything after token t) on entry:
 *   a. o = scale S^T q^        dS += scale q^ do^T        dq^ = scale S do
 *   b. S = S~ + k^ u^T         dk^ = dS u                 du  = dS^T k^
 *   c. u = beta e,             dv = beta du   dbeta = du . e
 *      e = v - S~^T k^         dS~ = dS - k^ (beta du)^T  dk^ -= S~ (beta du)
 *   d. S~ = Diag(a) S_(t-1),   dg_c = sum_j dS~_cj S~_cj  (a = e^g: da/dg = a)
 *      a = exp(g)              dS_(t-1) = Diag(a) dS~
 *   e. x^ = x r, r = (|x|^2 + eps)^(-1/2)   dx = r dx^ - r^3 (x . dx^) x
 *      for q and k when qk_l2norm is set (dx = dx^ otherwise)
 * Step a uses the updated state S_t, as the forward's read-out does.  The
 * sweep needs S_(t-1) at every token: the forward pass keeps the state at
 * every BWD_BLOCK-th token of the chain, and each block's states are
 * recomputed from the kept one by the same token step, so they are the
 * identical numbers a full store would hold.
 */
#define BWD_BLOCK 64

/* One forward token (steps 1-5) on S in place; no output. */
static void advance_state(const job_t* J, double* S, double* qh, double* kh, double* u,
                          int64_t row_k, int64_t row_v, int64_t bidx) {
    const int64_t dk = J->dk, dv = J->dv;
    double kk = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
        kh[c] = load_in(J->k, J->in_dtype, row_k + c);
        kk += kh[c] * kh[c];
    }
    if (J->qk_l2norm) {
        const double rk = 1.0 / sqrt(kk + ORACLE_EPS);
        for (int64_t c = 0; c < dk; ++c) kh[c] *= rk;
    }
    for (int64_t c = 0; c < dk; ++c) {
        const double a = exp((double)J->g[row_k + c]);
        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= a;
    }
    const double b = (double)J->beta[bidx];
    for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < dk; ++c) acc += S[c * dv + j] * kh[c];
        u[j] = b * (load_in(J->v, J->in_dtype, row_v + j) - acc);
    }
    for (int64_t c = 0; c < dk; ++c)
        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += kh[c] * u[j];
    (void)qh;
}

/* Reverse step of one token.  Sp = S_(t-1), Sn = S_t; dS holds dL/dS_t on
 * entry and dL/dS_(t-1) on exit.  w is scratch of dk*dv + 4*dk + 3*dv. */
static void reverse_token(const job_t* J, const double* Sp, const double* Sn, double* dS,
                          double* w, int64_t row_k, int64_t row_v, int64_t bidx) {
    const int64_t dk = J->dk, dv = J->dv;
    double* St = w;               /* S~ = Diag(a) S_(t-1)   dk x dv */
    double* qx = St + dk * dv;    /* raw q, then q^          dk */
    double* kx = qx + dk;         /* raw k, then k^          dk */
    double* dqh = kx + dk;        /* dL/dq^                  dk */
    double* dkh = dqh + dk;       /* dL/dk^                  dk */
    double* e = dkh + dk;         /* v - S~^T k^             dv */
    double* du = e + dv;          /* dL/du                   dv */
    double* don = du + dv;        /* do_t                    dv */
    double qq = 0.0, kk = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
        qx[c] = load_in(J->q, J->in_dtype, row_k + c);
        kx[c] = load_in(J->k, J->in_dtype, row_k + c);
        qq += qx[c] * qx[c];
        kk += kx[c] * kx[c];
    }
    const double rq = J->qk_l2norm ? 1.0 / sqrt(qq + ORACLE_EPS) : 1.0;
    const double rk = J->qk_l2norm ? 1.0 / sqrt(kk + ORACLE_EPS) : 1.0;
    double qh_c, kh_c;
    for (int64_t c = 0; c < dk; ++c) {
        const double a = exp((double)J->g[row_k + c]);
        for (int64_t j = 0; j < dv; ++j) St[c * dv + j] = a * Sp[c * dv + j];
    }
    const double b = (double)J->beta[bidx];
    for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < dk; ++c) acc += St[c * dv + j] * (kx[c] * rk);
        e[j] = load_in(J->v, J->in_dtype, row_v + j) - acc;
        don[j] = load_in(J->d_o, J->in_dtype, row_v + j);
    }
    /* a. read-out */
    for (int64_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) acc += Sn[c * dv + j] * don[j];
        dqh[c] = J->scale * acc;
        qh_c = qx[c] * rq;
        for (int64_t j = 0; j < dv; ++j) dS[c * dv + j] += J->scale * qh_c * don[j];
    }
    /* b. rank-1 write (u = beta e) */
    for (int64_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) acc += dS[c * dv + j] * (b * e[j]);
        dkh[c] = acc;
    }
    for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < dk; ++c) acc += dS[c * dv + j] * (kx[c] * rk);
        du[j] = acc;
    }
    /* c. correction */
    double db = 0.0;
    for (int64_t j = 0; j < dv; ++j) {
        J->grad_v[row_v + j] = b * du[j];
        db += du[j] * e[j];
    }
    J->grad_beta[bidx] = db;
    for (int64_t c = 0; c < dk; ++c) {
        kh_c = kx[c] * rk;
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) {
            dS[c * dv + j] -= kh_c * (b * du[j]);
            acc += St[c * dv + j] * (b * du[j]);
        }
        dkh[c] -= acc;
    }
    /* d. decay */
    for (int64_t c = 0; c < dk; ++c) {
        const double a = exp((double)J->g[row_k + c]);
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) acc += dS[c * dv + j] * St[c * dv + j];
        J->grad_g[row_k + c] = acc;
        for (int64_t j = 0; j < dv; ++j) dS[c * dv + j] *= a;
    }
    /* e. L2 normalisation */
    double qd = 0.0, kd = 0.0;
    for (int64_t c = 0; c < dk; ++c) { qd += qx[c] * dqh[c]; kd += kx[c] * dkh[c]; }
    for (int64_t c = 0; c < dk; ++c) {
        if (J->qk_l2norm) {
            J->grad_q[row_k + c] = rq * dqh[c] - rq * rq * rq * qd * qx[c];
            J->grad_k[row_k + c] = rk * dkh[c] - rk * rk * rk * kd * kx[c];
        } else {
            J->grad_q[row_k + c] = dqh[c];
            J->grad_k[row_k + c] = dkh[c];
        }
    }
}

/* Gradients of one (sequence, head) chain.  Returns nonzero on allocation
 * failure. */
static int run_bwd_chain(const job_t* J, int64_t n, int64_t h) {
    const int64_t H = J->heads, dk = J->dk, dv = J->dv, sz = dk * dv;
    int64_t tok0, len;
    if (J->cu_seqlens) {
        tok0 = J->cu_seqlens[n];
        len = (int64_t)J->cu_seqlens[n + 1] - tok0;
    } else {
        tok0 = n * J->seqlen;
        len = J->seqlen;
    }
    const int64_t nblk = (len + BWD_BLOCK - 1) / BWD_BLOCK;
    double* kept = (double*)malloc((size_t)(nblk > 0 ? nblk : 1) * sz * sizeof(double));
    double* blk = (double*)malloc((size_t)(BWD_BLOCK + 1) * sz * sizeof(double));
    double* dS = (double*)malloc((size_t)sz * sizeof(double));
    double* w = (double*)malloc((size_t)(sz + 4 * dk + 3 * dv) * sizeof(double));
    double* vec = (double*)malloc((size_t)(2 * dk + dv) * sizeof(double));
    if (!kept || !blk || !dS || !w || !vec) {
        free(kept); free(blk); free(dS); free(w); free(vec);
        return 1;
    }
    double *qh = vec, *kh = vec + dk, *u = vec + 2 * dk;
    const int64_t sidx = (n * H + h) * sz;
    /* forward sweep: keep the state entering every block */
    double* S = blk;
    for (int64_t i = 0; i < sz; ++i) S[i] = J->init_state ? (double)J->init_state[sidx + i] : 0.0;
    for (int64_t t = 0; t < len; ++t) {
        if (t % BWD_BLOCK == 0) memcpy(kept + (t / BWD_BLOCK) * sz, S, (size_t)sz * sizeof(double));
        const int64_t tok = tok0 + t;
        advance_state(J, S, qh, kh, u, (tok * H + h) * dk, (tok * H + h) * dv, tok * H + h);
    }
    /* reverse sweep */
    for (int64_t i = 0; i < sz; ++i) dS[i] = J->dfinal ? (double)J->dfinal[sidx + i] : 0.0;
    for (int64_t b = nblk - 1; b >= 0; --b) {
        const int64_t t0 = b * BWD_BLOCK;
        const int64_t t1 = (t0 + BWD_BLOCK < len) ? t0 + BWD_BLOCK : len;
        memcpy(blk, kept + b * sz, (size_t)sz * sizeof(double));
        for (int64_t t = t0; t < t1; ++t) {
            double* nxt = blk + (t - t0 + 1) * sz;
            memcpy(nxt, blk + (t - t0) * sz, (size_t)sz * sizeof(double));
            const int64_t tok = tok0 + t;
            advance_state(J, nxt, qh, kh, u, (tok * H + h) * dk, (tok * H + h) * dv, tok * H + h);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const int64_t tok = tok0 + t;
            reverse_token(J, blk + (t - t0) * sz, blk + (t - t0 + 1) * sz, dS, w,
                          (tok * H + h) * dk, (tok * H + h) * dv, tok * H + h);
        }
    }
    if (J->grad_init) memcpy(J->grad_init + sidx, dS, (size_t)sz * sizeof(double));
    free(kept); free(blk); free(dS); free(w); free(vec);
    return 0;
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int64_t sz = J->dk * J->dv;
    double* S = (double*)malloc((size_t)sz * sizeof(double));
    double* qh = (double*)malloc((size_t)J->dk * sizeof(double));
    double* kh = (double*)malloc((size_t)J->dk * sizeof(double));
    double* u = (double*)malloc((size_t)J->dv * sizeof(double));
    if (!S || !qh || !kh || !u) { free(S); free(qh); free(kh); free(u); return (void*)1; }
    const int64_t total = J->num_seqs * J->heads;
    int failed = 0;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t c = J->next_chain++;
        pthread_mutex_unlock(&J->mu);
        if (c >= total) break;
        const int64_t n = c / J->heads, h = c % J->heads;
        if (J->bwd) {
            if (run_bwd_chain(J, n, h)) { failed = 1; break; }
        } else if (J->steps > 0) {
            run_decode_chain(J, n, h, S, qh, kh, u);
        } else {
            run_fwd_chain(J, n, h, S, qh, kh, u);
        }
    }
    free(S); free(qh); free(kh); free(u);
    return failed ? (void*)1 : NULL;
}

static int run_job(job_t* J, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t tid[256];
    pthread_mutex_init(&J->mu, NULL);
    J->next_chain = 0;
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, J) != 0) break;
        ++started;
    }
    if (started == 0) {
        void* r = worker(J);
        rc = (r != NULL);
    }
    for (int i = 0; i < started; ++i) {
        void* r = NULL;
        pthread_join(tid[i], &r);
        if (r != NULL) rc = 1;
    }
    pthread_mutex_destroy(&J->mu);
    return rc;
}

/* Prefill oracle.  Returns 0 on success, nonzero on bad arguments or
 * allocation failure.  final_state and ckpt may be NULL.  Checkpoint j
 * (dense only) is the state after (j+1)*ckpt_every tokens of a sequence,
 * stored at ckpt[b, j, h, :, :] with T/ckpt_every slots per sequence. */
int kda_oracle_fwd_f64(int64_t batch, int64_t seqlen, int64_t num_seqs, int64_t heads,
                       int64_t dk, int64_t dv, int in_dtype, const void* q, const void* k,
                       const void* v, const float* g, const float* beta,
                       const float* init_state, const int32_t* cu_seqlens, int qk_l2norm,
                       double scale, int64_t ckpt_every, double* o, double* final_state,
                       double* ckpt, int nthreads) {
    if (batch < 1 || seqlen < 0 || heads < 1 || dk < 1 || dv < 1) return 2;
    if (in_dtype != 0 && in_dtype != 1) return 2;
    if (!q || !k || !v || !g || !beta || !o) return 2;
    if (cu_seqlens) {
        if (batch != 1 || num_seqs < 1) return 2;
        if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != seqlen) return 2;
        for (int64_t n = 0; n < num_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return 2;
        if (ckpt_every > 0) return 2;
    } else if (num_seqs != batch) {
        return 2;
    }
    if (ckpt_every < 0) return 2;
    job_t J;
    memset(&J, 0, sizeof J);
    J.batch = batch; J.seqlen = seqlen; J.num_seqs = num_seqs; J.heads = heads;
    J.dk = dk; J.dv = dv; J.in_dtype = in_dtype; J.qk_l2norm = qk_l2norm;
    J.scale = scale; J.ckpt_every = ckpt_every;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.init_state = init_state;
    J.cu_seqlens = cu_seqlens; J.o = o; J.final_state = final_state; J.ckpt = ckpt;
    J.steps = 0;
    return run_job(&J, nthreads) ? 3 : 0;
}

/* Decode oracle: `steps` single-token steps for N sequences x H heads.
 * Inputs are [steps, N, H, d] (q,k,g: d = dk; v: d = dv), beta [steps, N, H];
 * state_in [N, H, dk, dv] fp32 (NULL = zeros); o [steps, N, H, dv] fp64;
 * state_out [N, H, dk, dv] fp64.  Chains are independent, so each one runs
 * its steps back to back; the result equals the step-major order exactly. */
int kda_oracle_decode_f64(int64_t steps, int64_t num_seqs, int64_t heads, int64_t dk,
                          int64_t dv, int in_dtype, const void* q, const void* k,
                          const void* v, const float* g, const float* beta,
                          const float* state_in, int qk_l2norm, double scale, double* o,
                          double* state_out, int nthreads) {
    if (steps < 1 || num_seqs < 1 || heads < 1 || dk < 1 || dv < 1) return 2;
    if (in_dtype != 0 && in_dtype != 1) return 2;
    if (!q || !k || !v || !g || !beta || !o) return 2;
    job_t J;
    memset(&J, 0, sizeof J);
    J.batch = num_seqs; J.seqlen = 0; J.num_seqs = num_seqs; J.heads = heads;
    J.dk = dk; J.dv = dv; J.in_dtype = in_dtype; J.qk_l2norm = qk_l2norm;
    J.scale = scale; J.ckpt_every = 0;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.init_state = state_in;
    J.o = o; J.final_state = state_out; J.steps = steps;
    return run_job(&J, nthreads) ? 3 : 0;
}

/* Backward oracle: input gradients of the prefill operator for upstream
 * gradients d_o [B, T, H, dv] (in_dtype, like q/k/v) and dfinal [N, H, dk, dv]
 * (fp32; NULL = zero).  Outputs (fp64, all required except dinit): dq, dk
 * [B, T, H, dk], dv [B, T, H, dv], dg [B, T, H, dk], dbeta [B, T, H], dinit
 * [N, H, dk, dv] or NULL.  Other arguments as kda_oracle_fwd_f64.  Returns 0
 * on success, 2 on bad arguments, 3 on allocation failure. */
int kda_oracle_bwd_f64(int64_t batch, int64_t seqlen, int64_t num_seqs, int64_t heads,
                       int64_t dk, int64_t dv, int in_dtype, const void* q, const void* k,
                       const void* v, const float* g, const float* beta,
                       const float* init_state, const int32_t* cu_seqlens, int qk_l2norm,
                       double scale, const void* d_o, const float* dfinal, double* dq,
                       double* dkk, double* dvv, double* dg, double* dbeta, double* dinit,
                       int nthreads) {
    if (batch < 1 || seqlen < 0 || heads < 1 || dk < 1 || dv < 1) return 2;
    if (in_dtype != 0 && in_dtype != 1) return 2;
    if (!q || !k || !v || !g || !beta || !d_o || !dq || !dkk || !dvv || !dg || !dbeta) return 2;
    if (cu_seqlens) {
        if (batch != 1 || num_seqs < 1) return 2;
        if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != seqlen) return 2;
        for (int64_t n = 0; n < num_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return 2;
    } else if (num_seqs != batch) {
        return 2;
    }
    job_t J;
    memset(&J, 0, sizeof J);
    J.batch = batch; J.seqlen = seqlen; J.num_seqs = num_seqs; J.heads = heads;
    J.dk = dk; J.dv = dv; J.in_dtype = in_dtype; J.qk_l2norm = qk_l2norm;
    J.scale = scale;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.init_state = init_state;
    J.cu_seqlens = cu_seqlens;
    J.bwd = 1; J.d_o = d_o; J.dfinal = dfinal;
    J.grad_q = dq; J.grad_k = dkk; J.grad_v = dvv; J.grad_g = dg; J.grad_beta = dbeta;
    J.grad_init = dinit;
    return run_job(&J, nthreads) ? 3 : 0;
}

/* Output epilogue [XT §6.3 "Sigmoid output gate 控制读出"; XT §6 layer
 * diagram: the operator's output passes an RMSNorm, then a sigmoid output
 * gate, before the output projection].  The norm is head-wise: each (token,
 * head) row of d_v outputs is divided by its root mean square.  The gate is
 * a sigmoid of a value computed from the layer input, one per output
 * element.  The pages give neither the norm's eps nor its weight; this
 * project's reading: eps is a parameter (1e-6 in every workload) added to the
 * mean square under the root, and w is one weight per d_v channel, shared by
 * all heads (NULL means 1).  z is the gate's pre-activation.
 *   y_j = o_j / sqrt(mean_i o_i^2 + eps) * w_j * sigmoid(z_j)
 * o and z are fp32 (in_dtype 0) or bf16 bit patterns (in_dtype 1), rows x dv. */
int kda_oracle_gate_norm_f64(int64_t rows, int64_t dv, int in_dtype, const void* o,
                             const void* z, const float* w, double eps, double* y) {
    if (rows < 0 || dv < 1 || (in_dtype != 0 && in_dtype != 1)) return 2;
    if (rows > 0 && (!o || !z || !y)) return 2;
    for (int64_t r = 0; r < rows; ++r) {
        double ms = 0.0;
        for (int64_t j = 0; j < dv; ++j) {
            const double x = load_in(o, in_dtype, r * dv + j);
            ms += x * x;
        }
        ms /= (double)dv;
        const double inv_rms = 1.0 / sqrt(ms + eps);
        for (int64_t j = 0; j < dv; ++j) {
            const double x = load_in(o, in_dtype, r * dv + j);
            const double gate = 1.0 / (1.0 + exp(-load_in(z, in_dtype, r * dv + j)));
            const double wj = w ? (double)w[j] : 1.0;
            y[r * dv + j] = x * inv_rms * wj * gate;
        }
    }
    return 0;
}

/* ShortConv + Swish prologue [XT §6 layer diagram: the q, k and v
 * projections pass a ShortConv and a Swish before the operator (q and k then
 * the L2 norm); XT §6.1; XD, the preprocessing list: a small-window causal
 * convolution that mixes each position with the few tokens just before it].
 * The pages give no window; this project's reading: W taps (4 in every
 * workload), one filter per channel (depthwise), an optional bias, and
 * Swish(x) = x * sigmoid(x).  Per sequence n, channel c, token t:
 *   y_t[c] = swish(bias[c] + sum_{i<W} w[c][i] * x~[t - (W-1) + i][c])
 * where x~ is the sequence's own input, preceded by the carried state
 * state[n][c][0..W-2] (the W-1 inputs before the sequence, oldest first) or by
 * zeros when no state is given.  state_out[n][c][:] = the last W-1 entries of
 * x~ (carried state followed by the sequence's inputs).
 * x, y: [B, T, C] row-major (x fp32 or bf16; y fp64 out); varlen: B = 1 and
 * sequence n covers tokens cu[n] .. cu[n+1]-1.  w: [C][W] fp32; bias [C] fp32
 * or NULL; state [N][C][W-1] fp32 or NULL; state_out [N][C][W-1] fp64 or NULL. */
int kda_oracle_short_conv_f64(int64_t batch, int64_t seqlen, int64_t num_seqs, int64_t C,
                              int64_t W, int in_dtype, const void* x, const float* w,
                              const float* bias, const float* state, const int32_t* cu_seqlens,
                              double* y, double* state_out) {
    if (batch < 1 || seqlen < 0 || num_seqs < 0 || C < 1 || W < 1) return 2;
    if (in_dtype != 0 && in_dtype != 1) return 2;
    if (!w || (seqlen > 0 && (!x || !y))) return 2;
    const int64_t nseq = cu_seqlens ? num_seqs : batch;
    const int64_t H = W - 1;  /* carried inputs per channel */
    double* ext = (double*)malloc((size_t)(H + (seqlen > 0 ? seqlen : 1)) * sizeof(double));
    if (!ext) return 3;
    for (int64_t n = 0; n < nseq; ++n) {
        const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t len = cu_seqlens ? cu_seqlens[n + 1] - cu_seqlens[n] : seqlen;
        const int64_t rowbase = cu_seqlens ? 0 : n * seqlen;  /* token rows before sequence n */
        for (int64_t c = 0; c < C; ++c) {
            /* the extended input: carried state (or zeros), then the sequence */
            for (int64_t i = 0; i < H; ++i) ext[i] = state ? (double)state[(n * C + c) * H + i] : 0.0;
            for (int64_t t = 0; t < len; ++t)
                ext[H + t] = load_in(x, in_dtype, (rowbase + t0 + t) * C + c);
            for (int64_t t = 0; t < len; ++t) {
                double acc = bias ? (double)bias[c] : 0.0;
                for (int64_t i = 0; i < W; ++i) acc += (double)w[c * W + i] * ext[t + i];
                y[(rowbase + t0 + t) * C + c] = acc / (1.0 + exp(-acc));
            }
            if (state_out)
                for (int64_t i = 0; i < H; ++i) state_out[(n * C + c) * H + i] = ext[len + i];
        }
    }
    free(ext);
    return 0;
}

int kda_oracle_abi_version(void) { return 2; }
