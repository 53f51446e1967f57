/*
 * fp64 CPU oracle for exact attention and paged-cache decode.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain definition the
 * GPU kernels are checked against.  It shares no code with the GPU library
 * and is only called from the test suite, the smoke check and the
 * benchmark's CPU-baseline leg.
 *
 * What it computes (FlashAttention reaches this same result exactly, up to
 * rounding order -- NanoInfer page, "Flash Attention" section; inference
 * kernel cookbook page, recipe 01 notes):
 *
 *   s_ij = scale * sum_t q[i,t] k[j,t]                (Kernel-Inference-Engine
 *                                                      page, tile dataflow chart)
 *   valid(j) = j < n_b  and  (not causal or j <= i + Nk - Nq)
 *   m = max_valid s_ij,  e_j = exp(s_ij - m),  l = sum_valid e_j
 *   O[i,:] = sum_valid e_j v[j,:] / l,  LSE_i = m + ln l
 *
 * i.e. the safe three-pass softmax of the NanoInfer page ("Online Softmax"
 * section: find the max, exponentiate the shifted values, normalise) applied
 * to the masked score row, then multiplied by V.  Masks: causal and key
 * padding combined before the softmax (gpu-inference page, section 02).
 * Rows with no valid key give O = 0 and LSE = -inf.
 *
 * Decode (query length 1 over a sequence's cached tokens) is the same row
 * computation with every cached token valid; it reads the LOGICAL per
 * sequence K/V, never a paged pool.
 *
 * Grouped-query attention (the MQA / GQA variants of the llm-kernel-lib
 * page's "Ablation Study"): K and V have Hkv heads, H a multiple of Hkv, and
 * query head h attends with key/value head h / (H / Hkv) -- consecutive
 * query heads share one K/V head.  Hkv = H is ordinary multi-head attention.
 *
 * The backward (gradients of this same attention for a given dO) is the
 * chain rule written out term by term; see oracle_bwd.
 *
 * Inputs are raw f16 / bf16 bit patterns; they are widened exactly to
 * double here.  All arithmetic is IEEE double, libm exp/log, no fast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { OR_F16 = 0, OR_BF16 = 1 };

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double half_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double x;
    if (e == 0)
        x = ldexp((double)f, -24);                /* zero / subnormal */
    else if (e == 31)
        x = f ? NAN : INFINITY;
    else
        x = ldexp((double)(f | 0x400), e - 25);   /* 1.f * 2^(e-15) */
    return sign ? -x : x;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bfloat_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double widen(uint16_t x, int dtype)
{
    return dtype == OR_F16 ? half_to_double(x) : bfloat_to_double(x);
}

void oracle_widen(const uint16_t *src, int dtype, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = widen(src[i], dtype);
}

/*
 * One attention row: q (d doubles), keys/values (nk x d doubles, row-major),
 * nvalid leading keys valid.  Writes o[d] and *lse.  Returns 0, or 1 when the
 * softmax self-check (probabilities sum to one) fails.
 */
static int attention_row(const double *q, const double *kk, const double *vv, int nvalid,
                         int d, double scale, double *s, double *o, double *lse)
{
    for (int t = 0; t < d; ++t)
        o[t] = 0.0;
    if (nvalid <= 0) {
        *lse = -INFINITY;
        return 0;
    }
    /* scores */
    for (int j = 0; j < nvalid; ++j) {
        double dot = 0.0;
        for (int t = 0; t < d; ++t)
            dot += q[t] * kk[(int64_t)j * d + t];
        s[j] = scale * dot;
    }
    /* pass 1: max */
    double m = s[0];
    for (int j = 1; j < nvalid; ++j)
        if (s[j] > m)
            m = s[j];
    /* pass 2: exponentials and their sum */
    double l = 0.0;
    for (int j = 0; j < nvalid; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* pass 3: normalised probabilities times V */
    double psum = 0.0;
    for (int j = 0; j < nvalid; ++j) {
        double p = s[j] / l;
        psum += p;
        const double *vr = vv + (int64_t)j * d;
        for (int t = 0; t < d; ++t)
            o[t] += p * vr[t];
    }
    *lse = m + log(l);
    return fabs(psum - 1.0) > 1e-12 ? 1 : 0;
}

/* ------------------------------------------------------------- forward --- */

typedef struct {
    const uint16_t *q, *k, *v;
    int dtype, B, H, Hkv, Nq, Nk, d, causal;
    double scale;
    const int32_t *kv_lens;
    const int64_t *rows;   /* sorted flat row ids (b*H+h)*Nq+i, or NULL = all */
    int64_t nrows;
    double *o, *lse;
    int nthreads, tid;
    int bad;
} fwd_job;

static int64_t lower_bound64(const int64_t *a, int64_t n, int64_t key)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (a[mid] < key)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

static void *fwd_worker(void *arg)
{
    fwd_job *J = (fwd_job *)arg;
    const int d = J->d, Nq = J->Nq, Nk = J->Nk;
    double *kk = (double *)malloc(sizeof(double) * (size_t)Nk * d);
    double *vv = (double *)malloc(sizeof(double) * (size_t)Nk * d);
    double *qq = (double *)malloc(sizeof(double) * (size_t)d);
    double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
    if (!kk || !vv || !qq || !s) {
        J->bad = -1;
        goto done;
    }
    for (int64_t bh = J->tid; bh < (int64_t)J->B * J->H; bh += J->nthreads) {
        int b = (int)(bh / J->H), h = (int)(bh % J->H);
        int64_t kvh = (int64_t)b * J->Hkv + h / (J->H / J->Hkv);   /* K/V head of query head h */
        int64_t r0, r1;   /* positions in the output for this (b,h) */
        if (J->rows) {
            r0 = lower_bound64(J->rows, J->nrows, bh * Nq);
            r1 = lower_bound64(J->rows, J->nrows, (bh + 1) * Nq);
        } else {
            r0 = bh * Nq;
            r1 = (bh + 1) * Nq;
        }
        if (r0 == r1)
            continue;
        oracle_widen(J->k + kvh * Nk * d, J->dtype, (int64_t)Nk * d, kk);
        oracle_widen(J->v + kvh * Nk * d, J->dtype, (int64_t)Nk * d, vv);
        int nb = J->kv_lens ? J->kv_lens[b] : Nk;
        if (nb > Nk)
            nb = Nk;
        if (nb < 0)
            nb = 0;
        for (int64_t r = r0; r < r1; ++r) {
            int64_t flat = J->rows ? J->rows[r] : r;
            int i = (int)(flat - bh * Nq);
            int nvalid = nb;
            if (J->causal) {
                int64_t lim = (int64_t)i + (Nk - Nq) + 1;   /* keys j < lim */
                if (lim < nvalid)
                    nvalid = lim < 0 ? 0 : (int)lim;
            }
            oracle_widen(J->q + flat * d, J->dtype, d, qq);
            J->bad += attention_row(qq, kk, vv, nvalid, d, J->scale, s, J->o + r * d,
                                    J->lse + r);
        }
    }
done:
    free(kk);
    free(vv);
    free(qq);
    free(s);
    return NULL;
}

static int thread_count(int requested)
{
    if (requested > 0)
        return requested;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * Exact attention forward.  q [B,H,Nq,d], k/v [B,Hkv,Nk,d] (f16/bf16 bits),
 * H a multiple of Hkv.
 * rows: NULL for every row, else nrows sorted flat ids (b*H+h)*Nq+i; the
 * outputs o [nrows or B*H*Nq, d] and lse [nrows or B*H*Nq] follow that order.
 * Returns the number of rows failing the softmax self-check (0 expected),
 * or -1 on allocation failure.
 */
int oracle_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype, int B,
               int H, int Hkv, int Nq, int Nk, int d, double scale, int causal,
               const int32_t *kv_lens, const int64_t *rows, int64_t nrows, double *o,
               double *lse, int nthreads)
{
    if (Hkv < 1 || H % Hkv != 0)
        return -2;
    int nt = thread_count(nthreads);
    if ((int64_t)nt > (int64_t)B * H)
        nt = B * H > 0 ? B * H : 1;
    fwd_job *jobs = (fwd_job *)calloc((size_t)nt, sizeof(fwd_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int t = 0; t < nt; ++t) {
        fwd_job J = {q, k, v, dtype, B, H, Hkv, Nq, Nk, d, causal, scale, kv_lens,
                     rows, nrows, o, lse, nt, t, 0};
        jobs[t] = J;
        pthread_create(&th[t], NULL, fwd_worker, &jobs[t]);
    }
    int bad = 0;
    for (int t = 0; t < nt; ++t) {
        pthread_join(th[t], NULL);
        if (jobs[t].bad < 0)
            bad = -1;
        else if (bad >= 0)
            bad += jobs[t].bad;
    }
    free(jobs);
    free(th);
    return bad;
}

/* ------------------------------------------------------------ backward --- */

/*
 * Gradients of the attention above for a given output gradient dO (the
 * gpu-inference page, section 02: the backward recomputes the probabilities
 * and splits into a row term D, the K/V gradients and the Q gradient).  With
 * P_ij the softmax probabilities of row i (zero for masked keys):
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = dO_i . O_i          (equal to sum_j P_ij dP_ij)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * dK and dV of a K/V head sum over the query heads that read it.  This is the
 * chain rule through s_ij = scale q_i.k_j, the softmax and O = P V, written
 * out term by term.
 */
typedef struct {
    const uint16_t *q, *k, *v, *dout;
    int dtype, B, H, Hkv, Nq, Nk, d, causal;
    double scale;
    const int32_t *kv_lens;
    const int64_t *groups;   /* (b*Hkv + kvh) ids to compute, or NULL = all */
    int64_t ngroups;
    double *dq, *dk, *dv, *delta;
    int nthreads, tid;
    int bad;
} bwd_job;

static void *bwd_worker(void *arg)
{
    bwd_job *J = (bwd_job *)arg;
    const int d = J->d, Nq = J->Nq, Nk = J->Nk;
    const int grp = J->H / J->Hkv;
    double *kk = (double *)malloc(sizeof(double) * (size_t)Nk * d + 1);
    double *vv = (double *)malloc(sizeof(double) * (size_t)Nk * d + 1);
    double *qq = (double *)malloc(sizeof(double) * (size_t)d);
    double *gg = (double *)malloc(sizeof(double) * (size_t)d);   /* dO row */
    double *oo = (double *)malloc(sizeof(double) * (size_t)d);
    double *p = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
    if (!kk || !vv || !qq || !gg || !oo || !p) {
        J->bad = -1;
        goto done;
    }
    const int64_t total = J->groups ? J->ngroups : (int64_t)J->B * J->Hkv;
    for (int64_t gi = J->tid; gi < total; gi += J->nthreads) {
        const int64_t g = J->groups ? J->groups[gi] : gi;
        const int b = (int)(g / J->Hkv);
        const int64_t kvbase = g * Nk * d;
        oracle_widen(J->k + kvbase, J->dtype, (int64_t)Nk * d, kk);
        oracle_widen(J->v + kvbase, J->dtype, (int64_t)Nk * d, vv);
        double *dk = J->dk + kvbase, *dv = J->dv + kvbase;
        for (int64_t x = 0; x < (int64_t)Nk * d; ++x) {
            dk[x] = 0.0;
            dv[x] = 0.0;
        }
        int nb = J->kv_lens ? J->kv_lens[b] : Nk;
        if (nb > Nk)
            nb = Nk;
        if (nb < 0)
            nb = 0;
        for (int h = (int)(g % J->Hkv) * grp; h < (int)(g % J->Hkv) * grp + grp; ++h) {
            const int64_t bh = (int64_t)b * J->H + h;
            for (int i = 0; i < Nq; ++i) {
                const int64_t row = bh * Nq + i;
                double *dq = J->dq + row * d;
                int nvalid = nb;
                if (J->causal) {
                    int64_t lim = (int64_t)i + (Nk - Nq) + 1;
                    if (lim < nvalid)
                        nvalid = lim < 0 ? 0 : (int)lim;
                }
                for (int t = 0; t < d; ++t)
                    dq[t] = 0.0;
                J->delta[row] = 0.0;
                if (nvalid <= 0)
                    continue;
                oracle_widen(J->q + row * d, J->dtype, d, qq);
                oracle_widen(J->dout + row * d, J->dtype, d, gg);
                /* probabilities (safe softmax of the masked score row) */
                double m = -INFINITY;
                for (int j = 0; j < nvalid; ++j) {
                    double dot = 0.0;
                    for (int t = 0; t < d; ++t)
                        dot += qq[t] * kk[(int64_t)j * d + t];
                    p[j] = J->scale * dot;
                    if (p[j] > m)
                        m = p[j];
                }
                double l = 0.0;
                for (int j = 0; j < nvalid; ++j) {
                    p[j] = exp(p[j] - m);
                    l += p[j];
                }
                for (int t = 0; t < d; ++t)
                    oo[t] = 0.0;
                for (int j = 0; j < nvalid; ++j) {
                    p[j] /= l;
                    for (int t = 0; t < d; ++t)
                        oo[t] += p[j] * vv[(int64_t)j * d + t];
                }
                /* D_i = dO_i . O_i */
                double Di = 0.0;
                for (int t = 0; t < d; ++t)
                    Di += gg[t] * oo[t];
                J->delta[row] = Di;
                for (int j = 0; j < nvalid; ++j) {
                    const double *vj = vv + (int64_t)j * d;
                    const double *kj = kk + (int64_t)j * d;
                    double dp = 0.0;
                    for (int t = 0; t < d; ++t)
                        dp += gg[t] * vj[t];
                    const double ds = p[j] * (dp - Di);
                    double *dkj = dk + (int64_t)j * d, *dvj = dv + (int64_t)j * d;
                    for (int t = 0; t < d; ++t) {
                        dq[t] += J->scale * ds * kj[t];
                        dkj[t] += J->scale * ds * qq[t];
                        dvj[t] += p[j] * gg[t];
                    }
                }
            }
        }
    }
done:
    free(kk);
    free(vv);
    free(qq);
    free(gg);
    free(oo);
    free(p);
    return NULL;
}

/*
 * Attention backward.  q, dout [B,H,Nq,d]; k, v [B,Hkv,Nk,d] (f16/bf16 bits).
 * Writes dq [B,H,Nq,d], dk, dv [B,Hkv,Nk,d] and delta (D) [B,H,Nq] in double.
 * groups: NULL for everything, else ngroups ids b*Hkv + kvh: only those K/V
 * heads' dk/dv and the dq/delta rows of their query heads are written.
 * Returns 0, -1 on allocation failure, -2 on bad head counts.
 */
int oracle_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
               int dtype, int B, int H, int Hkv, int Nq, int Nk, int d, double scale,
               int causal, const int32_t *kv_lens, const int64_t *groups, int64_t ngroups,
               double *dq, double *dk, double *dv, double *delta, int nthreads)
{
    if (Hkv < 1 || H % Hkv != 0)
        return -2;
    const int64_t total = groups ? ngroups : (int64_t)B * Hkv;
    int nt = thread_count(nthreads);
    if ((int64_t)nt > total)
        nt = total > 0 ? (int)total : 1;
    bwd_job *jobs = (bwd_job *)calloc((size_t)nt, sizeof(bwd_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int t = 0; t < nt; ++t) {
        bwd_job J = {q, k, v, dout, dtype, B, H, Hkv, Nq, Nk, d, causal, scale, kv_lens,
                     groups, ngroups, dq, dk, dv, delta, nt, t, 0};
        jobs[t] = J;
        pthread_create(&th[t], NULL, bwd_worker, &jobs[t]);
    }
    int bad = 0;
    for (int t = 0; t < nt; ++t) {
        pthread_join(th[t], NULL);
        if (jobs[t].bad < 0)
            bad = -1;
    }
    free(jobs);
    free(th);
    return bad;
}

/* -------------------------------------------------------------- decode --- */

typedef struct {
    const uint16_t *q, *k, *v;
    const int64_t *seq_off;
    int dtype, S, H, Hkv, d;
    double scale;
    double *o, *lse;
    int nthreads, tid, bad;
} dec_job;

static void *dec_worker(void *arg)
{
    dec_job *J = (dec_job *)arg;
    const int d = J->d, H = J->H;
    int64_t maxlen = 0;
    for (int s = 0; s < J->S; ++s)
        if (J->seq_off[s + 1] - J->seq_off[s] > maxlen)
            maxlen = J->seq_off[s + 1] - J->seq_off[s];
    size_t cap = (size_t)(maxlen > 0 ? maxlen : 1);
    double *kk = (double *)malloc(sizeof(double) * cap * d);
    double *vv = (double *)malloc(sizeof(double) * cap * d);
    double *qq = (double *)malloc(sizeof(double) * (size_t)d);
    double *s = (double *)malloc(sizeof(double) * cap);
    if (!kk || !vv || !qq || !s) {
        J->bad = -1;
        goto done;
    }
    for (int64_t sh = J->tid; sh < (int64_t)J->S * H; sh += J->nthreads) {
        int sq = (int)(sh / H), h = (int)(sh % H);
        int kvh = h / (H / J->Hkv);   /* K/V head of query head h */
        int64_t a = J->seq_off[sq];
        int n = (int)(J->seq_off[sq + 1] - a);
        /* token t of sequence sq, K/V head kvh: row (a+t)*Hkv + kvh of the [T,Hkv,d] arrays */
        for (int t = 0; t < n; ++t) {
            oracle_widen(J->k + ((a + t) * J->Hkv + kvh) * d, J->dtype, d, kk + (int64_t)t * d);
            oracle_widen(J->v + ((a + t) * J->Hkv + kvh) * d, J->dtype, d, vv + (int64_t)t * d);
        }
        oracle_widen(J->q + sh * d, J->dtype, d, qq);
        J->bad += attention_row(qq, kk, vv, n, d, J->scale, s, J->o + sh * d, J->lse + sh);
    }
done:
    free(kk);
    free(vv);
    free(qq);
    free(s);
    return NULL;
}

/*
 * Decode attention: q [S,H,d]; k/v [T,Hkv,d] with sequence s owning tokens
 * seq_off[s] .. seq_off[s+1]-1 (all of them attended).  o [S,H,d], lse [S,H].
 */
int oracle_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const int64_t *seq_off, int dtype, int S, int H, int Hkv, int d, double scale,
                  double *o, double *lse, int nthreads)
{
    if (Hkv < 1 || H % Hkv != 0)
        return -2;
    int nt = thread_count(nthreads);
    if ((int64_t)nt > (int64_t)S * H)
        nt = S * H > 0 ? S * H : 1;
    dec_job *jobs = (dec_job *)calloc((size_t)nt, sizeof(dec_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int t = 0; t < nt; ++t) {
        dec_job J = {q, k, v, seq_off, dtype, S, H, Hkv, d, scale, o, lse, nt, t, 0};
        jobs[t] = J;
        pthread_create(&th[t], NULL, dec_worker, &jobs[t]);
    }
    int bad = 0;
    for (int t = 0; t < nt; ++t) {
        pthread_join(th[t], NULL);
        if (jobs[t].bad < 0)
            bad = -1;
        else if (bad >= 0)
            bad += jobs[t].bad;
    }
    free(jobs);
    free(th);
    return bad;
}
