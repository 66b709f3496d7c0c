/*
 * kda_oracle.c -- fp64 CPU oracle of the Kimi Delta Attention (KDA) mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: only the tests, the smoke check and the bench's CPU-baseline leg use it.  It
 * shares no code, header, table or constant generator with the HIP library.
 *
 * What it follows (page "colibri/c/kimi_k3.c", file header comment "KDA per-head
 * recurrence"; the same page's Kda weight struct, the model's KDA state and conv window
 * layout, and the rmsnorm_ helper):
 *   q,k,v = SiLU(ShortConv4(x))           conv taps stored oldest first, no bias
 *   q,k L2-normalised, eps added to the sum of squares inside the sqrt; q *= 128^-0.5
 *   gk    = gmin * sigmoid(exp(A_log[h]) * (z + dt_bias)),   gmin = -5,  alpha = exp(gk)
 *   beta  = sigmoid(b)
 *   S     = (I - beta k k^T) Diag(alpha) S + beta k v^T       S[k][v], key index = row
 *   o     = S^T q                                             read from the updated S
 *   out   = sigmoid(g) * RMSNorm_head(o)                      RMSNorm weight shared by heads
 *
 * Everything is plain fp64, token by token, one (sequence, head) at a time, in the
 * order the header comment states the steps.  The update is applied literally as three
 * passes over S (decay, delta-rule correction, write), so that it does not share the
 * single-pass shape of the GPU decode kernel.
 *
 * Pins (tests/test_oracle_*.py): brute-force products of explicit per-token transition
 * matrices, the beta=0/alpha=1 and alpha=1/beta=1 invariants, the Frobenius-norm bound,
 * closed forms (pure decay, orthonormal-key retrieval, one step from a zero state),
 * numpy.convolve for the conv, scipy's expit for sigmoid/SiLU, a constant-vector
 * RMSNorm, and an independent fp64 chunked (WY/UT) derivation.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#include "kda_oracle.h"

/* ---- scalar activations (page 3: sigmoidf_ / siluf_ helpers, here in fp64) ---- */

double kda_oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

double kda_oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/* ---- ShortConv4, one channel, one token ----
 * win[0..K-2] holds the K-1 previous pre-conv inputs, oldest first (page 3: conv
 * windows "oldest first"; taps "[proj*4] depthwise taps, oldest first").
 * y = sum_{j<K-1} w[j]*win[j] + w[K-1]*x ; afterwards the window is shifted by one and
 * x becomes its newest entry. */
double kda_oracle_conv_step(int K, const double *w, double *win, double x)
{
    double y = 0.0;
    for (int j = 0; j < K - 1; j++)
        y += w[j] * win[j];
    y += w[K - 1] * x;
    for (int j = 0; j < K - 2; j++)
        win[j] = win[j + 1];
    if (K > 1)
        win[K - 2] = x;
    return y;
}

/* ---- RMSNorm of one head's readout, then the sigmoid output gate ----
 * page 3 rmsnorm_: r = 1/sqrt(mean(o^2) + eps), y = o*r*w; then y *= sigmoid(g). */
void kda_oracle_rmsnorm_gate(int D, const double *o, const double *g, const double *w,
                             double eps, double *out)
{
    double ms = 0.0;
    for (int i = 0; i < D; i++)
        ms += o[i] * o[i];
    ms /= (double)D;
    double r = 1.0 / sqrt(ms + eps);
    for (int i = 0; i < D; i++)
        out[i] = kda_oracle_sigmoid(g[i]) * (o[i] * r * w[i]);
}

/* ---- the recurrence core: one token, one head, explicit gates ----
 * S[dk][dv] is updated in place; o[dv] = S^T q with the updated S.
 *   1. S <- Diag(alpha) S                       (row i scaled by alpha[i])
 *   2. S <- S - beta k (k^T S)                  ((I - beta k k^T) applied on the left)
 *   3. S <- S + beta k v^T
 *   4. o <- S^T q                                                                 */
void kda_oracle_core_step(int dk, int dv, double *S, const double *q, const double *k,
                          const double *v, const double *alpha, double beta, double *o)
{
    double *kts = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++)
            S[(size_t)i * dv + j] *= alpha[i];
    for (int j = 0; j < dv; j++) {
        double acc = 0.0;
        for (int i = 0; i < dk; i++)
            acc += k[i] * S[(size_t)i * dv + j];
        kts[j] = acc;
    }
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++)
            S[(size_t)i * dv + j] -= beta * k[i] * kts[j];
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++)
            S[(size_t)i * dv + j] += beta * k[i] * v[j];
    for (int j = 0; j < dv; j++) {
        double acc = 0.0;
        for (int i = 0; i < dk; i++)
            acc += S[(size_t)i * dv + j] * q[i];
        o[j] = acc;
    }
    free(kts);
}

/* ---- L2 normalisation, eps inside the sqrt, then a scale ---- */
static void l2norm_scale(int D, double *x, double eps, double scale)
{
    double ss = 0.0;
    for (int i = 0; i < D; i++)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < D; i++)
        x[i] = x[i] * inv * scale;
}

/* ---- the whole mixer for one (sequence, head), token by token ---- */
int kda_oracle_head_forward(const kda_oracle_params *p, const kda_oracle_job *jb)
{
    const int D = p->head_dim, K = p->conv_size;
    if (D < 1 || K < 1 || jb->T < 0)
        return -1;
    double q_scale = p->q_scale > 0.0 ? p->q_scale : 1.0 / sqrt((double)D);

    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *k = (double *)malloc(sizeof(double) * (size_t)D);
    double *v = (double *)malloc(sizeof(double) * (size_t)D);
    double *alpha = (double *)malloc(sizeof(double) * (size_t)D);
    double *o = (double *)malloc(sizeof(double) * (size_t)D);
    const double decay_rate = exp(jb->A_log);

    for (int t = 0; t < jb->T; t++) {
        const double *xq = jb->xq + (ptrdiff_t)t * jb->ld_x;
        const double *xk = jb->xk + (ptrdiff_t)t * jb->ld_x;
        const double *xv = jb->xv + (ptrdiff_t)t * jb->ld_x;
        const double *z = jb->z + (ptrdiff_t)t * jb->ld_z;
        const double *g = jb->g + (ptrdiff_t)t * jb->ld_g;
        const double b = jb->b[(ptrdiff_t)t * jb->ld_b];

        /* q,k,v = SiLU(ShortConv4(x)), channel by channel */
        for (int i = 0; i < D; i++) {
            q[i] = kda_oracle_silu(kda_oracle_conv_step(K, jb->wq + (size_t)i * K,
                                                        jb->cq + (size_t)i * (K - 1), xq[i]));
            k[i] = kda_oracle_silu(kda_oracle_conv_step(K, jb->wk + (size_t)i * K,
                                                        jb->ck + (size_t)i * (K - 1), xk[i]));
            v[i] = kda_oracle_silu(kda_oracle_conv_step(K, jb->wv + (size_t)i * K,
                                                        jb->cv + (size_t)i * (K - 1), xv[i]));
        }
        /* q,k L2-normalised; q scaled */
        l2norm_scale(D, q, p->l2_eps, q_scale);
        l2norm_scale(D, k, p->l2_eps, 1.0);
        /* per-key-channel decay gate and the per-head beta */
        for (int i = 0; i < D; i++) {
            double gk = p->gate_lower_bound * kda_oracle_sigmoid(decay_rate * (z[i] + jb->dt_bias[i]));
            alpha[i] = exp(gk);
        }
        double beta = kda_oracle_sigmoid(b);
        /* state update and readout */
        kda_oracle_core_step(D, D, jb->S, q, k, v, alpha, beta, o);
        /* output: sigmoid(g) * RMSNorm(o) */
        kda_oracle_rmsnorm_gate(D, o, g, p->norm_w, p->rms_eps, jb->out + (ptrdiff_t)t * jb->ld_out);
    }
    free(q);
    free(k);
    free(v);
    free(alpha);
    free(o);
    return 0;
}

/* ---- independent (sequence, head) jobs, spread over threads ---- */
int kda_oracle_run_jobs(const kda_oracle_params *p, const kda_oracle_job *jobs, int n_jobs,
                        int n_threads)
{
    int bad = 0;
    if (n_threads < 1)
        n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(| : bad)
    for (int j = 0; j < n_jobs; j++)
        bad |= (kda_oracle_head_forward(p, &jobs[j]) != 0);
    return bad ? -1 : 0;
}

int kda_oracle_job_size(void) { return (int)sizeof(kda_oracle_job); }
int kda_oracle_params_size(void) { return (int)sizeof(kda_oracle_params); }
