/*
 * kda_oracle.h -- fp64 CPU oracle of the KDA mixer (test infrastructure only; see
 * kda_oracle.c).  Not included by, and not including, anything of the HIP library.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int head_dim;             /* D (128 for the model; any D >= 1 here) */
    int conv_size;            /* ShortConv taps K (4 for the model) */
    double gate_lower_bound;  /* gmin = -5 */
    double l2_eps;            /* 1e-6, added to the sum of squares inside the sqrt */
    double rms_eps;           /* RMSNorm eps of the head norm */
    double q_scale;           /* <= 0 selects D^-0.5 */
    const double *norm_w;     /* [D] RMSNorm weight, shared by all heads */
} kda_oracle_params;

/* One (sequence, head): T tokens.  Every [T][D] array has its token rows ld_* apart
 * (in elements) and its D channels contiguous. */
typedef struct {
    int T;
    const double *xq, *xk, *xv;  /* pre-conv q/k/v, token t channel i at x[t*ld_x + i] */
    const double *z;             /* decay logits (before dt_bias)          [t*ld_z + i] */
    const double *g;             /* output-gate logits                     [t*ld_g + i] */
    const double *b;             /* beta logit of this head                [t*ld_b]     */
    ptrdiff_t ld_x, ld_z, ld_g, ld_b, ld_out;
    const double *wq, *wk, *wv;  /* [D][K] conv taps, oldest first */
    const double *dt_bias;       /* [D] */
    double A_log;
    double *S;                   /* [D][D] S[key][value]; in: initial state, out: final */
    double *cq, *ck, *cv;        /* [D][K-1] conv windows, oldest first; in/out */
    double *out;                 /* [t*ld_out + i] = sigmoid(g) * RMSNorm(o) */
} kda_oracle_job;

double kda_oracle_sigmoid(double x);
double kda_oracle_silu(double x);
double kda_oracle_conv_step(int K, const double *w, double *win, double x);
void kda_oracle_rmsnorm_gate(int D, const double *o, const double *g, const double *w,
                             double eps, double *out);
void kda_oracle_core_step(int dk, int dv, double *S, const double *q, const double *k,
                          const double *v, const double *alpha, double beta, double *o);
int kda_oracle_head_forward(const kda_oracle_params *p, const kda_oracle_job *jb);
int kda_oracle_run_jobs(const kda_oracle_params *p, const kda_oracle_job *jobs, int n_jobs,
                        int n_threads);
int kda_oracle_job_size(void);
int kda_oracle_params_size(void);

#ifdef __cplusplus
}
#endif
#endif
