/* Runs the fp64 oracle on a small varlen batch (sequences of 0, 1, 2 and 17 tokens,
 * 3 heads, D = 8) with nonzero initial states, for the address / undefined-behaviour
 * sanitizer build of the CPU tests.  Prints "ok" when every output and state is finite. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "kda_oracle.h"

static unsigned long long lcg = 12345;
static double urand(void) { /* uniform in [-1, 1) */
    lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(lcg >> 11) / (double)(1ULL << 52) - 1.0;
}
static double *fill(size_t n) {
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = urand();
    return p;
}

int main(void) {
    enum { D = 8, K = 4, H = 3, NSEQ = 4 };
    const int lens[NSEQ] = {0, 1, 2, 17};
    double *norm_w = fill(D);
    kda_oracle_params prm = {D, K, -5.0, 1e-6, 1e-5, 0.0, norm_w};
    kda_oracle_job jobs[NSEQ * H];
    double *bufs[NSEQ * H][12];
    for (int s = 0; s < NSEQ; ++s)
        for (int h = 0; h < H; ++h) {
            const int T = lens[s];
            const size_t n = (size_t)(T > 0 ? T : 1) * D;
            double **b = bufs[s * H + h];
            b[0] = fill(n); b[1] = fill(n); b[2] = fill(n); b[3] = fill(n); b[4] = fill(n);
            b[5] = fill(T > 0 ? T : 1);
            b[6] = fill(D * K); b[7] = fill(D * K); b[8] = fill(D * K);
            b[9] = fill(D * D);
            b[10] = fill(3 * D * (K - 1));
            b[11] = calloc(n, sizeof(double));
            kda_oracle_job *j = &jobs[s * H + h];
            j->T = T;
            j->xq = b[0]; j->xk = b[1]; j->xv = b[2]; j->z = b[3]; j->g = b[4]; j->b = b[5];
            j->ld_x = D; j->ld_z = D; j->ld_g = D; j->ld_b = 1; j->ld_out = D;
            j->wq = b[6]; j->wk = b[7]; j->wv = b[8];
            j->dt_bias = b[3];  /* any D values */
            j->A_log = -0.5;
            j->S = b[9];
            j->cq = b[10]; j->ck = b[10] + D * (K - 1); j->cv = b[10] + 2 * D * (K - 1);
            j->out = b[11];
        }
    if (kda_oracle_run_jobs(&prm, jobs, NSEQ * H, 2) != 0) {
        printf("oracle returned an error\n");
        return 1;
    }
    for (int i = 0; i < NSEQ * H; ++i) {
        for (int e = 0; e < jobs[i].T * D; ++e)
            if (!isfinite(jobs[i].out[e])) { printf("non-finite output\n"); return 1; }
        for (int e = 0; e < D * D; ++e)
            if (!isfinite(jobs[i].S[e])) { printf("non-finite state\n"); return 1; }
        for (int k = 0; k < 12; ++k) free(bufs[i][k]);
    }
    free(norm_w);
    printf("ok\n");
    return 0;
}
