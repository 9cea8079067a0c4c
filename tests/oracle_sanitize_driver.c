/* Drives every oracle function over special rows; built together with
 * oracle/oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitize.py (host code only).  It checks nothing itself:
 * a memory or undefined-behaviour error aborts the process. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_set_threads(int n);
void orc_softcap_fwd(const double* x, int64_t n, double cap, double* y);
void orc_softcap_bwd(const double* x, const double* gy, int64_t n, double cap, double* gx);
int orc_logp_fwd(const double* x, int64_t N, int64_t V, const int64_t* t, int64_t k,
                 double cap, double* out);
int orc_logp_bwd(const double* x, int64_t N, int64_t V, const int64_t* t, int64_t k,
                 double cap, const double* g, double* gx);
int orc_entropy_fwd(const double* x, int64_t N, int64_t V, double cap, double* out);
int orc_entropy_bwd(const double* x, int64_t N, int64_t V, double cap, const double* g,
                    double* gx);
int orc_kl_fwd(const double* pol, const double* ref, int64_t N, int64_t V, int dir,
               double cap_pol, double cap_ref, double* out);
int orc_kl_bwd(const double* pol, const double* ref, int64_t N, int64_t V, int dir,
               double cap_pol, double cap_ref, const double* g, double* gx);
int orc_kl_bwd_ref(const double* pol, const double* ref, int64_t N, int64_t V, int dir,
                   double cap_pol, double cap_ref, const double* g, double* gr);

static double* alloc(int64_t n) { return (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double)); }

/* rows: 0 plain, 1 masked columns, 2 all -inf, 3 +1000 offset, 4 one finite column */
static void fill(double* x, int64_t N, int64_t V, unsigned seed) {
    for (int64_t i = 0; i < N; ++i)
        for (int64_t v = 0; v < V; ++v) {
            seed = seed * 1103515245u + 12345u;
            double z = ((seed >> 8) & 0xffff) / 65536.0 * 6.0 - 3.0;
            if (i == 1 && v % 3 == 1) z = -INFINITY;
            if (i == 2) z = -INFINITY;
            if (i == 3) z += 1000.0;
            if (i == 4 && v != V - 1) z = -INFINITY;
            x[i * V + v] = z;
        }
}

static int run(int64_t N, int64_t V, int64_t k, double cap) {
    double *x = alloc(N * V), *y = alloc(N * V), *g = alloc(N * k), *gr = alloc(N);
    double *out = alloc(N * k), *gx = alloc(N * V), *gy = alloc(N * V);
    int64_t* t = (int64_t*)malloc((size_t)(N * k > 0 ? N * k : 1) * sizeof(int64_t));
    fill(x, N, V, 7u);
    fill(y, N, V, 11u);
    if (N > 0 && V > 1) y[V - 1] = -INFINITY; /* reference-only mask: mismatch in row 0 */
    for (int64_t i = 0; i < N * k; ++i) {
        t[i] = (i * 7) % (V + 2) - 1;         /* -1 and V: ignored / out of range */
        g[i] = 0.25 * (double)(i % 5) - 0.5;
    }
    if (N * k > 1) t[1] = t[0];                /* duplicate */
    for (int64_t i = 0; i < N; ++i) gr[i] = 1.0 - 0.1 * (double)i;
    for (int64_t i = 0; i < N * V; ++i) gy[i] = 0.5;
    int bad = 0;
    orc_softcap_fwd(x, N * V, cap > 0 ? cap : 30.0, gx);
    orc_softcap_bwd(x, gy, N * V, cap > 0 ? cap : 30.0, gx);
    bad |= orc_logp_fwd(x, N, V, t, k, cap, out);
    bad |= orc_logp_bwd(x, N, V, t, k, cap, g, gx);
    bad |= orc_entropy_fwd(x, N, V, cap, out);
    bad |= orc_entropy_bwd(x, N, V, cap, gr, gx);
    for (int dir = 0; dir < 2; ++dir) {
        bad |= orc_kl_fwd(x, y, N, V, dir, cap, 0.0, out);
        bad |= orc_kl_bwd(x, y, N, V, dir, cap, 0.0, gr, gx);
        bad |= orc_kl_bwd_ref(x, y, N, V, dir, 0.0, cap, gr, gy);
    }
    free(x); free(y); free(g); free(gr); free(out); free(gx); free(gy); free(t);
    return bad;
}

int main(void) {
    orc_set_threads(2);
    const double caps[] = {0.0, 20.0, 1e-7};
    int bad = 0;
    for (int c = 0; c < 3; ++c) {
        bad |= run(5, 7, 3, caps[c]);
        bad |= run(6, 1, 2, caps[c]);
        bad |= run(0, 9, 1, caps[c]);
        bad |= run(5, 300, 17, caps[c]);
    }
    printf("oracle sanitizer driver done (status %d)\n", bad);
    return bad ? 1 : 0;
}
