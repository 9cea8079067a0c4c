/*
 * oracle.c -- plain, slow fp64 CPU reference for the row-wise log-softmax
 * heads.  TEST INFRASTRUCTURE ONLY: it is linked by the test-suite, by the
 * smoke check and by the CPU-baseline leg of the benchmark, never by the
 * product library.  It shares no code, header, constant or helper with the
 * HIP path.
 *
 * Every head below has an exact closed definition, so the oracle is that
 * definition written out, row by row, in double precision, with the textbook
 * two-pass softmax (max first, then the sum of exponentials).  It does NOT
 * follow the single-read online algorithm that the GPU kernels use.
 *
 * Inputs are the exact fp64 values of the stored fp32/bf16 logits; outputs
 * are fp64 and are compared by the tests with the tolerance of the dtype the
 * GPU writes.
 *
 * Sources (web pages on the subject; cited by title and section):
 *   [SC]  "Final Logit Softcap" (RL-Kernel operator documentation):
 *         Summary (forward formula and its derivative), Tensor and Precision
 *         Contract, Accuracy and Invariance (fp64 derivative 1/cosh^2).
 *   [VP]  "Add Triton kernels for vocab-parallel logprobs, entropy and KL"
 *         (DeepSpeed pull request 8838): Changes (logprobs / entropy / KL
 *         heads, top-k one-hot terms), Tests (masked vocabulary, all -inf
 *         rows, support mismatch, duplicate / ignored top-k ids), and the
 *         review comment proposing a single pass over the logits for the
 *         entropy and KL forward (entropy H = log S - W/S, KL closed form,
 *         support-mismatch rule).
 *   [ZW]  "perf(logp): fused zero-workspace backward for the generic CUDA
 *         fused logp" (RL-Kernel pull request 495): Summary (gradient
 *         g * (onehot - softmax)), Behavior changes (targets outside [0, V)
 *         give output 0 and an exactly zero gradient row).
 *
 * Readings where the pages are silent:
 *   - a target is valid iff 0 <= t < V; any other value is ignored [ZW];
 *   - a logp row with no valid target has output 0 and an all-zero gradient,
 *     even if the row is empty (index handling comes first);
 *   - an empty row (every logit -inf) gives NaN outputs and NaN gradients;
 *   - a masked logit (-inf in a non-empty row) has probability exactly 0;
 *   - support mismatch is decided on the logits: KL(A||B) = +inf when some
 *     column is finite in A and -inf in B, even where p_A underflows [VP];
 *   - on a reverse-KL mismatch row the gradient is NaN on the policy's
 *     support and 0 elsewhere; forward KL keeps its finite gradient g(p - q);
 *   - the gradient with respect to the reference mirrors this: reverse KL
 *     keeps its finite g(q - p), forward KL gives NaN on the reference's
 *     support of a mismatch row and 0 elsewhere;
 *   - duplicate top-k ids each receive the same output; their upstream
 *     gradients add (ascending slot order) [VP];
 *   - softcap off is cap == 0; with a cap, -inf maps to -cap.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

/* Number of host threads used by every oracle call (rows are split among
 * them; each row is still computed by one thread in plain order). */
void orc_set_threads(int n) { g_threads = n > 0 ? n : 1; }
int orc_get_threads(void) { return g_threads; }

/* ---------------------------------------------------------------- softcap */

/* [SC] Summary: y = c * tanh(x / c). */
static double cap_value(double x, double c) { return c * tanh(x / c); }

/* [SC] Summary + Accuracy and Invariance: dy/dx = 1 - tanh^2(x/c), evaluated
 * as 1 / cosh^2(x/c) (the fp64 form the page uses); cosh overflow gives 0. */
static double cap_slope(double x, double c) {
    double ch = cosh(x / c);
    return 1.0 / (ch * ch);
}

void orc_softcap_fwd(const double* x, int64_t n, double cap, double* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = cap_value(x[i], cap);
}

void orc_softcap_bwd(const double* x, const double* gy, int64_t n, double cap, double* gx) {
    for (int64_t i = 0; i < n; ++i) gx[i] = gy[i] * cap_slope(x[i], cap);
}

/* ------------------------------------------------------- per-row softmax */

/* The capped row y (cap == 0: identity) and its slope s = dy/dx. */
static void row_prologue(const double* x, int64_t V, double cap, double* y, double* s) {
    for (int64_t v = 0; v < V; ++v) {
        if (cap != 0.0) {
            y[v] = cap_value(x[v], cap);
            s[v] = cap_slope(x[v], cap);
        } else {
            y[v] = x[v];
            s[v] = 1.0;
        }
    }
}

/* Textbook log-softmax of one row.  F = {v : y_v > -inf}.  Returns 1 if the
 * row is empty (F is empty).  Otherwise fills logp (-inf off F) and p (0 off
 * F) and returns 0. */
static int row_log_softmax(const double* y, int64_t V, double* logp, double* p) {
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v)
        if (y[v] > m) m = y[v];
    if (m == -INFINITY) return 1;
    double z = 0.0;
    for (int64_t v = 0; v < V; ++v)
        if (y[v] > -INFINITY) z += exp(y[v] - m);
    double lse = m + log(z);
    for (int64_t v = 0; v < V; ++v) {
        if (y[v] > -INFINITY) {
            logp[v] = y[v] - lse;
            p[v] = exp(logp[v]);
        } else {
            logp[v] = -INFINITY;
            p[v] = 0.0;
        }
    }
    return 0;
}

typedef struct {
    double* y;
    double* s;
    double* logp;
    double* p;
} row_buf;

static int buf_alloc(row_buf* b, int64_t V) {
    b->y = (double*)malloc(sizeof(double) * (size_t)V);
    b->s = (double*)malloc(sizeof(double) * (size_t)V);
    b->logp = (double*)malloc(sizeof(double) * (size_t)V);
    b->p = (double*)malloc(sizeof(double) * (size_t)V);
    return b->y && b->s && b->logp && b->p;
}

static void buf_free(row_buf* b) {
    free(b->y);
    free(b->s);
    free(b->logp);
    free(b->p);
}

static int target_valid(int64_t t, int64_t V) { return t >= 0 && t < V; }

/* ------------------------------------------------------------- logprobs */

/* [ZW] Behavior changes + [VP] Changes: out[i, j] = logp_i[t_ij] for a valid
 * target, exactly 0 for an ignored one; NaN for a valid target in an empty
 * row. */
int orc_logp_fwd(const double* x, int64_t N, int64_t V, const int64_t* t, int64_t k,
                 double cap, double* out) {
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads) reduction(| : bad)
    for (int64_t i = 0; i < N; ++i) {
        row_buf b;
        if (!buf_alloc(&b, V)) {
            bad |= 1;
            buf_free(&b);
            continue;
        }
        row_prologue(x + i * V, V, cap, b.y, b.s);
        int empty = row_log_softmax(b.y, V, b.logp, b.p);
        for (int64_t j = 0; j < k; ++j) {
            int64_t tj = t[i * k + j];
            if (!target_valid(tj, V))
                out[i * k + j] = 0.0;
            else if (empty)
                out[i * k + j] = NAN;
            else
                out[i * k + j] = b.logp[tj];
        }
        buf_free(&b);
    }
    return bad;
}

/* [ZW] Summary: d/dx of sum_j g_j logp[t_j] is (h - p * G) with
 * h_v = sum of g_j over valid slots j with t_j == v (ascending j) and
 * G = sum of g_j over valid slots; times the softcap slope [SC].  A row with
 * no valid slot is exactly zero; otherwise an empty row is NaN. */
int orc_logp_bwd(const double* x, int64_t N, int64_t V, const int64_t* t, int64_t k,
                 double cap, const double* g, double* gx) {
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads) reduction(| : bad)
    for (int64_t i = 0; i < N; ++i) {
        double* gr = gx + i * V;
        int any_valid = 0;
        for (int64_t j = 0; j < k; ++j) any_valid |= target_valid(t[i * k + j], V);
        if (!any_valid) {
            for (int64_t v = 0; v < V; ++v) gr[v] = 0.0;
            continue;
        }
        row_buf b;
        double* h = (double*)calloc((size_t)V, sizeof(double));
        if (!buf_alloc(&b, V) || !h) {
            bad |= 1;
            buf_free(&b);
            free(h);
            continue;
        }
        row_prologue(x + i * V, V, cap, b.y, b.s);
        int empty = row_log_softmax(b.y, V, b.logp, b.p);
        if (empty) {
            for (int64_t v = 0; v < V; ++v) gr[v] = NAN;
        } else {
            double G = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                int64_t tj = t[i * k + j];
                if (target_valid(tj, V)) {
                    G += g[i * k + j];
                    h[tj] += g[i * k + j];
                }
            }
            for (int64_t v = 0; v < V; ++v) gr[v] = (h[v] - b.p[v] * G) * b.s[v];
        }
        free(h);
        buf_free(&b);
    }
    return bad;
}

/* -------------------------------------------------------------- entropy */

/* [VP] review comment: H = -sum_v p_v log p_v over the support (0 log 0 = 0),
 * written here as sum_v p_v (lse - y_v).  NaN for an empty row. */
static double row_entropy(const row_buf* b, int64_t V) {
    double H = 0.0;
    for (int64_t v = 0; v < V; ++v)
        if (b->logp[v] > -INFINITY) H -= b->p[v] * b->logp[v];
    return H;
}

int orc_entropy_fwd(const double* x, int64_t N, int64_t V, double cap, double* out) {
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads) reduction(| : bad)
    for (int64_t i = 0; i < N; ++i) {
        row_buf b;
        if (!buf_alloc(&b, V)) {
            bad |= 1;
            buf_free(&b);
            continue;
        }
        row_prologue(x + i * V, V, cap, b.y, b.s);
        int empty = row_log_softmax(b.y, V, b.logp, b.p);
        out[i] = empty ? NAN : row_entropy(&b, V);
        buf_free(&b);
    }
    return bad;
}

/* dH/dy_v = -p_v (log p_v + H); masked columns (p = 0, log p = -inf) get 0. */
int orc_entropy_bwd(const double* x, int64_t N, int64_t V, double cap, const double* g,
                    double* gx) {
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads) reduction(| : bad)
    for (int64_t i = 0; i < N; ++i) {
        double* gr = gx + i * V;
        row_buf b;
        if (!buf_alloc(&b, V)) {
            bad |= 1;
            buf_free(&b);
            continue;
        }
        row_prologue(x + i * V, V, cap, b.y, b.s);
        int empty = row_log_softmax(b.y, V, b.logp, b.p);
        if (empty) {
            for (int64_t v = 0; v < V; ++v) gr[v] = NAN;
        } else {
            double H = row_entropy(&b, V);
            for (int64_t v = 0; v < V; ++v) {
                if (b.logp[v] == -INFINITY)
                    gr[v] = 0.0;
                else
                    gr[v] = g[i] * (-b.p[v] * (b.logp[v] + H)) * b.s[v];
            }
        }
        buf_free(&b);
    }
    return bad;
}

/* ------------------------------------------------------------------- KL */

/* Direction codes: 0 = reverse KL(P||R), 1 = forward KL(R||P), where P is the
 * policy (the differentiated input) and R the reference. */
enum { ORC_KL_REVERSE = 0, ORC_KL_FORWARD = 1 };

/* [VP] review comment: KL(A||B) = sum over A's support of
 * p_A (log p_A - log p_B); +inf when B masks a column A supports. */
static double row_kl(const row_buf* A, const row_buf* B, int64_t V) {
    for (int64_t v = 0; v < V; ++v)
        if (A->logp[v] > -INFINITY && B->logp[v] == -INFINITY) return INFINITY;
    double D = 0.0;
    for (int64_t v = 0; v < V; ++v)
        if (A->logp[v] > -INFINITY) D += A->p[v] * (A->logp[v] - B->logp[v]);
    return D;
}

int orc_kl_fwd(const double* pol, const double* ref, int64_t N, int64_t V, int dir,
               double cap_pol, double cap_ref, double* out) {
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads) reduction(| : bad)
    for (int64_t i = 0; i < N; ++i) {
        row_buf P, R;
        int okp = buf_alloc(&P, V), okr = buf_alloc(&R, V);
        if (!okp || !okr) {
            bad |= 1;
            buf_free(&P);
            buf_free(&R);
            continue;
        }
        row_prologue(pol + i * V, V, cap_pol, P.y, P.s);
        row_prologue(ref + i * V, V, cap_ref, R.y, R.s);
        int ep = row_log_softmax(P.y, V, P.logp, P.p);
        int er = row_log_softmax(R.y, V, R.logp, R.p);
        if (ep || er)
            out[i] = NAN;
        else
            out[i] = dir == ORC_KL_REVERSE ? row_kl(&P, &R, V) : row_kl(&R, &P, V);
        buf_free(&P);
        buf_free(&R);
    }
    return bad;
}

/* Gradient with respect to the policy logits only (the reference is treated
 * as detached).
 *   reverse: d/dy_v KL(P||R) = p_v (l_v - D),  l_v = log p_v - log q_v;
 *   forward: d/dy_v KL(R||P) = p_v - q_v.
 * Both times g and the policy's softcap slope. */
int orc_kl_bwd(const double* pol, const double* ref, int64_t N, int64_t V, int dir,
               double cap_pol, double cap_ref, const double* g, double* gx) {
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads) reduction(| : bad)
    for (int64_t i = 0; i < N; ++i) {
        double* gr = gx + i * V;
        row_buf P, R;
        int okp = buf_alloc(&P, V), okr = buf_alloc(&R, V);
        if (!okp || !okr) {
            bad |= 1;
            buf_free(&P);
            buf_free(&R);
            continue;
        }
        row_prologue(pol + i * V, V, cap_pol, P.y, P.s);
        row_prologue(ref + i * V, V, cap_ref, R.y, R.s);
        int ep = row_log_softmax(P.y, V, P.logp, P.p);
        int er = row_log_softmax(R.y, V, R.logp, R.p);
        if (ep || er) {
            for (int64_t v = 0; v < V; ++v) gr[v] = NAN;
        } else if (dir == ORC_KL_REVERSE) {
            double D = row_kl(&P, &R, V);
            for (int64_t v = 0; v < V; ++v) {
                if (P.logp[v] == -INFINITY)
                    gr[v] = 0.0;
                else if (D == INFINITY)
                    gr[v] = NAN;
                else
                    gr[v] = g[i] * P.p[v] * ((P.logp[v] - R.logp[v]) - D) * P.s[v];
            }
        } else {
            for (int64_t v = 0; v < V; ++v) gr[v] = g[i] * (P.p[v] - R.p[v]) * P.s[v];
        }
        buf_free(&P);
        buf_free(&R);
    }
    return bad;
}

/* Gradient with respect to the reference logits (a reference that is not
 * detached).  With log q_u = z_u - logsumexp(z) for the (capped) reference
 * logits z, d log q_u / d z_v = [u == v] - q_v, hence
 *   reverse: d/dz_v KL(P||R) = -sum_u p_u ([u == v] - q_v) = q_v - p_v,
 *            finite on every row where both distributions exist (a support
 *            mismatch included: no infinite term enters it);
 *   forward: d/dz_v KL(R||P) = q_v (log q_v - log p_v - D), 0 off the
 *            reference's support, and on a mismatch row (D = +inf) NaN on
 *            the reference's support -- the mirror images of the two policy
 *            gradients above.
 * Both times g and the reference's softcap slope; an empty row in either
 * tensor gives NaN everywhere. */
int orc_kl_bwd_ref(const double* pol, const double* ref, int64_t N, int64_t V, int dir,
                   double cap_pol, double cap_ref, const double* g, double* gr_out) {
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(g_threads) reduction(| : bad)
    for (int64_t i = 0; i < N; ++i) {
        double* gr = gr_out + i * V;
        row_buf P, R;
        int okp = buf_alloc(&P, V), okr = buf_alloc(&R, V);
        if (!okp || !okr) {
            bad |= 1;
            buf_free(&P);
            buf_free(&R);
            continue;
        }
        row_prologue(pol + i * V, V, cap_pol, P.y, P.s);
        row_prologue(ref + i * V, V, cap_ref, R.y, R.s);
        int ep = row_log_softmax(P.y, V, P.logp, P.p);
        int er = row_log_softmax(R.y, V, R.logp, R.p);
        if (ep || er) {
            for (int64_t v = 0; v < V; ++v) gr[v] = NAN;
        } else if (dir == ORC_KL_REVERSE) {
            for (int64_t v = 0; v < V; ++v) gr[v] = g[i] * (R.p[v] - P.p[v]) * R.s[v];
        } else {
            double D = row_kl(&R, &P, V);
            for (int64_t v = 0; v < V; ++v) {
                if (R.logp[v] == -INFINITY)
                    gr[v] = 0.0;
                else if (D == INFINITY)
                    gr[v] = NAN;
                else
                    gr[v] = g[i] * R.p[v] * ((R.logp[v] - P.logp[v]) - D) * R.s[v];
            }
        }
        buf_free(&P);
        buf_free(&R);
    }
    return bad;
}
