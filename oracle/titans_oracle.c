/*
 * titans_oracle.c -- plain fp64 CPU oracle of the Titans neural long-term
 * memory (chunked test-time update + retrieval).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU library is checked against.  Only the test suite, the package's smoke
 * check and the CPU-baseline leg of the benchmark may load or call it; the
 * product path never does.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes, and where the pages state it ("Titans: Learning to
 * Memorize at Test Time", mer.dev notes, page 1 of the source set):
 *
 *   section 3.1, "Objective":      loss l(M; x_t) = ||M(k_t) - v_t||^2
 *   section 3.1, "Learning Process and Surprise Metric":
 *                                   S_t = eta_t S_{t-1} - theta_t grad l
 *   section 3.1, "Forgetting Mechanism":
 *                                   M_t = (1 - alpha_t) M_{t-1} + S_t
 *   section 3.1, "Memory Architecture": M = W (matrix) or an MLP, L_M >= 2
 *   section 3.1, "Retrieving a Memory":  y_t = M*(q_t), a forward pass that
 *                                   does not change the weights
 *   section 3.2, "How to Parallelize the Long-term Memory Training": the
 *                                   sequence is cut into chunks of b tokens
 *                                   and every token's gradient is taken at
 *                                   the weights of the chunk start t'.
 * The German summary (lowest.today, "Gedaechtnisaktualisierungsmechanismus")
 * restates the same three update rules.
 *
 * Readings taken where the pages are silent or garbled:
 *   - gradient scale: the gradient used is (M(k) - v) dM/dW, i.e. the
 *     gradient of 0.5 ||M(k) - v||^2.  This is the form section 3.2 prints
 *     for the linear case, (W_0 x - x) x^T, without a factor 2.
 *   - chunk start: tokens are 0-indexed; chunk c covers [c b, c b + b) and
 *     every token of it differentiates at the state left by token c b - 1
 *     (the input state for c = 0).  A shorter last chunk follows the same
 *     rule.
 *   - order inside a token: S first, then M = (1 - alpha) M + S; alpha
 *     scales M only.
 *   - retrieval reads the state after the token's own write
 *     (read_mode 0, the write-then-read memory abstraction of section 2.1,
 *     "Modern Linear Models and Their Memory Perspective"); read_mode 1
 *     reads the chunk-start state instead.
 *   - MLP: no biases, widths d -> hidden -> ... -> hidden -> d, SiLU after
 *     every layer but the last; one layer is the matrix memory W.
 *
 * The algorithm is an iteration, so the oracle is that iteration written
 * token by token, with no blocking, reordering or closed-form coefficients.
 * Parameter layout per stream: layers 1..L concatenated, layer l stored
 * row-major as [n_l x n_{l-1}] (column-vector convention M(k) = W k).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TMO_MAX_LAYERS 16

typedef struct {
    int L;                        /* number of weight matrices */
    int w[TMO_MAX_LAYERS + 1];    /* widths n_0 .. n_L */
    int64_t off[TMO_MAX_LAYERS + 1]; /* offset of layer l (1-based) in the parameter vector */
    int64_t P;                    /* parameter count */
    int maxw;
} net_t;

static int net_init(net_t* n, int d, int hidden, int n_layers) {
    if (d <= 0 || n_layers <= 0 || n_layers > TMO_MAX_LAYERS) return -1;
    if (n_layers >= 2 && hidden <= 0) return -1;
    n->L = n_layers;
    n->w[0] = d;
    for (int l = 1; l < n_layers; ++l) n->w[l] = hidden;
    n->w[n_layers] = d;
    n->P = 0;
    n->maxw = d;
    for (int l = 1; l <= n_layers; ++l) {
        n->off[l] = n->P;
        n->P += (int64_t)n->w[l] * n->w[l - 1];
        if (n->w[l] > n->maxw) n->maxw = n->w[l];
    }
    return 0;
}

/* SiLU and its derivative, from the definition sigma(z) = z / (1 + e^-z). */
static double logistic(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu(double z) { return z * logistic(z); }
static double silu_prime(double z) {
    double s = logistic(z);
    return s * (1.0 + z * (1.0 - s));
}

/* Forward pass of the memory at weights W on input x.
 * z[l] (l = 1..L) receives the pre-activations and a[l] the activations
 * (a[0] = x, a[L] = z[L] = output).  Each z[l], a[l] has room for maxw. */
static void mem_forward(const net_t* n, const double* W, const double* x,
                        double** z, double** a) {
    memcpy(a[0], x, sizeof(double) * n->w[0]);
    for (int l = 1; l <= n->L; ++l) {
        const double* Wl = W + n->off[l];
        int rows = n->w[l], cols = n->w[l - 1];
        for (int r = 0; r < rows; ++r) {
            double acc = 0.0;
            for (int c = 0; c < cols; ++c) acc += Wl[(int64_t)r * cols + c] * a[l - 1][c];
            z[l][r] = acc;
            a[l][r] = (l < n->L) ? silu(acc) : acc;
        }
    }
}

/* Gradient of 0.5 ||M_W(k) - v||^2 with respect to every weight (layout of
 * W), by the chain rule written out layer by layer.  Returns the loss. */
static double mem_grad(const net_t* n, const double* W, const double* k, const double* v,
                       double* grad, double** z, double** a, double* delta, double* delta_prev) {
    mem_forward(n, W, k, z, a);
    int L = n->L;
    double loss = 0.0;
    for (int r = 0; r < n->w[L]; ++r) {
        delta[r] = a[L][r] - v[r];            /* residual M(k) - v */
        loss += 0.5 * delta[r] * delta[r];
    }
    for (int l = L; l >= 1; --l) {
        int rows = n->w[l], cols = n->w[l - 1];
        const double* Wl = W + n->off[l];
        double* gl = grad + n->off[l];
        for (int r = 0; r < rows; ++r)
            for (int c = 0; c < cols; ++c)
                gl[(int64_t)r * cols + c] = delta[r] * a[l - 1][c];   /* outer product */
        if (l > 1) {
            for (int c = 0; c < cols; ++c) {
                double acc = 0.0;
                for (int r = 0; r < rows; ++r) acc += Wl[(int64_t)r * cols + c] * delta[r];
                delta_prev[c] = acc * silu_prime(z[l - 1][c]);
            }
            memcpy(delta, delta_prev, sizeof(double) * cols);
        }
    }
    return loss;
}

typedef struct {
    double** z;
    double** a;
    double* zbuf;
    double* abuf;
    double* delta;
    double* delta_prev;
} work_t;

static int work_alloc(work_t* w, const net_t* n) {
    int L = n->L;
    w->z = (double**)calloc(L + 1, sizeof(double*));
    w->a = (double**)calloc(L + 1, sizeof(double*));
    w->zbuf = (double*)calloc((size_t)(L + 1) * n->maxw, sizeof(double));
    w->abuf = (double*)calloc((size_t)(L + 1) * n->maxw, sizeof(double));
    w->delta = (double*)calloc(n->maxw, sizeof(double));
    w->delta_prev = (double*)calloc(n->maxw, sizeof(double));
    if (!w->z || !w->a || !w->zbuf || !w->abuf || !w->delta || !w->delta_prev) return -1;
    for (int l = 0; l <= L; ++l) {
        w->z[l] = w->zbuf + (size_t)l * n->maxw;
        w->a[l] = w->abuf + (size_t)l * n->maxw;
    }
    return 0;
}

static void work_free(work_t* w) {
    free(w->z); free(w->a); free(w->zbuf); free(w->abuf); free(w->delta); free(w->delta_prev);
}

int64_t tmo_param_count(int d, int hidden, int n_layers) {
    net_t n;
    if (net_init(&n, d, hidden, n_layers)) return -1;
    return n.P;
}

/* y = M_W(x) for one vector x of width d. */
int tmo_memory_apply(int d, int hidden, int n_layers, const double* W, const double* x, double* y) {
    net_t n;
    work_t w;
    if (net_init(&n, d, hidden, n_layers)) return -1;
    if (work_alloc(&w, &n)) { work_free(&w); return -2; }
    mem_forward(&n, W, x, w.z, w.a);
    memcpy(y, w.a[n.L], sizeof(double) * d);
    work_free(&w);
    return 0;
}

/* grad = d/dW 0.5 ||M_W(k) - v||^2 ; *loss receives 0.5 ||M_W(k) - v||^2. */
int tmo_memory_grad(int d, int hidden, int n_layers, const double* W, const double* k,
                    const double* v, double* grad, double* loss) {
    net_t n;
    work_t w;
    if (net_init(&n, d, hidden, n_layers)) return -1;
    if (work_alloc(&w, &n)) { work_free(&w); return -2; }
    double l = mem_grad(&n, W, k, v, grad, w.z, w.a, w.delta, w.delta_prev);
    if (loss) *loss = l;
    work_free(&w);
    return 0;
}

/* One stream: the chunked recurrence, token by token. */
static int run_stream(const net_t* n, int N, int chunk, int read_mode,
                      const double* k, const double* v, const double* q,
                      const double* alpha, const double* eta, const double* theta,
                      const double* W_in, const double* S_in,
                      double* y, double* W_out, double* S_out, double* w_norm) {
    int64_t P = n->P;
    int d = n->w[0];
    double* W = (double*)malloc(sizeof(double) * P);
    double* S = (double*)malloc(sizeof(double) * P);
    double* Wc = (double*)malloc(sizeof(double) * P);   /* chunk-start weights M_{t'} */
    double* g = (double*)malloc(sizeof(double) * P);
    work_t w;
    int rc = 0;
    if (!W || !S || !Wc || !g || work_alloc(&w, n)) { rc = -2; goto done; }
    memcpy(W, W_in, sizeof(double) * P);
    memcpy(S, S_in, sizeof(double) * P);
    for (int t = 0; t < N; ++t) {
        if (t % chunk == 0) memcpy(Wc, W, sizeof(double) * P);
        /* momentary surprise: gradient of the associative loss at M_{t'} */
        mem_grad(n, Wc, k + (int64_t)t * d, v + (int64_t)t * d, g, w.z, w.a, w.delta, w.delta_prev);
        double a_t = alpha[t], e_t = eta[t], th_t = theta[t];
        for (int64_t p = 0; p < P; ++p) S[p] = e_t * S[p] - th_t * g[p];      /* surprise momentum */
        for (int64_t p = 0; p < P; ++p) W[p] = (1.0 - a_t) * W[p] + S[p];     /* forget-gated write */
        /* retrieval: forward pass on the query, weights unchanged */
        mem_forward(n, read_mode == 1 ? Wc : W, q + (int64_t)t * d, w.z, w.a);
        memcpy(y + (int64_t)t * d, w.a[n->L], sizeof(double) * d);
        if (w_norm && ((t + 1) % chunk == 0 || t == N - 1)) {
            double s2 = 0.0;
            for (int64_t p = 0; p < P; ++p) s2 += W[p] * W[p];
            w_norm[t / chunk] = sqrt(s2);
        }
    }
    memcpy(W_out, W, sizeof(double) * P);
    memcpy(S_out, S, sizeof(double) * P);
    work_free(&w);
done:
    free(W); free(S); free(Wc); free(g);
    return rc;
}

/*
 * Chunked memory over `streams` independent (batch, head) streams.
 *   k, v, q, y:          [streams, N, d]
 *   alpha, eta, theta:   [streams, N]
 *   W_in, S_in, W_out, S_out: [streams, P]
 *   w_norm (optional):   [streams, ceil(N / chunk)], ||W||_F after each chunk
 * Returns 0, -1 for bad arguments, -2 for allocation failure.
 */
int tmo_forward(int streams, int N, int d, int hidden, int n_layers, int chunk, int read_mode,
                const double* k, const double* v, const double* q,
                const double* alpha, const double* eta, const double* theta,
                const double* W_in, const double* S_in,
                double* y, double* W_out, double* S_out, double* w_norm, int n_threads) {
    net_t n;
    if (net_init(&n, d, hidden, n_layers)) return -1;
    if (streams < 0 || N < 0 || chunk <= 0 || (read_mode != 0 && read_mode != 1)) return -1;
    int64_t P = n.P;
    int64_t n_chunks = (N + chunk - 1) / chunk;
    int rc = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(min : rc)
    for (int s = 0; s < streams; ++s) {
        int r = run_stream(&n, N, chunk, read_mode,
                           k + (int64_t)s * N * d, v + (int64_t)s * N * d, q + (int64_t)s * N * d,
                           alpha + (int64_t)s * N, eta + (int64_t)s * N, theta + (int64_t)s * N,
                           W_in + s * P, S_in + s * P,
                           y + (int64_t)s * N * d, W_out + s * P, S_out + s * P,
                           w_norm ? w_norm + s * n_chunks : NULL);
        if (r < rc) rc = r;
    }
    return rc;
}

int tmo_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
