/*
 * oracle.c - plain, slow, double-precision CPU oracle for the selective
 * state-space scan (the S6 core of Mamba) and its two vision variants.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load this; the library's product path never does, and
 * this file shares no code, header or table with the HIP kernels.
 *
 * Passages followed (page title, then section):
 *  [MS] "Mamba Series from Selective State Spaces to Visual State Space Models"
 *       - section "选择性 SSM 的数学形式" (mathematical form of the selective SSM):
 *         continuous system h' = A h + B x, y = C h; zero-order-hold discretisation
 *         Abar = exp(dA), Bbar = (dA)^-1 (exp(dA) - I) dB; selection
 *         delta = softplus(W x + b), B = W_B x, C = W_C x, A a fixed diagonal.
 *       - section "关键代码" (key code), cross_scan_fwd and SS2Dv0.forwardv0: the four
 *         scan orders (row-major, column-major and the reversal of each), the scan
 *         call with per-direction A, Ds, delta_bias and delta_softplus, the merge of the
 *         four outputs back to pixel order by flip / transpose and sum, the SiLU gate.
 *       - section "核心洞察", insight 1: the time-varying recurrence is evaluated as a
 *         scan (here: the plain sequential recurrence, which the parallel scan
 *         reassociates).
 *  [LM] "从LSTM到Mamba：双向状态空间模型如何重塑视觉序列建模"
 *       - §2.1: h' = A h + B x, y = C h + D x (the D skip term).
 *       - §3.1: bidirectional SSM, a forward scan and a scan over reverse(x).
 *
 * Readings where the pages are silent or disagree (each listed in the design notes):
 *  - Bbar: the default is Bbar = delta * B (Euler; what the workload statement uses);
 *    zoh != 0 selects the [MS] zero-order-hold Bbar = expm1(delta*A)/A * B (delta*B at A = 0),
 *    in the forward and in the backward (input_coef).
 *  - initial state is zero unless h0 is given; D, z, delta_bias may be absent.
 *  - bidirectional fusion is the SUM of the forward output and the backward output
 *    re-reversed to token order (the page concatenates); one gate on the sum.
 *  - SS2D per-direction delta, B, C are stored in pixel order; direction k visits pixel
 *    pi_k(l) at scan step l (see ss2d_pixel below); outputs are added at the same pixel.
 *
 * Every function returns 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---- scalar helpers ---------------------------------------------------- */

/* softplus(w) = log(1 + e^w), written so that neither branch overflows. */
static double softplus(double w) { return w > 0.0 ? w + log1p(exp(-w)) : log1p(exp(w)); }

/* silu(z) = z * sigmoid(z); sigmoid evaluated on the side where exp cannot overflow. */
static double silu(double z) {
    if (z >= 0.0) return z / (1.0 + exp(-z));
    double e = exp(z);
    return z * e / (1.0 + e);
}

/* ---- one direction of the scan over [batch][L][dim] --------------------- */

typedef struct {
    const double *x, *delta, *A, *B, *C, *D, *delta_bias, *h0;
    double *y_pre; /* sum_n C h + D x, before any gate */
    double *h_last;
    int64_t batch, L, dim, N;
    int softplus, zoh;
} scan_t;

/* The recurrence for stream (b, d), in the order the method writes it:
 *   delta_t = softplus(delta[b,t,d] + bias[d])           (when enabled)
 *   h_t[n]  = exp(delta_t A[d,n]) h_{t-1}[n] + Bbar_t[n] x[b,t,d]
 *   y_t     = sum_n C[b,t,n] h_t[n] + D[d] x[b,t,d]                              */
static void scan_stream(const scan_t *s, int64_t b, int64_t d, double *h) {
    const int64_t N = s->N, dim = s->dim, L = s->L;
    for (int64_t n = 0; n < N; ++n) h[n] = s->h0 ? s->h0[(b * dim + d) * N + n] : 0.0;
    const double Dd = s->D ? s->D[d] : 0.0;
    const double *Arow = s->A + d * N;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t i = (b * L + t) * dim + d;
        double dt = s->delta[i];
        if (s->delta_bias) dt += s->delta_bias[d];
        if (s->softplus) dt = softplus(dt);
        const double xv = s->x[i];
        const double *Bt = s->B + (b * L + t) * N;
        const double *Ct = s->C + (b * L + t) * N;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a = Arow[n];
            const double Abar = exp(dt * a);
            double Bbar;
            if (s->zoh)
                Bbar = (a != 0.0 ? expm1(dt * a) / a : dt) * Bt[n];
            else
                Bbar = dt * Bt[n];
            h[n] = Abar * h[n] + Bbar * xv;
            acc += Ct[n] * h[n];
        }
        s->y_pre[i] = acc + Dd * xv;
    }
    if (s->h_last)
        for (int64_t n = 0; n < N; ++n) s->h_last[(b * dim + d) * N + n] = h[n];
}

typedef struct {
    const scan_t *s;
    int64_t first, last; /* stream range [first, last) over batch*dim */
} job_t;

static void *scan_worker(void *p) {
    const job_t *j = (const job_t *)p;
    double *h = (double *)malloc(sizeof(double) * (size_t)j->s->N);
    if (!h) return (void *)1;
    for (int64_t q = j->first; q < j->last; ++q) scan_stream(j->s, q / j->s->dim, q % j->s->dim, h);
    free(h);
    return NULL;
}

static int resolve_threads(int nthreads, int64_t streams) {
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 0 ? (int)c : 1;
    }
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > streams) nthreads = (int)(streams > 0 ? streams : 1);
    return nthreads;
}

static int run_scan(const scan_t *s, int nthreads) {
    const int64_t streams = s->batch * s->dim;
    if (streams == 0 || s->L == 0) {
        if (s->h_last && s->L == 0)
            for (int64_t q = 0; q < streams * s->N; ++q) s->h_last[q] = s->h0 ? s->h0[q] : 0.0;
        return 0;
    }
    nthreads = resolve_threads(nthreads, streams);
    pthread_t tid[256];
    int live[256];
    job_t jobs[256];
    int rc = 0;
    for (int k = 0; k < nthreads; ++k) {
        jobs[k].s = s;
        jobs[k].first = streams * k / nthreads;
        jobs[k].last = streams * (k + 1) / nthreads;
        live[k] = 0;
    }
    /* threads 1..n-1 run in the background, share 0 runs here; a thread that cannot be
     * started has its share run here too */
    for (int k = 1; k < nthreads; ++k) live[k] = pthread_create(&tid[k], NULL, scan_worker, &jobs[k]) == 0;
    if (scan_worker(&jobs[0])) rc = -1;
    for (int k = 1; k < nthreads; ++k) {
        void *ret = NULL;
        if (live[k]) {
            if (pthread_join(tid[k], &ret) != 0 || ret) rc = -1;
        } else if (scan_worker(&jobs[k])) {
            rc = -1;
        }
    }
    return rc;
}

static int bad_common(const void *x, const void *delta, const void *A, const void *B, const void *C,
                      const void *y, int64_t batch, int64_t L, int64_t dim, int64_t N) {
    return !x || !delta || !A || !B || !C || !y || batch < 0 || L < 0 || dim < 0 || N <= 0;
}

/* ---- public entry points ------------------------------------------------ */

/* Single-direction scan.  x, delta, z, y: [batch][L][dim]; B, C: [batch][L][N];
 * A: [dim][N]; D, delta_bias: [dim]; h0, h_last: [batch][dim][N].  D, z, delta_bias,
 * h0, h_last may be NULL.  y = (sum_n C h + D x) * silu(z), the gate only if z is given. */
int oracle_selscan(const double *x, const double *delta, const double *A, const double *B, const double *C,
                   const double *D, const double *z, const double *delta_bias, int delta_softplus, int zoh,
                   const double *h0, double *h_last, double *y, int64_t batch, int64_t L, int64_t dim,
                   int64_t N, int nthreads) {
    if (bad_common(x, delta, A, B, C, y, batch, L, dim, N)) return -1;
    scan_t s = {x, delta, A, B, C, D, delta_bias, h0, y, h_last, batch, L, dim, N, delta_softplus, zoh};
    if (run_scan(&s, nthreads)) return -1;
    if (z) {
        const int64_t tot = batch * L * dim;
        for (int64_t i = 0; i < tot; ++i) y[i] *= silu(z[i]);
    }
    return 0;
}

/* reverse the time axis of a [batch][L][w] array into out */
static void reverse_time(const double *in, double *out, int64_t batch, int64_t L, int64_t w) {
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t t = 0; t < L; ++t)
            memcpy(out + (b * L + t) * w, in + (b * L + (L - 1 - t)) * w, sizeof(double) * (size_t)w);
}

/* Bidirectional scan ([LM] §3.1).  delta, B, C, A, D, delta_bias carry a leading
 * direction axis of 2: [0] forward, [1] backward; all per-token arrays are in token
 * order.  Direction 1 is the same scan run over the time-reversed sequence with its own
 * parameters; its output is reversed back to token order and added to direction 0's.
 * y = (y_fwd + y_bwd) * silu(z).                                                        */
int oracle_selscan_bidir(const double *x, const double *delta, const double *A, const double *B,
                         const double *C, const double *D, const double *z, const double *delta_bias,
                         int delta_softplus, int zoh, double *y, int64_t batch, int64_t L, int64_t dim,
                         int64_t N, int nthreads) {
    if (bad_common(x, delta, A, B, C, y, batch, L, dim, N)) return -1;
    const int64_t tok = batch * L * dim, bc = batch * L * N;
    int rc = 0;
    double *yf = (double *)malloc(sizeof(double) * (size_t)(tok ? tok : 1));
    double *xr = (double *)malloc(sizeof(double) * (size_t)(tok ? tok : 1));
    double *dr = (double *)malloc(sizeof(double) * (size_t)(tok ? tok : 1));
    double *yr = (double *)malloc(sizeof(double) * (size_t)(tok ? tok : 1));
    double *Br = (double *)malloc(sizeof(double) * (size_t)(bc ? bc : 1));
    double *Cr = (double *)malloc(sizeof(double) * (size_t)(bc ? bc : 1));
    if (!yf || !xr || !dr || !yr || !Br || !Cr) { rc = -1; goto done; }
    {
        /* forward direction, in token order */
        scan_t f = {x, delta, A, B, C, D, delta_bias, NULL, yf, NULL, batch, L, dim, N, delta_softplus, zoh};
        if (run_scan(&f, nthreads)) { rc = -1; goto done; }
        /* backward direction: reverse(x) and direction-1 parameters reversed */
        reverse_time(x, xr, batch, L, dim);
        reverse_time(delta + tok, dr, batch, L, dim);
        reverse_time(B + bc, Br, batch, L, N);
        reverse_time(C + bc, Cr, batch, L, N);
        scan_t r = {xr, dr, A + dim * N, Br, Cr, D ? D + dim : NULL, delta_bias ? delta_bias + dim : NULL,
                    NULL, yr, NULL, batch, L, dim, N, delta_softplus, zoh};
        if (run_scan(&r, nthreads)) { rc = -1; goto done; }
        reverse_time(yr, y, batch, L, dim); /* back to token order */
        for (int64_t i = 0; i < tok; ++i) y[i] += yf[i];
        if (z)
            for (int64_t i = 0; i < tok; ++i) y[i] *= silu(z[i]);
    }
done:
    free(yf); free(xr); free(dr); free(yr); free(Br); free(Cr);
    return rc;
}

/* Pixel visited at scan step l by direction k on an H x W map stored row-major
 * (pixel p = h*W + w, L = H*W), as the [MS] cross-scan builds the sequences:
 *   k = 0: row-major flatten                      -> p = l
 *   k = 1: transpose(H, W) then flatten           -> l = w*H + h, so p = (l % H)*W + l / H
 *   k = 2: k = 0 flipped along the sequence       -> step L-1-l of k = 0
 *   k = 3: k = 1 flipped along the sequence       -> step L-1-l of k = 1                    */
static int64_t ss2d_pixel(int k, int64_t l, int64_t H, int64_t W) {
    const int64_t L = H * W;
    if (k >= 2) l = L - 1 - l;
    if (k == 0 || k == 2) return l;
    return (l % H) * W + l / H;
}

/* Pixel visited at scan step l by direction k of the windowed cross-scan on an H x W map cut
 * into square windows of side w (w divides H and W): [DP] LocalMamba, the image is divided
 * into windows and the selective scan runs inside each window.  The pages give no more, so
 * the reading is the SS2D cross-scan with windows:
 *   k = 0: windows in row-major order, the pixels of each window in row-major order;
 *   k = 1: the same on the transposed map (windows and pixels column-major);
 *   k = 2, 3: k = 0, 1 reversed.
 * With w = 1, or one window (w = H = W), this is the SS2D cross-scan.                        */
static void win_rowmajor(int64_t l, int64_t Ww, int64_t w, int64_t *row, int64_t *col) {
    const int64_t per = w * w, nwx = Ww / w;
    const int64_t wi = l / per, r = l % per;
    *row = (wi / nwx) * w + r / w;
    *col = (wi % nwx) * w + r % w;
}

static int64_t local_pixel(int k, int64_t l, int64_t H, int64_t W, int64_t w) {
    const int64_t L = H * W;
    int64_t r, c;
    if (k >= 2) l = L - 1 - l;
    if (k == 0 || k == 2) {
        win_rowmajor(l, W, w, &r, &c);
        return r * W + c;
    }
    win_rowmajor(l, H, w, &r, &c); /* on the transposed (W x H) map: its row r is column r here */
    return c * W + r;
}

/* SS2D four-direction scan with merge ([MS] cross_scan_fwd, SS2Dv0.forwardv0).
 * x, z, y: [batch][H*W][dim] (pixels row-major); delta: [4][batch][H*W][dim];
 * B, C: [4][batch][H*W][N]; A: [4][dim][N]; D, delta_bias: [4][dim].  Per-direction
 * arrays are in pixel order.  For each direction k the sequence of pixels pi_k(0..L-1)
 * is gathered, scanned with direction k's parameters, and each output is added at the
 * pixel it came from.  The page gates after a normalisation outside the scan, so z is
 * normally absent; if given, it gates the merged sum.                                    */
static int cross_scan(const double *x, const double *delta, const double *A, const double *B, const double *C,
                      const double *D, const double *z, const double *delta_bias, int delta_softplus, int zoh,
                      double *y, int64_t batch, int64_t H, int64_t W, int64_t win, int64_t dim, int64_t N,
                      int nthreads) {
    if (H < 0 || W < 0) return -1;
    const int64_t L = H * W;
    if (bad_common(x, delta, A, B, C, y, batch, L, dim, N)) return -1;
    const int64_t tok = batch * L * dim, bc = batch * L * N;
    int rc = 0;
    double *xs = (double *)malloc(sizeof(double) * (size_t)(tok ? tok : 1));
    double *ds = (double *)malloc(sizeof(double) * (size_t)(tok ? tok : 1));
    double *os = (double *)malloc(sizeof(double) * (size_t)(tok ? tok : 1));
    double *Bs = (double *)malloc(sizeof(double) * (size_t)(bc ? bc : 1));
    double *Cs = (double *)malloc(sizeof(double) * (size_t)(bc ? bc : 1));
    if (!xs || !ds || !os || !Bs || !Cs) { rc = -1; goto done; }
    for (int64_t i = 0; i < tok; ++i) y[i] = 0.0;
    for (int k = 0; k < 4; ++k) {
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t l = 0; l < L; ++l) {
                const int64_t p = win ? local_pixel(k, l, H, W, win) : ss2d_pixel(k, l, H, W);
                memcpy(xs + (b * L + l) * dim, x + (b * L + p) * dim, sizeof(double) * (size_t)dim);
                memcpy(ds + (b * L + l) * dim, delta + k * tok + (b * L + p) * dim, sizeof(double) * (size_t)dim);
                memcpy(Bs + (b * L + l) * N, B + k * bc + (b * L + p) * N, sizeof(double) * (size_t)N);
                memcpy(Cs + (b * L + l) * N, C + k * bc + (b * L + p) * N, sizeof(double) * (size_t)N);
            }
        scan_t s = {xs, ds, A + k * dim * N, Bs, Cs, D ? D + k * dim : NULL,
                    delta_bias ? delta_bias + k * dim : NULL, NULL, os, NULL, batch, L, dim, N,
                    delta_softplus, zoh};
        if (run_scan(&s, nthreads)) { rc = -1; goto done; }
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t l = 0; l < L; ++l) {
                const int64_t p = win ? local_pixel(k, l, H, W, win) : ss2d_pixel(k, l, H, W);
                for (int64_t d = 0; d < dim; ++d) y[(b * L + p) * dim + d] += os[(b * L + l) * dim + d];
            }
    }
    if (z)
        for (int64_t i = 0; i < tok; ++i) y[i] *= silu(z[i]);
done:
    free(xs); free(ds); free(os); free(Bs); free(Cs);
    return rc;
}

int oracle_ss2d(const double *x, const double *delta, const double *A, const double *B, const double *C,
                const double *D, const double *z, const double *delta_bias, int delta_softplus, int zoh,
                double *y, int64_t batch, int64_t H, int64_t W, int64_t dim, int64_t N, int nthreads) {
    return cross_scan(x, delta, A, B, C, D, z, delta_bias, delta_softplus, zoh, y, batch, H, W, 0, dim, N,
                      nthreads);
}

/* Windowed (local) four-direction scan with merge: as oracle_ss2d, with local_pixel's orders
 * for window side win (win >= 1 dividing H and W).                                        */
int oracle_local_ss2d(const double *x, const double *delta, const double *A, const double *B, const double *C,
                      const double *D, const double *z, const double *delta_bias, int delta_softplus, int zoh,
                      double *y, int64_t batch, int64_t H, int64_t W, int64_t win, int64_t dim, int64_t N,
                      int nthreads) {
    if (win < 1 || H % win || W % win) return -1;
    return cross_scan(x, delta, A, B, C, D, z, delta_bias, delta_softplus, zoh, y, batch, H, W, win, dim, N,
                      nthreads);
}

/* The pixel (token) each direction visits at each scan step, as the scans above use it:
 * kind 1 bidirectional (k = 0, 1), 2 SS2D (k = 0..3), 3 windowed cross-scan (k = 0..3,
 * window win).  Fills order[l], l = 0..L-1, for direction k; returns -1 on a bad argument. */
int oracle_scan_order(int kind, int k, int64_t H, int64_t W, int64_t win, int64_t L, int64_t *order) {
    if (!order || L < 0) return -1;
    for (int64_t l = 0; l < L; ++l) {
        if (kind == 1) {
            if (k < 0 || k > 1) return -1;
            order[l] = k == 0 ? l : L - 1 - l;
        } else if (kind == 2) {
            if (k < 0 || k > 3 || H * W != L) return -1;
            order[l] = ss2d_pixel(k, l, H, W);
        } else if (kind == 3) {
            if (k < 0 || k > 3 || H * W != L || win < 1 || H % win || W % win) return -1;
            order[l] = local_pixel(k, l, H, W, win);
        } else {
            return -1;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------
 * The convolution in front of the scan.
 *  [MS] "Mamba Series ...", section 方法设计 (architecture diagram): in the Mamba block the
 *       scan's input branch is Linear -> Conv1D(k=4) -> SiLU -> SSM; in the VSS block it is
 *       Linear -> DWConv 3x3 -> SiLU -> SS2D (also SS2Dv0.forwardv0 in section 关键代码:
 *       conv2d, then act).
 * Readings (the pages give only the kernel sizes): the 1-D convolution is depthwise (one
 * filter per channel, as the 2-D one is named) and causal, the output at step t seeing
 * inputs t-(K-1) .. t with zeros (or a carried state) before the sequence; the 2-D one keeps
 * the map size (zero padding (ks-1)/2, stride 1) and, like the framework layers the code
 * calls, is a cross-correlation; both add a per-channel bias when one is given.
 * --------------------------------------------------------------------------------- */

/* out[b,t,d] = act(bias[d] + sum_{i<K} w[d*K+i] * xin(b, t-(K-1)+i, d)), act = silu or identity,
 * xin(b,s,d) = x[b,s,d] for s >= 0 and, for -(K-1) <= s < 0, state_in[b][K-1+s][d] (zero when
 * state_in is NULL).  state_out [batch][K-1][dim], if given, receives the last K-1 rows of
 * (state_in rows ++ x rows).  Layout [batch][L][dim]; w [dim][K]. */
int oracle_causal_conv1d(const double *x, const double *w, const double *bias, const double *state_in,
                         double *state_out, int silu_, double *out, int64_t batch, int64_t L, int64_t dim,
                         int64_t K) {
    if (batch < 0 || L < 0 || dim < 0 || K < 1 || !w || (L > 0 && (!x || !out))) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            for (int64_t t = 0; t < L; ++t) {
                double v = bias ? bias[d] : 0.0;
                for (int64_t i = 0; i < K; ++i) {
                    const int64_t s = t - (K - 1) + i;
                    double xv = 0.0;
                    if (s >= 0) xv = x[(b * L + s) * dim + d];
                    else if (state_in) xv = state_in[(b * (K - 1) + (K - 1) + s) * dim + d];
                    v += w[d * K + i] * xv;
                }
                out[(b * L + t) * dim + d] = silu_ ? silu(v) : v;
            }
            if (state_out) {
                for (int64_t r = 0; r < K - 1; ++r) {
                    const int64_t s = L - (K - 1) + r; /* row of the concatenation, relative to x */
                    double xv = 0.0;
                    if (s >= 0) xv = x[(b * L + s) * dim + d];
                    else if (state_in) xv = state_in[(b * (K - 1) + (K - 1) + s) * dim + d];
                    state_out[(b * (K - 1) + r) * dim + d] = xv;
                }
            }
        }
    }
    return 0;
}

/* out[b,h,w,d] = act(bias[d] + sum_{i,j<ks} wt[(d*ks+i)*ks+j] * x[b, h+i-p, w+j-p, d]), p = (ks-1)/2,
 * x read as zero outside the H x W map.  Layout [batch][H][W][dim]; wt [dim][ks][ks]; ks odd. */
int oracle_dwconv2d(const double *x, const double *wt, const double *bias, int silu_, double *out, int64_t batch,
                    int64_t H, int64_t W, int64_t dim, int64_t ks) {
    if (batch < 0 || H < 0 || W < 0 || dim < 0 || ks < 1 || ks % 2 == 0 || !wt) return -1;
    if (batch * H * W > 0 && (!x || !out)) return -1;
    const int64_t p = (ks - 1) / 2;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t w = 0; w < W; ++w)
                for (int64_t d = 0; d < dim; ++d) {
                    double v = bias ? bias[d] : 0.0;
                    for (int64_t i = 0; i < ks; ++i) {
                        const int64_t hh = h + i - p;
                        if (hh < 0 || hh >= H) continue;
                        for (int64_t j = 0; j < ks; ++j) {
                            const int64_t ww = w + j - p;
                            if (ww < 0 || ww >= W) continue;
                            v += wt[(d * ks + i) * ks + j] * x[((b * H + hh) * W + ww) * dim + d];
                        }
                    }
                    out[((b * H + h) * W + w) * dim + d] = silu_ ? silu(v) : v;
                }
    return 0;
}

/* number of hardware threads the oracle would use for nthreads <= 0 */
int oracle_default_threads(void) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c > 0 ? (int)c : 1;
}

/* ---- backward of the single-direction scan ------------------------------ */

/* sigmoid without overflow on either side */
static double sigmoid(double z) {
    if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

typedef struct {
    const double *x, *delta, *A, *B, *C, *D, *z, *delta_bias, *h0, *dy;
    double *dx, *ddelta, *dz, *dh0;           /* per stream: written by the stream's thread */
    int64_t batch, L, dim, N;
    int softplus, zoh;
} bwd_t;

/* The input coefficient of one step and its two partial derivatives.  Euler: beta = delta.
 * Zero-order hold ([MS] "选择性 SSM 的数学形式"): beta = (exp(delta a) - 1) / a, i.e.
 * delta * phi(y) with y = delta a and phi(y) = (e^y - 1) / y (beta = delta at a = 0).  Then
 *   d beta / d delta = e^y
 *   d beta / d a     = delta^2 phi'(y),  phi'(y) = (e^y (y - 1) + 1) / y^2
 *                                                = sum_k (k + 1) y^k / (k + 2)!
 * (the series near y = 0, where the closed form cancels; 1/2 at y = 0).                  */
static void input_coef(int zoh, double dt, double a, double *beta, double *dbeta_ddt, double *dbeta_da) {
    if (!zoh) {
        *beta = dt;
        *dbeta_ddt = 1.0;
        *dbeta_da = 0.0;
        return;
    }
    const double y = dt * a;
    *beta = a != 0.0 ? expm1(y) / a : dt;
    *dbeta_ddt = exp(y);
    double dphi;
    if (fabs(y) < 0.5) {
        double term = 1.0, fact = 2.0; /* y^k and (k + 2)! */
        dphi = 0.0;
        for (int k = 0; k < 30; ++k) {
            dphi += (k + 1) * term / fact;
            term *= y;
            fact *= k + 3;
        }
    } else {
        dphi = (exp(y) * (y - 1.0) + 1.0) / (y * y);
    }
    *dbeta_da = dt * dt * dphi;
}

typedef struct {
    const bwd_t *s;
    int64_t first, last;
    double *dB, *dC;   /* [batch][L][N] private partial sums */
    double *dA;        /* [dim][N] */
    double *dD, *dbias;/* [dim] */
    double *h;         /* (L + 1) x N states of one stream */
    double *dt, *w;    /* L: delta_t after bias/softplus, and its pre-softplus argument */
    int failed;
} bwd_job_t;

/* Reverse-mode derivative of the recurrence of scan_stream, for stream (b, d), given dL/dy.
 * The forward is rerun and every state kept; then, from t = L-1 down to 0, with g[n] the
 * derivative of L with respect to h_t[n]:
 *   y_t = yp_t * silu(z_t), yp_t = sum_n C_t[n] h_t[n] + D x_t
 *   h_t[n] = e_t[n] h_{t-1}[n] + beta_t[n] B_t[n] x_t,   e_t[n] = exp(delta_t A[n])
 * (beta = delta for Euler, the zero-order-hold coefficient otherwise; input_coef) so
 * g_t += C_t dyp_t;  then the parameters of step t take their share of g_t and
 * g_{t-1} = e_t g_t.                                                                       */
static void bwd_stream(bwd_job_t *j, int64_t b, int64_t d) {
    const bwd_t *s = j->s;
    const int64_t N = s->N, dim = s->dim, L = s->L;
    double *h = j->h; /* h + (t + 1) * N holds h_t; h holds h_{-1} */
    for (int64_t n = 0; n < N; ++n) h[n] = s->h0 ? s->h0[(b * dim + d) * N + n] : 0.0;
    const double Dd = s->D ? s->D[d] : 0.0;
    const double *Arow = s->A + d * N;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t i = (b * L + t) * dim + d;
        double w = s->delta[i];
        if (s->delta_bias) w += s->delta_bias[d];
        const double dt = s->softplus ? softplus(w) : w;
        j->w[t] = w;
        j->dt[t] = dt;
        const double xv = s->x[i];
        const double *Bt = s->B + (b * L + t) * N;
        for (int64_t n = 0; n < N; ++n) {
            double beta, dbdt, dbda;
            input_coef(s->zoh, dt, Arow[n], &beta, &dbdt, &dbda);
            h[(t + 1) * N + n] = exp(dt * Arow[n]) * h[t * N + n] + beta * Bt[n] * xv;
        }
    }
    double *g = (double *)calloc((size_t)N, sizeof(double));
    if (!g) { j->failed = 1; return; }
    for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t i = (b * L + t) * dim + d;
        const double xv = s->x[i], dt = j->dt[t];
        const double *Bt = s->B + (b * L + t) * N;
        const double *Ct = s->C + (b * L + t) * N;
        const double *ht = h + (t + 1) * N, *hp = h + t * N;
        double yp = Dd * xv;
        for (int64_t n = 0; n < N; ++n) yp += Ct[n] * ht[n];
        double dyp = s->dy[i];
        if (s->z) {
            const double zv = s->z[i], sg = sigmoid(zv);
            if (s->dz) s->dz[i] = s->dy[i] * yp * sg * (1.0 + zv * (1.0 - sg));
            dyp = s->dy[i] * zv * sg;
        }
        j->dD[d] += dyp * xv;
        double dxv = Dd * dyp, ddt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            g[n] += Ct[n] * dyp;
            j->dC[(b * L + t) * N + n] += dyp * ht[n];
            const double e = exp(dt * Arow[n]);
            double beta, dbdt, dbda;
            input_coef(s->zoh, dt, Arow[n], &beta, &dbdt, &dbda);
            ddt += g[n] * (Arow[n] * e * hp[n] + dbdt * Bt[n] * xv);
            j->dA[d * N + n] += g[n] * (dt * e * hp[n] + dbda * Bt[n] * xv);
            j->dB[(b * L + t) * N + n] += g[n] * beta * xv;
            dxv += g[n] * beta * Bt[n];
            g[n] *= e;
        }
        s->dx[i] = dxv;
        const double dw = s->softplus ? ddt * sigmoid(j->w[t]) : ddt;
        s->ddelta[i] = dw;
        j->dbias[d] += dw;
    }
    if (s->dh0)
        for (int64_t n = 0; n < N; ++n) s->dh0[(b * dim + d) * N + n] = g[n];
    free(g);
}

static void *bwd_worker(void *p) {
    bwd_job_t *j = (bwd_job_t *)p;
    for (int64_t q = j->first; q < j->last && !j->failed; ++q) bwd_stream(j, q / j->s->dim, q % j->s->dim);
    return NULL;
}

/* Backward of oracle_selscan (Euler Bbar, or the zero-order hold when zoh != 0).  Inputs as
 * for oracle_selscan plus dy [batch][L][dim].  Outputs: dx, ddelta [batch][L][dim] (derivative
 * with respect to the delta argument, before bias and softplus); dA [dim][N]; dB, dC
 * [batch][L][N]; dD, ddelta_bias [dim]; dz [batch][L][dim]; dh0 [batch][dim][N].  dx,
 * ddelta, dA, dB, dC are required; dD, dz, ddelta_bias, dh0 may be NULL (not written).    */
int oracle_selscan_bwd(const double *x, const double *delta, const double *A, const double *B,
                       const double *C, const double *D, const double *z, const double *delta_bias,
                       int delta_softplus, int zoh, const double *h0, const double *dy, double *dx, double *ddelta,
                       double *dA, double *dB, double *dC, double *dD, double *dz, double *ddelta_bias,
                       double *dh0, int64_t batch, int64_t L, int64_t dim, int64_t N, int nthreads) {
    if (bad_common(x, delta, A, B, C, dy, batch, L, dim, N) || !dx || !ddelta || !dA || !dB || !dC) return -1;
    const int64_t streams = batch * dim, bc = batch * L * N;
    memset(dA, 0, sizeof(double) * (size_t)(dim * N));
    memset(dB, 0, sizeof(double) * (size_t)bc);
    memset(dC, 0, sizeof(double) * (size_t)bc);
    if (dD) memset(dD, 0, sizeof(double) * (size_t)dim);
    if (ddelta_bias) memset(ddelta_bias, 0, sizeof(double) * (size_t)dim);
    if (dh0) {
        for (int64_t q = 0; q < streams * N; ++q) dh0[q] = 0.0;
    }
    if (streams == 0 || L == 0) return 0;
    bwd_t s = {x, delta, A, B, C, D, z, delta_bias, h0, dy, dx, ddelta, dz, dh0, batch, L, dim, N,
               delta_softplus, zoh};
    nthreads = resolve_threads(nthreads, streams);
    bwd_job_t jobs[256];
    pthread_t tid[256];
    int live[256];
    int rc = 0;
    for (int k = 0; k < nthreads; ++k) {
        bwd_job_t *j = &jobs[k];
        memset(j, 0, sizeof(*j));
        j->s = &s;
        j->first = streams * k / nthreads;
        j->last = streams * (k + 1) / nthreads;
        j->dB = (double *)calloc((size_t)bc, sizeof(double));
        j->dC = (double *)calloc((size_t)bc, sizeof(double));
        j->dA = (double *)calloc((size_t)(dim * N), sizeof(double));
        j->dD = (double *)calloc((size_t)dim, sizeof(double));
        j->dbias = (double *)calloc((size_t)dim, sizeof(double));
        j->h = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));
        j->dt = (double *)malloc(sizeof(double) * (size_t)L);
        j->w = (double *)malloc(sizeof(double) * (size_t)L);
        if (!j->dB || !j->dC || !j->dA || !j->dD || !j->dbias || !j->h || !j->dt || !j->w) j->failed = 1;
    }
    for (int k = 1; k < nthreads; ++k) live[k] = !jobs[k].failed && pthread_create(&tid[k], NULL, bwd_worker, &jobs[k]) == 0;
    if (!jobs[0].failed) bwd_worker(&jobs[0]);
    for (int k = 1; k < nthreads; ++k) {
        if (live[k]) pthread_join(tid[k], NULL);
        else if (!jobs[k].failed) bwd_worker(&jobs[k]);
    }
    /* shared sums, added in a fixed thread order */
    for (int k = 0; k < nthreads; ++k) {
        bwd_job_t *j = &jobs[k];
        if (j->failed) rc = -1;
        if (!rc) {
            for (int64_t q = 0; q < bc; ++q) { dB[q] += j->dB[q]; dC[q] += j->dC[q]; }
            for (int64_t q = 0; q < dim * N; ++q) dA[q] += j->dA[q];
            for (int64_t q = 0; q < dim; ++q) {
                if (dD) dD[q] += j->dD[q];
                if (ddelta_bias) ddelta_bias[q] += j->dbias[q];
            }
        }
        free(j->dB); free(j->dC); free(j->dA); free(j->dD); free(j->dbias); free(j->h); free(j->dt); free(j->w);
    }
    return rc;
}

/* ---- backward of the convolutions -------------------------------------- */

/* d act / dv at v: silu'(v) = sigmoid(v) (1 + v (1 - sigmoid(v))), or 1 without the SiLU */
static double act_grad(int silu_, double v) {
    if (!silu_) return 1.0;
    const double s = sigmoid(v);
    return s * (1.0 + v * (1.0 - s));
}

/* Backward of oracle_causal_conv1d for dL/dout = dout.  Per (b, t, d) the pre-activation v is
 * recomputed and dv = dout act'(v); tap i read input row t-(K-1)+i of xin = state_in ++ x, so
 *   d xin[b, t-(K-1)+i, d] += w[d,i] dv,   dw[d,i] += xin[b, t-(K-1)+i, d] dv,   dbias[d] += dv.
 * The rows of xin before step 0 are state_in's: their derivative is dstate_in.  dx [batch][L][dim]
 * and dw [dim][K] are required; dbias [dim] and dstate_in [batch][K-1][dim] may be NULL.       */
int oracle_causal_conv1d_bwd(const double *x, const double *w, const double *bias, const double *state_in,
                             const double *dout, int silu_, double *dx, double *dw, double *dbias,
                             double *dstate_in, int64_t batch, int64_t L, int64_t dim, int64_t K) {
    if (batch < 0 || L < 0 || dim < 0 || K < 1 || !w || !dw || (L > 0 && (!x || !dout || !dx))) return -1;
    memset(dw, 0, sizeof(double) * (size_t)(dim * K));
    if (dbias) memset(dbias, 0, sizeof(double) * (size_t)dim);
    if (L > 0) memset(dx, 0, sizeof(double) * (size_t)(batch * L * dim));
    if (dstate_in) memset(dstate_in, 0, sizeof(double) * (size_t)(batch * (K - 1) * dim));
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < dim; ++d)
            for (int64_t t = 0; t < L; ++t) {
                double v = bias ? bias[d] : 0.0;
                for (int64_t i = 0; i < K; ++i) {
                    const int64_t s = t - (K - 1) + i;
                    double xv = 0.0;
                    if (s >= 0) xv = x[(b * L + s) * dim + d];
                    else if (state_in) xv = state_in[(b * (K - 1) + (K - 1) + s) * dim + d];
                    v += w[d * K + i] * xv;
                }
                const double dv = dout[(b * L + t) * dim + d] * act_grad(silu_, v);
                if (dbias) dbias[d] += dv;
                for (int64_t i = 0; i < K; ++i) {
                    const int64_t s = t - (K - 1) + i;
                    double xv = 0.0;
                    if (s >= 0) {
                        xv = x[(b * L + s) * dim + d];
                        dx[(b * L + s) * dim + d] += w[d * K + i] * dv;
                    } else {
                        if (state_in) xv = state_in[(b * (K - 1) + (K - 1) + s) * dim + d];
                        if (dstate_in) dstate_in[(b * (K - 1) + (K - 1) + s) * dim + d] += w[d * K + i] * dv;
                    }
                    dw[d * K + i] += xv * dv;
                }
            }
    return 0;
}

/* Backward of oracle_dwconv2d for dL/dout = dout: dv = dout act'(v) with v recomputed; tap (i, j)
 * of output pixel (h, w) read input pixel (h+i-p, w+j-p) when it lies in the map, so
 *   dx[b, h+i-p, w+j-p, d] += wt[d,i,j] dv,   dwt[d,i,j] += x[b, h+i-p, w+j-p, d] dv,   dbias[d] += dv.
 * dx and dwt are required, dbias may be NULL.                                                   */
int oracle_dwconv2d_bwd(const double *x, const double *wt, const double *bias, const double *dout, int silu_,
                        double *dx, double *dwt, double *dbias, int64_t batch, int64_t H, int64_t W, int64_t dim,
                        int64_t ks) {
    if (batch < 0 || H < 0 || W < 0 || dim < 0 || ks < 1 || ks % 2 == 0 || !wt || !dwt) return -1;
    if (batch * H * W > 0 && (!x || !dout || !dx)) return -1;
    const int64_t p = (ks - 1) / 2;
    memset(dwt, 0, sizeof(double) * (size_t)(dim * ks * ks));
    if (dbias) memset(dbias, 0, sizeof(double) * (size_t)dim);
    if (batch * H * W > 0) memset(dx, 0, sizeof(double) * (size_t)(batch * H * W * dim));
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t w = 0; w < W; ++w)
                for (int64_t d = 0; d < dim; ++d) {
                    double v = bias ? bias[d] : 0.0;
                    for (int64_t i = 0; i < ks; ++i) {
                        const int64_t hh = h + i - p;
                        if (hh < 0 || hh >= H) continue;
                        for (int64_t j = 0; j < ks; ++j) {
                            const int64_t ww = w + j - p;
                            if (ww < 0 || ww >= W) continue;
                            v += wt[(d * ks + i) * ks + j] * x[((b * H + hh) * W + ww) * dim + d];
                        }
                    }
                    const double dv = dout[((b * H + h) * W + w) * dim + d] * act_grad(silu_, v);
                    if (dbias) dbias[d] += dv;
                    for (int64_t i = 0; i < ks; ++i) {
                        const int64_t hh = h + i - p;
                        if (hh < 0 || hh >= H) continue;
                        for (int64_t j = 0; j < ks; ++j) {
                            const int64_t ww = w + j - p;
                            if (ww < 0 || ww >= W) continue;
                            const int64_t q = ((b * H + hh) * W + ww) * dim + d;
                            dx[q] += wt[(d * ks + i) * ks + j] * dv;
                            dwt[(d * ks + i) * ks + j] += x[q] * dv;
                        }
                    }
                }
    return 0;
}
