/*
 * ttt_oracle.c -- plain fp64 reference of the multi-head test-time-training
 * (TTT) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library; it consumes the exact (already quantised) inputs widened to
 * double and returns double results.
 *
 * Sources (the pages the method is described on):
 *  - "Vision-TTT: Efficient and Expressive Visual Representation Learning
 *    with Test-Time Training" (papernotes reading notes), section "关键设计"
 *    item 1: the L2 reconstruction loss l(W;x_t) = ||W x_t^K - x_t^V||^2,
 *    its gradient G_t = 2 (W x_t^K - x_t^V)(x_t^K)^T and the output
 *    z_t = W_t x_t^Q; item 2: the reversed ("dual") dataset t = T..1; item 4:
 *    per-head d x d states and mini-batches of b tokens with
 *    W_t = W_0 - eta * sum_{s<=t} G_s inside a batch; "一个完整示例": b = 16,
 *    ceil(196/16) = 13 steps per direction.
 *  - "CVPR 2026 Oral | ... ViT3" (ccvip repost), observation 2 (one
 *    full-batch step), observation 6 (depthwise 3x3 convolution as the inner
 *    model), observation 1 (end-to-end training differentiates the inner
 *    gradient: the "gradient of the gradient").
 *
 * Readings where the pages are silent (the kernels use the same ones):
 *  - full-batch loss is the token mean: L(W) = (1/N) sum_i ||W k_i - v_i||^2,
 *    so G = (2/N) sum_i (W0 k_i - v_i) k_i^T;
 *  - a mini-batch of n_c tokens scales each G_s by 1/n_c, gradients are taken
 *    at the batch-start state, and z_t uses the state after token t;
 *  - the reverse scan is the same procedure on the flipped sequence, its
 *    outputs are mapped back to their positions and the two directions are
 *    averaged (the trained gate is not modelled);
 *  - the token grid is row-major (n = y * grid_w + x); the depthwise kernel is
 *    a cross-correlation with zero padding, stride 1, no bias.
 *
 * Layouts: K, Q, V, Z, dZ, dK, dQ, dV are [B][H][N][d] contiguous;
 * W0 is [H][d][d] row-major with W[r][c] mapping input channel c to output
 * channel r (z = W q); w0 is [H][d][3][3]; eta is [H].
 *
 * Every function returns 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX4(b, h, n, c) ((((size_t)(b) * H + (h)) * N + (n)) * d + (c))

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * One full-batch gradient step of the linear inner model, then apply.
 *   r_i = W0 k_i - v_i                       (residual of the L2 loss)
 *   G   = (2/N) sum_i r_i k_i^T              (gradient of the mean loss)
 *   W1  = W0 - eta_h G
 *   z_i = W1 q_i
 * G_out (nullable) receives G per slice, [B][H][d][d].
 * ---------------------------------------------------------------------- */
int oracle_linear_fullbatch(int B, int H, int N, int d,
                            const double* K, const double* Q, const double* V,
                            const double* W0, const double* eta,
                            double* Z, double* G_out, int nthreads) {
    if (B < 0 || H < 0 || N <= 0 || d <= 0) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        int b = (int)(s / H), h = (int)(s % H);
        const double* W = W0 + (size_t)h * d * d;
        double* G = (double*)calloc((size_t)d * d, sizeof(double));
        double* W1 = (double*)malloc((size_t)d * d * sizeof(double));
        double* r = (double*)malloc((size_t)d * sizeof(double));
        for (int i = 0; i < N; ++i) {
            const double* k = K + IDX4(b, h, i, 0);
            const double* v = V + IDX4(b, h, i, 0);
            for (int o = 0; o < d; ++o) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += W[(size_t)o * d + c] * k[c];
                r[o] = acc - v[o];
            }
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c) G[(size_t)o * d + c] += r[o] * k[c];
        }
        for (size_t e = 0; e < (size_t)d * d; ++e) {
            G[e] *= 2.0 / (double)N;
            W1[e] = W[e] - eta[h] * G[e];
        }
        for (int i = 0; i < N; ++i) {
            const double* q = Q + IDX4(b, h, i, 0);
            double* z = Z + IDX4(b, h, i, 0);
            for (int o = 0; o < d; ++o) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += W1[(size_t)o * d + c] * q[c];
                z[o] = acc;
            }
        }
        if (G_out) memcpy(G_out + (size_t)s * d * d, G, (size_t)d * d * sizeof(double));
        free(G);
        free(W1);
        free(r);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Depthwise 3x3 convolution inner model, one full-batch step, then apply.
 * Per channel c on the grid (y, x), token n = y * gw + x, zero padding:
 *   P[y][x] = sum_{i,j in 0..2} w0[c][i][j] K[y+i-1][x+j-1]
 *   R       = P - V
 *   g[c][i][j] = (2/N) sum_{y,x} R[y][x] K[y+i-1][x+j-1]
 *   w1 = w0 - eta_h g ;  Z[y][x] = sum_{i,j} w1[c][i][j] Q[y+i-1][x+j-1]
 * g_out (nullable) receives g per slice, [B][H][d][3][3].
 * ---------------------------------------------------------------------- */
static double tap(const double* X, int H, int N, int d, int b, int h, int gh, int gw,
                  int y, int x, int c) {
    if (y < 0 || y >= gh || x < 0 || x >= gw) return 0.0;
    return X[IDX4(b, h, y * gw + x, c)];
}

int oracle_dwconv3x3_fullbatch(int B, int H, int gh, int gw, int d,
                               const double* K, const double* Q, const double* V,
                               const double* w0, const double* eta,
                               double* Z, double* g_out, int nthreads) {
    if (B < 0 || H < 0 || gh <= 0 || gw <= 0 || d <= 0) return -1;
    int N = gh * gw;
    set_threads(nthreads);
    long nwork = (long)B * H * d; /* each channel of each slice is independent */
#pragma omp parallel for schedule(dynamic, 4)
    for (long wkey = 0; wkey < nwork; ++wkey) {
        int c = (int)(wkey % d);
        long s = wkey / d;
        int b = (int)(s / H), h = (int)(s % H);
        const double* w = w0 + ((size_t)h * d + c) * 9;
        double g[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double p = 0.0;
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j)
                        p += w[i * 3 + j] * tap(K, H, N, d, b, h, gh, gw, y + i - 1, x + j - 1, c);
                double rr = p - V[IDX4(b, h, y * gw + x, c)];
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j)
                        g[i * 3 + j] += rr * tap(K, H, N, d, b, h, gh, gw, y + i - 1, x + j - 1, c);
            }
        double w1[9];
        for (int t = 0; t < 9; ++t) {
            g[t] *= 2.0 / (double)N;
            w1[t] = w[t] - eta[h] * g[t];
        }
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double z = 0.0;
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j)
                        z += w1[i * 3 + j] * tap(Q, H, N, d, b, h, gh, gw, y + i - 1, x + j - 1, c);
                Z[IDX4(b, h, y * gw + x, c)] = z;
            }
        if (g_out)
            for (int t = 0; t < 9; ++t) g_out[(((size_t)b * H + h) * d + c) * 9 + t] = g[t];
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Mini-batch scans.  Number of mini-batches of one scan direction:
 * ceil(N / b); the last one holds N - (nchunks-1)*b tokens.
 * ---------------------------------------------------------------------- */
int oracle_num_chunks(int N, int b) {
    if (N <= 0 || b <= 0) return -1;
    return (N + b - 1) / b;
}

/* One direction of one (b,h) chain, token by token, as the definition reads:
 * inside a mini-batch of n_c tokens with start state Ws,
 *   G_t  = (2/n_c) (Ws k_t - v_t) k_t^T
 *   acc += G_t ;  W_t = Ws - eta * acc ;  z_t = W_t q_t
 * and after the mini-batch Ws <- Ws - eta * acc.
 * reverse != 0 scans the flipped sequence (position N-1 first). */
static void scan_one(int N, int d, int bsz, int reverse, const double* K, const double* Q,
                     const double* V, const double* W0, double eta, double* Zout) {
    size_t dd = (size_t)d * d;
    double* Ws = (double*)malloc(dd * sizeof(double));
    double* acc = (double*)malloc(dd * sizeof(double));
    double* Wt = (double*)malloc(dd * sizeof(double));
    double* r = (double*)malloc((size_t)d * sizeof(double));
    memcpy(Ws, W0, dd * sizeof(double));
    for (int c0 = 0; c0 < N; c0 += bsz) {
        int nc = (N - c0 < bsz) ? (N - c0) : bsz;
        memset(acc, 0, dd * sizeof(double));
        for (int t = 0; t < nc; ++t) {
            int pos = reverse ? (N - 1 - (c0 + t)) : (c0 + t);
            const double* k = K + (size_t)pos * d;
            const double* v = V + (size_t)pos * d;
            const double* q = Q + (size_t)pos * d;
            for (int o = 0; o < d; ++o) {
                double a = 0.0;
                for (int c = 0; c < d; ++c) a += Ws[(size_t)o * d + c] * k[c];
                r[o] = a - v[o];
            }
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c)
                    acc[(size_t)o * d + c] += (2.0 / (double)nc) * r[o] * k[c];
            for (size_t e = 0; e < dd; ++e) Wt[e] = Ws[e] - eta * acc[e];
            double* z = Zout + (size_t)pos * d;
            for (int o = 0; o < d; ++o) {
                double a = 0.0;
                for (int c = 0; c < d; ++c) a += Wt[(size_t)o * d + c] * q[c];
                z[o] = a;
            }
        }
        for (size_t e = 0; e < dd; ++e) Ws[e] -= eta * acc[e];
    }
    free(Ws);
    free(acc);
    free(Wt);
    free(r);
}

/* mode 0: average of the forward and the reverse scan; 1: forward only;
 * 2: reverse only. */
int oracle_linear_minibatch(int B, int H, int N, int d, int bsz, int mode,
                            const double* K, const double* Q, const double* V,
                            const double* W0, const double* eta, double* Z,
                            int nthreads) {
    if (B < 0 || H < 0 || N <= 0 || d <= 0 || bsz <= 0 || mode < 0 || mode > 2) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
    int ndir = (mode == 0) ? 2 : 1;
    size_t slice_elems = (size_t)N * d;
    double* tmp = NULL;
    if (mode == 0) tmp = (double*)malloc((size_t)nslice * slice_elems * sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (long job = 0; job < nslice * ndir; ++job) {
        long s = job / ndir;
        int dir = (int)(job % ndir);
        int h = (int)(s % H);
        size_t off = (size_t)s * slice_elems;
        int reverse = (mode == 2) ? 1 : (mode == 1 ? 0 : dir);
        double* out = (mode == 0 && dir == 1) ? tmp + off : Z + off;
        scan_one(N, d, bsz, reverse, K + off, Q + off, V + off, W0 + (size_t)h * d * d,
                 eta[h], out);
    }
    if (mode == 0) {
        size_t total = (size_t)nslice * slice_elems;
        for (size_t e = 0; e < total; ++e) Z[e] = 0.5 * (Z[e] + tmp[e]);
        free(tmp);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Gradient of L = sum <dZ, Z> through the full-batch linear step, by
 * reverse-mode differentiation of the residual form, token by token:
 *   forward : r_i = W0 k_i - v_i ; G = (2/N) sum r_i k_i^T ;
 *             W1 = W0 - eta G ; z_i = W1 q_i
 *   reverse : dW1  = sum_i dz_i q_i^T ;  dq_i = W1^T dz_i
 *             dG   = -eta dW1 ;          deta += -<dW1, G>
 *             dr_i = (2/N) dG k_i
 *             dk_i = (2/N) dG^T r_i + W0^T dr_i ;  dv_i = -dr_i
 *             dW0 += dW1 + sum_i dr_i k_i^T
 * dW0 [H][d][d] and deta [H] are sums over the batch (b ascending).
 * ---------------------------------------------------------------------- */
int oracle_linear_fullbatch_bwd(int B, int H, int N, int d,
                                const double* K, const double* Q, const double* V,
                                const double* W0, const double* eta, const double* dZ,
                                double* dK, double* dQ, double* dV,
                                double* dW0, double* deta, int nthreads) {
    if (B < 0 || H < 0 || N <= 0 || d <= 0) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
    size_t dd = (size_t)d * d;
    double* pW0 = (double*)calloc((size_t)(nslice > 0 ? nslice : 1) * dd, sizeof(double));
    double* peta = (double*)calloc((size_t)(nslice > 0 ? nslice : 1), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        int b = (int)(s / H), h = (int)(s % H);
        const double* W = W0 + (size_t)h * dd;
        double e = eta[h];
        double* R = (double*)malloc((size_t)N * d * sizeof(double));
        double* G = (double*)calloc(dd, sizeof(double));
        double* W1 = (double*)malloc(dd * sizeof(double));
        double* dW1 = (double*)calloc(dd, sizeof(double));
        double* dG = (double*)malloc(dd * sizeof(double));
        double* dr = (double*)malloc((size_t)d * sizeof(double));
        double* gW0 = pW0 + (size_t)s * dd;
        /* forward */
        for (int i = 0; i < N; ++i) {
            const double* k = K + IDX4(b, h, i, 0);
            const double* v = V + IDX4(b, h, i, 0);
            double* r = R + (size_t)i * d;
            for (int o = 0; o < d; ++o) {
                double a = 0.0;
                for (int c = 0; c < d; ++c) a += W[(size_t)o * d + c] * k[c];
                r[o] = a - v[o];
            }
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c) G[(size_t)o * d + c] += r[o] * k[c];
        }
        for (size_t t = 0; t < dd; ++t) {
            G[t] *= 2.0 / (double)N;
            W1[t] = W[t] - e * G[t];
        }
        /* reverse: output z_i = W1 q_i */
        for (int i = 0; i < N; ++i) {
            const double* q = Q + IDX4(b, h, i, 0);
            const double* dz = dZ + IDX4(b, h, i, 0);
            double* dq = dQ + IDX4(b, h, i, 0);
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c) dW1[(size_t)o * d + c] += dz[o] * q[c];
            for (int c = 0; c < d; ++c) {
                double a = 0.0;
                for (int o = 0; o < d; ++o) a += W1[(size_t)o * d + c] * dz[o];
                dq[c] = a;
            }
        }
        /* reverse: W1 = W0 - eta G */
        double de = 0.0;
        for (size_t t = 0; t < dd; ++t) {
            dG[t] = -e * dW1[t];
            de -= dW1[t] * G[t];
            gW0[t] = dW1[t];
        }
        peta[s] = de;
        /* reverse: G = (2/N) sum r_i k_i^T, r_i = W0 k_i - v_i */
        for (int i = 0; i < N; ++i) {
            const double* k = K + IDX4(b, h, i, 0);
            const double* r = R + (size_t)i * d;
            double* dk = dK + IDX4(b, h, i, 0);
            double* dv = dV + IDX4(b, h, i, 0);
            for (int o = 0; o < d; ++o) {
                double a = 0.0;
                for (int c = 0; c < d; ++c) a += dG[(size_t)o * d + c] * k[c];
                dr[o] = (2.0 / (double)N) * a;
            }
            for (int c = 0; c < d; ++c) {
                double a = 0.0, w = 0.0;
                for (int o = 0; o < d; ++o) {
                    a += dG[(size_t)o * d + c] * r[o];
                    w += W[(size_t)o * d + c] * dr[o];
                }
                dk[c] = (2.0 / (double)N) * a + w;
            }
            for (int o = 0; o < d; ++o) dv[o] = -dr[o];
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c) gW0[(size_t)o * d + c] += dr[o] * k[c];
        }
        free(R);
        free(G);
        free(W1);
        free(dW1);
        free(dG);
        free(dr);
    }
    /* fixed-order sum over the batch */
    for (int h = 0; h < H; ++h) {
        double* o = dW0 + (size_t)h * dd;
        memset(o, 0, dd * sizeof(double));
        deta[h] = 0.0;
        for (int b = 0; b < B; ++b) {
            long s = (long)b * H + h;
            for (size_t t = 0; t < dd; ++t) o[t] += pW0[(size_t)s * dd + t];
            deta[h] += peta[s];
        }
    }
    free(pW0);
    free(peta);
    return 0;
}

/* ------------------------------------------------------------------------
 * Gradient of L = sum <dZ, Z> through the depthwise 3x3 full-batch step
 * (end-to-end training goes through the inner gradient: the ViT3 article,
 * observation 1; the conv inner model: observation 6).  Per channel c of
 * slice (b, h), reverse mode through the forward's steps in order
 *   P[p] = sum_t w0[t] K[p+t] ; R = P - V ; g[t] = (2/N) sum_p R[p] K[p+t]
 *   w1 = w0 - eta g ;           Z[p] = sum_t w1[t] Q[p+t]
 * (t runs over the 9 taps (i-1, j-1); K, Q are zero outside the grid and a
 * gradient aimed outside the grid is dropped):
 *   dw1[t] = sum_p dZ[p] Q[p+t] ;       dQ[p+t] += w1[t] dZ[p]
 *   dg = -eta dw1 ;  deta -= sum_t dw1[t] g[t] ;  dw0 += dw1
 *   dR[p] = (2/N) sum_t dg[t] K[p+t] ;  dK[p+t] += (2/N) dg[t] R[p]
 *   dV = -dR ;  dw0[t] += sum_p dR[p] K[p+t] ;  dK[p+t] += w0[t] dR[p]
 * dw0 [H][d][3][3] and deta [H] are sums over the batch (b ascending).
 * ---------------------------------------------------------------------- */
int oracle_dwconv3x3_fullbatch_bwd(int B, int H, int gh, int gw, int d,
                                   const double* K, const double* Q, const double* V,
                                   const double* w0, const double* eta, const double* dZ,
                                   double* dK, double* dQ, double* dV,
                                   double* dw0, double* deta, int nthreads) {
    if (B < 0 || H < 0 || gh <= 0 || gw <= 0 || d <= 0) return -1;
    int N = gh * gw;
    set_threads(nthreads);
    long nwork = (long)B * H * d;
    double* pw0 = (double*)calloc((size_t)(nwork > 0 ? nwork : 1) * 9, sizeof(double));
    double* peta = (double*)calloc((size_t)(nwork > 0 ? nwork : 1), sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (long wkey = 0; wkey < nwork; ++wkey) {
        int c = (int)(wkey % d);
        long s = wkey / d;
        int b = (int)(s / H), h = (int)(s % H);
        const double* w = w0 + ((size_t)h * d + c) * 9;
        double e = eta[h];
        double* R = (double*)malloc((size_t)N * sizeof(double));
        double* dR = (double*)malloc((size_t)N * sizeof(double));
        double g[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0}, w1[9], dw1[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0}, dg[9];
        double* gw0 = pw0 + (size_t)wkey * 9;
        /* forward: R and g */
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double pp = 0.0;
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j)
                        pp += w[i * 3 + j] * tap(K, H, N, d, b, h, gh, gw, y + i - 1, x + j - 1, c);
                R[y * gw + x] = pp - V[IDX4(b, h, y * gw + x, c)];
            }
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x)
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j)
                        g[i * 3 + j] += R[y * gw + x] * tap(K, H, N, d, b, h, gh, gw, y + i - 1, x + j - 1, c);
        for (int t = 0; t < 9; ++t) {
            g[t] *= 2.0 / (double)N;
            w1[t] = w[t] - e * g[t];
        }
        /* reverse: Z = w1 conv Q */
        for (int p = 0; p < N; ++p) dQ[IDX4(b, h, p, c)] = 0.0;
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double dz = dZ[IDX4(b, h, y * gw + x, c)];
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j) {
                        int yy = y + i - 1, xx = x + j - 1;
                        if (yy < 0 || yy >= gh || xx < 0 || xx >= gw) continue;
                        dw1[i * 3 + j] += dz * Q[IDX4(b, h, yy * gw + xx, c)];
                        dQ[IDX4(b, h, yy * gw + xx, c)] += w1[i * 3 + j] * dz;
                    }
            }
        /* reverse: w1 = w0 - eta g */
        double de = 0.0;
        for (int t = 0; t < 9; ++t) {
            dg[t] = -e * dw1[t];
            de -= dw1[t] * g[t];
            gw0[t] = dw1[t];
        }
        peta[wkey] = de;
        /* reverse: g = (2/N) sum_p R[p] K[p+t] */
        for (int p = 0; p < N; ++p) dK[IDX4(b, h, p, c)] = 0.0;
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double a = 0.0;
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j) {
                        int yy = y + i - 1, xx = x + j - 1;
                        if (yy < 0 || yy >= gh || xx < 0 || xx >= gw) continue;
                        a += dg[i * 3 + j] * K[IDX4(b, h, yy * gw + xx, c)];
                        dK[IDX4(b, h, yy * gw + xx, c)] += (2.0 / (double)N) * dg[i * 3 + j] * R[y * gw + x];
                    }
                dR[y * gw + x] = (2.0 / (double)N) * a;
            }
        /* reverse: R = P - V, P = w0 conv K */
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double r = dR[y * gw + x];
                dV[IDX4(b, h, y * gw + x, c)] = -r;
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j) {
                        int yy = y + i - 1, xx = x + j - 1;
                        if (yy < 0 || yy >= gh || xx < 0 || xx >= gw) continue;
                        gw0[i * 3 + j] += r * K[IDX4(b, h, yy * gw + xx, c)];
                        dK[IDX4(b, h, yy * gw + xx, c)] += w[i * 3 + j] * r;
                    }
            }
        free(R);
        free(dR);
    }
    /* fixed-order sum over the batch */
    for (int h = 0; h < H; ++h) {
        deta[h] = 0.0;
        for (int c = 0; c < d; ++c)
            for (int t = 0; t < 9; ++t) dw0[((size_t)h * d + c) * 9 + t] = 0.0;
        for (int b = 0; b < B; ++b)
            for (int c = 0; c < d; ++c) {
                long wkey = ((long)b * H + h) * d + c;
                for (int t = 0; t < 9; ++t) dw0[((size_t)h * d + c) * 9 + t] += pw0[(size_t)wkey * 9 + t];
                deta[h] += peta[wkey];
            }
    }
    free(pw0);
    free(peta);
    return 0;
}

/* ========================================================================
 * Variants of the inner training (the ViT3 article's design space and its
 * final recipe; the Vision-TTT notes' ablation on the initial state and its
 * gradient-magnitude map).
 *
 * loss: 0 = the L2 reconstruction loss of the definitions above;
 *       1 = the dot-product loss of the ViT3 recipe ("点积损失函数"),
 *           read as l(W; k, v) = -<W k, v> (its token mean over the batch),
 *           so G = -(1/N) sum_i v_i k_i^T: no W-dependent term.
 * ====================================================================== */

/* One full-batch gradient of the linear model at W (residual form for L2). */
static void lin_grad(int N, int d, int loss, const double* K, const double* V, const double* W,
                     double* G, double* r) {
    memset(G, 0, (size_t)d * d * sizeof(double));
    for (int i = 0; i < N; ++i) {
        const double* k = K + (size_t)i * d;
        const double* v = V + (size_t)i * d;
        if (loss == 0) {
            for (int o = 0; o < d; ++o) {
                double a = 0.0;
                for (int c = 0; c < d; ++c) a += W[(size_t)o * d + c] * k[c];
                r[o] = a - v[o];
            }
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c) G[(size_t)o * d + c] += (2.0 / (double)N) * r[o] * k[c];
        } else {
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c) G[(size_t)o * d + c] -= (1.0 / (double)N) * v[o] * k[c];
        }
    }
}

/* `steps` full-batch gradient steps (epochs over the whole token set; the
 * ViT3 article, observation 2), each gradient taken at the current W:
 *   W <- W - eta_h G(W), steps times, from W0;  z_i = W q_i.
 * W_out (nullable) receives the final W per slice, [B][H][d][d]. */
int oracle_linear_fullbatch_ex(int B, int H, int N, int d, int loss, int steps,
                               const double* K, const double* Q, const double* V,
                               const double* W0, const double* eta,
                               double* Z, double* W_out, int nthreads) {
    if (B < 0 || H < 0 || N <= 0 || d <= 0 || loss < 0 || loss > 1 || steps < 1) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
    size_t dd = (size_t)d * d;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        int b = (int)(s / H), h = (int)(s % H);
        double* W = (double*)malloc(dd * sizeof(double));
        double* G = (double*)malloc(dd * sizeof(double));
        double* r = (double*)malloc((size_t)d * sizeof(double));
        memcpy(W, W0 + (size_t)h * dd, dd * sizeof(double));
        for (int e = 0; e < steps; ++e) {
            lin_grad(N, d, loss, K + IDX4(b, h, 0, 0), V + IDX4(b, h, 0, 0), W, G, r);
            for (size_t t = 0; t < dd; ++t) W[t] -= eta[h] * G[t];
        }
        for (int i = 0; i < N; ++i) {
            const double* q = Q + IDX4(b, h, i, 0);
            double* z = Z + IDX4(b, h, i, 0);
            for (int o = 0; o < d; ++o) {
                double a = 0.0;
                for (int c = 0; c < d; ++c) a += W[(size_t)o * d + c] * q[c];
                z[o] = a;
            }
        }
        if (W_out) memcpy(W_out + (size_t)s * dd, W, dd * sizeof(double));
        free(W);
        free(G);
        free(r);
    }
    return 0;
}

/* Backward of one full-batch step under either loss (reverse mode as in
 * oracle_linear_fullbatch_bwd).  Dot loss: G = -(1/N) sum v_i k_i^T, so
 *   dG = -eta dW1 ; dv_i = -(1/N) dG k_i ; dk_i = -(1/N) dG^T v_i ; dW0 = dW1. */
int oracle_linear_fullbatch_bwd_ex(int B, int H, int N, int d, int loss,
                                   const double* K, const double* Q, const double* V,
                                   const double* W0, const double* eta, const double* dZ,
                                   double* dK, double* dQ, double* dV,
                                   double* dW0, double* deta, int nthreads) {
    if (loss == 0)
        return oracle_linear_fullbatch_bwd(B, H, N, d, K, Q, V, W0, eta, dZ, dK, dQ, dV, dW0, deta, nthreads);
    if (B < 0 || H < 0 || N <= 0 || d <= 0 || loss != 1) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
    size_t dd = (size_t)d * d;
    double* pW0 = (double*)calloc((size_t)(nslice > 0 ? nslice : 1) * dd, sizeof(double));
    double* peta = (double*)calloc((size_t)(nslice > 0 ? nslice : 1), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        int b = (int)(s / H), h = (int)(s % H);
        const double* W = W0 + (size_t)h * dd;
        double e = eta[h];
        double* G = (double*)malloc(dd * sizeof(double));
        double* W1 = (double*)malloc(dd * sizeof(double));
        double* dW1 = (double*)calloc(dd, sizeof(double));
        double* dG = (double*)malloc(dd * sizeof(double));
        double* r = (double*)malloc((size_t)d * sizeof(double));
        lin_grad(N, d, 1, K + IDX4(b, h, 0, 0), V + IDX4(b, h, 0, 0), W, G, r);
        for (size_t t = 0; t < dd; ++t) W1[t] = W[t] - e * G[t];
        for (int i = 0; i < N; ++i) {
            const double* q = Q + IDX4(b, h, i, 0);
            const double* dz = dZ + IDX4(b, h, i, 0);
            double* dq = dQ + IDX4(b, h, i, 0);
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c) dW1[(size_t)o * d + c] += dz[o] * q[c];
            for (int c = 0; c < d; ++c) {
                double a = 0.0;
                for (int o = 0; o < d; ++o) a += W1[(size_t)o * d + c] * dz[o];
                dq[c] = a;
            }
        }
        double de = 0.0;
        for (size_t t = 0; t < dd; ++t) {
            dG[t] = -e * dW1[t];
            de -= dW1[t] * G[t];
            pW0[(size_t)s * dd + t] = dW1[t];
        }
        peta[s] = de;
        for (int i = 0; i < N; ++i) {
            const double* k = K + IDX4(b, h, i, 0);
            const double* v = V + IDX4(b, h, i, 0);
            double* dk = dK + IDX4(b, h, i, 0);
            double* dv = dV + IDX4(b, h, i, 0);
            for (int o = 0; o < d; ++o) {
                double a = 0.0;
                for (int c = 0; c < d; ++c) a += dG[(size_t)o * d + c] * k[c];
                dv[o] = -(1.0 / (double)N) * a;
            }
            for (int c = 0; c < d; ++c) {
                double a = 0.0;
                for (int o = 0; o < d; ++o) a += dG[(size_t)o * d + c] * v[o];
                dk[c] = -(1.0 / (double)N) * a;
            }
        }
        free(G);
        free(W1);
        free(dW1);
        free(dG);
        free(r);
    }
    for (int h = 0; h < H; ++h) {
        double* o = dW0 + (size_t)h * dd;
        memset(o, 0, dd * sizeof(double));
        deta[h] = 0.0;
        for (int b = 0; b < B; ++b) {
            long s = (long)b * H + h;
            for (size_t t = 0; t < dd; ++t) o[t] += pW0[(size_t)s * dd + t];
            deta[h] += peta[s];
        }
    }
    free(pW0);
    free(peta);
    return 0;
}

/* Depthwise 3x3 full-batch step under either loss.  Dot loss:
 *   g[t] = -(1/N) sum_p V[p] K[p+t]   (no w0-dependent term). */
int oracle_dwconv3x3_fullbatch_ex(int B, int H, int gh, int gw, int d, int loss,
                                  const double* K, const double* Q, const double* V,
                                  const double* w0, const double* eta,
                                  double* Z, double* g_out, int nthreads) {
    if (loss == 0) return oracle_dwconv3x3_fullbatch(B, H, gh, gw, d, K, Q, V, w0, eta, Z, g_out, nthreads);
    if (B < 0 || H < 0 || gh <= 0 || gw <= 0 || d <= 0 || loss != 1) return -1;
    int N = gh * gw;
    set_threads(nthreads);
    long nwork = (long)B * H * d;
#pragma omp parallel for schedule(dynamic, 4)
    for (long wkey = 0; wkey < nwork; ++wkey) {
        int c = (int)(wkey % d);
        long s = wkey / d;
        int b = (int)(s / H), h = (int)(s % H);
        const double* w = w0 + ((size_t)h * d + c) * 9;
        double g[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0}, w1[9];
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double vv = V[IDX4(b, h, y * gw + x, c)];
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j)
                        g[i * 3 + j] -= vv * tap(K, H, N, d, b, h, gh, gw, y + i - 1, x + j - 1, c);
            }
        for (int t = 0; t < 9; ++t) {
            g[t] *= 1.0 / (double)N;
            w1[t] = w[t] - eta[h] * g[t];
        }
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double z = 0.0;
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j)
                        z += w1[i * 3 + j] * tap(Q, H, N, d, b, h, gh, gw, y + i - 1, x + j - 1, c);
                Z[IDX4(b, h, y * gw + x, c)] = z;
            }
        if (g_out)
            for (int t = 0; t < 9; ++t) g_out[(((size_t)b * H + h) * d + c) * 9 + t] = g[t];
    }
    return 0;
}

/* Backward of the depthwise step under either loss.  Dot loss, reverse mode
 * through g[t] = -(1/N) sum_p V[p] K[p+t]:
 *   dV[p] = -(1/N) sum_t dg[t] K[p+t] ;  dK[p+t] += -(1/N) dg[t] V[p] ;
 *   dw0 = dw1 ;  dQ, dw1, dg, deta as for L2. */
int oracle_dwconv3x3_fullbatch_bwd_ex(int B, int H, int gh, int gw, int d, int loss,
                                      const double* K, const double* Q, const double* V,
                                      const double* w0, const double* eta, const double* dZ,
                                      double* dK, double* dQ, double* dV,
                                      double* dw0, double* deta, int nthreads) {
    if (loss == 0)
        return oracle_dwconv3x3_fullbatch_bwd(B, H, gh, gw, d, K, Q, V, w0, eta, dZ, dK, dQ, dV, dw0, deta,
                                              nthreads);
    if (B < 0 || H < 0 || gh <= 0 || gw <= 0 || d <= 0 || loss != 1) return -1;
    int N = gh * gw;
    set_threads(nthreads);
    long nwork = (long)B * H * d;
    double* pw0 = (double*)calloc((size_t)(nwork > 0 ? nwork : 1) * 9, sizeof(double));
    double* peta = (double*)calloc((size_t)(nwork > 0 ? nwork : 1), sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (long wkey = 0; wkey < nwork; ++wkey) {
        int c = (int)(wkey % d);
        long s = wkey / d;
        int b = (int)(s / H), h = (int)(s % H);
        const double* w = w0 + ((size_t)h * d + c) * 9;
        double e = eta[h];
        double g[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0}, w1[9], dw1[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0}, dg[9];
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double vv = V[IDX4(b, h, y * gw + x, c)];
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j)
                        g[i * 3 + j] -= vv * tap(K, H, N, d, b, h, gh, gw, y + i - 1, x + j - 1, c);
            }
        for (int t = 0; t < 9; ++t) {
            g[t] *= 1.0 / (double)N;
            w1[t] = w[t] - e * g[t];
        }
        for (int p = 0; p < N; ++p) {
            dQ[IDX4(b, h, p, c)] = 0.0;
            dK[IDX4(b, h, p, c)] = 0.0;
        }
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double dz = dZ[IDX4(b, h, y * gw + x, c)];
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j) {
                        int yy = y + i - 1, xx = x + j - 1;
                        if (yy < 0 || yy >= gh || xx < 0 || xx >= gw) continue;
                        dw1[i * 3 + j] += dz * Q[IDX4(b, h, yy * gw + xx, c)];
                        dQ[IDX4(b, h, yy * gw + xx, c)] += w1[i * 3 + j] * dz;
                    }
            }
        double de = 0.0;
        for (int t = 0; t < 9; ++t) {
            dg[t] = -e * dw1[t];
            de -= dw1[t] * g[t];
            pw0[(size_t)wkey * 9 + t] = dw1[t];
        }
        peta[wkey] = de;
        for (int y = 0; y < gh; ++y)
            for (int x = 0; x < gw; ++x) {
                double vv = V[IDX4(b, h, y * gw + x, c)], a = 0.0;
                for (int i = 0; i < 3; ++i)
                    for (int j = 0; j < 3; ++j) {
                        int yy = y + i - 1, xx = x + j - 1;
                        if (yy < 0 || yy >= gh || xx < 0 || xx >= gw) continue;
                        a += dg[i * 3 + j] * K[IDX4(b, h, yy * gw + xx, c)];
                        dK[IDX4(b, h, yy * gw + xx, c)] += -(1.0 / (double)N) * dg[i * 3 + j] * vv;
                    }
                dV[IDX4(b, h, y * gw + x, c)] = -(1.0 / (double)N) * a;
            }
    }
    for (int h = 0; h < H; ++h) {
        deta[h] = 0.0;
        for (int c = 0; c < d; ++c)
            for (int t = 0; t < 9; ++t) dw0[((size_t)h * d + c) * 9 + t] = 0.0;
        for (int b = 0; b < B; ++b)
            for (int c = 0; c < d; ++c) {
                long wkey = ((long)b * H + h) * d + c;
                for (int t = 0; t < 9; ++t) dw0[((size_t)h * d + c) * 9 + t] += pw0[(size_t)wkey * 9 + t];
                deta[h] += peta[wkey];
            }
    }
    free(pw0);
    free(peta);
    return 0;
}

/* Mini-batch scans with a separate initial state per direction (the
 * Vision-TTT ablation's best variant): W0 is [2][H][d][d], the forward
 * scan starts from W0[0][h] and the reverse scan from W0[1][h]. */
int oracle_linear_minibatch_2w0(int B, int H, int N, int d, int bsz, int mode,
                                const double* K, const double* Q, const double* V,
                                const double* W0, const double* eta, double* Z,
                                int nthreads) {
    if (B < 0 || H < 0 || N <= 0 || d <= 0 || bsz <= 0 || mode < 0 || mode > 2) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
    int ndir = (mode == 0) ? 2 : 1;
    size_t slice_elems = (size_t)N * d;
    size_t dd = (size_t)d * d;
    double* tmp = NULL;
    if (mode == 0) tmp = (double*)malloc((size_t)nslice * slice_elems * sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (long job = 0; job < nslice * ndir; ++job) {
        long s = job / ndir;
        int dir = (int)(job % ndir);
        int h = (int)(s % H);
        size_t off = (size_t)s * slice_elems;
        int reverse = (mode == 2) ? 1 : (mode == 1 ? 0 : dir);
        double* out = (mode == 0 && dir == 1) ? tmp + off : Z + off;
        scan_one(N, d, bsz, reverse, K + off, Q + off, V + off,
                 W0 + ((size_t)reverse * H + h) * dd, eta[h], out);
    }
    if (mode == 0) {
        size_t total = (size_t)nslice * slice_elems;
        for (size_t e = 0; e < total; ++e) Z[e] = 0.5 * (Z[e] + tmp[e]);
        free(tmp);
    }
    return 0;
}

/* Gradient magnitude map (the Vision-TTT notes: the per-token gradient's
 * size marks how much new information the token carries): for every token,
 * the Frobenius norm of its own gradient at W0, with the outer product
 * written out entry by entry:
 *   L2:  G_t = 2 (W0 k_t - v_t) k_t^T ;   dot:  G_t = -v_t k_t^T.
 * out: [B][H][N]. */
int oracle_linear_gradient_magnitude(int B, int H, int N, int d, int loss,
                                     const double* K, const double* V, const double* W0,
                                     double* out, int nthreads) {
    if (B < 0 || H < 0 || N <= 0 || d <= 0 || loss < 0 || loss > 1) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        int b = (int)(s / H), h = (int)(s % H);
        const double* W = W0 + (size_t)h * d * d;
        double* r = (double*)malloc((size_t)d * sizeof(double));
        for (int i = 0; i < N; ++i) {
            const double* k = K + IDX4(b, h, i, 0);
            const double* v = V + IDX4(b, h, i, 0);
            for (int o = 0; o < d; ++o) {
                if (loss == 0) {
                    double a = 0.0;
                    for (int c = 0; c < d; ++c) a += W[(size_t)o * d + c] * k[c];
                    r[o] = 2.0 * (a - v[o]);
                } else {
                    r[o] = -v[o];
                }
            }
            double f = 0.0;
            for (int o = 0; o < d; ++o)
                for (int c = 0; c < d; ++c) f += (r[o] * k[c]) * (r[o] * k[c]);
            out[(size_t)s * N + i] = sqrt(f);
        }
        free(r);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Gradient of L = sum <dZ, Z> through the mini-batch scans (end-to-end
 * training of Vision-TTT goes through the inner updates; the notes' key
 * design 4 recomputes the states in the backward).  One chain (one
 * direction), reverse mode through the token-by-token procedure of
 * scan_one, with the chunk-start states recomputed by a forward pass.
 * Inside a chunk of n_c tokens with start state Ws, a = 2/n_c:
 *   r_t = Ws k_t - v_t ; acc_t = sum_{s<=t} a r_s k_s^T ;
 *   W_t = Ws - eta acc_t ; z_t = W_t q_t ;  next Ws = Ws - eta acc_last.
 * Reverse, with dWn the gradient reaching the next chunk's start state:
 *   dW_t = dz_t q_t^T ; dq_t = W_t^T dz_t ; deta -= <dW_t, acc_t> ;
 *   E_s = dWn + sum_{t>=s} dW_t ;  dG_s = -eta E_s ; deta -= <dWn, acc_last>
 *   dr_s = a dG_s k_s ; dk_s = a dG_s^T r_s + Ws^T dr_s ; dv_s = -dr_s ;
 *   dWs = dWn + sum_t dW_t + sum_s dr_s k_s^T.
 * dzs: this chain's output gradient (position order); dK, dQ, dV are
 * accumulated (+=); *dW0_out and *deta_out receive the chain's terms.
 * ---------------------------------------------------------------------- */
static void scan_one_bwd(int N, int d, int bsz, int reverse, const double* K, const double* Q,
                         const double* V, const double* W0, double eta, const double* dzs,
                         double* dK, double* dQ, double* dV, double* dW0_out, double* deta_out) {
    size_t dd = (size_t)d * d;
    int nch = (N + bsz - 1) / bsz;
    double* Wst = (double*)malloc((size_t)nch * dd * sizeof(double)); /* chunk-start states */
    double* acc = (double*)malloc(dd * sizeof(double));
    double* r = (double*)malloc((size_t)bsz * d * sizeof(double));
    double* accs = (double*)malloc((size_t)bsz * dd * sizeof(double)); /* acc_t of the chunk */
    double* dWn = (double*)calloc(dd, sizeof(double));
    double* dWs = (double*)malloc(dd * sizeof(double));
    double* E = (double*)malloc(dd * sizeof(double));
    double* Wt = (double*)malloc(dd * sizeof(double));
    double* dr = (double*)malloc((size_t)d * sizeof(double));
    double de = 0.0;
    /* forward: chunk-start states */
    memcpy(Wst, W0, dd * sizeof(double));
    for (int c = 0; c < nch; ++c) {
        int c0 = c * bsz, nc = (N - c0 < bsz) ? (N - c0) : bsz;
        const double* Ws = Wst + (size_t)c * dd;
        memset(acc, 0, dd * sizeof(double));
        for (int t = 0; t < nc; ++t) {
            int pos = reverse ? (N - 1 - (c0 + t)) : (c0 + t);
            const double* k = K + (size_t)pos * d;
            const double* v = V + (size_t)pos * d;
            for (int o = 0; o < d; ++o) {
                double x = 0.0;
                for (int cc = 0; cc < d; ++cc) x += Ws[(size_t)o * d + cc] * k[cc];
                double rr = x - v[o];
                for (int cc = 0; cc < d; ++cc) acc[(size_t)o * d + cc] += (2.0 / (double)nc) * rr * k[cc];
            }
        }
        if (c + 1 < nch)
            for (size_t e = 0; e < dd; ++e) Wst[(size_t)(c + 1) * dd + e] = Ws[e] - eta * acc[e];
    }
    /* reverse over the chunks */
    for (int c = nch - 1; c >= 0; --c) {
        int c0 = c * bsz, nc = (N - c0 < bsz) ? (N - c0) : bsz;
        double a = 2.0 / (double)nc;
        const double* Ws = Wst + (size_t)c * dd;
        /* recompute r_t and acc_t of the chunk */
        memset(acc, 0, dd * sizeof(double));
        for (int t = 0; t < nc; ++t) {
            int pos = reverse ? (N - 1 - (c0 + t)) : (c0 + t);
            const double* k = K + (size_t)pos * d;
            const double* v = V + (size_t)pos * d;
            for (int o = 0; o < d; ++o) {
                double x = 0.0;
                for (int cc = 0; cc < d; ++cc) x += Ws[(size_t)o * d + cc] * k[cc];
                r[(size_t)t * d + o] = x - v[o];
                for (int cc = 0; cc < d; ++cc) acc[(size_t)o * d + cc] += a * r[(size_t)t * d + o] * k[cc];
            }
            memcpy(accs + (size_t)t * dd, acc, dd * sizeof(double));
        }
        /* the chunk-end update: W_next = Ws - eta acc_last */
        for (size_t e = 0; e < dd; ++e) de -= dWn[e] * acc[e];
        memcpy(dWs, dWn, dd * sizeof(double));
        memcpy(E, dWn, dd * sizeof(double));
        /* tokens in reverse: E becomes dWn + sum_{t' >= t} dW_t' */
        for (int t = nc - 1; t >= 0; --t) {
            int pos = reverse ? (N - 1 - (c0 + t)) : (c0 + t);
            const double* k = K + (size_t)pos * d;
            const double* q = Q + (size_t)pos * d;
            const double* dz = dzs + (size_t)pos * d;
            const double* at = accs + (size_t)t * dd;
            /* z_t = W_t q_t, W_t = Ws - eta acc_t */
            for (size_t e = 0; e < dd; ++e) Wt[e] = Ws[e] - eta * at[e];
            for (int cc = 0; cc < d; ++cc) {
                double x = 0.0;
                for (int o = 0; o < d; ++o) x += Wt[(size_t)o * d + cc] * dz[o];
                dQ[(size_t)pos * d + cc] += x;
            }
            for (int o = 0; o < d; ++o)
                for (int cc = 0; cc < d; ++cc) {
                    double dw = dz[o] * q[cc];
                    de -= dw * at[(size_t)o * d + cc];
                    dWs[(size_t)o * d + cc] += dw;
                    E[(size_t)o * d + cc] += dw;
                }
            /* G_t = a r_t k_t^T with dG_t = -eta E */
            const double* rt = r + (size_t)t * d;
            for (int o = 0; o < d; ++o) {
                double x = 0.0;
                for (int cc = 0; cc < d; ++cc) x += E[(size_t)o * d + cc] * k[cc];
                dr[o] = a * (-eta) * x;
            }
            for (int cc = 0; cc < d; ++cc) {
                double x = 0.0, y = 0.0;
                for (int o = 0; o < d; ++o) {
                    x += E[(size_t)o * d + cc] * rt[o];
                    y += Ws[(size_t)o * d + cc] * dr[o];
                }
                dK[(size_t)pos * d + cc] += a * (-eta) * x + y;
            }
            for (int o = 0; o < d; ++o) {
                dV[(size_t)pos * d + o] -= dr[o];
                for (int cc = 0; cc < d; ++cc) dWs[(size_t)o * d + cc] += dr[o] * k[cc];
            }
        }
        memcpy(dWn, dWs, dd * sizeof(double));
    }
    memcpy(dW0_out, dWn, dd * sizeof(double));
    *deta_out = de;
    free(Wst);
    free(acc);
    free(r);
    free(accs);
    free(dWn);
    free(dWs);
    free(E);
    free(Wt);
    free(dr);
}

/* Gradient of L = sum <dZ, Z> through oracle_linear_minibatch (mode 0: Z is
 * the average of the two scans, so each chain sees dZ / 2).  dK, dQ, dV
 * [B][H][N][d] are overwritten; dW0 [H][d][d] and deta [H] are sums over
 * the batch and both directions (b ascending, forward before reverse). */
int oracle_linear_minibatch_bwd(int B, int H, int N, int d, int bsz, int mode,
                                const double* K, const double* Q, const double* V,
                                const double* W0, const double* eta, const double* dZ,
                                double* dK, double* dQ, double* dV, double* dW0, double* deta,
                                int nthreads) {
    if (B < 0 || H < 0 || N <= 0 || d <= 0 || bsz <= 0 || mode < 0 || mode > 2) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
    int ndir = (mode == 0) ? 2 : 1;
    size_t slice_elems = (size_t)N * d, dd = (size_t)d * d;
    double* pW0 = (double*)calloc((size_t)(nslice > 0 ? nslice : 1) * ndir * dd, sizeof(double));
    double* peta = (double*)calloc((size_t)(nslice > 0 ? nslice : 1) * ndir, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        int h = (int)(s % H);
        size_t off = (size_t)s * slice_elems;
        double* dzs = (double*)malloc(slice_elems * sizeof(double));
        for (size_t e = 0; e < slice_elems; ++e) {
            dzs[e] = (mode == 0 ? 0.5 : 1.0) * dZ[off + e];
            dK[off + e] = dQ[off + e] = dV[off + e] = 0.0;
        }
        for (int dir = 0; dir < ndir; ++dir) {
            int reverse = (mode == 2) ? 1 : (mode == 1 ? 0 : dir);
            scan_one_bwd(N, d, bsz, reverse, K + off, Q + off, V + off, W0 + (size_t)h * dd, eta[h], dzs,
                         dK + off, dQ + off, dV + off, pW0 + ((size_t)s * ndir + dir) * dd,
                         peta + (size_t)s * ndir + dir);
        }
        free(dzs);
    }
    for (int h = 0; h < H; ++h) {
        double* o = dW0 + (size_t)h * dd;
        memset(o, 0, dd * sizeof(double));
        deta[h] = 0.0;
        for (int b = 0; b < B; ++b)
            for (int dir = 0; dir < ndir; ++dir) {
                long s = (long)b * H + h;
                for (size_t t = 0; t < dd; ++t) o[t] += pW0[((size_t)s * ndir + dir) * dd + t];
                deta[h] += peta[(size_t)s * ndir + dir];
            }
    }
    free(pW0);
    free(peta);
    return 0;
}

/* ------------------------------------------------------------------------
 * Two-layer SiLU MLP inner model (the ViT3 article, observation 4: width
 * ratio r = hidden / input from 1 to 4): f(k) = W2 silu(W1 k), W1 [rd][d],
 * W2 [d][rd], silu(x) = x / (1 + e^-x).  One full-batch step of the L2
 * loss L = (1/N) sum_i ||f(k_i) - v_i||^2 by backpropagation per token:
 *   h = W1 k ; a = silu(h) ; e = W2 a - v
 *   dW2 = (2/N) sum e a^T ;  g = (W2^T e) * silu'(h) ;  dW1 = (2/N) sum g k^T
 *   W1' = W1 - eta dW1 ;  W2' = W2 - eta dW2 ;  z = W2' silu(W1' q).
 * W1: [H][rd][d], W2: [H][d][rd].  G1_out / G2_out (nullable): dW1, dW2
 * per slice.
 * ---------------------------------------------------------------------- */
static double silu(double x) { return x / (1.0 + exp(-x)); }
static double silu_grad(double x) {
    double sg = 1.0 / (1.0 + exp(-x));
    return sg * (1.0 + x * (1.0 - sg));
}

int oracle_mlp_fullbatch(int B, int H, int N, int d, int hid,
                         const double* K, const double* Q, const double* V,
                         const double* W1, const double* W2, const double* eta,
                         double* Z, double* G1_out, double* G2_out, int nthreads) {
    if (B < 0 || H < 0 || N <= 0 || d <= 0 || hid <= 0) return -1;
    set_threads(nthreads);
    long nslice = (long)B * H;
    size_t n1 = (size_t)hid * d;
#pragma omp parallel for schedule(dynamic, 1)
    for (long s = 0; s < nslice; ++s) {
        int b = (int)(s / H), h = (int)(s % H);
        const double* w1 = W1 + (size_t)h * n1;
        const double* w2 = W2 + (size_t)h * n1;
        double* g1 = (double*)calloc(n1, sizeof(double));
        double* g2 = (double*)calloc(n1, sizeof(double));
        double* hv = (double*)malloc((size_t)hid * sizeof(double));
        double* av = (double*)malloc((size_t)hid * sizeof(double));
        double* ev = (double*)malloc((size_t)d * sizeof(double));
        double* w1n = (double*)malloc(n1 * sizeof(double));
        double* w2n = (double*)malloc(n1 * sizeof(double));
        for (int i = 0; i < N; ++i) {
            const double* k = K + IDX4(b, h, i, 0);
            const double* v = V + IDX4(b, h, i, 0);
            for (int j = 0; j < hid; ++j) {
                double x = 0.0;
                for (int c = 0; c < d; ++c) x += w1[(size_t)j * d + c] * k[c];
                hv[j] = x;
                av[j] = silu(x);
            }
            for (int o = 0; o < d; ++o) {
                double x = 0.0;
                for (int j = 0; j < hid; ++j) x += w2[(size_t)o * hid + j] * av[j];
                ev[o] = x - v[o];
            }
            for (int o = 0; o < d; ++o)
                for (int j = 0; j < hid; ++j) g2[(size_t)o * hid + j] += (2.0 / (double)N) * ev[o] * av[j];
            for (int j = 0; j < hid; ++j) {
                double x = 0.0;
                for (int o = 0; o < d; ++o) x += w2[(size_t)o * hid + j] * ev[o];
                double gj = x * silu_grad(hv[j]);
                for (int c = 0; c < d; ++c) g1[(size_t)j * d + c] += (2.0 / (double)N) * gj * k[c];
            }
        }
        for (size_t e = 0; e < n1; ++e) {
            w1n[e] = w1[e] - eta[h] * g1[e];
            w2n[e] = w2[e] - eta[h] * g2[e];
        }
        for (int i = 0; i < N; ++i) {
            const double* q = Q + IDX4(b, h, i, 0);
            double* z = Z + IDX4(b, h, i, 0);
            for (int j = 0; j < hid; ++j) {
                double x = 0.0;
                for (int c = 0; c < d; ++c) x += w1n[(size_t)j * d + c] * q[c];
                av[j] = silu(x);
            }
            for (int o = 0; o < d; ++o) {
                double x = 0.0;
                for (int j = 0; j < hid; ++j) x += w2n[(size_t)o * hid + j] * av[j];
                z[o] = x;
            }
        }
        if (G1_out) memcpy(G1_out + (size_t)s * n1, g1, n1 * sizeof(double));
        if (G2_out) memcpy(G2_out + (size_t)s * n1, g2, n1 * sizeof(double));
        free(g1);
        free(g2);
        free(hv);
        free(av);
        free(ev);
        free(w1n);
        free(w2n);
    }
    return 0;
}
