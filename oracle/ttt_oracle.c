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
