/*
 * ttt.h -- C ABI of the MI355X (gfx950) multi-head test-time-training layer.
 *
 * The layer (ViT3 / Vision-TTT) treats the key/value views of a token
 * sequence as a small training set, takes gradient steps of an L2
 * reconstruction loss on a per-head inner model, and applies the updated
 * model to the query view.  Definitions, per slice (image b, head h), with
 * token i's key, value and query as column vectors k_i, v_i, q_i in R^d:
 *
 *   loss      l(W) = (1/N) sum_i ||W k_i - v_i||^2                (*)
 *   gradient  G    = (2/N) sum_i (W0 k_i - v_i) k_i^T
 *   update    W1   = W0 - eta_h G
 *   output    z_i  = W1 q_i
 *
 * Sources: Vision-TTT reading notes (papernotes), section "关键设计" item 1
 * (loss, per-token gradient G_t, output z_t = W_t x_t^Q), item 2 (reversed
 * dataset), item 4 (per-head d x d state, mini-batch b = 16); ViT3 article
 * (ccvip repost), observation 2 (one full-batch step), observation 6 (3x3
 * depthwise-conv inner model), observation 1 (end-to-end training goes
 * through the inner gradient).  (*) the 1/N token mean is a reading: the
 * pages print the per-token loss only.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer is a DEVICE pointer on the current HIP device.  The
 *   caller owns all buffers; the library never allocates, frees or
 *   synchronises.  Work is enqueued on `stream` (NULL = the null stream) and
 *   the call returns without waiting for it.
 * Views.  K, Q, V, Z, dZ, dK, dQ, dV are ttt_view: element (b, h, n, c) of a
 *   view lives at ((T*)ptr)[b*stride_b + h*stride_h + n*stride_n + c], with
 *   strides in elements and unit stride along the d channels.  All views of
 *   one call share ttt_problem.dtype.  A call covers heads [0, H) of its
 *   views: to run a sub-range of a larger tensor's heads, offset ptr (and
 *   W0 / w0 / eta) to the first head.
 * Parameters.  W0 is float [H][d][d] row-major, W[r][c] maps input channel c
 *   to output channel r (z = W q).  w0 is float [H][d][3][3].  eta is
 *   float [H].  All fp32 regardless of dtype.
 * Precision.  dtype TTT_F32: fp32 inputs, fp32 arithmetic.  dtype TTT_BF16:
 *   bf16 inputs and outputs, fp32 accumulation; the fp32 inner weights are
 *   rounded to bf16 only where they enter a matrix-core product.
 * Workspace.  `ws` is device scratch of at least ttt_workspace_size(op, p)
 *   bytes (0 is possible; then ws may be NULL).  It must be zero-filled
 *   before its first use; every call leaves its synchronisation counters at
 *   zero again, so one zeroed workspace can serve any sequence of calls on
 *   one stream.  Calls that overlap in time must not share a workspace.
 * Errors.  All validation happens before any HIP call or launch and has no
 *   side effect; on error nothing is written.  B == 0 or H == 0 returns
 *   TTT_OK without a launch.  N <= 0, or d <= 0, is TTT_ERR_BAD_SHAPE;
 *   d != 64 is TTT_ERR_UNSUPPORTED.  Negative strides, or strides under
 *   which two elements of one view coincide, are TTT_ERR_BAD_STRIDE.  Every
 *   view pointer and stride*element-size must be 16-byte aligned, W0 / w0
 *   16-byte and eta / saved / dW0 / deta 4-byte aligned, else
 *   TTT_ERR_MISALIGNED.  An output view or buffer that overlaps any input
 *   or any other output is TTT_ERR_ALIASING (Q may alias K: the shared
 *   Q/K projection of the Vision-TTT ablation).  A failed launch returns
 *   TTT_ERR_HIP.  No C++ exception crosses this interface.
 * Determinism.  For a fixed device, problem and input, results are bitwise
 *   identical from run to run (fixed-order reductions, no float atomics).
 */
#ifndef TTT_H_
#define TTT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* ttt_stream_t; /* same object as hipStream_t */

typedef enum {
    TTT_OK = 0,
    TTT_ERR_NULL_POINTER = 1,
    TTT_ERR_BAD_SHAPE = 2,
    TTT_ERR_BAD_STRIDE = 3,
    TTT_ERR_MISALIGNED = 4,
    TTT_ERR_UNSUPPORTED = 5,
    TTT_ERR_ALIASING = 6,
    TTT_ERR_WORKSPACE_TOO_SMALL = 7,
    TTT_ERR_HIP = 8
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* Direction(s) of the mini-batch scan: the average of the forward scan and
 * the scan of the reversed sequence (mapped back to token positions), or one
 * of them alone. */
typedef enum {
    TTT_BIDIR_AVG = 0,
    TTT_FORWARD_ONLY = 1,
    TTT_BACKWARD_ONLY = 2
} ttt_scan_mode;

typedef enum {
    TTT_OP_LINEAR_FULLBATCH = 0,
    TTT_OP_DWCONV3X3_FULLBATCH = 1,
    TTT_OP_LINEAR_MINIBATCH_BIDIR = 2,
    TTT_OP_LINEAR_FULLBATCH_BWD = 3
} ttt_op;

typedef struct {
    void* ptr;
    int64_t stride_b, stride_h, stride_n; /* in elements; channel stride is 1 */
} ttt_view;

typedef struct {
    int32_t B, H, N, d;      /* images, heads in this call, tokens, head dim  */
    ttt_dtype dtype;         /* element type of every view of the call        */
    int32_t grid_h, grid_w;  /* dwconv only: token n sits at (n / grid_w,
                                n % grid_w); grid_h * grid_w == N            */
    int32_t minibatch;       /* minibatch scan only: tokens per mini-batch b  */
    ttt_scan_mode mode;      /* minibatch scan only                           */
} ttt_problem;

/* Bytes of workspace `op` needs for problem `p` (0 for a bad problem). */
size_t ttt_workspace_size(ttt_op op, const ttt_problem* p);

/* Human-readable name of a status code (static storage). */
const char* ttt_status_string(ttt_status s);

/*
 * One full-batch gradient step of the linear d x d inner model, then apply
 * (ViT3 observation 2; Vision-TTT "关键设计" item 1).  Per slice:
 *   A = sum_i k_i k_i^T, C = sum_i v_i k_i^T  (so G = (2/N)(W0 A - C)),
 *   W1 = W0 - eta_h G, z_i = W1 q_i.
 * In: K, Q, V [B,H,N,d]; W0 [H][d][d]; eta [H].  Out: Z [B,H,N,d].
 * saved: NULL, or float [B][H][2][d][d] receiving A then G of each slice
 *   (what ttt_linear_fullbatch_bwd can reuse).
 */
ttt_status ttt_linear_fullbatch(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                const float* W0, const float* eta, ttt_view Z,
                                float* saved, void* ws, size_t ws_bytes,
                                ttt_stream_t stream);

/*
 * One full-batch gradient step of the 3x3 depthwise-conv inner model, then
 * apply (ViT3 observation 6; the article's layer recipe with one depthwise
 * conv head).  Tokens form a row-major grid_h x grid_w map per channel;
 * conv is cross-correlation with zero padding, stride 1, no bias:
 *   P = conv(K, w0), R = P - V,
 *   g[c][i][j] = (2/N) sum_{y,x} R[c,y,x] K[c, y+i-1, x+j-1],
 *   w1 = w0 - eta_h g, Z = conv(Q, w1).
 * In: K, Q, V [B,H,N,d]; w0 [H][d][3][3]; eta [H].  Out: Z.
 * saved: NULL, or float [B][H][d][3][3] receiving g of each slice.
 * grid_h * grid_w must equal N (else TTT_ERR_BAD_SHAPE).
 */
ttt_status ttt_dwconv3x3_fullbatch(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                   const float* w0, const float* eta, ttt_view Z,
                                   float* saved, void* ws, size_t ws_bytes,
                                   ttt_stream_t stream);

/*
 * One layer's full-batch steps in one call (the ViT3 layer recipe: linear
 * and depthwise-conv inner models on different heads of the same tokens):
 * exactly ttt_linear_fullbatch(lin, Kl, Ql, Vl, W0, eta_l, Zl) and
 * ttt_dwconv3x3_fullbatch(conv, Kc, Qc, Vc, w0, eta_c, Zc), without saved
 * outputs, with the same results bit for bit.  When both fit (bf16, the
 * linear heads' tokens split over workgroups exchanging through one XCD,
 * the conv heads one tile per workgroup) they run as one kernel, in which
 * each workgroup's conv work starts as soon as its linear work ends;
 * otherwise as the two kernels of those calls.  Either problem may
 * have B or H zero.  All ten views/buffers are inputs except Zl and Zc; no
 * output may overlap another argument.
 * ws: ttt_layer_workspace_size(lin, conv) bytes, 256-byte aligned,
 * zero-filled before its first use (the library leaves it reusable), not
 * shared by calls that may run concurrently.
 */
size_t ttt_layer_workspace_size(const ttt_problem* lin, const ttt_problem* conv);
ttt_status ttt_layer_fullbatch(const ttt_problem* lin, ttt_view Kl, ttt_view Ql, ttt_view Vl,
                               const float* W0, const float* eta_l, ttt_view Zl,
                               const ttt_problem* conv, ttt_view Kc, ttt_view Qc, ttt_view Vc,
                               const float* w0, const float* eta_c, ttt_view Zc,
                               void* ws, size_t ws_bytes, ttt_stream_t stream);

/*
 * Causal mini-batch gradient descent of the linear inner model over the
 * token sequence and over the reversed sequence (Vision-TTT "关键设计"
 * items 2 and 4).  Mini-batches of b = p->minibatch tokens, the last one
 * possibly shorter (n_c tokens); with batch-start state Ws, for token t of
 * the batch:
 *   G_t = (2/n_c)(Ws k_t - v_t) k_t^T,  W_t = Ws - eta_h sum_{s<=t} G_s,
 *   z_t = W_t q_t,  and after the batch Ws <- W_last.
 * Both directions start from W0.  TTT_BIDIR_AVG writes
 * Z = (Z_forward + Z_reverse)/2; the other modes write one direction.
 * b must be in [1, 16] on this device (larger: TTT_ERR_UNSUPPORTED).
 * (N + 512) * stride_n * 2 bytes must stay under 2^31 for K, Q, V and Z
 * (a slice's rows are addressed with 32-bit offsets; else
 * TTT_ERR_UNSUPPORTED).
 */
ttt_status ttt_linear_minibatch_bidir(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                      const float* W0, const float* eta, ttt_view Z,
                                      void* ws, size_t ws_bytes, ttt_stream_t stream);

/*
 * Backward of ttt_linear_fullbatch for L = sum <dZ, Z> (end-to-end training
 * through the inner update: ViT3 observation 1).  With beta = 2 eta_h / N,
 * dW1 = dZ^T Q and M = W0^T dW1 + dW1^T W0, per slice:
 *   dQ = dZ W1,  dK = beta (V dW1 - K M),  dV = beta K dW1^T,
 * and summed over the batch in b order:
 *   dW0[h] = sum_b dW1 (I - beta A),  deta[h] = -sum_b <dW1, G>.
 * saved: the forward's [B][H][2][d][d] A/G buffer, or NULL to recompute A
 *   and G from K and V.
 * Out: dK, dQ, dV (views, dtype); dW0 float [H][d][d] and deta float [H]
 *   (overwritten, not accumulated).
 */
ttt_status ttt_linear_fullbatch_bwd(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                    const float* W0, const float* eta, ttt_view dZ,
                                    const float* saved, ttt_view dK, ttt_view dQ, ttt_view dV,
                                    float* dW0, float* deta, void* ws, size_t ws_bytes,
                                    ttt_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H_ */
