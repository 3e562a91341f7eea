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
    TTT_OP_LINEAR_FULLBATCH_BWD = 3,
    TTT_OP_LAYER_FULLBATCH = 4, /* workspace of ttt_layer_fullbatch (sized by
                                   ttt_layer_workspace_size; ttt_workspace_size
                                   returns 0 for it) */
    TTT_OP_DWCONV3X3_FULLBATCH_BWD = 5,
    TTT_OP_LINEAR_MINIBATCH_BIDIR_BWD = 6,
    TTT_OP_MLP_FULLBATCH = 7
} ttt_op;

typedef struct {
    void* ptr;
    int64_t stride_b, stride_h, stride_n; /* in elements; channel stride is 1 */
} ttt_view;

/* Inner loss.  TTT_LOSS_L2: l(W; k, v) = ||W k - v||^2 (the definitions
 * above).  TTT_LOSS_DOT: the dot-product loss of the ViT3 recipe, read as
 * l(W; k, v) = -<W k, v>, so the full-batch gradient is
 * G = -(1/N) sum_i v_i k_i^T (depthwise: g[t] = -(1/N) sum_p V[p] K[p+t])
 * and one step is linear attention added to W0's output.  Full-batch
 * linear and depthwise steps and their backward take either; the
 * mini-batch scan takes L2 only. */
typedef enum { TTT_LOSS_L2 = 0, TTT_LOSS_DOT = 1 } ttt_loss;

typedef struct {
    int32_t B, H, N, d;      /* images, heads in this call, tokens, head dim  */
    ttt_dtype dtype;         /* element type of every view of the call        */
    int32_t grid_h, grid_w;  /* dwconv only: token n sits at (n / grid_w,
                                n % grid_w); grid_h * grid_w == N            */
    int32_t minibatch;       /* minibatch scan only: tokens per mini-batch b  */
    ttt_scan_mode mode;      /* minibatch scan only                           */
    ttt_loss loss;           /* inner loss (0 = L2)                           */
    int32_t steps;           /* ttt_linear_fullbatch only: full-batch gradient
                                steps (epochs), each at the current W; 0 and
                                1 mean one step; other ops require <= 1      */
    int32_t w0_per_direction;/* minibatch scan only: 1 = W0 is
                                [2][H][d][d], the forward scan starting from
                                W0[0] and the reversed one from W0[1]; 0 =
                                one shared [H][d][d]                         */
    int32_t hidden;          /* ttt_mlp_fullbatch only: hidden width of the
                                two-layer inner model (r d, r = 1..4)        */
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
 * p->loss selects the L2 or the dot-product loss.  p->steps = E > 1 takes E
 * full-batch steps (ViT3 observation 2, more inner epochs): W_{e+1} =
 * W_e - eta_h G(W_e), then z_i = W_E q_i; three launches (the Gram pass
 * saving A and G(W0) in the workspace, the d x d steps per slice, the
 * apply); saved must then be NULL (the backward covers one step).
 */
ttt_status ttt_linear_fullbatch(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                const float* W0, const float* eta, ttt_view Z,
                                float* saved, void* ws, size_t ws_bytes,
                                ttt_stream_t stream);

/*
 * ttt_linear_fullbatch for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results bit for bit, without a caller
 * workspace.  Its scratch is a fixed 10.5 MiB device array inside the
 * library (enough for every problem shape), one copy per device, held
 * until the process ends; the call allocates and frees nothing.  Before its
 * kernel each call zeroes the scratch's counters with a small kernel (no
 * memset node), so a failed exchange of one call does not carry over.
 * Every call on a device shares that device's scratch: calls that may
 * overlap in time on one device (two streams, two threads) race and must
 * not be issued.  Arguments, errors and outputs as ttt_linear_fullbatch; a
 * problem needing more scratch than the array holds would be
 * TTT_ERR_WORKSPACE_TOO_SMALL (no valid shape does).
 */
ttt_status ttt_linear_fullbatch_noalloc(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                        const float* W0, const float* eta, ttt_view Z,
                                        float* saved, ttt_stream_t stream);

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
 * Backward of ttt_dwconv3x3_fullbatch for L = sum <dZ, Z> (end-to-end
 * training through the inner update: ViT3 observation 1; the depthwise
 * conv inner model: observation 6).  Per channel of a slice, t over the 9
 * taps, with dw1[t] = sum_p dZ[p] Q[p+t] and dg = -eta_h dw1:
 *   dQ[q] = sum_t w1[t] dZ[q-t],  dR[p] = (2/N) sum_t dg[t] K[p+t],
 *   dV = -dR,  dK[q] = sum_t ((2/N) dg[t] R[q-t] + w0[t] dR[q-t])
 *   (R = conv(K, w0) - V; R and dR are zero off the grid),
 * and summed over the batch in b order:
 *   dw0[h] = sum_b (dw1 + sum_p dR[p] K[p+t]),  deta[h] = -sum_b <dw1, g>.
 * saved: the forward's g ([B][H][d][3][3], its saved output) or NULL to
 *   recompute g from K and V.
 * Out: dK, dQ, dV (views, dtype); dw0 float [H][d][3][3] and deta float [H]
 *   (overwritten).  grid_h * grid_w must equal N.  Each view's slice must
 *   span less than 512 MiB (N * stride_n * element size < 2^29 bytes), or
 *   TTT_ERR_UNSUPPORTED.
 * ws: ttt_workspace_size(TTT_OP_DWCONV3X3_FULLBATCH_BWD, p) bytes (no
 *   zero-fill needed: every word is written before it is read).
 */
ttt_status ttt_dwconv3x3_fullbatch_bwd(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                       const float* w0, const float* eta, ttt_view dZ,
                                       const float* saved, ttt_view dK, ttt_view dQ, ttt_view dV,
                                       float* dw0, float* deta, void* ws, size_t ws_bytes,
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
 * b: any value >= 1 (b >= N is one mini-batch: the full-batch step's
 * gradients, applied causally).
 * When the chains (slice x direction) would leave most compute units idle,
 * each chain is cut into segments that run in parallel (chunk-parallel
 * scan: over a mini-batch the state update is affine, W <- W M + U, so the
 * segments' maps are walked first, their start states composed in order,
 * then every segment walked from its start state); the results agree with
 * the single walk to rounding.  The environment variable
 * TTT_SCAN_SEGMENTS=n (a test switch) forces n segments (at most 8).
 * bf16 views run on the matrix cores (bf16 products, fp32 accumulation and
 * state); fp32 views on the vector ALUs in fp32 throughout (no segments).
 * bf16: (N + 512) * stride_n * 2 bytes must stay under 2^31 for K, Q, V and
 * Z (a slice's rows are addressed with 32-bit offsets; else
 * TTT_ERR_UNSUPPORTED).
 */
ttt_status ttt_linear_minibatch_bidir(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                      const float* W0, const float* eta, ttt_view Z,
                                      void* ws, size_t ws_bytes, ttt_stream_t stream);

/*
 * Gradient magnitude map (Vision-TTT notes, key design item 1: the size of
 * each token's gradient marks the information it adds): per token, the
 * Frobenius norm of its own full-batch gradient at W0,
 *   L2:  ||2 (W0 k_t - v_t) k_t^T||_F = 2 ||W0 k_t - v_t|| ||k_t||,
 *   dot: ||v_t k_t^T||_F = ||v_t|| ||k_t||   (p->loss).
 * In: K, V [B,H,N,d]; W0 [H][d][d].  Out: gmm float [B][H][N] (contiguous,
 * 4-byte aligned).  No workspace.  bf16 inputs: W0 k_t on the matrix cores
 * with W0 rounded to bf16; fp32 inputs: fp32 products.
 */
ttt_status ttt_linear_gradient_magnitude(const ttt_problem* p, ttt_view K, ttt_view V, const float* W0,
                                         float* gmm, ttt_stream_t stream);

/*
 * Two-layer SiLU MLP inner model (ViT3 article, observation 4: widening the
 * inner model from hidden = d to 4d keeps improving the layer), one
 * full-batch step of the L2 loss, then applied to the queries.  Per slice
 * (b, h), with f(k) = W2 silu(W1 k) and e_t = f(k_t) - v_t:
 *   dW2 = (2/N) sum_t e_t a_t^T,  a_t = silu(W1 k_t),
 *   dW1 = (2/N) sum_t ((W2^T e_t) * silu'(W1 k_t)) k_t^T,
 *   W1' = W1[h] - eta[h] dW1,  W2' = W2[h] - eta[h] dW2,
 *   Z[b,h,t] = W2' silu(W1' q_t).
 * p->hidden in {64, 128, 192, 256}; bf16 views only; p->loss L2; one step.
 * In: K, Q, V [B,H,N,d] views; W1 float [H][hidden][d]; W2 float
 * [H][d][hidden]; eta float [H].  Out: Z [B,H,N,d] view.  Every product on
 * the matrix cores with bf16 operands (the weights, the activations, the
 * errors and the back-propagated gradients rounded to bf16) and fp32
 * accumulation; the per-split gradient partials are summed in a fixed order
 * (deterministic).  ws: ttt_workspace_size(TTT_OP_MLP_FULLBATCH, p) bytes
 * (bf16 weights and fp32 gradient partials), no zero-fill needed.
 * Errors: TTT_ERR_UNSUPPORTED for fp32, other widths or the dot loss,
 * TTT_ERR_BAD_SHAPE for hidden <= 0, then as ttt_linear_fullbatch.
 */
ttt_status ttt_mlp_fullbatch(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V, const float* W1,
                             const float* W2, const float* eta, ttt_view Z, void* ws, size_t ws_bytes,
                             ttt_stream_t stream);

/*
 * Backward of ttt_linear_minibatch_bidir for L = sum <dZ, Z> (end-to-end
 * training of Vision-TTT through the inner updates; the states are
 * recomputed, key design item 4).  Per chain (slice, direction) and
 * mini-batch of n_c tokens with start state Ws, alpha = -2 eta_h / n_c,
 * token rows R = K Ws^T - V, S = Q K^T and P = dZ R^T (both kept where the
 * key token does not follow the query token), dWn the gradient at the next
 * start state:
 *   dR = alpha (K dWn^T + S^T dZ),  dV = -dR,  dQ = dZ Ws + alpha P K,
 *   dK = dR Ws + alpha (R dWn + P^T Q),  dWs = dWn + dZ^T Q + dR^T K;
 * with both directions each scan receives dZ / 2.  Summed over the batch
 * (and the directions): dW0 = the walks' final dWs (with
 * p->w0_per_direction dW0 is [2][H][d][d], each direction's own),
 * deta = sum over mini-batches of (-2/n_c)(<R dWn, K> + <P, S>).
 * p->minibatch in [1, 32] (else TTT_ERR_UNSUPPORTED); bf16 or fp32 views;
 * p->loss must be L2.  Out: dK, dQ, dV (views, dtype), dW0 and deta fp32
 * (overwritten).  ws: ttt_workspace_size(TTT_OP_LINEAR_MINIBATCH_BIDIR_BWD,
 * p) bytes (every mini-batch's start state and gradient state, fp32: about
 * 2 * slices * directions * ceil(N/b) * 16 KB), no zero-fill needed.
 */
ttt_status ttt_linear_minibatch_bidir_bwd(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                          const float* W0, const float* eta, ttt_view dZ,
                                          ttt_view dK, ttt_view dQ, ttt_view dV, float* dW0,
                                          float* deta, void* ws, size_t ws_bytes, ttt_stream_t stream);

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

/*
 * Diagnostics
 * -----------
 * Which kernel a call would launch on the current device, and how the
 * tokens of a slice are split over workgroups.  Pure functions of the
 * problem and the device (no launch, no state).
 *   kernel: TTT_KERNEL_LIN_RESIDENT -- one resident kernel exchanging
 *             [A; C] partials (fp32 inputs, saved A/G, device-wide exchange
 *             or one workgroup per slice);
 *           TTT_KERNEL_LIN_RESIDENT_GX -- the bf16 resident kernel whose
 *             splits exchange G_s = W0 A_s - C_s through one XCD's L2 (taken
 *             when no saved buffer is passed);
 *           TTT_KERNEL_LIN_STREAM -- token ranges too long to stay in LDS;
 *           TTT_KERNEL_DWCONV -- the depthwise-conv kernel.
 *   splits: workgroups per (image, head) slice; xcd_local: 1 when the
 *   splits of a slice exchange through one XCD's L2, 0 for device-scope
 *   atomics; fused (layer query): 1 when ttt_layer_fullbatch is one launch;
 *   fused (linear query, p->steps > 1): 1 when the steps run inside the one
 *   launch of TTT_KERNEL_LIN_RESIDENT_GX (each split keeps its A_s and C_s,
 *   every further step is one more exchange round), 0 when they take three
 *   launches (the Gram pass saving A and G, the steps, the apply).
 * op TTT_OP_LINEAR_FULLBATCH (with_saved: whether a saved buffer is passed)
 * or TTT_OP_DWCONV3X3_FULLBATCH; other ops are TTT_ERR_UNSUPPORTED.
 * B == 0 or H == 0 gives all zeros.
 *
 * Environment switches read at every call: TTT_EXCHANGE=device makes split
 * slices use the device-scope exchange (plain block mapping) even where
 * the XCD-local one applies; TTT_TEST_EXCHANGE_GIVEUP=1 makes every slice
 * barrier give up after a few polls (the failure path below, for tests);
 * TTT_SPLIT_STEPS=1 sends several full-batch steps down the three-launch
 * path.
 */
enum {
    TTT_KERNEL_LIN_RESIDENT = 1,
    TTT_KERNEL_LIN_RESIDENT_GX = 2,
    TTT_KERNEL_LIN_STREAM = 3,
    TTT_KERNEL_DWCONV = 4
};
typedef struct {
    int32_t kernel, splits, xcd_local, fused;
} ttt_plan_info;
ttt_status ttt_plan_query(ttt_op op, const ttt_problem* p, int with_saved, ttt_plan_info* out);
ttt_status ttt_layer_plan_query(const ttt_problem* lin, const ttt_problem* conv, int32_t* fused);

/*
 * Exchange failures.  The workgroups of a split slice meet at barriers in
 * the workspace; a wait is bounded (about a second).  A slice whose
 * workgroups never all arrive (the device did not keep the grid resident,
 * e.g. other kernels occupied it) marks its counter line failed: that
 * slice's outputs (Z, and A/G or g when saved) are NaN in that call and in
 * every later call on the same workspace, and the call still returns
 * TTT_OK (the failure happens after the launch).
 * ttt_workspace_exchange_failed: *failed = 1 when any counter line of the
 *   workspace `ws` of operation `op` has failed.  Waits for `stream`
 *   (hipStreamSynchronize) and copies the failure words to the host.
 * ttt_workspace_reset: zero-fills ws (hipMemsetAsync on `stream`): the
 *   workspace is then as good as a fresh zero-filled one.  Not for use
 *   inside HIP graph capture.
 */
ttt_status ttt_workspace_exchange_failed(ttt_op op, const void* ws, size_t ws_bytes, int32_t* failed,
                                         ttt_stream_t stream);
ttt_status ttt_workspace_reset(void* ws, size_t ws_bytes, ttt_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H_ */
