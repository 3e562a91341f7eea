// minibatch_scan_bwd.hip -- gradient of the mini-batch scans (Vision-TTT:
// end-to-end training through the inner updates; the notes' key design 4
// recomputes the states in the backward instead of storing per-token ones).
//
// One chain = one (slice, direction).  With walk position w (token
// w or N-1-w), mini-batch c of n_c <= 32 tokens, start state Ws and
// alpha = -2 eta / n_c, the forward is, per mini-batch (token rows):
//   R = K Ws^T - V,  Z = Q Ws^T + alpha tril(Q K^T) R,  Ws' = Ws + alpha R^T K.
// Backward of L = <dZ, Z> with dWn the gradient at the next start state
// (S = Q K^T and P = dZ R^T, both kept where s <= t):
//   dR  = alpha (K dWn^T + S^T dZ)           dV = -dR
//   dQ  = dZ Ws + alpha P K
//   dK  = dR Ws + alpha (R dWn + P^T Q)
//   dWs = dWn + dZ^T Q + dR^T K              (the recurrence, run backwards)
//   d(alpha) = <R dWn, K> + <P, S>           deta += (-2/n_c) d(alpha)
// The rows of W evolve independently in both recurrences, so the serial
// walks run per 16-row block of W (four workgroups per chain); everything
// else is per mini-batch and runs in parallel:
//   states   per (chain, row block): the forward walk, storing every
//            mini-batch's start state Ws (fp32);
//   chain    per (chain, row block): the backward walk, storing each
//            mini-batch's dR and the gradient dWn at its end;
//   outputs  per (chain, mini-batch): dQ, dK, dV and the deta term;
//   sums     per head: dW0 (the walks' final dWs) and deta over the batch
//            and the directions, in a fixed order; with both directions
//            the two directions' fp32 gradient planes are added.
// Two implementations.  bf16 views with b <= 16: both walks on the matrix
// cores (minibatch_scan.hip: states and gradient states kept in bf16), the
// outputs on the matrix cores per token block, both directions in one
// workgroup when their mini-batches cover the same tokens (no fp32 planes).
// Otherwise fp32 arithmetic on the vector ALUs throughout (bf16 or fp32
// views); the serial walks prefetch the next mini-batch's rows into
// registers while the current one is computed.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace ttt {
namespace {

constexpr int kSbMax = 32;  // tokens per mini-batch handled here
constexpr int kSbT = 256;   // threads per workgroup
constexpr int kP = 65;      // LDS pitch (floats) of 64-wide rows: lanes reading a column of
                            // different rows hit different banks

struct SbArgs {
    View4 K, Q, V, dZ, dK, dQ, dV;
    const float* W0;   // [H][64][64] (or [2][H][64][64] with w0dir)
    const float* eta;
    float* dW0;        // [H][64][64] (or [2][H][64][64])
    float* deta;       // [H]
    float* ws_state;   // [chains][nch][64][64]: forward start states (fp32; bf16 from the matrix-core walks)
    float* dwn_state;  // [chains][nch][64][64]: gradient at each mini-batch's end (likewise)
    float* dRp;        // [chains][N][64]: dR by walk position
    float* dW0c;       // [chains][64][64]
    float* detac;      // [chains][nch]
    float* planes;     // both directions: [2][3][slices][N][64] fp32 (dQ, dK, dV)
    int B, H, N, b, nch, mode, nd, w0dir, bf16;
};

__device__ __forceinline__ int chain_dir(const SbArgs& a, int di) { return a.mode == 2 ? 1 : (a.mode == 0 ? di : 0); }

// element (token pos, channel c) of a view of slice (bb, h); the element
// type is a template parameter (a branch on it around a load would make
// the load wait where the branches join)
template <bool BF>
__device__ __forceinline__ float ldv(const View4& v, int bb, int h, int pos, int c) {
    const long long e = (long long)bb * v.sb + (long long)h * v.sh + (long long)pos * v.sn + c;
    if constexpr (BF) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(v.ptr)[e] << 16);
    else return reinterpret_cast<const float*>(v.ptr)[e];
}
template <bool BF>
__device__ __forceinline__ void stv(const View4& v, int bb, int h, int pos, int c, float x) {
    const long long e = (long long)bb * v.sb + (long long)h * v.sh + (long long)pos * v.sn + c;
    if constexpr (BF) reinterpret_cast<uint16_t*>(v.ptr)[e] = f2bf(x);
    else reinterpret_cast<float*>(v.ptr)[e] = x;
}

struct ChainId {
    int ch, slice, bb, h, di, dir;
};
__device__ __forceinline__ ChainId chain_of(const SbArgs& a, int ch) {
    ChainId c;
    c.ch = ch;
    c.slice = ch / a.nd;
    c.di = ch % a.nd;
    c.dir = chain_dir(a, c.di);
    c.bb = c.slice / a.H;
    c.h = c.slice % a.H;
    return c;
}
__device__ __forceinline__ int pos_of(const SbArgs& a, const ChainId& c, int w) { return c.dir ? a.N - 1 - w : w; }
__device__ __forceinline__ int nc_of(const SbArgs& a, int c) { return min(a.b, a.N - c * a.b); }

// The mini-batch's token rows (all 64 channels) into registers: thread t
// holds elements t + 256 j (row (t + 256 j) / 64, channel % 64) of the
// n_c x 64 tile, zeros past n_c.
struct Tile {
    float x[kSbMax * 64 / kSbT];
};
// Branch-free: rows past n_c load the last row and are zeroed afterwards.
template <bool BF>
__device__ __forceinline__ void load_tile(const SbArgs& a, const View4& v, const ChainId& c, int mb, float scale,
                                          Tile& t) {
    const int n = nc_of(a, mb);
#pragma unroll
    for (int j = 0; j < kSbMax * 64 / kSbT; ++j) {
        const int e = threadIdx.x + kSbT * j, r = e >> 6, ch = e & 63;
        const float x = ldv<BF>(v, c.bb, c.h, pos_of(a, c, mb * a.b + min(r, n - 1)), ch);
        t.x[j] = r < n ? scale * x : 0.f;
    }
}
__device__ __forceinline__ void tile_to_lds(const Tile& t, float* dst) {
#pragma unroll
    for (int j = 0; j < kSbMax * 64 / kSbT; ++j) {
        const int e = threadIdx.x + kSbT * j;
        dst[(e >> 6) * kP + (e & 63)] = t.x[j];
    }
}

// ---- forward states per (chain, row block) ------------------------------
template <bool BF>
__global__ __launch_bounds__(kSbT) void sbwd_states(SbArgs a) {
    __shared__ float Wr[16 * kP];      // rows 16 rb .. of the start state
    __shared__ float Kt[kSbMax * kP];
    __shared__ float Vt[kSbMax * kP];
    __shared__ float Rt[kSbMax * 16];
    const int rb = blockIdx.x & 3, tid = threadIdx.x;
    const ChainId c = chain_of(a, blockIdx.x >> 2);
    const float eta = a.eta[c.h];
    const float* W0 = a.W0 + ((a.w0dir && c.dir ? (long long)a.H : 0) + c.h) * 4096 + rb * 1024;
    for (int e = tid; e < 1024; e += kSbT) Wr[(e >> 6) * kP + (e & 63)] = W0[e];
    Tile kn, vn;
    load_tile<BF>(a, a.K, c, 0, 1.f, kn);
    load_tile<BF>(a, a.V, c, 0, 1.f, vn);
    for (int mb = 0; mb < a.nch; ++mb) {
        const int n = nc_of(a, mb);
        const float alpha = -2.f * eta / (float)n;
        __syncthreads(); // Wr complete; the previous tiles are read
        float* st = a.ws_state + ((long long)c.ch * a.nch + mb) * 4096 + rb * 1024;
        for (int e = tid; e < 1024; e += kSbT) st[e] = Wr[(e >> 6) * kP + (e & 63)];
        tile_to_lds(kn, Kt);
        tile_to_lds(vn, Vt);
        if (mb + 1 < a.nch) {
            load_tile<BF>(a, a.K, c, mb + 1, 1.f, kn);
            load_tile<BF>(a, a.V, c, mb + 1, 1.f, vn);
        }
        __syncthreads();
        // R[s][r] = Ws[r] . k_s - v_s[16 rb + r]
        for (int e = tid; e < n * 16; e += kSbT) {
            const int s = e >> 4, r = e & 15;
            float x = 0.f;
#pragma unroll 16
            for (int j = 0; j < 64; ++j) x = fmaf(Wr[r * kP + j], Kt[s * kP + j], x);
            Rt[e] = x - Vt[s * kP + 16 * rb + r];
        }
        __syncthreads();
        // Ws[r][j] += alpha sum_s R[s][r] K[s][j]
        for (int e = tid; e < 1024; e += kSbT) {
            const int r = e >> 6, j = e & 63;
            float x = 0.f;
            for (int s = 0; s < n; ++s) x = fmaf(Rt[s * 16 + r], Kt[s * kP + j], x);
            Wr[r * kP + j] = fmaf(alpha, x, Wr[r * kP + j]);
        }
    }
}

// ---- backward chain per (chain, row block) --------------------------------
template <bool BF>
__global__ __launch_bounds__(kSbT) void sbwd_chain(SbArgs a) {
    __shared__ float Gr[16 * kP];      // rows 16 rb .. of dWn
    __shared__ float Kt[kSbMax * kP];
    __shared__ float Qt[kSbMax * kP];
    __shared__ float Dt[kSbMax * kP];  // dZ (this chain's share)
    __shared__ float St[kSbMax * kSbMax];
    __shared__ float dRt[kSbMax * 16];
    const int rb = blockIdx.x & 3, tid = threadIdx.x;
    const ChainId c = chain_of(a, blockIdx.x >> 2);
    const float eta = a.eta[c.h];
    const float dzs = a.mode == 0 ? 0.5f : 1.f;
    for (int e = tid; e < 16 * kP; e += kSbT) Gr[e] = 0.f;
    Tile kn, qn, dn;
    const int last = a.nch - 1;
    load_tile<BF>(a, a.K, c, last, 1.f, kn);
    load_tile<BF>(a, a.Q, c, last, 1.f, qn);
    load_tile<BF>(a, a.dZ, c, last, dzs, dn);
    for (int mb = last; mb >= 0; --mb) {
        const int n = nc_of(a, mb);
        const float alpha = -2.f * eta / (float)n;
        __syncthreads();
        float* st = a.dwn_state + ((long long)c.ch * a.nch + mb) * 4096 + rb * 1024;
        for (int e = tid; e < 1024; e += kSbT) st[e] = Gr[(e >> 6) * kP + (e & 63)];
        tile_to_lds(kn, Kt);
        tile_to_lds(qn, Qt);
        tile_to_lds(dn, Dt);
        if (mb > 0) {
            load_tile<BF>(a, a.K, c, mb - 1, 1.f, kn);
            load_tile<BF>(a, a.Q, c, mb - 1, 1.f, qn);
            load_tile<BF>(a, a.dZ, c, mb - 1, dzs, dn);
        }
        __syncthreads();
        // S[t][s] = q_t . k_s for s <= t
        for (int e = tid; e < n * n; e += kSbT) {
            const int t = e / n, s = e % n;
            float x = 0.f;
            if (s <= t) {
#pragma unroll 16
                for (int j = 0; j < 64; ++j) x = fmaf(Qt[t * kP + j], Kt[s * kP + j], x);
            }
            St[t * kSbMax + s] = x;
        }
        __syncthreads();
        // dR[s][r] = alpha (dWn[r] . k_s + sum_{t >= s} S[t][s] dz_t[r])
        for (int e = tid; e < n * 16; e += kSbT) {
            const int s = e >> 4, r = e & 15;
            float x = 0.f;
#pragma unroll 16
            for (int j = 0; j < 64; ++j) x = fmaf(Gr[r * kP + j], Kt[s * kP + j], x);
            for (int t = s; t < n; ++t) x = fmaf(St[t * kSbMax + s], Dt[t * kP + 16 * rb + r], x);
            const float d = alpha * x;
            dRt[e] = d;
            a.dRp[((long long)c.ch * a.N + mb * a.b + s) * 64 + 16 * rb + r] = d;
        }
        __syncthreads();
        // dWs[r][j] = dWn[r][j] + sum_t dz_t[r] q_t[j] + sum_s dR[s][r] k_s[j]
        for (int e = tid; e < 1024; e += kSbT) {
            const int r = e >> 6, j = e & 63;
            float x = Gr[r * kP + j];
            for (int t = 0; t < n; ++t) x = fmaf(Dt[t * kP + 16 * rb + r], Qt[t * kP + j], x);
            for (int s = 0; s < n; ++s) x = fmaf(dRt[s * 16 + r], Kt[s * kP + j], x);
            Gr[r * kP + j] = x;
        }
    }
    __syncthreads();
    float* o = a.dW0c + (long long)c.ch * 4096 + rb * 1024;
    for (int e = tid; e < 1024; e += kSbT) o[e] = Gr[(e >> 6) * kP + (e & 63)];
}

// ---- outputs per (chain, mini-batch) ---------------------------------------
template <bool BF>
__global__ __launch_bounds__(kSbT) void sbwd_outputs(SbArgs a) {
    __shared__ float Wt[64 * 65];      // Ws (padded rows)
    __shared__ float Gt[64 * 65];      // dWn
    __shared__ float Kt[kSbMax * kP], Qt[kSbMax * kP], Dt[kSbMax * kP], Rt[kSbMax * kP], dRt[kSbMax * kP];
    __shared__ float St[kSbMax * kSbMax], Pt[kSbMax * kSbMax];
    __shared__ float red[kSbT];
    const int tid = threadIdx.x;
    const int mb = blockIdx.x % a.nch;
    const ChainId c = chain_of(a, blockIdx.x / a.nch);
    const int n = nc_of(a, mb);
    const float eta = a.eta[c.h];
    const float alpha = -2.f * eta / (float)n;
    const float dzs = a.mode == 0 ? 0.5f : 1.f;
    {
        const float* ws = a.ws_state + ((long long)c.ch * a.nch + mb) * 4096;
        const float* gs = a.dwn_state + ((long long)c.ch * a.nch + mb) * 4096;
        for (int e = tid; e < 4096; e += kSbT) {
            Wt[(e >> 6) * 65 + (e & 63)] = ws[e];
            Gt[(e >> 6) * 65 + (e & 63)] = gs[e];
        }
        Tile t;
        load_tile<BF>(a, a.K, c, mb, 1.f, t);
        tile_to_lds(t, Kt);
        load_tile<BF>(a, a.Q, c, mb, 1.f, t);
        tile_to_lds(t, Qt);
        load_tile<BF>(a, a.dZ, c, mb, dzs, t);
        tile_to_lds(t, Dt);
        for (int e = tid; e < kSbMax * 64; e += kSbT) {
            const int s = e >> 6;
            dRt[s * kP + (e & 63)] = s < n ? a.dRp[((long long)c.ch * a.N + mb * a.b + s) * 64 + (e & 63)] : 0.f;
        }
    }
    __syncthreads();
    // R = K Ws^T - V
    for (int e = tid; e < n * 64; e += kSbT) {
        const int s = e >> 6, r = e & 63;
        float x = 0.f;
#pragma unroll 16
        for (int j = 0; j < 64; ++j) x = fmaf(Wt[r * 65 + j], Kt[s * kP + j], x);
        Rt[s * kP + r] = x - ldv<BF>(a.V, c.bb, c.h, pos_of(a, c, mb * a.b + s), r);
    }
    // S = Q K^T (s <= t)
    for (int e = tid; e < n * n; e += kSbT) {
        const int t = e / n, s = e % n;
        float x = 0.f;
        if (s <= t) {
#pragma unroll 16
            for (int j = 0; j < 64; ++j) x = fmaf(Qt[t * kP + j], Kt[s * kP + j], x);
        }
        St[t * kSbMax + s] = x;
    }
    __syncthreads();
    // P = dZ R^T (s <= t)
    for (int e = tid; e < n * n; e += kSbT) {
        const int t = e / n, s = e % n;
        float x = 0.f;
        if (s <= t) {
#pragma unroll 16
            for (int r = 0; r < 64; ++r) x = fmaf(Dt[t * kP + r], Rt[s * kP + r], x);
        }
        Pt[t * kSbMax + s] = x;
    }
    __syncthreads();
    float dal = 0.f; // this thread's share of d(alpha)
    for (int e = tid; e < n * 64; e += kSbT) {
        const int i = e >> 6, j = e & 63; // token row i, channel j
        // dQ[i][j] = dz_i . Ws[:, j] + alpha sum_{s <= i} P[i][s] k_s[j]
        float q = 0.f, kk = 0.f, rd = 0.f;
#pragma unroll 16
        for (int r = 0; r < 64; ++r) {
            q = fmaf(Dt[i * kP + r], Wt[r * 65 + j], q);
            kk = fmaf(dRt[i * kP + r], Wt[r * 65 + j], kk);
            rd = fmaf(Rt[i * kP + r], Gt[r * 65 + j], rd);
        }
        float pk = 0.f, pq = 0.f;
        for (int s = 0; s <= i; ++s) pk = fmaf(Pt[i * kSbMax + s], Kt[s * kP + j], pk);
        for (int t = i; t < n; ++t) pq = fmaf(Pt[t * kSbMax + i], Qt[t * kP + j], pq);
        const float dq = fmaf(alpha, pk, q);
        // dK[i][j] = dR_i . Ws[:, j] + alpha (R_i . dWn[:, j] + sum_{t >= i} P[t][i] q_t[j])
        const float dk = fmaf(alpha, rd + pq, kk);
        dal = fmaf(rd, Kt[i * kP + j], dal);
        const int pos = pos_of(a, c, mb * a.b + i);
        const float dv = -dRt[i * kP + j];
        if (a.nd == 1) {
            stv<BF>(a.dQ, c.bb, c.h, pos, j, dq);
            stv<BF>(a.dK, c.bb, c.h, pos, j, dk);
            stv<BF>(a.dV, c.bb, c.h, pos, j, dv);
        } else {
            const long long pl = (long long)a.B * a.H * a.N * 64, o = ((long long)c.slice * a.N + pos) * 64 + j;
            float* pb = a.planes + (long long)c.di * 3 * pl;
            pb[o] = dq;
            pb[pl + o] = dk;
            pb[2 * pl + o] = dv;
        }
    }
    for (int e = tid; e < n * n; e += kSbT) dal = fmaf(Pt[(e / n) * kSbMax + e % n], St[(e / n) * kSbMax + e % n], dal);
    red[tid] = dal;
    __syncthreads();
    for (int s = kSbT / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    if (tid == 0) a.detac[(long long)c.ch * a.nch + mb] = (-2.f / (float)n) * red[0];
}

// ---- outputs on the matrix cores (bf16 views, b <= 16) ---------------------
// One workgroup of four waves per token block, rows in token order: the
// tokens of one mini-batch of one direction (PLANES: that direction's fp32
// plane, the planes summed afterwards), or, when every direction's
// mini-batches cover the same tokens (one direction, or both with N a
// multiple of b: the reverse walk's mini-batch nch-1-c holds the forward
// mini-batch c's tokens), all of them, summed in registers and stored once.
// In the reverse direction walk slot s is row n-1-s, so the kept pairs
// "s <= t" become "row_s >= row_t"; nothing else depends on the order.
// Wave w forms output channels 16w .. 16w+15 and R's channels there.  bf16
// operands (the states and R, P rounded), fp32 accumulation; dV = -dR in
// fp32.  Sums of products of different matrix-core shapes are added on the
// vector unit.
constexpr int kMcRow = 144;          // bytes per staged 64-channel bf16 row (+16: banks)
constexpr int kMcTile = 16 * kMcRow; // 16 token rows
constexpr int kMcW = 64 * kMcRow;    // a 64 x 64 state

__device__ __forceinline__ v4s_t tr4(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
}
__device__ __forceinline__ u32x4 cat_tr(const v4s_t& lo, const v4s_t& hi) {
    const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
    return u32x4{l[0], l[1], h[0], h[1]};
}
__device__ __forceinline__ float bfe(const v4s_t& v, int i) {
    return __uint_as_float((uint32_t)(uint16_t)v[i] << 16);
}

template <bool PLANES>
__global__ __launch_bounds__(kSbT) void sbwd_outputs_mc(SbArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[6 * kMcTile + 2 * kMcW];
    __shared__ float red[4];
    char* const tK = lds;
    char* const tQ = lds + kMcTile;
    char* const tV = lds + 2 * kMcTile;
    char* const tZ = lds + 3 * kMcTile; // dZ, scaled as the direction receives it
    char* const tD = lds + 4 * kMcTile; // dR
    char* const tR = lds + 5 * kMcTile; // R
    char* const sW = lds + 6 * kMcTile; // Ws  [r][j]
    char* const sG = sW + kMcW;         // dWn [r][j]
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int e = m >> 2, aa = m & 3;
    int slice, c, di0, ndi;
    if (PLANES) {
        const int ch = blockIdx.x / a.nch;
        c = blockIdx.x % a.nch;
        slice = ch / a.nd;
        di0 = ch % a.nd;
        ndi = 1;
    } else {
        slice = blockIdx.x / a.nch;
        c = blockIdx.x % a.nch;
        di0 = 0;
        ndi = a.nd;
    }
    const int bb = slice / a.H, h = slice % a.H;
    const float eta = a.eta[h];
    const float zs = a.mode == 0 ? 0.5f : 1.f;
    const v4f z4{0.f, 0.f, 0.f, 0.f};
    // operand reads: a 16-row tile's row m, channels 8g.. (+32 kb) -- the
    // A operand, and the B operand whose columns are the tile's rows;
    // a state's rows 32kb + 8g .. +7 at channel 16w + m (B operand, k over
    // the state's rows); a tile's rows 4g .. 4g+3 at channel 16w + m
    auto rowop = [&](const char* t, int kb) { return *reinterpret_cast<const u32x4*>(t + m * kMcRow + 64 * kb + 16 * g); };
    auto colop = [&](const char* st, int kb) {
        const char* p = st + (32 * kb + 8 * g + e) * kMcRow + 2 * (16 * w + 4 * aa);
        return cat_tr(tr4(p), tr4(p + 4 * kMcRow));
    };
    auto col16 = [&](const char* t) { return tr4(t + (4 * g + e) * kMcRow + 2 * (16 * w + 4 * aa)); };
    v4f oQ = z4, oK = z4, oV = z4; // outputs at rows 4g+i, channel 16w+m
    // One pass per direction.  Every load of both passes is issued before
    // the first pass's products (registers), so the second pass does not
    // wait for memory again.  Loads are branch-free: a row past n loads a
    // clamped row and is zeroed after the load.
    struct Pass {
        int dir, ch, mb, n, tok_lo;
        u32x4 rows[2];  // K, Q, V, dZ rows: thread t holds 16-byte chunks t and t + 256
        f32x4 dr;       // dR, row tid / 16, channels 4 (tid % 16) ..
        u32x4 ws[2], gs[2]; // Ws, dWn chunks t and t + 256
        float dv[4];    // dR at rows 4g+i, channel 16w+m
    };
    auto pass_of = [&](int p) __attribute__((always_inline)) {
        Pass q;
        const int di = di0 + p;
        q.dir = chain_dir(a, di);
        q.ch = slice * a.nd + di;
        q.mb = (!PLANES && a.nd == 2 && q.dir == 1) ? a.nch - 1 - c : c;
        q.n = nc_of(a, q.mb);
        q.tok_lo = q.dir ? a.N - q.mb * a.b - q.n : q.mb * a.b;
        return q;
    };
    auto issue = [&](Pass& q) __attribute__((always_inline)) {
        // the views are picked by value (a reference picked at run time
        // would copy the arguments to scratch)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + kSbT * j, t = e >> 7, r = (e >> 3) & 15, ck = e & 7;
            const View4 v = j == 0 ? (t == 0 ? a.K : a.Q) : (t == 2 ? a.V : a.dZ);
            q.rows[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(v.ptr) + bb * v.sb + h * v.sh +
                                                        (long long)(q.tok_lo + min(r, q.n - 1)) * v.sn + 8 * ck);
        }
        {
            const int r = min(tid >> 4, q.n - 1), c4 = tid & 15;
            const int pos = q.dir ? a.N - 1 - (q.tok_lo + r) : q.tok_lo + r;
            q.dr = *reinterpret_cast<const f32x4*>(a.dRp + ((long long)q.ch * a.N + pos) * 64 + 4 * c4);
        }
        const u32x4* ws = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(a.ws_state) +
                                                         ((long long)q.ch * a.nch + q.mb) * 4096);
        const u32x4* gs = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(a.dwn_state) +
                                                         ((long long)q.ch * a.nch + q.mb) * 4096);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            q.ws[j] = ws[tid + kSbT * j];
            q.gs[j] = gs[tid + kSbT * j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = min(4 * g + i, q.n - 1);
            const int pos = q.dir ? a.N - 1 - (q.tok_lo + r) : q.tok_lo + r;
            q.dv[i] = a.dRp[((long long)q.ch * a.N + pos) * 64 + 16 * w + m];
        }
    };
    // (the two passes are separate variables: an array indexed by the pass
    // would live in scratch memory)
    Pass p0 = pass_of(0), p1 = p0;
    issue(p0);
    if (ndi > 1) {
        p1 = pass_of(1);
        issue(p1);
    }
    int tok_lo = 0, n = 0;
    auto run = [&](const Pass& q, bool later) __attribute__((always_inline)) {
        const int dir = q.dir, ch = q.ch, mb = q.mb;
        n = q.n;
        tok_lo = q.tok_lo;
        const float alpha = -2.f * eta / (float)n;
        if (later) __syncthreads(); // the previous pass has read every tile
        // K, Q, V, dZ rows (zeros past n; dZ scaled as the direction
        // receives it)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + kSbT * j, t = e >> 7, r = (e >> 3) & 15, ck = e & 7;
            u32x4 x = q.rows[j];
            if (t == 3)
#pragma unroll
                for (int k = 0; k < 4; ++k) x[k] = pack_bf2(zs * bflo(x[k]), zs * bfhi(x[k]));
            if (r >= n) x = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(lds + t * kMcTile + r * kMcRow + 16 * ck) = x;
        }
        // dR rows (bf16 in LDS)
        {
            const int r = tid >> 4, c4 = tid & 15;
            const f32x4 x = r < n ? q.dr : f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<u32x2*>(tD + r * kMcRow + 8 * c4) = u32x2{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3])};
        }
        // Ws and dWn (bf16, stored so by the matrix-core walks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + kSbT * j, o = (e >> 3) * kMcRow + 16 * (e & 7);
            *reinterpret_cast<u32x4*>(sW + o) = q.ws[j];
            *reinterpret_cast<u32x4*>(sG + o) = q.gs[j];
        }
        // dV = -dR (fp32)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * g + i < n) oV[i] -= q.dv[i];
        __syncthreads();
        // R = K Ws^T - V at channels 16w + m (B operand: Ws row 16w+m), to LDS
        {
            const char* wr = sW + (16 * w + m) * kMcRow + 16 * g;
            const v4f KW = mfma32(as_v8bf(rowop(tK, 1)), as_v8bf(*reinterpret_cast<const u32x4*>(wr + 64)),
                                  mfma32(as_v8bf(rowop(tK, 0)), as_v8bf(*reinterpret_cast<const u32x4*>(wr)), z4));
            const v4s_t vv = col16(tV);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<bf16_t*>(tR + (4 * g + i) * kMcRow + 2 * (16 * w + m)) = f2bf(KW[i] - bfe(vv, i));
        }
        __syncthreads();
        // S = Q K^T and P = dZ R^T at (t = 4g+i, s = m); P^T at (s = 4g+i, t = m)
        const v4f S = mfma32(as_v8bf(rowop(tQ, 1)), as_v8bf(rowop(tK, 1)), mfma32(as_v8bf(rowop(tQ, 0)), as_v8bf(rowop(tK, 0)), z4));
        const v4f P = mfma32(as_v8bf(rowop(tZ, 1)), as_v8bf(rowop(tR, 1)), mfma32(as_v8bf(rowop(tZ, 0)), as_v8bf(rowop(tR, 0)), z4));
        const v4f Pt = mfma32(as_v8bf(rowop(tR, 1)), as_v8bf(rowop(tZ, 1)), mfma32(as_v8bf(rowop(tR, 0)), as_v8bf(rowop(tZ, 0)), z4));
        float kp[4], kt[4]; // kept pairs: P layout (t = 4g+i, s = m), P^T layout (t = m, s = 4g+i)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            kp[i] = (dir ? m >= r : m <= r) ? 1.f : 0.f;
            kt[i] = (dir ? r >= m : r <= m) ? 1.f : 0.f;
        }
        const u32x2 Pk{pack_bf2(kp[0] * P[0], kp[1] * P[1]), pack_bf2(kp[2] * P[2], kp[3] * P[3])};
        const u32x2 Ptk{pack_bf2(kt[0] * Pt[0], kt[1] * Pt[1]), pack_bf2(kt[2] * Pt[2], kt[3] * Pt[3])};
        // the state operands, k over r, at channel 16w + m
        const u32x4 W0b = colop(sW, 0), W1b = colop(sW, 1), G0b = colop(sG, 0), G1b = colop(sG, 1);
        const v4s_t kc = col16(tK), qc = col16(tQ);
        // dQ = dZ Ws + alpha P_kept K
        const v4f q1 = mfma32(as_v8bf(rowop(tZ, 1)), as_v8bf(W1b), mfma32(as_v8bf(rowop(tZ, 0)), as_v8bf(W0b), z4));
        const v4f q2 = mfma16(as_v4s(Ptk), kc, z4);
        // dK = dR Ws + alpha (R dWn + P_kept^T Q)
        const v4f k1 = mfma32(as_v8bf(rowop(tD, 1)), as_v8bf(W1b), mfma32(as_v8bf(rowop(tD, 0)), as_v8bf(W0b), z4));
        const v4f k2 = mfma32(as_v8bf(rowop(tR, 1)), as_v8bf(G1b), mfma32(as_v8bf(rowop(tR, 0)), as_v8bf(G0b), z4));
        const v4f k3 = mfma16(as_v4s(Pk), qc, z4);
        // d(alpha) = <R dWn, K> + <P_kept, S>
        float dal = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            oQ[i] += q1[i] + alpha * q2[i];
            oK[i] += k1[i] + alpha * (k2[i] + k3[i]);
            dal = fmaf(k2[i], bfe(kc, i), dal);
            if (w == 0) dal = fmaf(kp[i] * P[i], S[i], dal);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) dal += __shfl_xor(dal, o);
        if (lane == 0) red[w] = dal;
        __syncthreads();
        if (tid == 0) a.detac[(long long)ch * a.nch + mb] = (-2.f / (float)n) * (((red[0] + red[1]) + red[2]) + red[3]);
    };
    run(p0, false);
    if (ndi > 1) run(p1, true);
    if (PLANES) {
        const long long pl = (long long)a.B * a.H * a.N * 64;
        float* pb = a.planes + (long long)di0 * 3 * pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            if (r < n) {
                const long long o = ((long long)slice * a.N + tok_lo + r) * 64 + 16 * w + m;
                pb[o] = oQ[i];
                pb[pl + o] = oK[i];
                pb[2 * pl + o] = oV[i];
            }
        }
        return;
    }
    // bf16 rows through LDS (the tiles are free once every wave is past the
    // d(alpha) barrier), stored 16 bytes a thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int o = (4 * g + i) * kMcRow + 2 * (16 * w + m);
        *reinterpret_cast<bf16_t*>(tK + o) = f2bf(oQ[i]);
        *reinterpret_cast<bf16_t*>(tQ + o) = f2bf(oK[i]);
        *reinterpret_cast<bf16_t*>(tV + o) = f2bf(oV[i]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = tid + kSbT * j, t = q >> 7, r = (q >> 3) & 15, ck = q & 7;
        if (q >= 3 * 128 || r >= n) continue;
        const View4 v = j == 0 ? (t == 0 ? a.dQ : a.dK) : a.dV;
        *reinterpret_cast<u32x4*>(reinterpret_cast<bf16_t*>(v.ptr) + bb * v.sb + h * v.sh + (long long)(tok_lo + r) * v.sn +
                                  8 * ck) = *reinterpret_cast<const u32x4*>(lds + t * kMcTile + r * kMcRow + 16 * ck);
    }
}

// ---- sums ------------------------------------------------------------------
// dW0 and deta per head, in fixed orders (dW0: chains in (b, direction) order).
__global__ __launch_bounds__(kSbT) void sbwd_sums(SbArgs a) {
    const int h = blockIdx.x / 16, part = blockIdx.x % 16, tid = threadIdx.x;
    const int ndw = a.w0dir ? 2 : 1;
    const int nchain = a.B * a.nd; // the head's chains, in (b, direction) order
    // Loads are issued eight at a time before their adds (a chain of the
    // other direction, or one past the end, adds zero: x + 0 is x, so the
    // order of the sums is the plain one)
    for (int wd = 0; wd < ndw; ++wd) {
        const int e = part * 256 + tid;
        float s = 0.f;
        for (int c0 = 0; c0 < nchain; c0 += 8) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = min(c0 + j, nchain - 1), bb = c / a.nd, di = c % a.nd;
                const bool use = c0 + j < nchain && (!a.w0dir || chain_dir(a, di) == wd);
                const float x = a.dW0c[(((long long)bb * a.H + h) * a.nd + di) * 4096 + e];
                t[j] = use ? x : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) s += t[j];
        }
        a.dW0[((long long)wd * a.H + h) * 4096 + e] = s;
    }
    if (part == 0) {
        // thread t sums mini-batches t, t + 256, ... of every chain of the
        // head (chains in (b, direction) order), then a fixed tree
        __shared__ float red[kSbT];
        const int per = (a.nch + kSbT - 1) / kSbT; // mini-batches of one chain per thread
        const int nitem = nchain * per;              // item i: chain i / per, mini-batch tid + 256 (i % per)
        float s = 0.f;
        for (int i0 = 0; i0 < nitem; i0 += 8) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = min(i0 + j, nitem - 1), c = i / per, mb = tid + kSbT * (i % per);
                const int bb = c / a.nd, di = c % a.nd;
                const float x = a.detac[(((long long)bb * a.H + h) * a.nd + di) * a.nch + min(mb, a.nch - 1)];
                t[j] = i0 + j < nitem && mb < a.nch ? x : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) s += t[j];
        }
        red[tid] = s;
        __syncthreads();
        for (int o = kSbT / 2; o > 0; o >>= 1) {
            if (tid < o) red[tid] += red[tid + o];
            __syncthreads();
        }
        if (tid == 0) a.deta[h] = red[0];
    }
}

// both directions: dQ, dK, dV = forward plane + reverse plane
template <bool BF>
__global__ __launch_bounds__(kSbT) void sbwd_planes(SbArgs a) {
    const long long pl = (long long)a.B * a.H * a.N * 64;
    const long long e = (long long)blockIdx.x * kSbT + threadIdx.x;
    if (e >= 3 * pl) return;
    const int which = (int)(e / pl);
    const long long o = e % pl;
    const int j = (int)(o & 63);
    const long long st = o >> 6;
    const int pos = (int)(st % a.N), slice = (int)(st / a.N);
    const float x = a.planes[which * pl + o] + a.planes[3 * pl + which * pl + o];
    const View4& v = which == 0 ? a.dQ : (which == 1 ? a.dK : a.dV);
    stv<BF>(v, slice / a.H, slice % a.H, pos, j, x);
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

} // namespace

bool scan_bwd_supported(int b) { return b >= 1 && b <= kSbMax; }

size_t scan_bwd_ws_bytes(int B, int H, int N, int b, int mode) {
    if (b < 1 || N < 1) return 0;
    const size_t slices = (size_t)B * H, nd = mode == 0 ? 2 : 1, chains = slices * nd;
    const size_t nch = (N + b - 1) / b;
    size_t bytes = 2 * a256(chains * nch * 4096 * 4);      // states, gradient states
    bytes += a256(chains * (size_t)N * 64 * 4);              // dR
    bytes += a256(chains * 4096 * 4) + a256(chains * nch * 4); // dW0, deta per chain
    if (nd == 2) bytes += a256(2 * 3 * slices * (size_t)N * 64 * 4);
    return bytes;
}

hipError_t launch_scan_bwd(const ScanBwdLaunch& s, hipStream_t stream) {
    SbArgs a{};
    a.K = s.K; a.Q = s.Q; a.V = s.V; a.dZ = s.dZ;
    a.dK = s.dK; a.dQ = s.dQ; a.dV = s.dV;
    a.W0 = s.W0; a.eta = s.eta; a.dW0 = s.dW0; a.deta = s.deta;
    a.B = s.B; a.H = s.H; a.N = s.N; a.b = s.b; a.mode = s.mode;
    a.nd = s.mode == 0 ? 2 : 1;
    a.nch = (s.N + s.b - 1) / s.b;
    a.w0dir = s.w0dir;
    a.bf16 = s.bf16;
    const size_t slices = (size_t)s.B * s.H, chains = slices * a.nd;
    char* w = (char*)s.ws;
    a.ws_state = (float*)w;
    w += a256(chains * a.nch * 4096 * 4);
    a.dwn_state = (float*)w;
    w += a256(chains * a.nch * 4096 * 4);
    a.dRp = (float*)w;
    w += a256(chains * (size_t)s.N * 64 * 4);
    a.dW0c = (float*)w;
    w += a256(chains * 4096 * 4);
    a.detac = (float*)w;
    w += a256(chains * a.nch * 4);
    a.planes = a.nd == 2 ? (float*)w : nullptr;
    const dim3 block(kSbT);
    const dim3 walks((unsigned)(chains * 4)), per_mb((unsigned)(chains * a.nch));
    // matrix-core outputs: one workgroup per token block covers every
    // direction when the directions' mini-batches coincide
    const bool fused = a.nd == 1 || s.N % s.b == 0;
    if (a.bf16) {
        if (s.walks) {
            ScanBwdWalks wk{};
            wk.K = s.K; wk.Q = s.Q; wk.V = s.V; wk.dZ = s.dZ;
            wk.W0 = s.W0; wk.eta = s.eta;
            // bf16 states in the first half of the fp32 state buffers
            wk.states = reinterpret_cast<uint16_t*>(a.ws_state);
            wk.dwn = reinterpret_cast<uint16_t*>(a.dwn_state);
            wk.dRp = a.dRp; wk.dW0c = a.dW0c;
            wk.B = s.B; wk.H = s.H; wk.N = s.N; wk.b = s.b; wk.mode = s.mode; wk.w0dir = s.w0dir;
            wk.cus = s.cus;
            const hipError_t e = launch_scan_bwd_walks(wk, stream);
            if (e != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL(sbwd_states<true>, walks, block, 0, stream, a);
            hipLaunchKernelGGL(sbwd_chain<true>, walks, block, 0, stream, a);
        }
        if (!s.walks) hipLaunchKernelGGL(sbwd_outputs<true>, per_mb, block, 0, stream, a);
        else if (fused) hipLaunchKernelGGL(sbwd_outputs_mc<false>, dim3((unsigned)(slices * a.nch)), block, 0, stream, a);
        else hipLaunchKernelGGL(sbwd_outputs_mc<true>, per_mb, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL(sbwd_states<false>, walks, block, 0, stream, a);
        hipLaunchKernelGGL(sbwd_chain<false>, walks, block, 0, stream, a);
        hipLaunchKernelGGL(sbwd_outputs<false>, per_mb, block, 0, stream, a);
    }
    hipLaunchKernelGGL(sbwd_sums, dim3((unsigned)(s.H * 16)), block, 0, stream, a);
    if (a.nd == 2 && !(a.bf16 && s.walks && fused)) {
        const long long n = 3LL * slices * s.N * 64;
        const dim3 g((unsigned)((n + kSbT - 1) / kSbT));
        if (a.bf16) hipLaunchKernelGGL(sbwd_planes<true>, g, block, 0, stream, a);
        else hipLaunchKernelGGL(sbwd_planes<false>, g, block, 0, stream, a);
    }
    return hipGetLastError();
}

} // namespace ttt
