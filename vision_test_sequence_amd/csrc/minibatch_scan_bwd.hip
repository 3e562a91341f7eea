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
// fp32 arithmetic on the vector ALUs throughout (bf16 or fp32 views); the
// serial walks prefetch the next mini-batch's rows into registers while
// the current one is computed.
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
    float* ws_state;   // [chains][nch][64][64]: forward start states
    float* dwn_state;  // [chains][nch][64][64]: gradient at each mini-batch's end
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

// ---- sums ------------------------------------------------------------------
// dW0 and deta per head: chains in (b, direction) order, mini-batches in order.
__global__ __launch_bounds__(kSbT) void sbwd_sums(SbArgs a) {
    const int h = blockIdx.x / 16, part = blockIdx.x % 16, tid = threadIdx.x;
    const int ndw = a.w0dir ? 2 : 1;
    for (int wd = 0; wd < ndw; ++wd) {
        const int e = part * 256 + tid;
        float s = 0.f;
        for (int bb = 0; bb < a.B; ++bb)
            for (int di = 0; di < a.nd; ++di) {
                if (a.w0dir && chain_dir(a, di) != wd) continue;
                const long long ch = ((long long)bb * a.H + h) * a.nd + di;
                s += a.dW0c[ch * 4096 + e];
            }
        a.dW0[((long long)wd * a.H + h) * 4096 + e] = s;
    }
    if (part == 0 && tid == 0) {
        float s = 0.f;
        for (int bb = 0; bb < a.B; ++bb)
            for (int di = 0; di < a.nd; ++di) {
                const long long ch = ((long long)bb * a.H + h) * a.nd + di;
                for (int mb = 0; mb < a.nch; ++mb) s += a.detac[ch * a.nch + mb];
            }
        a.deta[h] = s;
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
    if (a.bf16) {
        if (s.walks) {
            ScanBwdWalks wk{};
            wk.K = s.K; wk.Q = s.Q; wk.V = s.V; wk.dZ = s.dZ;
            wk.W0 = s.W0; wk.eta = s.eta;
            wk.states = a.ws_state; wk.dwn = a.dwn_state; wk.dRp = a.dRp; wk.dW0c = a.dW0c;
            wk.B = s.B; wk.H = s.H; wk.N = s.N; wk.b = s.b; wk.mode = s.mode; wk.w0dir = s.w0dir;
            const hipError_t e = launch_scan_bwd_walks(wk, stream);
            if (e != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL(sbwd_states<true>, walks, block, 0, stream, a);
            hipLaunchKernelGGL(sbwd_chain<true>, walks, block, 0, stream, a);
        }
        hipLaunchKernelGGL(sbwd_outputs<true>, per_mb, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL(sbwd_states<false>, walks, block, 0, stream, a);
        hipLaunchKernelGGL(sbwd_chain<false>, walks, block, 0, stream, a);
        hipLaunchKernelGGL(sbwd_outputs<false>, per_mb, block, 0, stream, a);
    }
    hipLaunchKernelGGL(sbwd_sums, dim3((unsigned)(s.H * 16)), block, 0, stream, a);
    if (a.nd == 2) {
        const long long n = 3LL * slices * s.N * 64;
        const dim3 g((unsigned)((n + kSbT - 1) / kSbT));
        if (a.bf16) hipLaunchKernelGGL(sbwd_planes<true>, g, block, 0, stream, a);
        else hipLaunchKernelGGL(sbwd_planes<false>, g, block, 0, stream, a);
    }
    return hipGetLastError();
}

} // namespace ttt
