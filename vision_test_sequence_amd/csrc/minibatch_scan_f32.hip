// minibatch_scan_f32.hip -- the bidirectional mini-batch scan for fp32
// views, on the vector ALUs in fp32 throughout (the bf16 path runs on the
// matrix cores in minibatch_scan.hip).  Vision-TTT notes, key designs 2
// and 4: per direction, mini-batches of b walk positions (the last one
// n_c <= b), with mini-batch start state Ws and alpha = -2 eta / n_c,
//   R_s = Ws k_s - v_s,   z_t = W_t q_t,   W_t = Ws + alpha sum_{s <= t} R_s k_s^T,
// and after the mini-batch Ws <- W_last.
//
// The 64 rows of W (output channels) evolve independently, so one
// workgroup per (chain, 16-row block of W) walks the whole chain and forms
// its 16 output channels of every token; no workgroups meet.  A mini-batch
// is walked in sub-blocks of up to 32 positions: the residuals of every
// sub-block use Ws, the outputs use the running state (Ws plus the earlier
// sub-blocks' updates) and the sub-block's own causal term,
//   z_t = W_run q_t + alpha sum_{s <= t, s in the sub-block} (q_t . k_s) R_s,
// which together are W_t q_t for any b.  Both directions: fp32 planes per
// direction in the workspace, averaged by a second kernel.
#include "common.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kFT = 256; // threads per workgroup
constexpr int kFS = 32;  // positions per sub-block
constexpr int kFP = 65;  // LDS pitch (floats) of 64-wide rows

struct F32Args {
    View4 K, Q, V, Z;
    const float* W0;
    const float* eta;
    float* P;  // both directions: [slices][N][64] forward outputs
    float* P2; // [slices][N][64] reverse outputs
    int B, H, N, b, mode, w0dir, nd;
};

__device__ __forceinline__ const float* row_of(const View4& v, int bb, int h, long long tok) {
    return reinterpret_cast<const float*>(v.ptr) + bb * v.sb + h * v.sh + tok * v.sn;
}

__global__ __launch_bounds__(kFT) void scan_f32(F32Args a) {
    __shared__ float Ws[16 * kFP], Wr[16 * kFP]; // rows 16 rb .. of the start and running states
    __shared__ float Kt[kFS * kFP], Qt[kFS * kFP];
    __shared__ float Vt[kFS * 17], Rt[kFS * 17], St[kFS * kFS];
    const int tid = threadIdx.x, rb = blockIdx.x & 3, ch = blockIdx.x >> 2;
    const int slice = ch / a.nd, di = ch % a.nd;
    const int dir = a.mode == 2 ? 1 : (a.mode == 0 ? di : 0);
    const int bb = slice / a.H, h = slice % a.H;
    const float eta = a.eta[h];
    const float* W0 = a.W0 + ((a.w0dir && dir ? (long long)a.H : 0) + h) * 4096 + rb * 1024;
    for (int e = tid; e < 1024; e += kFT) Ws[(e >> 6) * kFP + (e & 63)] = Wr[(e >> 6) * kFP + (e & 63)] = W0[e];
    float* plane = a.mode == 0 ? (dir ? a.P2 : a.P) + (long long)slice * a.N * 64 : nullptr;
    const int nch = (a.N + a.b - 1) / a.b;
    for (int c = 0; c < nch; ++c) {
        const int n = min(a.b, a.N - c * a.b);
        const float alpha = -2.f * eta / (float)n;
        for (int j0 = 0; j0 < n; j0 += kFS) {
            const int m = min(kFS, n - j0);
            __syncthreads(); // the previous sub-block's reads and the state update are done
            // K, Q rows (64 channels), V's 16 channels of the block; zeros past m
            for (int e = tid; e < kFS * 64; e += kFT) {
                const int s = e >> 6, cc = e & 63;
                const long long pos = (long long)c * a.b + j0 + s;
                const long long tok = dir ? a.N - 1 - pos : pos;
                const bool ok = s < m;
                Kt[s * kFP + cc] = ok ? row_of(a.K, bb, h, tok)[cc] : 0.f;
                Qt[s * kFP + cc] = ok ? row_of(a.Q, bb, h, tok)[cc] : 0.f;
                if (cc < 16) Vt[s * 17 + cc] = ok ? row_of(a.V, bb, h, tok)[16 * rb + cc] : 0.f;
            }
            __syncthreads();
            // R[s][r] = Ws[r] . k_s - v_s[r];  S[t][s] = q_t . k_s (s <= t)
            for (int e = tid; e < m * 16; e += kFT) {
                const int s = e >> 4, r = e & 15;
                float x = 0.f;
#pragma unroll 16
                for (int j = 0; j < 64; ++j) x = fmaf(Ws[r * kFP + j], Kt[s * kFP + j], x);
                Rt[s * 17 + r] = x - Vt[s * 17 + r];
            }
            for (int e = tid; e < m * m; e += kFT) {
                const int t = e / m, s = e % m;
                float x = 0.f;
                if (s <= t) {
#pragma unroll 16
                    for (int j = 0; j < 64; ++j) x = fmaf(Qt[t * kFP + j], Kt[s * kFP + j], x);
                }
                St[t * kFS + s] = x;
            }
            __syncthreads();
            // z_t[r] = W_run[r] . q_t + alpha sum_{s <= t} S[t][s] R[s][r]
            for (int e = tid; e < m * 16; e += kFT) {
                const int t = e >> 4, r = e & 15;
                float x = 0.f;
#pragma unroll 16
                for (int j = 0; j < 64; ++j) x = fmaf(Wr[r * kFP + j], Qt[t * kFP + j], x);
                float y = 0.f;
                for (int s = 0; s <= t; ++s) y = fmaf(St[t * kFS + s], Rt[s * 17 + r], y);
                const float z = fmaf(alpha, y, x);
                const long long pos = (long long)c * a.b + j0 + t;
                const long long tok = dir ? a.N - 1 - pos : pos;
                if (plane) plane[tok * 64 + 16 * rb + r] = z;
                else reinterpret_cast<float*>(a.Z.ptr)[bb * a.Z.sb + h * a.Z.sh + tok * a.Z.sn + 16 * rb + r] = z;
            }
            __syncthreads(); // W_run is read; now its update
            // W_run[r][j] += alpha sum_s R[s][r] K[s][j]
            for (int e = tid; e < 1024; e += kFT) {
                const int r = e >> 6, j = e & 63;
                float x = 0.f;
                for (int s = 0; s < m; ++s) x = fmaf(Rt[s * 17 + r], Kt[s * kFP + j], x);
                Wr[r * kFP + j] = fmaf(alpha, x, Wr[r * kFP + j]);
            }
        }
        __syncthreads();
        // the mini-batch ends: its last running state starts the next one
        for (int e = tid; e < 1024; e += kFT) Ws[(e >> 6) * kFP + (e & 63)] = Wr[(e >> 6) * kFP + (e & 63)];
    }
}

// Both directions: Z = (P + P2) / 2, one float4 per thread.
__global__ __launch_bounds__(kFT) void scan_f32_average(F32Args a) {
    const long long e = (long long)blockIdx.x * kFT + threadIdx.x; // (slice, token, channel quad)
    const long long n = (long long)a.B * a.H * a.N * 16;
    if (e >= n) return;
    const int q = (int)(e & 15);
    const long long st = e >> 4;
    const int tok = (int)(st % a.N), slice = (int)(st / a.N);
    const f32x4 x = reinterpret_cast<const f32x4*>(a.P)[e], y = reinterpret_cast<const f32x4*>(a.P2)[e];
    float* z = reinterpret_cast<float*>(a.Z.ptr) + (slice / a.H) * a.Z.sb + (slice % a.H) * a.Z.sh +
               (long long)tok * a.Z.sn + 4 * q;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = 0.5f * (x[i] + y[i]);
}

} // namespace

hipError_t launch_scan_f32(const ScanLaunch& s, hipStream_t stream) {
    F32Args a{};
    a.K = s.K; a.Q = s.Q; a.V = s.V; a.Z = s.Z;
    a.W0 = s.W0; a.eta = s.eta;
    a.B = s.B; a.H = s.H; a.N = s.N; a.b = s.b; a.mode = s.mode; a.w0dir = s.w0dir;
    a.nd = s.mode == 0 ? 2 : 1;
    // workspace: [256 bytes reserved][P][P2] (the layout of the bf16 scan's)
    float* cur = (float*)s.ws + 64;
    if (s.mode == 0) {
        a.P = cur;
        a.P2 = a.P + (size_t)s.B * s.H * s.N * 64;
    }
    const long long chains = (long long)s.B * s.H * a.nd;
    hipLaunchKernelGGL(scan_f32, dim3((unsigned)(4 * chains)), dim3(kFT), 0, stream, a);
    if (s.mode == 0) {
        const long long n = (long long)s.B * s.H * s.N * 16;
        hipLaunchKernelGGL(scan_f32_average, dim3((unsigned)((n + kFT - 1) / kFT)), dim3(kFT), 0, stream, a);
    }
    return hipGetLastError();
}

} // namespace ttt
