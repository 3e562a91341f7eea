// minibatch_scan.hip -- mini-batch bidirectional TTT scan (Vision-TTT's
// linear inner model), gfx950.
//
// Per chain (slice, direction) the scan walks chunks of b <= 16 tokens with
// a 64x64 fp32 state W (Vision-TTT page, section on mini-batch parallel
// inference and its update equations).  With X = W^T held in fp32 matrix
// accumulators, one chunk is the dual form
//   R  = K_c X - V_c                          (16 x 64 residuals)
//   R' = -(2 eta / n_c) R
//   Z_c^T = X^T Q_c^T + R'^T tril(Q_c K_c^T)^T
//   X <- X + K_c^T R'
// which equals the token-by-token definition (each token's output sees the
// gradients of the chunk up to and including itself, all taken at the
// chunk-start state).  The 64 output rows of W evolve independently, so a
// chain is split into four 16-column blocks of X, one wave each; a wave
// never exchanges data with the other column blocks.
//
// Matrix-core plumbing (16x16 MFMA tiles, lane l = 16 g + m):
//  * X tile ct (ct = 0..3) holds X[pi(ct, 4g+i)][16 rt + m], where the row
//    permutation pi makes the eight k-slots of a lane in a 16x16x32 product
//    the contiguous channels 32 kb + 8 g .. +7.  One bf16 copy of X serves
//    as the B operand of K_c X and as the A operand of X^T Q_c^T.
//  * R comes out with lane (g, m) holding R[t = 4g+i][r = m]: exactly the B
//    operand of the 16x16x16 update and the A operand of R'^T (...).
//  * The update's A operand is K_c transposed (channel-major); each wave
//    writes its chunk of K to LDS channel-major and reads it back as 8-byte
//    rows.  V is transposed the same way for the initial value of R.
//  * tril(Q_c K_c^T)^T comes straight out of K_c Q_c^T's accumulator.
//
// Bidirectional average: the forward and backward waves of a column block
// share a workgroup and step in lockstep.  For each token, the direction
// that reaches it first stores its fp32 output in the workspace; the other
// one reads it back kPre chunks ahead of use (register prefetch), averages
// and stores the bf16 result.  Visibility: vector-memory operations of a
// wave complete in issue order, so a wave that has received the data of
// chunk j (loaded after its stores of step j - kPre) has completed those
// stores; a workgroup barrier then publishes them to its partner.  A
// prefetch issued at step j may therefore read outputs stored at steps
// <= j - kPre, i.e. tokens whose two arrivals are >= 2 kPre chunks apart.
// Tokens closer to the middle of the sequence are averaged after the scan
// from both stored fp32 outputs.
#include "common.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kPre = 6;       // chunks in flight per wave (register prefetch depth)
constexpr int kChunk = 16;    // token slots of one chunk (MFMA tile rows)
constexpr int kKtPitch = 20;  // LDS row pitch (bf16) of the channel-major K / V
constexpr int kLdsPerWave = (64 + 16) * kKtPitch; // bf16 elements

// Row permutation of the X tiles (see header).
__device__ __forceinline__ int pi_row(int ct, int rho) {
    return 32 * (ct >> 1) + 8 * (rho >> 2) + 4 * (ct & 1) + (rho & 3);
}

struct ScanArgs {
    View4 K, Q, V, Z;
    const float* W0;
    const float* eta;
    float* P;     // [slices][N][64] fp32: first-arrival outputs
    float* P2;    // [slices][N][64] fp32: second-arrival outputs near the middle
    float* dummy; // [blocks][2 waves][64 lanes][8] fp32: sink of masked-off stores
    int H, N, b, nch, slices, mode, ndir, xcd;
};

// One chunk's operands of one lane (token slot m): K and Q channels
// 32 kb + 8 g .. +7, V channels 16 rt + 4 g .. +3, and the partner's fp32
// output for the same token and channels (bidirectional mode).
struct ChunkRegs {
    u32x4 k[2], q[2];
    u32x2 v;
    f32x4 pp;
};

struct Lane {
    int lane, g, m, rt, dir, slice, h;
    const bf16_t *K, *Q, *V;
    bf16_t* Z;
    long long Ksn, Qsn, Vsn, Zsn;
    float* P;
    float* P2;
    float* sink;
};

// Reversed-sequence index -> token, and the chunk in which the partner
// direction meets the same token.
__device__ __forceinline__ int token_of(const ScanArgs& a, int dir, int rho) {
    return dir ? a.N - 1 - rho : rho;
}
__device__ __forceinline__ int partner_chunk(const ScanArgs& a, int dir, int p) {
    return (dir ? p : a.N - 1 - p) / a.b;
}
__device__ __forceinline__ bool defer_window(int j, int jp) {
    const int d = j - jp;
    return d < 2 * kPre && d > -2 * kPre;
}

__device__ __forceinline__ void issue_loads(const ScanArgs& a, const Lane& L, int j, ChunkRegs& r) {
    const int jc = min(j, a.nch - 1);
    const int rho = jc * a.b + L.m;
    const bool valid = L.m < a.b && rho < a.N;
    const int p = token_of(a, L.dir, valid ? rho : 0);
    const bf16_t* kp = L.K + (long long)p * L.Ksn + 8 * L.g;
    const bf16_t* qp = L.Q + (long long)p * L.Qsn + 8 * L.g;
    r.k[0] = *reinterpret_cast<const u32x4*>(kp);
    r.k[1] = *reinterpret_cast<const u32x4*>(kp + 32);
    r.q[0] = *reinterpret_cast<const u32x4*>(qp);
    r.q[1] = *reinterpret_cast<const u32x4*>(qp + 32);
    r.v = *reinterpret_cast<const u32x2*>(L.V + (long long)p * L.Vsn + 16 * L.rt + 4 * L.g);
    if (a.ndir == 2) {
        const int jp = partner_chunk(a, L.dir, p);
        const bool second = jc > jp || (jc == jp && L.dir == 1);
        const bool use = valid && j < a.nch && second && !defer_window(jc, jp);
        const float* src = use ? L.P + (long long)p * 64 + 16 * L.rt + 4 * L.g : L.sink;
        r.pp = *reinterpret_cast<const f32x4*>(src);
    }
}

__device__ __forceinline__ uint32_t sel0(bool keep, uint32_t v) { return keep ? v : 0u; }

template <int D>
__device__ __forceinline__ void scan_chain(const ScanArgs& a, const Lane& L, bf16_t* kt, bf16_t* vt) {
    const int g = L.g, m = L.m;
    const float eta = a.eta[L.h];

    // X = W0^T in accumulator layout
    v4f X[4];
    {
        const float* w = a.W0 + (long long)L.h * 4096 + (16 * L.rt + m) * 64 + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(w + 32 * kb);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(w + 32 * kb + 4);
            X[2 * kb] = v4f{lo[0], lo[1], lo[2], lo[3]};
            X[2 * kb + 1] = v4f{hi[0], hi[1], hi[2], hi[3]};
        }
    }

    ChunkRegs cr[D];
#pragma unroll
    for (int u = 0; u < D; ++u) issue_loads(a, L, u, cr[u]);

    const bool ragged_all = a.b < kChunk;
    const int nsteps = ((a.nch + D - 1) / D) * D;
    for (int j0 = 0; j0 < nsteps; j0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int j = j0 + u;
            ChunkRegs& r = cr[u];
            const int rho = j * a.b + m;
            const bool valid = j < a.nch && m < a.b && rho < a.N;
            const int nc = min(a.b, a.N - j * a.b);
            if (ragged_all || j >= a.nch - 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    r.k[0][e] = sel0(valid, r.k[0][e]);
                    r.k[1][e] = sel0(valid, r.k[1][e]);
                    r.q[0][e] = sel0(valid, r.q[0][e]);
                    r.q[1][e] = sel0(valid, r.q[1][e]);
                }
                r.v[0] = sel0(valid, r.v[0]);
                r.v[1] = sel0(valid, r.v[1]);
            }
            const float alpha = nc > 0 ? -2.0f * eta / (float)nc : 0.f;

            // channel-major K and V of this chunk into the wave's LDS
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = r.k[kb][e];
                    const int c = 32 * kb + 8 * g + 2 * e;
                    kt[c * kKtPitch + m] = (bf16_t)(w & 0xffffu);
                    kt[(c + 1) * kKtPitch + m] = (bf16_t)(w >> 16);
                }
            vt[(4 * g + 0) * kKtPitch + m] = (bf16_t)(r.v[0] & 0xffffu);
            vt[(4 * g + 1) * kKtPitch + m] = (bf16_t)(r.v[0] >> 16);
            vt[(4 * g + 2) * kKtPitch + m] = (bf16_t)(r.v[1] & 0xffffu);
            vt[(4 * g + 3) * kKtPitch + m] = (bf16_t)(r.v[1] >> 16);
            u32x2 ktA[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                ktA[ct] = *reinterpret_cast<const u32x2*>(kt + pi_row(ct, m) * kKtPitch + 4 * g);
            const u32x2 vin = *reinterpret_cast<const u32x2*>(vt + m * kKtPitch + 4 * g);

            // bf16 copy of the chunk-start state
            v8bf xb[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 u4{pack_bf2(X[2 * kb][0], X[2 * kb][1]), pack_bf2(X[2 * kb][2], X[2 * kb][3]),
                               pack_bf2(X[2 * kb + 1][0], X[2 * kb + 1][1]),
                               pack_bf2(X[2 * kb + 1][2], X[2 * kb + 1][3])};
                xb[kb] = as_v8bf(u4);
            }
            // R = K X - V
            v4f R = v4f{-bflo(vin[0]), -bfhi(vin[0]), -bflo(vin[1]), -bfhi(vin[1])};
            R = mfma32(as_v8bf(r.k[0]), xb[0], R);
            R = mfma32(as_v8bf(r.k[1]), xb[1], R);
            const u32x2 rp2{pack_bf2(alpha * R[0], alpha * R[1]), pack_bf2(alpha * R[2], alpha * R[3])};
            const v4s rp = as_v4s(rp2);
            // X += K^T R'
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) X[ct] = mfma16(as_v4s(ktA[ct]), rp, X[ct]);

            // Z^T = X^T Q^T + R'^T tril(Q K^T)^T   (chunk-start X)
            v4f S = v4f{0.f, 0.f, 0.f, 0.f};
            S = mfma32(as_v8bf(r.k[0]), as_v8bf(r.q[0]), S);
            S = mfma32(as_v8bf(r.k[1]), as_v8bf(r.q[1]), S);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * g + i > m) S[i] = 0.f;
            const u32x2 sb2{pack_bf2(S[0], S[1]), pack_bf2(S[2], S[3])};
            v4f Zt = v4f{0.f, 0.f, 0.f, 0.f};
            Zt = mfma32(xb[0], as_v8bf(r.q[0]), Zt);
            Zt = mfma32(xb[1], as_v8bf(r.q[1]), Zt);
            Zt = mfma16(rp, as_v4s(sb2), Zt);

            // outputs of token slot m, channels 16 rt + 4 g .. +3
            const int p = token_of(a, L.dir, valid ? rho : 0);
            const long long zoff = (long long)p * L.Zsn + 16 * L.rt + 4 * g;
            const long long poff = (long long)p * 64 + 16 * L.rt + 4 * g;
            if (a.ndir == 1) {
                bf16_t* dz = valid ? L.Z + zoff : reinterpret_cast<bf16_t*>(L.sink);
                __builtin_nontemporal_store(u32x2{pack_bf2(Zt[0], Zt[1]), pack_bf2(Zt[2], Zt[3])},
                                            reinterpret_cast<u32x2*>(dz));
            } else {
                const int jp = partner_chunk(a, L.dir, p);
                const bool first = j < jp || (j == jp && L.dir == 0);
                const bool defer = defer_window(j, jp);
                float* dp = !valid ? L.sink : (first ? L.P + poff : (defer ? L.P2 + poff : L.sink));
                *reinterpret_cast<f32x4*>(dp) = f32x4{Zt[0], Zt[1], Zt[2], Zt[3]};
                const bool fin = valid && !first && !defer;
                const f32x4 o = r.pp;
                bf16_t* dz = fin ? L.Z + zoff : reinterpret_cast<bf16_t*>(L.sink + 4);
                __builtin_nontemporal_store(u32x2{pack_bf2(0.5f * (Zt[0] + o[0]), 0.5f * (Zt[1] + o[1])),
                                                  pack_bf2(0.5f * (Zt[2] + o[2]), 0.5f * (Zt[3] + o[3]))},
                                            reinterpret_cast<u32x2*>(dz));
                // partner's stores of steps <= j - kPre are complete: publish
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            issue_loads(a, L, j + D, r);
        }
    }
}

__global__ __launch_bounds__(128, 1) void scan_kernel(ScanArgs a) {
    __shared__ __attribute__((aligned(16))) bf16_t lds[2 * kLdsPerWave];
    const SliceSplit ss = map_block(blockIdx.x, 4, a.xcd);
    if (ss.slice >= a.slices) return; // padding block of the XCD-aware grid
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= a.ndir) return;
    Lane L;
    L.lane = threadIdx.x & 63;
    L.g = L.lane >> 4;
    L.m = L.lane & 15;
    L.rt = ss.split;
    L.dir = a.ndir == 2 ? w : (a.mode == 2 ? 1 : 0);
    L.slice = ss.slice;
    const int bb = ss.slice / a.H;
    L.h = ss.slice % a.H;
    L.K = (const bf16_t*)a.K.ptr + bb * a.K.sb + L.h * a.K.sh;
    L.Q = (const bf16_t*)a.Q.ptr + bb * a.Q.sb + L.h * a.Q.sh;
    L.V = (const bf16_t*)a.V.ptr + bb * a.V.sb + L.h * a.V.sh;
    L.Z = (bf16_t*)a.Z.ptr + bb * a.Z.sb + L.h * a.Z.sh;
    L.Ksn = a.K.sn; L.Qsn = a.Q.sn; L.Vsn = a.V.sn; L.Zsn = a.Z.sn;
    L.P = a.P ? a.P + (long long)ss.slice * a.N * 64 : nullptr;
    L.P2 = a.P2 ? a.P2 + (long long)ss.slice * a.N * 64 : nullptr;
    L.sink = a.dummy + ((long long)blockIdx.x * 2 + w) * 512 + L.lane * 8;
    bf16_t* kt = lds + w * kLdsPerWave;
    scan_chain<kPre>(a, L, kt, kt + 64 * kKtPitch);

    if (a.ndir == 2) {
        // tokens whose two arrivals are < 2 kPre chunks apart: average the
        // two stored fp32 outputs
        drain_vmem();
        __syncthreads();
        const int span = (2 * kPre + 1) * a.b;
        const int lo = max(0, (a.N - 1) / 2 - span), hi = min(a.N, a.N / 2 + span + 1);
        for (int e = threadIdx.x; e < (hi - lo) * 4; e += 64 * a.ndir) {
            const int p = lo + (e >> 2), c = 16 * L.rt + 4 * (e & 3);
            const int jf = p / a.b, jb = (a.N - 1 - p) / a.b;
            if (!defer_window(jf, jb)) continue;
            const f32x4 x = *reinterpret_cast<const f32x4*>(L.P + (long long)p * 64 + c);
            const f32x4 y = *reinterpret_cast<const f32x4*>(L.P2 + (long long)p * 64 + c);
            *reinterpret_cast<u32x2*>(L.Z + (long long)p * L.Zsn + c) =
                u32x2{pack_bf2(0.5f * (x[0] + y[0]), 0.5f * (x[1] + y[1])),
                      pack_bf2(0.5f * (x[2] + y[2]), 0.5f * (x[3] + y[3]))};
        }
    }
}

long long padded_slices(int B, int H) {
    const long long s = (long long)B * H;
    return (s + 7) / 8 * 8;
}

} // namespace

size_t scan_ws_bytes(int B, int H, int N, int mode) {
    const long long blocks = padded_slices(B, H) * 4;
    size_t bytes = (size_t)blocks * 2 * 512 * sizeof(float);
    if (mode == 0) bytes += 2 * (size_t)B * H * N * 64 * sizeof(float);
    return bytes;
}

hipError_t launch_scan(ScanLaunch s, hipStream_t stream) {
    if (!s.bf16) return hipErrorNotSupported;
    ScanArgs a{};
    a.K = s.K; a.Q = s.Q; a.V = s.V; a.Z = s.Z;
    a.W0 = s.W0; a.eta = s.eta;
    a.H = s.H; a.N = s.N; a.b = s.b;
    a.nch = (s.N + s.b - 1) / s.b;
    a.slices = s.B * s.H;
    a.mode = s.mode;
    a.ndir = s.mode == 0 ? 2 : 1;
    a.xcd = 1;
    const long long blocks = padded_slices(s.B, s.H) * 4;
    float* base = (float*)s.ws;
    a.dummy = base;
    if (a.ndir == 2) {
        a.P = base + blocks * 2 * 512;
        a.P2 = a.P + (size_t)a.slices * s.N * 64;
    }
    hipLaunchKernelGGL(scan_kernel, dim3((unsigned)blocks), dim3(64 * a.ndir), 0, stream, a);
    return hipGetLastError();
}

} // namespace ttt
