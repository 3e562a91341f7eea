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

constexpr int kPre = 4;    // chunks in flight per wave (register prefetch depth)
constexpr int kChunk = 16; // token slots of one chunk (MFMA tile rows)
constexpr int kKRow = 144; // bytes per staged K row (64 channels + pad)
constexpr int kVRow = 48;  // bytes per staged V row (this block's 16 channels + pad)
constexpr int kWaveLds = kChunk * (kKRow + kVRow);

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s;

struct ScanArgs {
    View4 K, Q, V, Z;
    const float* W0;
    const float* eta;
    float* P;     // [slices][N][64] fp32: first-arrival outputs
    float* P2;    // [slices][N][64] fp32: second-arrival outputs near the middle
    float* dummy; // [blocks][2 waves][64 lanes][8] fp32: sink of masked-off stores
    const char* zeros; // 256 zero bytes (never written): the rows of empty slots
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

// Per-lane walk of one chain.  Token slot m of chunk j is token
// p = j*b + m (forward) or N-1-(j*b + m) (reverse); the chunk in which the
// partner direction meets that token is c0 - j with c0 = (N-1-m) / b, in
// both directions.
struct Walk {
    int g, m, rt, dir, b, N, nch;
    int c0;                   // partner chunk of slot m at chunk 0
    long long step;           // +-1 token per chunk step of b tokens, as +-b
    const char *K, *Q, *V;    // token 0 row + this lane's channel offset
    const char *Kn, *Qn, *Vn; // running: rows of the next chunk to load
    long long Ksn, Qsn, Vsn;  // bytes per token
    const float* Pn;          // running: partner's output of the next chunk
    const float* Pbase;
    const char* zeros;
    char* Z;                  // token 0 + channel offset (bytes)
    long long Zsn;
    float *P, *P2;            // token 0 + channel offset
    float* sink;
};

__device__ __forceinline__ int token_of(const Walk& L, int rho) { return L.dir ? L.N - 1 - rho : rho; }
__device__ __forceinline__ bool defer_d(int d) { return d < 2 * kPre && d > -2 * kPre; }

__device__ __forceinline__ void issue_loads(const ScanArgs& a, Walk& L, int jj, ChunkRegs& r) {
    const char *kp, *qp, *vp;
    const float* pp = L.sink;
    const bool inrange = jj < L.nch - 1 || (jj == L.nch - 1 && jj * L.b + kChunk - 1 < L.N);
    if (inrange && L.m < L.b) { // every slot a token of this chunk (uniform but for m)
        kp = L.Kn;
        qp = L.Qn;
        vp = L.Vn;
        if (a.ndir == 2 && 2 * jj - L.c0 >= 2 * kPre) pp = L.Pn;
    } else { // ragged or past the end: clamp to a valid token
        const int jc = min(jj, L.nch - 1);
        const int rho = jc * L.b + L.m;
        const bool valid = jj < L.nch && L.m < L.b && rho < L.N;
        const int p = token_of(L, valid ? rho : 0);
        // a slot without a token reads zero rows: it then adds nothing to
        // the state or to the other slots' outputs
        kp = valid ? L.K + p * L.Ksn : L.zeros;
        qp = valid ? L.Q + p * L.Qsn : L.zeros;
        vp = valid ? L.V + p * L.Vsn : L.zeros;
        if (a.ndir == 2 && valid && jj < L.nch && 2 * jc - L.c0 >= 2 * kPre) pp = L.Pbase + (long long)p * 64;
    }
    r.k[0] = *reinterpret_cast<const u32x4*>(kp);
    r.k[1] = *reinterpret_cast<const u32x4*>(kp + 64);
    r.q[0] = *reinterpret_cast<const u32x4*>(qp);
    r.q[1] = *reinterpret_cast<const u32x4*>(qp + 64); // (the zero block is 256 bytes)
    r.v = *reinterpret_cast<const u32x2*>(vp);
    if (a.ndir == 2) r.pp = *reinterpret_cast<const f32x4*>(pp);
    L.Kn += L.step * L.Ksn;
    L.Qn += L.step * L.Qsn;
    L.Vn += L.step * L.Vsn;
    L.Pn += L.step * 64;
}

__device__ __forceinline__ v4s_t tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
}

template <int D>
__device__ __forceinline__ void scan_chain(const ScanArgs& a, Walk& L, char* kt, char* vt, const float* W0h,
                                           float eta) {
    const int g = L.g, m = L.m, lane = 16 * g + m;

    // X = W0^T in accumulator layout
    v4f X[4];
    {
        const float* w = W0h + (16 * L.rt + m) * 64 + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(w + 32 * kb);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(w + 32 * kb + 4);
            X[2 * kb] = v4f{lo[0], lo[1], lo[2], lo[3]};
            X[2 * kb + 1] = v4f{hi[0], hi[1], hi[2], hi[3]};
        }
    }
    // LDS addresses.  Writes: this lane's K row chunks and V row piece.
    // Transposing reads (in each 16-lane group, lane 4e + a points at a
    // 4-element row piece; lane m of the group receives element m % 4 of
    // the pieces of lanes 4e + m/4, e = 0..3):
    //  * update operand of X tile ct: lane (g, 4e + a) points at token
    //    4g + e, channels pi(ct, 4a) .. +3 = 32(ct>>1) + 8a + 4(ct&1);
    //  * initial R (= -V^T): token 4g + e, channels 4a .. +3 of the block.
    const int e = (lane & 15) >> 2, aa = lane & 3;
    char* kw = kt + m * kKRow + 16 * g;
    char* vw = vt + m * kVRow + 8 * g;
    const char* kr = kt + (4 * g + e) * kKRow + 16 * aa;
    const char* vr = vt + (4 * g + e) * kVRow + 8 * aa;

    ChunkRegs cr[D];
#pragma unroll
    for (int u = 0; u < D; ++u) issue_loads(a, L, u, cr[u]);

    const float alpha_full = -2.0f * eta / (float)L.b;
    const int nlast = L.N - (L.nch - 1) * L.b;
    const float alpha_last = -2.0f * eta / (float)nlast;
    const bool ragged_all = L.b < kChunk;
    // running output pointers of chunk j
    const long long zst = L.step * L.Zsn;
    char* zp = L.Z + (long long)token_of(L, m) * L.Zsn;
    float* p1 = L.P + (long long)token_of(L, m) * 64;
    float* p2 = L.P2 + (long long)token_of(L, m) * 64;
    const long long pst = L.step * 64;
    const int nsteps = ((L.nch + D - 1) / D) * D;
    for (int j0 = 0; j0 < nsteps; j0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int j = j0 + u;
            ChunkRegs& r = cr[u];
            // slots without a token hold zero rows (see issue_loads)
            const bool valid = (!ragged_all && j < L.nch - 1) || (j < L.nch && m < L.b && j * L.b + m < L.N);
            const float alpha = j < L.nch - 1 ? alpha_full : (j == L.nch - 1 ? alpha_last : 0.f);

            // this chunk's K rows and V piece into the wave's LDS, read back
            // transposed
            *reinterpret_cast<u32x4*>(kw) = r.k[0];
            *reinterpret_cast<u32x4*>(kw + 64) = r.k[1];
            *reinterpret_cast<u32x2*>(vw) = r.v;
            v4s_t ktA[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) ktA[ct] = tr_read(kr + 64 * (ct >> 1) + 8 * (ct & 1));
            const v4s_t vin = tr_read(vr);

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
            v4f R;
#pragma unroll
            for (int i = 0; i < 4; ++i) R[i] = -bf2f((bf16_t)vin[i]);
            R = mfma32(as_v8bf(r.k[0]), xb[0], R);
            R = mfma32(as_v8bf(r.k[1]), xb[1], R);
            const u32x2 rp2{pack_bf2(alpha * R[0], alpha * R[1]), pack_bf2(alpha * R[2], alpha * R[3])};
            const v4s rp = as_v4s(rp2);
            // X += K^T R'
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) X[ct] = mfma16(ktA[ct], rp, X[ct]);

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
            if (a.ndir == 1) {
                bf16_t* dz = valid ? reinterpret_cast<bf16_t*>(zp) : reinterpret_cast<bf16_t*>(L.sink);
                __builtin_nontemporal_store(u32x2{pack_bf2(Zt[0], Zt[1]), pack_bf2(Zt[2], Zt[3])},
                                            reinterpret_cast<u32x2*>(dz));
            } else {
                const int d = 2 * j - L.c0; // own chunk minus the partner's
                const bool first = d < 0 || (d == 0 && L.dir == 0);
                const bool defer = defer_d(d);
                float* dp = !valid ? L.sink : (first ? p1 : (defer ? p2 : L.sink));
                *reinterpret_cast<f32x4*>(dp) = f32x4{Zt[0], Zt[1], Zt[2], Zt[3]};
                const bool fin = valid && !first && !defer;
                const f32x4 o = r.pp;
                bf16_t* dz = fin ? reinterpret_cast<bf16_t*>(zp) : reinterpret_cast<bf16_t*>(L.sink + 4);
                __builtin_nontemporal_store(u32x2{pack_bf2(0.5f * (Zt[0] + o[0]), 0.5f * (Zt[1] + o[1])),
                                                  pack_bf2(0.5f * (Zt[2] + o[2]), 0.5f * (Zt[3] + o[3]))},
                                            reinterpret_cast<u32x2*>(dz));
                // partner's stores of steps <= j - kPre are complete: publish
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            zp += zst;
            p1 += pst;
            p2 += pst;
            issue_loads(a, L, j + D, r);
        }
    }
}

__global__ __launch_bounds__(128, 1) void scan_kernel(ScanArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[2 * kWaveLds];
    const SliceSplit ss = map_block(blockIdx.x, 4, a.xcd);
    if (ss.slice >= a.slices) return; // padding block of the XCD-aware grid
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= a.ndir) return;
    const int lane = threadIdx.x & 63;
    Walk L;
    L.g = lane >> 4;
    L.m = lane & 15;
    L.rt = ss.split;
    L.dir = a.ndir == 2 ? w : (a.mode == 2 ? 1 : 0);
    L.b = a.b;
    L.N = a.N;
    L.nch = a.nch;
    L.c0 = (a.N - 1 - L.m) / a.b;
    L.step = L.dir ? -(long long)a.b : (long long)a.b;
    const int bb = ss.slice / a.H, h = ss.slice % a.H;
    L.Ksn = a.K.sn * 2;
    L.Qsn = a.Q.sn * 2;
    L.Vsn = a.V.sn * 2;
    L.Zsn = a.Z.sn * 2;
    L.K = (const char*)a.K.ptr + (bb * a.K.sb + h * a.K.sh) * 2 + 16 * L.g;
    L.Q = (const char*)a.Q.ptr + (bb * a.Q.sb + h * a.Q.sh) * 2 + 16 * L.g;
    L.V = (const char*)a.V.ptr + (bb * a.V.sb + h * a.V.sh) * 2 + (16 * L.rt + 4 * L.g) * 2;
    L.Z = (char*)a.Z.ptr + (bb * a.Z.sb + h * a.Z.sh) * 2 + (16 * L.rt + 4 * L.g) * 2;
    const int ch = 16 * L.rt + 4 * L.g;
    L.P = a.P ? a.P + (long long)ss.slice * a.N * 64 + ch : nullptr;
    L.P2 = a.P2 ? a.P2 + (long long)ss.slice * a.N * 64 + ch : nullptr;
    L.Pbase = L.P;
    L.zeros = a.zeros;
    L.sink = a.dummy + ((long long)blockIdx.x * 2 + w) * 512 + lane * 8;
    // running load pointers start at chunk 0, slot m (clamped when slot m
    // holds no token of chunk 0; the ragged path never uses them then)
    const int p0 = L.dir ? max(a.N - 1 - L.m, 0) : min(L.m, a.N - 1);
    L.Kn = L.K + p0 * L.Ksn;
    L.Qn = L.Q + p0 * L.Qsn;
    L.Vn = L.V + p0 * L.Vsn;
    L.Pn = L.P ? L.P + (long long)p0 * 64 : L.sink;
    char* kt = lds + w * kWaveLds;
    scan_chain<kPre>(a, L, kt, kt + kChunk * kKRow, a.W0 + (long long)h * 4096, a.eta[h]);

    if (a.ndir == 2) {
        // tokens whose two arrivals are < 2 kPre chunks apart: average the
        // two stored fp32 outputs
        drain_vmem();
        __syncthreads();
        const int span = (2 * kPre + 1) * a.b;
        const int lo = max(0, (a.N - 1) / 2 - span), hi = min(a.N, a.N / 2 + span + 1);
        const float* P = a.P + (long long)ss.slice * a.N * 64;
        const float* P2 = a.P2 + (long long)ss.slice * a.N * 64;
        bf16_t* Z = (bf16_t*)a.Z.ptr + bb * a.Z.sb + h * a.Z.sh;
        for (int e2 = threadIdx.x; e2 < (hi - lo) * 4; e2 += 64 * a.ndir) {
            const int p = lo + (e2 >> 2), c = 16 * L.rt + 4 * (e2 & 3);
            const int jf = p / a.b, jb = (a.N - 1 - p) / a.b;
            if (!defer_d(jf - jb)) continue;
            const f32x4 x = *reinterpret_cast<const f32x4*>(P + (long long)p * 64 + c);
            const f32x4 y = *reinterpret_cast<const f32x4*>(P2 + (long long)p * 64 + c);
            *reinterpret_cast<u32x2*>(Z + (long long)p * a.Z.sn + c) =
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
    size_t bytes = (size_t)blocks * 2 * 512 * sizeof(float) + 256;
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
    // workspace: [zero block, 256 bytes][sink][P][P2].  The zero block sits
    // at offset 0 whatever the shape, so no call's outputs ever land on it.
    float* base = (float*)s.ws;
    a.zeros = (const char*)base;
    a.dummy = base + 64;
    if (a.ndir == 2) {
        a.P = a.dummy + blocks * 2 * 512;
        a.P2 = a.P + (size_t)a.slices * s.N * 64;
    }
    hipLaunchKernelGGL(scan_kernel, dim3((unsigned)blocks), dim3(64 * a.ndir), 0, stream, a);
    return hipGetLastError();
}

} // namespace ttt
