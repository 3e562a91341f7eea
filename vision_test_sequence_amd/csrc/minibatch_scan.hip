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
// Two waves per (slice, direction, column block): the chain wave carries
// the recurrence alone (R, R', the X update: the serial path of the scan)
// and publishes each chunk's K rows, bf16 chunk-start X and R' in LDS; the
// output wave, behind it, forms Z from them.  One workgroup barrier per
// two chunks hands them from chain wave to output wave (the two waves meet
// half as often, and the output wave's work on the two chunks overlaps);
// the output products are chained on the matrix cores, with the causal
// mask applied to the packed bf16 operand as a bit mask.
//
// Bidirectional average: each direction of a column block runs in a
// workgroup of its own and stores every token's output in the workspace as
// bf16 (P forward, P2 backward); a second kernel (scan_average) forms
// Z = (P + P2) / 2 in fp32 and rounds it to bf16.  (With the two directions in one workgroup, stepping
// in lockstep and averaging as they go, the 1280x1280 workload took 162 us
// against 122 us: the lockstep paced both chains by the slowest wave.)
#include "common.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kPre = 12;   // chunks in flight per wave (register prefetch depth)
static_assert(kPre % 12 == 0, "buffer rotation: j % 4 and j % 6 follow the unrolled index");
constexpr int kChunk = 16; // token slots of one chunk (MFMA tile rows)
constexpr int kKRow = 144; // bytes per staged K row (64 channels + pad)
constexpr int kVRow = 48;  // bytes per staged V row (this block's 16 channels + pad)
constexpr int kXLane = 48; // bytes per lane of a published chunk: X (32) and R' (8)
// LDS per direction: K rows x6 (between two barriers the output wave reads
// chunks j, j+1 while the chain stages j+3, j+4 and j+2 waits), V rows x2
// (chain wave only), published X/R' x4.  The prefetch depth is a multiple
// of 12 so that buffer indices are compile-time constants in the unrolled
// loop.
constexpr int kKBuf = kChunk * kKRow;
constexpr int kVBuf = kChunk * kVRow;
constexpr int kXBuf = 64 * kXLane;
constexpr int kNK = 6; // K buffers (chunk c in c % 6)
constexpr int kNX = 4; // published X/R' buffers (chunk c in c % 4)
constexpr int kDirLds = kNK * kKBuf + 2 * kVBuf + kNX * kXBuf;
constexpr int kXOff = kNK * kKBuf + 2 * kVBuf;
constexpr int kOneCuLds = 96 * 1024; // LDS that keeps a second workgroup off the CU
static_assert(kDirLds <= kOneCuLds, "scan LDS");


typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s;

struct ScanArgs {
    View4 K, Q, V, Z;
    const float* W0;
    const float* eta;
    bf16_t* P;         // [slices][N][64]: forward-direction outputs (both directions)
    bf16_t* P2;        // [slices][N][64]: backward-direction outputs
    int H, N, b, nch, slices, mode, xcd;
    int split;         // both directions: outputs to P / P2 (then scan_average)
    int blocks;        // workgroups per direction
};

// Per-lane walk of one chain.  Token slot m of chunk j is token
// p = j*b + m (forward) or N-1-(j*b + m) (reverse).
struct Walk {
    int g, m, rt, dir, b, N, nch;
    long long step; // token step per chunk: +-b
};
__device__ __forceinline__ int token_of(const Walk& L, int rho) { return L.dir ? L.N - 1 - rho : rho; }
// Loads are branch-free (so the compiler can schedule them into the
// matrix-core latencies): a slot's buffer offset advances by one chunk per
// call, and a slot without a token falls outside the slice's descriptor.
__device__ __forceinline__ v4s_t tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
}
// Workgroup barrier for the chunk hand-over: LDS writes before it are
// visible to LDS reads after it (lds_barrier waits for this wave's LDS
// operations, not for its global loads), and the compiler moves no global
// access across it.
__device__ __forceinline__ void chunk_barrier() {
    asm volatile("" ::: "memory");
    lds_barrier();
    asm volatile("" ::: "memory");
}

// Buffer descriptor over [base, base + bytes): a raw buffer access whose
// offset lies outside it returns zeros (load) or is dropped (store).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, long long bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr unsigned kOffSlice = 0x80000000u; // an offset outside every slice span

// ------------------------------------------------------------ chain wave --
// K, V: the slice's token 0, channel 0; Ksn, Vsn: token strides in bytes.
template <int D>
__device__ void chain_wave(const ScanArgs& a, const Walk& L, const char* K, const char* V, long long Ksn,
                           long long Vsn, const float* W0h, float eta, char* lds) {
    const int g = L.g, m = L.m, lane = 16 * g + m;
    const int e = (lane & 15) >> 2, aa = lane & 3;
    char* vbuf = lds + kNK * kKBuf;
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
    // K and V rows through buffer descriptors over the slice, as in the
    // output wave: an overrun token or an empty slot loads zeros
    const bool slot = L.m < L.b;
    const long long p0 = token_of(L, m);
    const int ch = 16 * L.rt + 4 * g; // this lane's V channels
    const __amdgpu_buffer_rsrc_t krs = span_rsrc(K, (long long)(L.N - 1) * Ksn + 128);
    const __amdgpu_buffer_rsrc_t vrs = span_rsrc(V, (long long)(L.N - 1) * Vsn + 128);
    unsigned koff = slot ? (unsigned)(p0 * Ksn + 16 * g) : kOffSlice;
    unsigned voff = slot ? (unsigned)(p0 * Vsn + 2 * ch) : kOffSlice;
    const unsigned kst = slot ? (unsigned)(L.step * Ksn) : 0u, vst = slot ? (unsigned)(L.step * Vsn) : 0u;
    struct Regs {
        u32x4 k[2];
        u32x2 v;
    } cr[D];
    auto issue = [&](Regs& r) __attribute__((always_inline)) {
        r.k[0] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff, 0, 0);
        r.k[1] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff + 64u, 0, 0);
        r.v = __builtin_amdgcn_raw_buffer_load_b64(vrs, voff, 0, 0);
        koff += kst;
        voff += vst;
    };
#pragma unroll
    for (int u = 0; u < D; ++u) issue(cr[u]);

    const float alpha_full = -2.0f * eta / (float)L.b;
    const float alpha_last = -2.0f * eta / (float)(L.N - (L.nch - 1) * L.b);
    // LDS addresses: this lane's K row chunks and V row piece; transposing
    // reads (in each 16-lane group lane 4e + a points at a 4-element row
    // piece, lane m of the group receives element m % 4 of the pieces of
    // lanes 4e + m/4, e = 0..3): the update operand of X tile ct is token
    // 4g + e, channels pi(ct, 4a) .. +3; -V^T is token 4g + e, channels
    // 4a .. +3 of the block.
    const int kw = m * kKRow + 16 * g, kr = (4 * g + e) * kKRow + 16 * aa;
    const int vw = m * kVRow + 8 * g, vr = (4 * g + e) * kVRow + 8 * aa;
    // stage chunk jj (registers r) in K buffer jj % 3 / V buffer jj % 2 and
    // read its transposed operands back
    auto stage = [&](const Regs& r, int kbi, int vbi, v4s_t* ktA, v4s_t& vin) __attribute__((always_inline)) {
        char* kb = lds + kbi * kKBuf;
        char* vb = vbuf + vbi * kVBuf;
        *reinterpret_cast<u32x4*>(kb + kw) = r.k[0];
        *reinterpret_cast<u32x4*>(kb + kw + 64) = r.k[1];
        *reinterpret_cast<u32x2*>(vb + vw) = r.v;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) ktA[ct] = tr_read(kb + kr + 64 * (ct >> 1) + 8 * (ct & 1));
        vin = tr_read(vb + vr);
    };
    v4s_t ktA[4], vin;
    stage(cr[0], 0, 0, ktA, vin);
    const int nsteps = ((L.nch + D - 1) / D) * D;
    for (int j0 = 0; j0 < nsteps; j0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int j = j0 + u;
            Regs& r = cr[u];
            char* xo = lds + kXOff + (u % kNX) * kXBuf + lane * kXLane;
            // the next chunk's operands, one step ahead of their use
            v4s_t ktN[4], vinN;
            stage(cr[(u + 1) % D], (u + 1) % kNK, (u + 1) & 1, ktN, vinN);
            const float alpha = j < L.nch - 1 ? alpha_full : (j == L.nch - 1 ? alpha_last : 0.f);

            // bf16 copy of the chunk-start state
            u32x4 xu[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
                xu[kb2] = u32x4{pack_bf2(X[2 * kb2][0], X[2 * kb2][1]), pack_bf2(X[2 * kb2][2], X[2 * kb2][3]),
                                pack_bf2(X[2 * kb2 + 1][0], X[2 * kb2 + 1][1]),
                                pack_bf2(X[2 * kb2 + 1][2], X[2 * kb2 + 1][3])};
            // R = K X - V ;  R' = alpha R, the two halves of the channel
            // contraction chained on the matrix cores (fewer vector
            // instructions: the waves' instruction streams bound the scan)
            // -V from the transposed bf16 pairs: one sign flip per pair
            const u32x2 vneg = __builtin_bit_cast(u32x2, vin) ^ u32x2{0x80008000u, 0x80008000u};
            const v4f Rv{bflo(vneg[0]), bfhi(vneg[0]), bflo(vneg[1]), bfhi(vneg[1])};
            const v4f R = mfma32(as_v8bf(r.k[1]), as_v8bf(xu[1]), mfma32(as_v8bf(r.k[0]), as_v8bf(xu[0]), Rv));
            const u32x2 rp2{pack_bf2(alpha * R[0], alpha * R[1]), pack_bf2(alpha * R[2], alpha * R[3])};
            // X += K^T R'
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) X[ct] = mfma16(ktA[ct], as_v4s(rp2), X[ct]);
            // publish the chunk for the output wave
            *reinterpret_cast<u32x4*>(xo) = xu[0];
            *reinterpret_cast<u32x4*>(xo + 16) = xu[1];
            *reinterpret_cast<u32x2*>(xo + 32) = rp2;
            if (u & 1) chunk_barrier(); // chunks j-1, j published
            issue(r);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) ktA[ct] = ktN[ct];
            vin = vinN;
        }
    }
}

// ----------------------------------------------------------- output wave --
// Q, Z (or P, this direction's [N][64] bf16 rows): the slice's token 0,
// channel 0; Qsn, Zsn: token strides in bytes.
template <int D>
__device__ void output_wave(const ScanArgs& a, const Walk& L, const char* Q, long long Qsn, char* Z,
                            long long Zsn, bf16_t* P, const char* lds) {
    const int g = L.g, m = L.m, lane = 16 * g + m;
    const int ch = 16 * L.rt + 4 * g; // this lane's output channels
    // Q rows, Z / P outputs through buffer descriptors over the slice: a
    // slot whose token lies outside the slice (the walk's overrun past
    // either end: the offset then exceeds the span or wraps negative, as
    // the host bounds the spans) or an empty slot (m >= b) reads zeros and
    // stores nothing, with no per-chunk selects.
    const bool slot = L.m < L.b;
    const long long p0 = token_of(L, m);
    const __amdgpu_buffer_rsrc_t qrs = span_rsrc(Q, (long long)(L.N - 1) * Qsn + 128);
    unsigned qoff = slot ? (unsigned)(p0 * Qsn + 16 * g) : kOffSlice;
    const unsigned qst = slot ? (unsigned)(L.step * Qsn) : 0u;
    struct Regs {
        u32x4 q[2];
    } cr[D];
    auto issue = [&](Regs& r) __attribute__((always_inline)) {
        r.q[0] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff, 0, 0);
        r.q[1] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 64u, 0, 0);
        qoff += qst;
    };
#pragma unroll
    for (int u = 0; u < D; ++u) issue(cr[u]);

    // causal mask of K Q^T's accumulator (lane (g, m): rows 4g+i, column
    // m), kept where 4g+i <= m, as bit masks of the packed bf16 pairs
    const u32x2 tril{(4 * g <= m ? 0xFFFFu : 0u) | (4 * g + 1 <= m ? 0xFFFF0000u : 0u),
                     (4 * g + 2 <= m ? 0xFFFFu : 0u) | (4 * g + 3 <= m ? 0xFFFF0000u : 0u)};
    // outputs: this direction's bf16 rows of P ([N][64] per slice), or Z
    const __amdgpu_buffer_rsrc_t zrs = a.split ? span_rsrc(P, (long long)L.N * 128)
                                               : span_rsrc(Z, (long long)(L.N - 1) * Zsn + 128);
    const long long zsn = a.split ? 128 : Zsn;
    unsigned zoff = slot ? (unsigned)(p0 * zsn + 2 * ch) : kOffSlice;
    const unsigned zst = slot ? (unsigned)(L.step * zsn) : 0u;
    const int nsteps = ((L.nch + D - 1) / D) * D;
    for (int j0 = 0; j0 < nsteps; j0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            Regs& r = cr[u];
            if ((u & 1) == 0) chunk_barrier(); // chunks j, j+1 published
            const char* kb = lds + (u % kNK) * kKBuf + m * kKRow + 16 * g;
            const char* xi = lds + kXOff + (u % kNX) * kXBuf + lane * kXLane;
            const u32x4 k0 = *reinterpret_cast<const u32x4*>(kb);
            const u32x4 k1 = *reinterpret_cast<const u32x4*>(kb + 64);
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(xi);
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(xi + 16);
            const u32x2 rp2 = *reinterpret_cast<const u32x2*>(xi + 32);

            // Z^T = X^T Q^T + R'^T tril(Q K^T)^T   (chunk-start X), all
            // accumulated on the matrix cores
            const v4f zero4{0.f, 0.f, 0.f, 0.f};
            const v4f S = mfma32(as_v8bf(k1), as_v8bf(r.q[1]), mfma32(as_v8bf(k0), as_v8bf(r.q[0]), zero4));
            const v4f Zq = mfma32(as_v8bf(x1), as_v8bf(r.q[1]), mfma32(as_v8bf(x0), as_v8bf(r.q[0]), zero4));
            const u32x2 sb2{pack_bf2(S[0], S[1]) & tril[0], pack_bf2(S[2], S[3]) & tril[1]};
            const v4f Zt = mfma16(as_v4s(rp2), as_v4s(sb2), Zq);

            // outputs of token slot m, channels 16 rt + 4 g .. +3 (Z
            // streamed past the caches; P is read back by the average)
            const u32x2 zv{pack_bf2(Zt[0], Zt[1]), pack_bf2(Zt[2], Zt[3])};
            if (a.split) __builtin_amdgcn_raw_buffer_store_b64(zv, zrs, zoff, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b64(zv, zrs, zoff, 0, 2 /* nt */);
            asm volatile("" ::: "memory"); // stores of chunk j before the loads of chunk j + D
            zoff += zst;
            issue(r);
        }
    }
}

// One (slice, direction, 16-column block) per workgroup: wave 0 the chain,
// wave 1 the output.  With both directions (split), blocks [0, blocks)
// walk forward and the rest backward.  Spread: the workgroup takes more
// than half a CU's LDS, so no two share a CU -- used when the grid fits the
// device one workgroup per CU (two chains on one CU share its SIMDs: 127
// against 121 us at 1280x1280).
template <bool Spread>
__global__ __launch_bounds__(128, 1) void scan_kernel(ScanArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[Spread ? kOneCuLds : kDirLds];
    const int dsplit = a.split && (int)blockIdx.x >= a.blocks ? 1 : 0;
    const int bidx = (int)blockIdx.x - dsplit * a.blocks;
    const SliceSplit ss = map_block(bidx, 4, a.xcd);
    if (ss.slice >= a.slices) return; // padding block of the XCD-aware grid
    const int role = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // chain / output wave
    const int lane = threadIdx.x & 63;
    Walk L;
    L.g = lane >> 4;
    L.m = lane & 15;
    L.rt = ss.split;
    L.dir = a.split ? dsplit : (a.mode == 2 ? 1 : 0);
    L.b = a.b;
    L.N = a.N;
    L.nch = a.nch;
    L.step = L.dir ? -(long long)a.b : (long long)a.b;
    const int bb = ss.slice / a.H, h = ss.slice % a.H;
    if (role == 0) {
        // slice bases: wave-uniform, so the buffer descriptors need no
        // per-lane resolution (lane offsets go into the buffer offsets)
        const char* K = (const char*)a.K.ptr + (bb * a.K.sb + h * a.K.sh) * 2;
        const char* V = (const char*)a.V.ptr + (bb * a.V.sb + h * a.V.sh) * 2;
        chain_wave<kPre>(a, L, K, V, a.K.sn * 2, a.V.sn * 2, a.W0 + (long long)h * 4096, a.eta[h], lds);
    } else {
        const char* Q = (const char*)a.Q.ptr + (bb * a.Q.sb + h * a.Q.sh) * 2;
        char* Z = (char*)a.Z.ptr + (bb * a.Z.sb + h * a.Z.sh) * 2;
        bf16_t* P = a.split ? (dsplit ? a.P2 : a.P) + (long long)ss.slice * a.N * 64 : nullptr;
        output_wave<kPre>(a, L, Q, a.Q.sn * 2, Z, a.Z.sn * 2, P, lds);
    }
}

// Z = (forward + backward) / 2 from the two directions' outputs, 8
// channels (16 bytes of each) per thread.
__global__ __launch_bounds__(256) void scan_average(ScanArgs a) {
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x; // (slice, token, channel octet)
    if (e >= (long long)a.slices * a.N * 8) return;
    const int c8 = (int)(e & 7);
    const long long st = e >> 3;
    const int p = (int)(st % a.N), slice = (int)(st / a.N);
    const int bb = slice / a.H, h = slice % a.H;
    const u32x4 x = *reinterpret_cast<const u32x4*>(a.P + st * 64 + 8 * c8);
    const u32x4 y = *reinterpret_cast<const u32x4*>(a.P2 + st * 64 + 8 * c8);
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        o[k] = pack_bf2(0.5f * (bflo(x[k]) + bflo(y[k])), 0.5f * (bfhi(x[k]) + bfhi(y[k])));
    bf16_t* z = (bf16_t*)a.Z.ptr + bb * a.Z.sb + h * a.Z.sh + (long long)p * a.Z.sn + 8 * c8;
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(z));
}

long long padded_slices(int B, int H) {
    const long long s = (long long)B * H;
    return (s + 7) / 8 * 8;
}

} // namespace

size_t scan_ws_bytes(int B, int H, int N, int mode) {
    size_t bytes = 256;
    if (mode == 0) bytes += 2 * (size_t)B * H * N * 64 * sizeof(bf16_t);
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
    // both directions: each in workgroups of its own, bf16 outputs averaged
    // by a second kernel
    a.split = s.mode == 0 ? 1 : 0;
    a.xcd = 1;
    const long long blocks = padded_slices(s.B, s.H) * 4;
    a.blocks = (int)blocks;
    // workspace: [256 bytes reserved][P][P2]
    float* base = (float*)s.ws;
    if (a.split) {
        a.P = reinterpret_cast<bf16_t*>(base + 64);
        a.P2 = a.P + (size_t)a.slices * s.N * 64;
    }
    const long long grid = blocks * (a.split ? 2 : 1);
    if (grid <= s.cus) hipLaunchKernelGGL(scan_kernel<true>, dim3((unsigned)grid), dim3(128), 0, stream, a);
    else hipLaunchKernelGGL(scan_kernel<false>, dim3((unsigned)grid), dim3(128), 0, stream, a);
    if (a.split) {
        const long long n = (long long)a.slices * s.N * 8;
        hipLaunchKernelGGL(scan_average, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

} // namespace ttt
