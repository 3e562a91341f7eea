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
// workgroup of its own and stores every token's output in the workspace in
// fp32 (P forward, P2 backward); a second kernel (scan_average) forms
// Z = (P + P2) / 2 and rounds it to bf16 once.  (With the two directions in
// one workgroup, stepping in lockstep and averaging as they go, the
// 1280x1280 workload took 162 us against 122 us: the lockstep paced both
// chains by the slowest wave.)
//
// Chunk-parallel scan: over one mini-batch X <- (I + alpha K^T K) X
// - alpha K^T V, an affine map of X.  When the chains leave most CUs idle,
// each is cut into segments: scan_maps walks the state [M | U] from [I | 0]
// through every segment but the last (eight 16-column blocks, V = 0 for the
// M columns: the chain wave's own arithmetic), scan_starts composes the
// start states in order (W_s = W_{s-1} M^T + U^T), and the scan kernel
// walks every segment from its start state.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

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
    float* P;          // [slices][N][64]: forward-direction outputs (both directions)
    float* P2;         // [slices][N][64]: backward-direction outputs
    int H, N, b, nch, slices, mode, xcd;
    int split;         // both directions: outputs to P / P2 (then scan_average)
    int blocks;        // workgroups per direction
    int w0dir;         // W0 is [2][H][64][64]: forward, then reverse scan
    int tb;            // tokens per tile: b (b <= 16) or 16
    int T;             // tiles per mini-batch: 1 (b <= 16) or ceil(min(b, N) / 16)
    int ntile;         // tiles of one walk: ceil(N / tb)
    int nseg;          // segments per chain (chunk-parallel scan), 1 = one walk
    float* maps;       // [chains][nseg-1][2][64][64]: segment maps (S_M, S_U), W layout
    float* starts;     // [chains][nseg][64][64]: segment start states W_s (s >= 1)
};

// Segment s of a chain: mini-batches [s nmb / nseg, (s+1) nmb / nseg), as tiles.
__device__ __forceinline__ int seg_mb(const ScanArgs& a, int s) { return (int)((long long)s * a.nch / a.nseg); }
__device__ __forceinline__ int seg_tile(const ScanArgs& a, int s) {
    const int t = seg_mb(a, s) * a.T;
    return t < a.ntile ? t : a.ntile;
}

// Per-lane walk of one chain over tiles of tb tokens.  Token slot m of
// tile j is token p = j*tb + m (forward) or N-1-(j*tb + m) (reverse).  A
// mini-batch is one tile (b <= 16) or T consecutive 16-token tiles (b a
// multiple of 16, or b >= N: then every mini-batch but the walk's last is
// T whole tiles).
struct Walk {
    int g, m, rt, dir, b, N, nch; // nch: tiles of this walk
    int j0, mb0;                  // the walk's first tile and first mini-batch
    long long step;               // token step per tile: +-tb
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
// Ragged mini-batches (RG: b > 16, not a multiple of 16, b < N): tile j is
// sub-tile s = j % T of mini-batch c = j / T and holds walk positions
// c b + 16 s .. +15, of which those below the mini-batch's count n_c are
// tokens.  A cursor (c, s) over the walk's tiles replaces the fixed
// offset step of the uniform walks.
struct TileCur {
    int c, s;
};
__device__ __forceinline__ void cur_next(TileCur& t, int T) {
    if (++t.s == T) {
        t.s = 0;
        ++t.c;
    }
}
// This lane's buffer offset for slot m of the cursor's tile (row stride
// sn bytes, lane_bytes within the row), or kOffSlice for an empty slot.
template <typename A>
__device__ __forceinline__ unsigned cur_off(const A& a, const Walk& L, const TileCur& t, long long sn,
                                            unsigned lane_bytes) {
    const int nc = min(a.b, L.N - t.c * a.b);
    const int q = 16 * t.s + L.m;
    if (q >= nc) return kOffSlice;
    const long long pos = (long long)t.c * a.b + q;
    const long long tok = L.dir ? L.N - 1 - pos : pos;
    return (unsigned)(tok * sn) + lane_bytes;
}

// ------------------------------------------------------------ chain wave --
// K, V: the slice's token 0, channel 0; Ksn, Vsn: token strides in bytes.
// Ws: the walk's start state W (row-major [64][64], W = X^T), or null for a
// segment map's block (MAP): the identity (columns of M, vzero: no V term)
// or zero (columns of U).  MAP walks publish nothing and store their final
// state, transposed like Ws, to out (rows 16 rt + m).
// states (MAP walks only; may be null): every mini-batch's start state is
// stored there in bf16 (the precision the backward's products take it in),
// transposed like Ws, 4096 values per mini-batch.
template <int D, bool MAP, bool RG = false>
__device__ void chain_wave(const ScanArgs& a, const Walk& L, const char* K, const char* V, long long Ksn,
                           long long Vsn, const float* Ws, float eta, char* lds, bool vzero = false,
                           float* out = nullptr, bf16_t* states = nullptr) {
    const int g = L.g, m = L.m, lane = 16 * g + m;
    const int e = (lane & 15) >> 2, aa = lane & 3;
    char* vbuf = lds + kNK * kKBuf;
    // X = W^T in accumulator layout: tile 2kb + h holds rows 32 kb + 8g + 4h + i
    v4f X[4];
    if (Ws) {
        const float* w = Ws + (16 * L.rt + m) * 64 + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(w + 32 * kb);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(w + 32 * kb + 4);
            X[2 * kb] = v4f{lo[0], lo[1], lo[2], lo[3]};
            X[2 * kb + 1] = v4f{hi[0], hi[1], hi[2], hi[3]};
        }
    } else {
        const float one = vzero ? 1.f : 0.f; // identity block of M, or U = 0
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                X[ct][i] = (32 * (ct >> 1) + 8 * g + 4 * (ct & 1) + i == 16 * L.rt + m) ? one : 0.f;
    }
    // K and V rows through buffer descriptors over the slice, as in the
    // output wave: an overrun token or an empty slot loads zeros
    const bool slot = L.m < L.b;
    const long long p0 = token_of(L, L.j0 * L.b + m);
    const int ch = 16 * L.rt + 4 * g; // this lane's V channels
    const __amdgpu_buffer_rsrc_t krs = span_rsrc(K, (long long)(L.N - 1) * Ksn + 128);
    const __amdgpu_buffer_rsrc_t vrs = span_rsrc(V, (long long)(L.N - 1) * Vsn + 128);
    TileCur icur{L.mb0, 0}; // RG: the next tile to issue
    unsigned koff = slot ? (unsigned)(p0 * Ksn + 16 * g) : kOffSlice;
    unsigned voff = slot && !vzero ? (unsigned)(p0 * Vsn + 2 * ch) : kOffSlice;
    if constexpr (RG) {
        koff = cur_off(a, L, icur, Ksn, 16 * g);
        voff = vzero ? kOffSlice : cur_off(a, L, icur, Vsn, 2 * ch);
    }
    const unsigned kst = slot ? (unsigned)(L.step * Ksn) : 0u, vst = slot && !vzero ? (unsigned)(L.step * Vsn) : 0u;
    struct Regs {
        u32x4 k[2];
        u32x2 v;
    } cr[D];
    auto issue = [&](Regs& r) __attribute__((always_inline)) {
        r.k[0] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff, 0, 0);
        r.k[1] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff + 64u, 0, 0);
        r.v = __builtin_amdgcn_raw_buffer_load_b64(vrs, voff, 0, 0);
        if constexpr (RG) {
            cur_next(icur, a.T);
            koff = cur_off(a, L, icur, Ksn, 16 * g);
            voff = vzero ? kOffSlice : cur_off(a, L, icur, Vsn, 2 * ch);
        } else {
            koff += kst;
            voff += vst;
        }
    };
#pragma unroll
    for (int u = 0; u < D; ++u) issue(cr[u]);

    // step of each mini-batch: -2 eta / n_c (the last one may be shorter)
    const float alpha_full = -2.0f * eta / (float)a.b;
    const float alpha_last = -2.0f * eta / (float)(L.N - (a.nch - 1) * a.b);
    // mini-batch of the current tile and the tile's place in it (wave-
    // uniform counters); xs: the mini-batch's start state in bf16, the B
    // operand of its residuals R = K X_s - V, while X runs on through the
    // batch's tiles (the output wave needs the running state)
    int chunk = L.mb0, sub = 0, left = L.nch;
    u32x4 xs[2];
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
        // the rows are written as 16-byte words and read back as 16-bit
        // elements: keep the compiler from reordering them across chunks
        asm volatile("" ::: "memory");
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
            Regs& r = cr[u];
            char* xo = lds + kXOff + (u % kNX) * kXBuf + lane * kXLane;
            // the next tile's operands, one step ahead of their use
            v4s_t ktN[4], vinN;
            stage(cr[(u + 1) % D], (u + 1) % kNK, (u + 1) & 1, ktN, vinN);
            // past the walk's last tile (the prefetch pipeline's tail) alpha is 0
            const float alpha =
                left <= 0 ? 0.f : (chunk < a.nch - 1 ? alpha_full : (chunk == a.nch - 1 ? alpha_last : 0.f));
            --left;

            // bf16 copy of the running state (published), and of the
            // mini-batch's start state at its first tile
            u32x4 xu[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
                xu[kb2] = u32x4{pack_bf2(X[2 * kb2][0], X[2 * kb2][1]), pack_bf2(X[2 * kb2][2], X[2 * kb2][3]),
                                pack_bf2(X[2 * kb2 + 1][0], X[2 * kb2 + 1][1]),
                                pack_bf2(X[2 * kb2 + 1][2], X[2 * kb2 + 1][3])};
            if (sub == 0) {
                xs[0] = xu[0];
                xs[1] = xu[1];
                if (MAP && states && chunk < a.nch) {
                    bf16_t* o = states + (long long)chunk * 4096 + (16 * L.rt + m) * 64 + 8 * g;
#pragma unroll
                    for (int kb2 = 0; kb2 < 2; ++kb2) *reinterpret_cast<u32x4*>(o + 32 * kb2) = xu[kb2];
                }
            }
            if (++sub == a.T) {
                sub = 0;
                ++chunk;
            }
            // R = K X_s - V ;  R' = alpha R, the two halves of the channel
            // contraction chained on the matrix cores (fewer vector
            // instructions: the waves' instruction streams bound the scan)
            // -V from the transposed bf16 pairs: one sign flip per pair
            const u32x2 vneg = __builtin_bit_cast(u32x2, vin) ^ u32x2{0x80008000u, 0x80008000u};
            const v4f Rv{bflo(vneg[0]), bfhi(vneg[0]), bflo(vneg[1]), bfhi(vneg[1])};
            const v4f R = mfma32(as_v8bf(r.k[1]), as_v8bf(xs[1]), mfma32(as_v8bf(r.k[0]), as_v8bf(xs[0]), Rv));
            const u32x2 rp2{pack_bf2(alpha * R[0], alpha * R[1]), pack_bf2(alpha * R[2], alpha * R[3])};
            // X += K^T R'
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) X[ct] = mfma16(ktA[ct], as_v4s(rp2), X[ct]);
            if (!MAP) {
                // publish the chunk for the output wave
                *reinterpret_cast<u32x4*>(xo) = xu[0];
                *reinterpret_cast<u32x4*>(xo + 16) = xu[1];
                *reinterpret_cast<u32x2*>(xo + 32) = rp2;
                if (u & 1) chunk_barrier(); // chunks j-1, j published
            }
            issue(r);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) ktA[ct] = ktN[ct];
            vin = vinN;
        }
    }
    if (MAP && out) {
        // the final state, transposed as the start states are read
        float* o = out + (16 * L.rt + m) * 64 + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            *reinterpret_cast<f32x4*>(o + 32 * kb) = f32x4{X[2 * kb][0], X[2 * kb][1], X[2 * kb][2], X[2 * kb][3]};
            *reinterpret_cast<f32x4*>(o + 32 * kb + 4) =
                f32x4{X[2 * kb + 1][0], X[2 * kb + 1][1], X[2 * kb + 1][2], X[2 * kb + 1][3]};
        }
    }
}

// ----------------------------------------------------------- output wave --
// Q, Z (or P, this direction's [N][64] fp32 rows): the slice's token 0,
// channel 0; Qsn, Zsn: token strides in bytes.
template <int D, bool RG = false>
__device__ void output_wave(const ScanArgs& a, const Walk& L, const char* Q, long long Qsn, char* Z,
                            long long Zsn, float* P, const char* lds) {
    const int g = L.g, m = L.m, lane = 16 * g + m;
    const int ch = 16 * L.rt + 4 * g; // this lane's output channels
    // Q rows, Z / P outputs through buffer descriptors over the slice: a
    // slot whose token lies outside the slice (the walk's overrun past
    // either end: the offset then exceeds the span or wraps negative, as
    // the host bounds the spans) or an empty slot (m >= b) reads zeros and
    // stores nothing, with no per-chunk selects.
    const bool slot = L.m < L.b;
    const long long p0 = token_of(L, L.j0 * L.b + m);
    const __amdgpu_buffer_rsrc_t qrs = span_rsrc(Q, (long long)(L.N - 1) * Qsn + 128);
    TileCur icur{L.mb0, 0}, zcur{L.mb0, 0}; // RG: the next tile to issue / to store
    unsigned qoff = slot ? (unsigned)(p0 * Qsn + 16 * g) : kOffSlice;
    if constexpr (RG) qoff = cur_off(a, L, icur, Qsn, 16 * g);
    const unsigned qst = slot ? (unsigned)(L.step * Qsn) : 0u;
    struct Regs {
        u32x4 q[2];
    } cr[D];
    auto issue = [&](Regs& r) __attribute__((always_inline)) {
        r.q[0] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff, 0, 0);
        r.q[1] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 64u, 0, 0);
        if constexpr (RG) {
            cur_next(icur, a.T);
            qoff = cur_off(a, L, icur, Qsn, 16 * g);
        } else {
            qoff += qst;
        }
    };
#pragma unroll
    for (int u = 0; u < D; ++u) issue(cr[u]);

    // causal mask of K Q^T's accumulator (lane (g, m): rows 4g+i, column
    // m), kept where 4g+i <= m, as bit masks of the packed bf16 pairs
    const u32x2 tril{(4 * g <= m ? 0xFFFFu : 0u) | (4 * g + 1 <= m ? 0xFFFF0000u : 0u),
                     (4 * g + 2 <= m ? 0xFFFFu : 0u) | (4 * g + 3 <= m ? 0xFFFF0000u : 0u)};
    // outputs: this direction's fp32 rows of P ([N][64] per slice), or Z
    const __amdgpu_buffer_rsrc_t zrs = a.split ? span_rsrc(P, (long long)L.N * 256)
                                               : span_rsrc(Z, (long long)(L.N - 1) * Zsn + 128);
    const long long zsn = a.split ? 256 : Zsn;
    unsigned zoff = slot ? (unsigned)(p0 * zsn + (a.split ? 4 : 2) * ch) : kOffSlice;
    if constexpr (RG) zoff = cur_off(a, L, zcur, zsn, (a.split ? 4 : 2) * ch);
    const unsigned zst = slot ? (unsigned)(L.step * zsn) : 0u;
    int left = L.nch; // tiles of the walk still to store (a segment ends before the slice does)
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
            // (added on the vector unit: never chain one matrix-core shape's
            // result into another shape's accumulator)
            const v4f Zr = mfma16(as_v4s(rp2), as_v4s(sb2), zero4);
            const v4f Zt{Zq[0] + Zr[0], Zq[1] + Zr[1], Zq[2] + Zr[2], Zq[3] + Zr[3]};

            // outputs of token slot m, channels 16 rt + 4 g .. +3 (Z
            // streamed past the caches; P, in fp32, is read back by the
            // average, so each direction's output is rounded once, in Z)
            const unsigned zo = left-- > 0 ? zoff : kOffSlice;
            if (a.split) {
                const u32x4 pv{__float_as_uint(Zt[0]), __float_as_uint(Zt[1]), __float_as_uint(Zt[2]),
                               __float_as_uint(Zt[3])};
                __builtin_amdgcn_raw_buffer_store_b128(pv, zrs, zo, 0, 0);
            } else {
                const u32x2 zv{pack_bf2(Zt[0], Zt[1]), pack_bf2(Zt[2], Zt[3])};
                __builtin_amdgcn_raw_buffer_store_b64(zv, zrs, zo, 0, 2 /* nt */);
            }
            asm volatile("" ::: "memory"); // stores of chunk j before the loads of chunk j + D
            if constexpr (RG) {
                cur_next(zcur, a.T);
                zoff = cur_off(a, L, zcur, zsn, (a.split ? 4 : 2) * ch);
            } else {
                zoff += zst;
            }
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
template <bool Spread, bool RG>
__global__ __launch_bounds__(128, 1) void scan_kernel(ScanArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[Spread ? kOneCuLds : kDirLds];
    const int dsplit = a.split && (int)blockIdx.x >= a.blocks ? 1 : 0;
    const int bidx = (int)blockIdx.x - dsplit * a.blocks;
    // unit = (slice, segment); its 4 column blocks share an XCD (and the
    // L2 that serves their common K and Q rows), consecutive units go to
    // different XCDs
    const SliceSplit us = map_block(bidx, 4, a.xcd);
    if (us.slice >= a.slices * a.nseg) return; // padding block of the XCD-aware grid
    SliceSplit ss;
    ss.slice = us.slice / a.nseg;
    ss.split = us.split;
    const int seg = us.slice % a.nseg;
    const int role = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // chain / output wave
    const int lane = threadIdx.x & 63;
    Walk L;
    L.g = lane >> 4;
    L.m = lane & 15;
    L.rt = ss.split;
    L.dir = a.split ? dsplit : (a.mode == 2 ? 1 : 0);
    L.b = a.tb;
    L.N = a.N;
    L.j0 = seg_tile(a, seg);
    L.nch = seg_tile(a, seg + 1) - L.j0;
    L.mb0 = seg_mb(a, seg);
    L.step = L.dir ? -(long long)a.tb : (long long)a.tb;
    const int bb = ss.slice / a.H, h = ss.slice % a.H;
    if (role == 0) {
        // slice bases: wave-uniform, so the buffer descriptors need no
        // per-lane resolution (lane offsets go into the buffer offsets)
        const char* K = (const char*)a.K.ptr + (bb * a.K.sb + h * a.K.sh) * 2;
        const char* V = (const char*)a.V.ptr + (bb * a.V.sb + h * a.V.sh) * 2;
        // segment 0 starts from W0 (the reverse scan from its own when one is
        // given per direction), segment s from the state the maps gave it
        const float* Ws = seg == 0 ? a.W0 + ((a.w0dir && L.dir ? (long long)a.H : 0) + h) * 4096
                                   : a.starts + ((long long)(dsplit * a.slices + ss.slice) * a.nseg + seg) * 4096;
        chain_wave<kPre, false, RG>(a, L, K, V, a.K.sn * 2, a.V.sn * 2, Ws, a.eta[h], lds);
    } else {
        const char* Q = (const char*)a.Q.ptr + (bb * a.Q.sb + h * a.Q.sh) * 2;
        char* Z = (char*)a.Z.ptr + (bb * a.Z.sb + h * a.Z.sh) * 2;
        float* P = a.split ? (dsplit ? a.P2 : a.P) + (long long)ss.slice * a.N * 64 : nullptr;
        output_wave<kPre, RG>(a, L, Q, a.Q.sn * 2, Z, a.Z.sn * 2, P, lds);
    }
}

// Chunk-parallel scan, first pass: the affine map of each segment but the
// last.  Over a mini-batch the state update X <- X + K^T R',
// R' = alpha (K X - V), is X <- (I + alpha K^T K) X - alpha K^T V, so a
// segment maps its start state to M X + U; walking the state [M | U] from
// [I | 0] through the segment's mini-batches (V = 0 for the M columns)
// gives both.  One wave per (chain, segment, 16-column block of [M | U]):
// blocks 0-3 the columns of M, blocks 4-7 those of U.  Stored transposed
// (S_M = M^T, S_U = U^T), so that W_end = W_start S_M + S_U.
template <bool RG>
__global__ __launch_bounds__(64, 1) void scan_maps(ScanArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kNK * kKBuf + 2 * kVBuf];
    // unit = (slice, segment but the last), 8 column blocks of [M | U] each
    const int units = a.slices * (a.nseg - 1);
    const int per_dir = (units + 7) / 8 * 8 * 8;
    const int dsplit = a.split && (int)blockIdx.x >= per_dir ? 1 : 0;
    const int bidx = (int)blockIdx.x - dsplit * per_dir;
    const SliceSplit us = map_block(bidx, 8, a.xcd);
    if (us.slice >= units) return;
    SliceSplit ss;
    ss.slice = us.slice / (a.nseg - 1);
    const int blk = us.split, seg = us.slice % (a.nseg - 1);
    const int lane = threadIdx.x & 63;
    Walk L;
    L.g = lane >> 4;
    L.m = lane & 15;
    L.rt = blk & 3;
    L.dir = a.split ? dsplit : (a.mode == 2 ? 1 : 0);
    L.b = a.tb;
    L.N = a.N;
    L.j0 = seg_tile(a, seg);
    L.nch = seg_tile(a, seg + 1) - L.j0;
    L.mb0 = seg_mb(a, seg);
    L.step = L.dir ? -(long long)a.tb : (long long)a.tb;
    const int bb = ss.slice / a.H, h = ss.slice % a.H;
    const char* K = (const char*)a.K.ptr + (bb * a.K.sb + h * a.K.sh) * 2;
    const char* V = (const char*)a.V.ptr + (bb * a.V.sb + h * a.V.sh) * 2;
    float* out = a.maps + (((long long)(dsplit * a.slices + ss.slice) * (a.nseg - 1) + seg) * 2 + (blk >> 2)) * 4096;
    chain_wave<kPre, true, RG>(a, L, K, V, a.K.sn * 2, a.V.sn * 2, nullptr, a.eta[h], lds, blk < 4, out);
}

// ------------------------------------------------ backward: forward states --
// Every mini-batch's start state of every chain (b <= 16): the chain wave of
// the scan, storing the state at each mini-batch start.  One wave per
// (chain, 16-column block), wid = 4 ch + block; chain ch = slice * nd +
// direction index.
__device__ __forceinline__ void states_wave(const ScanArgs& a, bf16_t* states, int nd, int wid) {
    __shared__ __attribute__((aligned(16))) char lds[kNK * kKBuf + 2 * kVBuf];
    // the four column blocks of a chain on one XCD, whose L2 serves their
    // common K rows once (wid: the XCD-aware block index)
    const SliceSplit cs = map_block(wid, 4, 1);
    if (cs.slice >= a.slices * nd) return; // padding of the XCD-aware grid
    const int ch = cs.slice, rt = cs.split;
    const int slice = ch / nd, di = ch % nd;
    const int lane = threadIdx.x & 63;
    Walk L;
    L.g = lane >> 4;
    L.m = lane & 15;
    L.rt = rt;
    L.dir = a.mode == 2 ? 1 : (a.mode == 0 ? di : 0);
    L.b = a.tb;
    L.N = a.N;
    L.j0 = 0;
    L.nch = a.ntile;
    L.mb0 = 0;
    L.step = L.dir ? -(long long)a.tb : (long long)a.tb;
    const int bb = slice / a.H, h = slice % a.H;
    const char* K = (const char*)a.K.ptr + (bb * a.K.sb + h * a.K.sh) * 2;
    const char* V = (const char*)a.V.ptr + (bb * a.V.sb + h * a.V.sh) * 2;
    const float* W0h = a.W0 + ((a.w0dir && L.dir ? (long long)a.H : 0) + h) * 4096;
    chain_wave<kPre, true>(a, L, K, V, a.K.sn * 2, a.V.sn * 2, W0h, a.eta[h], lds, false, nullptr,
                           states + (long long)ch * a.nch * 4096);
}

// ------------------------------------------------ backward: gradient walk --
// The backward walk of the scan (b <= 16), per chain and 16-row block of
// dW, on the matrix cores.  With Y = dW^T (the gradient at the next
// mini-batch start, zero after the last), S = Q K^T (kept for s <= t),
// alpha = -2 eta / n_c and dZ scaled by zs (1/2 per direction of the
// average), per mini-batch walked from the last:
//   dR = alpha (K Y + S^T dZ),   Y <- Y + K^T dR + Q^T dZ,
// storing Y before the update (dwn, bf16) and dR (fp32, by walk position).  The
// operand layouts are the chain wave's: Y tiles as X's, K Y as K X, S^T
// straight out of Q K^T's accumulator, K^T and Q^T from staged rows read
// back transposed, dZ's 16 columns like V's.
struct BwdWalkArgs {
    ScanArgs s;
    View4 Q, dZ;
    bf16_t* dwn;  // [chains][nch][64][64]
    float* dRp;   // [chains][N][64]
    float* dW0c;  // [chains][64][64]
    int nd;
};
constexpr int kBD = 8; // chunks in flight (register prefetch depth)
static_assert(kBD % 2 == 0, "LDS buffer sets alternate with the unrolled index");
__device__ __forceinline__ void grad_wave(const BwdWalkArgs& w, int wid) {
    const ScanArgs& a = w.s;
    // two sets of buffers, alternating mini-batches (kBD is even), and the
    // wave's dR tile (16 tokens x 16 channels fp32, rows of 20 floats)
    __shared__ __attribute__((aligned(16))) char lds[2 * (2 * kKBuf + kVBuf)];
    __shared__ __attribute__((aligned(16))) float drt[16 * 20];
    // the four row blocks of a chain on one XCD (see states_wave)
    const SliceSplit cs = map_block(wid, 4, 1);
    if (cs.slice >= a.slices * w.nd) return; // padding of the XCD-aware grid
    const int ch = cs.slice, rb = cs.split;
    const int slice = ch / w.nd, di = ch % w.nd;
    const int dir = a.mode == 2 ? 1 : (a.mode == 0 ? di : 0);
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const int e = m >> 2, aa = m & 3;
    const int bb = slice / a.H, h = slice % a.H;
    const float eta = a.eta[h];
    const float zs = a.mode == 0 ? 0.5f : 1.f;
    const int b = a.tb, N = a.N, nch = a.nch;
    // walk position of slot m in mini-batch c: c b + m; token N-1-pos for
    // the reverse scan.  Rows through buffer descriptors over the slice: a
    // slot past either end of the slice reads zeros.
    const bool slot = m < b;
    const long long pos0 = (long long)(nch - 1) * b + m;
    const long long tok0 = dir ? N - 1 - pos0 : pos0;
    const long long tstep = dir ? b : -b; // token step from one mini-batch to the previous
    const char* Kp = (const char*)a.K.ptr + (bb * a.K.sb + h * a.K.sh) * 2;
    const char* Qp = (const char*)w.Q.ptr + (bb * w.Q.sb + h * w.Q.sh) * 2;
    const char* Zp = (const char*)w.dZ.ptr + (bb * w.dZ.sb + h * w.dZ.sh) * 2;
    const long long Ksn = a.K.sn * 2, Qsn = w.Q.sn * 2, Zsn = w.dZ.sn * 2;
    const __amdgpu_buffer_rsrc_t krs = span_rsrc(Kp, (long long)(N - 1) * Ksn + 128);
    const __amdgpu_buffer_rsrc_t qrs = span_rsrc(Qp, (long long)(N - 1) * Qsn + 128);
    const __amdgpu_buffer_rsrc_t zrs = span_rsrc(Zp, (long long)(N - 1) * Zsn + 128);
    unsigned koff = slot ? (unsigned)(tok0 * Ksn + 16 * g) : kOffSlice;
    unsigned qoff = slot ? (unsigned)(tok0 * Qsn + 16 * g) : kOffSlice;
    unsigned zoff = slot ? (unsigned)(tok0 * Zsn + 2 * (16 * rb + 4 * g)) : kOffSlice;
    const unsigned kst = slot ? (unsigned)(tstep * Ksn) : 0u, qst = slot ? (unsigned)(tstep * Qsn) : 0u,
                   zst = slot ? (unsigned)(tstep * Zsn) : 0u;
    struct Regs {
        u32x4 k[2], q[2];
        u32x2 z;
    } cr[kBD];
    auto issue = [&](Regs& r) __attribute__((always_inline)) {
        r.k[0] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff, 0, 0);
        r.k[1] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff + 64u, 0, 0);
        r.q[0] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff, 0, 0);
        r.q[1] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 64u, 0, 0);
        r.z = __builtin_amdgcn_raw_buffer_load_b64(zrs, zoff, 0, 0);
        koff += kst;
        qoff += qst;
        zoff += zst;
    };
#pragma unroll
    for (int u = 0; u < kBD; ++u) issue(cr[u]);
    // transposed operands of a staged mini-batch: K^T, Q^T for the four Y
    // tiles (token 4g + e, channels pi(ct, 4a) .. +3) and dZ (token 4g + e,
    // channels 16 rb + 4a .. +3), as in the chain wave
    const int kw = m * kKRow + 16 * g, kr = (4 * g + e) * kKRow + 16 * aa;
    const int vw = m * kVRow + 8 * g, vr = (4 * g + e) * kVRow + 8 * aa;
    auto stage = [&](const Regs& r, int set, v4s_t* ktA, v4s_t* qtA, v4s_t& zin) __attribute__((always_inline)) {
        // the rows are written as 16-byte words and read back as 16-bit
        // elements, which the compiler may treat as unrelated: nothing may
        // move across these points
        asm volatile("" ::: "memory");
        char* kbuf = lds + set * (2 * kKBuf + kVBuf);
        char* qbuf = kbuf + kKBuf;
        char* zbuf = kbuf + 2 * kKBuf;
        *reinterpret_cast<u32x4*>(kbuf + kw) = r.k[0];
        *reinterpret_cast<u32x4*>(kbuf + kw + 64) = r.k[1];
        *reinterpret_cast<u32x4*>(qbuf + kw) = r.q[0];
        *reinterpret_cast<u32x4*>(qbuf + kw + 64) = r.q[1];
        // dZ scaled by zs (exact in bf16 for 1/2 and 1 away from the denormals)
        const u32x2 zv{pack_bf2(zs * bflo(r.z[0]), zs * bfhi(r.z[0])), pack_bf2(zs * bflo(r.z[1]), zs * bfhi(r.z[1]))};
        *reinterpret_cast<u32x2*>(zbuf + vw) = zv;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            ktA[ct] = tr_read(kbuf + kr + 64 * (ct >> 1) + 8 * (ct & 1));
            qtA[ct] = tr_read(qbuf + kr + 64 * (ct >> 1) + 8 * (ct & 1));
        }
        zin = tr_read(zbuf + vr);
        asm volatile("" ::: "memory");
    };
    v4f Y[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) Y[ct] = v4f{0.f, 0.f, 0.f, 0.f};
    // S^T for the A operand: lane (g, m) holds S[t = 4g+i][s = m], kept for t >= s
    const u32x2 keep{(4 * g >= m ? 0xFFFFu : 0u) | (4 * g + 1 >= m ? 0xFFFF0000u : 0u),
                     (4 * g + 2 >= m ? 0xFFFFu : 0u) | (4 * g + 3 >= m ? 0xFFFF0000u : 0u)};
    const float alpha_full = -2.f * eta / (float)b;
    const float alpha_last = -2.f * eta / (float)(N - (nch - 1) * b);
    bf16_t* dwn = w.dwn + (long long)ch * nch * 4096;
    float* dRp = w.dRp + (long long)ch * N * 64;
    v4s_t ktA[4], qtA[4], zin;
    stage(cr[0], 0, ktA, qtA, zin);
    const int nsteps = (nch + kBD - 1) / kBD * kBD;
    int c = nch - 1; // mini-batch being walked
    for (int j0 = 0; j0 < nsteps; j0 += kBD) {
#pragma unroll
        for (int u = 0; u < kBD; ++u) {
            Regs& r = cr[u];
            const bool live = c >= 0;
            const float alpha = !live ? 0.f : (c == nch - 1 ? alpha_last : alpha_full);
            // bf16 copy of Y for K Y; store Y (the gradient at this mini-batch's end)
            u32x4 ys[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                ys[kb] = u32x4{pack_bf2(Y[2 * kb][0], Y[2 * kb][1]), pack_bf2(Y[2 * kb][2], Y[2 * kb][3]),
                               pack_bf2(Y[2 * kb + 1][0], Y[2 * kb + 1][1]), pack_bf2(Y[2 * kb + 1][2], Y[2 * kb + 1][3])};
            if (live) {
                bf16_t* o = dwn + (long long)c * 4096 + (16 * rb + m) * 64 + 8 * g;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) *reinterpret_cast<u32x4*>(o + 32 * kb) = ys[kb];
            }
            // S = Q K^T (lane: S[4g+i][m]); dR = alpha (S^T dZ + K Y), all on
            // 16x16x32 products chained through one accumulator: S^T dZ has
            // only 16 tokens, so its k slots 8g+4 .. 8g+7 are zero (the
            // slots 8g .. 8g+3 take token 4g+i: the kept S^T of the lane's
            // accumulator, dZ of the transposed read), then K Y over the 64
            // channels.  (One product shape only: a 16x16x16 result chained
            // into a 16x16x32 accumulator is read before it is complete.)
            const v4f zero4{0.f, 0.f, 0.f, 0.f};
            const v4f S = mfma32(as_v8bf(r.q[1]), as_v8bf(r.k[1]), mfma32(as_v8bf(r.q[0]), as_v8bf(r.k[0]), zero4));
            const u32x2 zb = __builtin_bit_cast(u32x2, zin);
            const u32x4 sA{pack_bf2(S[0], S[1]) & keep[0], pack_bf2(S[2], S[3]) & keep[1], 0u, 0u};
            const u32x4 zB{zb[0], zb[1], 0u, 0u};
            const v4f KY = mfma32(as_v8bf(r.k[1]), as_v8bf(ys[1]),
                                  mfma32(as_v8bf(r.k[0]), as_v8bf(ys[0]), mfma32(as_v8bf(sA), as_v8bf(zB), zero4)));
            const v4f dR{alpha * KY[0], alpha * KY[1], alpha * KY[2], alpha * KY[3]};
            // dR by walk position (token slot 4g+i of mini-batch c, channel
            // 16 rb + m), turned through LDS so that a lane holds four
            // channels of one token and the wave stores it with one
            // instruction: a wave can keep only so many memory operations in
            // flight, and with one store per token slot they, not the loads
            // a few mini-batches ahead, bounded the walk
#pragma unroll
            for (int i = 0; i < 4; ++i) drt[(4 * g + i) * 20 + m] = dR[i];
            if (live) {
                const int n = c == nch - 1 ? N - (nch - 1) * b : b;
                const int t = lane >> 2, q4 = lane & 3;
                const f32x4 x = *reinterpret_cast<const f32x4*>(drt + t * 20 + 4 * q4);
                if (t < n) *reinterpret_cast<f32x4*>(dRp + ((long long)c * b + t) * 64 + 16 * rb + 4 * q4) = x;
            }
            const u32x2 dr2{pack_bf2(dR[0], dR[1]), pack_bf2(dR[2], dR[3])};
            // the next mini-batch's operands, one step ahead of their use
            v4s_t ktN[4], qtN[4], zN;
            stage(cr[(u + 1) % kBD], (u + 1) & 1, ktN, qtN, zN);
            // Y += K^T dR + Q^T dZ as one 16x16x32 product per tile: k slots
            // 8g .. 8g+3 are token 4g+i of the K^T dR term, 8g+4 .. 8g+7 the
            // same token of the Q^T dZ term (the lane holds both operand
            // pieces already: the transposed reads and dR, dZ of slot 4g+i)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const u32x2 ka = __builtin_bit_cast(u32x2, ktA[ct]), qa = __builtin_bit_cast(u32x2, qtA[ct]);
                const u32x4 A{ka[0], ka[1], qa[0], qa[1]}, B{dr2[0], dr2[1], zb[0], zb[1]};
                Y[ct] = mfma32(as_v8bf(A), as_v8bf(B), Y[ct]);
            }
            issue(r);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                ktA[ct] = ktN[ct];
                qtA[ct] = qtN[ct];
            }
            zin = zN;
            --c;
        }
    }
    // the chain's dW0 contribution: Y at the walk's end (W layout, rows 16 rb + m)
    float* o = w.dW0c + (long long)ch * 4096 + (16 * rb + m) * 64 + 8 * g;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        *reinterpret_cast<f32x4*>(o + 32 * kb) = f32x4{Y[2 * kb][0], Y[2 * kb][1], Y[2 * kb][2], Y[2 * kb][3]};
        *reinterpret_cast<f32x4*>(o + 32 * kb + 4) = f32x4{Y[2 * kb + 1][0], Y[2 * kb + 1][1], Y[2 * kb + 1][2], Y[2 * kb + 1][3]};
    }
}

// The two walks do not depend on each other (the gradient walk reads K, Q
// and dZ only): one workgroup per (chain, 16-row block) runs both, wave 0
// the forward states, wave 1 the gradient walk, on two SIMDs of one CU.
// Spread: the workgroup takes more than half a CU's LDS, so no two share a
// CU (used when the grid fits the device one workgroup per CU; single-wave
// workgroups of the two walks packed onto shared SIMDs ran 252 us against
// 88 + 179 us apart).
constexpr int kWalksLds = kNK * kKBuf + 2 * kVBuf + 2 * (2 * kKBuf + kVBuf) + 16 * 20 * 4; // the two waves' own LDS
template <bool Spread>
__global__ __launch_bounds__(128, 1) void scan_bwd_walks(BwdWalkArgs w, bf16_t* states) {
    __shared__ char spread[Spread ? kOneCuLds - kWalksLds : 16];
    if (threadIdx.x == 0) asm volatile("" ::"v"(spread)); // kept: it only reserves LDS
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave == 0) states_wave(w.s, states, w.nd, (int)blockIdx.x);
    else grad_wave(w, (int)blockIdx.x);
}
static_assert(kWalksLds < kOneCuLds, "backward walks LDS");

// Chunk-parallel scan, second pass: segment start states in order,
// W_s = W_{s-1} S_M(s-1) + S_U(s-1), W_0 = W0 (fp32 matrix cores, 16x16x4
// tiles).  The rows of W (output channels) are independent: one workgroup
// per (chain, 16-row block), wave w forming columns 16w .. 16w+15; the maps
// are loaded two steps ahead.
__global__ __launch_bounds__(256) void scan_starts(ScanArgs a) {
    __shared__ __attribute__((aligned(16))) float Wl[16 * 68];
    __shared__ __attribute__((aligned(16))) float Ml[64 * 68];
    const int chains = a.slices * (a.split ? 2 : 1);
    const int c = blockIdx.x >> 2, rb = blockIdx.x & 3;
    if (c >= chains) return;
    const int dir = a.split ? (c >= a.slices ? 1 : 0) : (a.mode == 2 ? 1 : 0);
    const int slice = c % a.slices, h = slice % a.H;
    const float* W0h = a.W0 + ((a.w0dir && dir ? (long long)a.H : 0) + h) * 4096;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, g = lane >> 4, m = lane & 15;
    // this thread's share of a map: float4s t + 256 j of S_M, and the four
    // S_U entries of its output tile
    struct MapRegs {
        f32x4 mr[4];
        float ur[4];
    } rg[2];
    auto fetch = [&](MapRegs& r, int s) __attribute__((always_inline)) {
        if (s >= a.nseg) return;
        const float* SM = a.maps + ((long long)c * (a.nseg - 1) + (s - 1)) * 2 * 4096;
        const float* SU = SM + 4096;
#pragma unroll
        for (int j = 0; j < 4; ++j) r.mr[j] = reinterpret_cast<const f32x4*>(SM)[t + 256 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i) r.ur[i] = SU[(16 * rb + 4 * g + i) * 64 + 16 * w + m];
    };
    auto step = [&](MapRegs& r, int s) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = t + 256 * j; // float4 q: row q / 16, columns 4 (q % 16) ..
            *reinterpret_cast<f32x4*>(Ml + (q >> 4) * 68 + 4 * (q & 15)) = r.mr[j];
        }
        v4f acc{r.ur[0], r.ur[1], r.ur[2], r.ur[3]};
        fetch(r, s + 2);
        lds_barrier(); // W_{s-1} rows and S_M in LDS
#pragma unroll
        for (int k = 0; k < 16; ++k) // D[16rb + 4g+i][16w + m] += W[16rb + m][4k + g] S_M[4k + g][16w + m]
            acc = mfma4(Wl[m * 68 + 4 * k + g], Ml[(4 * k + g) * 68 + 16 * w + m], acc);
        lds_barrier(); // every wave has read W_{s-1} and S_M
        float* out = a.starts + ((long long)c * a.nseg + s) * 4096 + 16 * rb * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Wl[(4 * g + i) * 68 + 16 * w + m] = acc[i];
            out[(4 * g + i) * 64 + 16 * w + m] = acc[i];
        }
    };
    fetch(rg[0], 1);
    fetch(rg[1], 2);
    for (int e = t; e < 1024; e += 256) Wl[(e >> 6) * 68 + (e & 63)] = W0h[16 * rb * 64 + e];
    for (int s = 1; s < a.nseg; s += 2) {
        step(rg[0], s);
        if (s + 1 < a.nseg) step(rg[1], s + 1);
    }
}

// Z = (forward + backward) / 2 from the two directions' fp32 outputs,
// rounded to bf16 once; 8 channels per thread.
__global__ __launch_bounds__(256) void scan_average(ScanArgs a) {
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x; // (slice, token, channel octet)
    if (e >= (long long)a.slices * a.N * 8) return;
    const int c8 = (int)(e & 7);
    const long long st = e >> 3;
    const int p = (int)(st % a.N), slice = (int)(st / a.N);
    const int bb = slice / a.H, h = slice % a.H;
    const f32x4* xp = reinterpret_cast<const f32x4*>(a.P + st * 64 + 8 * c8);
    const f32x4* yp = reinterpret_cast<const f32x4*>(a.P2 + st * 64 + 8 * c8);
    const f32x4 x0 = xp[0], x1 = xp[1], y0 = yp[0], y1 = yp[1];
    u32x4 o;
    o[0] = pack_bf2(0.5f * (x0[0] + y0[0]), 0.5f * (x0[1] + y0[1]));
    o[1] = pack_bf2(0.5f * (x0[2] + y0[2]), 0.5f * (x0[3] + y0[3]));
    o[2] = pack_bf2(0.5f * (x1[0] + y1[0]), 0.5f * (x1[1] + y1[1]));
    o[3] = pack_bf2(0.5f * (x1[2] + y1[2]), 0.5f * (x1[3] + y1[3]));
    bf16_t* z = (bf16_t*)a.Z.ptr + bb * a.Z.sb + h * a.Z.sh + (long long)p * a.Z.sn + 8 * c8;
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(z));
}

} // namespace

// Segments of the chunk-parallel scan.  A chain's walk is bound by the
// throughput of the CU it runs on, not by the recurrence's latency: cut
// into segments that share CUs, the 1280x1280 scan (48 chains, 192
// workgroups) took 164 us at 4 segments against 95 us in one walk (maps and
// walks both slowed by the sharing).  So a chain is cut only while its
// segments' workgroups still get a CU each: P = CUs / (4 chains), at most
// kMaxSeg, with at least 8 mini-batches per segment.  forced > 0 (a test
// switch) takes that count within the same limits.
constexpr int kMaxSeg = 8;
int scan_segments(long long chains, int nmb, int cus, int forced) {
    if (chains <= 0 || chains * 4 >= 1024) return 1;
    long long P = forced > 0 ? forced : (long long)(cus > 0 ? cus : 256) / (chains * 4);
    if (P > kMaxSeg) P = kMaxSeg;
    if (forced <= 0 && P > nmb / 8) P = nmb / 8;
    if (P > nmb) P = nmb;
    return P < 1 ? 1 : (int)P;
}

size_t scan_ws_bytes(int B, int H, int N, int mode) {
    size_t bytes = 256;
    if (mode == 0) bytes += 2 * (size_t)B * H * N * 64 * sizeof(float);
    const long long chains = (long long)B * H * (mode == 0 ? 2 : 1);
    if (chains * 4 < 1024) // room for kMaxSeg segments: maps, then start states
        bytes += (size_t)chains * ((kMaxSeg - 1) * 2 + kMaxSeg) * 4096 * sizeof(float);
    return bytes;
}

bool scan_minibatch_supported(int b, int N) { return b >= 1 && N >= 0; }

hipError_t launch_scan_bwd_walks(const ScanBwdWalks& l, hipStream_t stream) {
    if (l.b < 1 || l.b > 16) return hipErrorNotSupported;
    ScanArgs a{};
    a.K = l.K; a.V = l.V; a.Q = l.Q;
    a.W0 = l.W0; a.eta = l.eta;
    a.w0dir = l.w0dir;
    a.H = l.H; a.N = l.N; a.b = l.b;
    a.nch = (l.N + l.b - 1) / l.b;
    a.tb = l.b;
    a.T = 1;
    a.ntile = a.nch;
    a.slices = l.B * l.H;
    a.mode = l.mode;
    a.nseg = 1;
    const int nd = l.mode == 0 ? 2 : 1;
    // chains padded to whole XCD groups, 4 row blocks each
    const unsigned blocks = (unsigned)(((4LL * a.slices * nd + 31) / 32) * 32);
    BwdWalkArgs w{};
    w.s = a;
    w.Q = l.Q;
    w.dZ = l.dZ;
    w.dwn = l.dwn;
    w.dRp = l.dRp;
    w.dW0c = l.dW0c;
    w.nd = nd;
    if ((int)blocks <= l.cus) hipLaunchKernelGGL(scan_bwd_walks<true>, dim3(blocks), dim3(128), 0, stream, w, l.states);
    else hipLaunchKernelGGL(scan_bwd_walks<false>, dim3(blocks), dim3(128), 0, stream, w, l.states);
    return hipGetLastError();
}

hipError_t launch_scan(ScanLaunch s, hipStream_t stream) {
    if (!s.bf16) return hipErrorNotSupported;
    ScanArgs a{};
    a.K = s.K; a.Q = s.Q; a.V = s.V; a.Z = s.Z;
    a.W0 = s.W0; a.eta = s.eta;
    a.w0dir = s.w0dir;
    a.H = s.H; a.N = s.N; a.b = s.b;
    a.nch = (s.N + s.b - 1) / s.b;
    // tiles: a mini-batch of b <= 16 tokens is one tile; a larger one is
    // T = ceil(min(b, N) / 16) tiles of 16 positions, the last of them
    // ragged unless b is a multiple of 16 (or b >= N: one mini-batch)
    a.tb = s.b <= 16 ? s.b : 16;
    a.T = s.b <= 16 ? 1 : (std::min(s.b, s.N) + 15) / 16;
    const int nlast = s.N - (a.nch - 1) * s.b;
    a.ntile = (a.nch - 1) * a.T + (nlast + a.tb - 1) / a.tb;
    const bool rg = s.b > 16 && s.b % 16 != 0 && s.b < s.N;
    a.slices = s.B * s.H;
    a.mode = s.mode;
    // both directions: each in workgroups of its own, fp32 outputs averaged
    // by a second kernel
    a.split = s.mode == 0 ? 1 : 0;
    a.xcd = 1;
    const long long chains = (long long)a.slices * (a.split ? 2 : 1);
    a.nseg = scan_segments(chains, a.nch, s.cus, s.segs);
    // per direction: (slice, segment) units padded to whole XCD groups, 4 blocks each
    const long long blocks = ((long long)a.slices * a.nseg + 7) / 8 * 8 * 4;
    a.blocks = (int)blocks;
    // workspace: [256 bytes reserved][P][P2][segment maps][segment starts]
    float* cur = (float*)s.ws + 64;
    if (a.split) {
        a.P = cur;
        a.P2 = a.P + (size_t)a.slices * s.N * 64;
        cur = a.P2 + (size_t)a.slices * s.N * 64;
    }
    const int dirs = a.split ? 2 : 1;
    if (a.nseg > 1) {
        a.maps = cur;
        a.starts = cur + (size_t)chains * (kMaxSeg - 1) * 2 * 4096;
        const long long mblocks = ((long long)a.slices * (a.nseg - 1) + 7) / 8 * 8 * 8;
        if (rg) hipLaunchKernelGGL(scan_maps<true>, dim3((unsigned)(dirs * mblocks)), dim3(64), 0, stream, a);
        else hipLaunchKernelGGL(scan_maps<false>, dim3((unsigned)(dirs * mblocks)), dim3(64), 0, stream, a);
        hipLaunchKernelGGL(scan_starts, dim3((unsigned)(4 * chains)), dim3(256), 0, stream, a);
    }
    const long long grid = blocks * dirs;
    const dim3 gd((unsigned)grid), bd(128);
    if (grid <= s.cus) {
        if (rg) hipLaunchKernelGGL((scan_kernel<true, true>), gd, bd, 0, stream, a);
        else hipLaunchKernelGGL((scan_kernel<true, false>), gd, bd, 0, stream, a);
    } else {
        if (rg) hipLaunchKernelGGL((scan_kernel<false, true>), gd, bd, 0, stream, a);
        else hipLaunchKernelGGL((scan_kernel<false, false>), gd, bd, 0, stream, a);
    }
    if (a.split) {
        const long long n = (long long)a.slices * s.N * 8;
        hipLaunchKernelGGL(scan_average, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

} // namespace ttt
