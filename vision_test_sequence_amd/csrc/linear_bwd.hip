// linear_bwd.hip -- gradient of the full-batch linear TTT step, gfx950.
//
// Forward (ViT^3 page, the inner linear model and its one full-batch
// gradient step; the gradient itself is what end-to-end training needs,
// the page's section on the "gradient of the gradient"):
//   G = (2/N) (W0 A - C),  A = K^T K,  C = V^T K,  W1 = W0 - eta G,  Z = Q W1^T.
// Backward of L(dZ) = <dZ, Z>, with beta = 2 eta / N:
//   dW1 = dZ^T Q                          (reduction over the tokens)
//   dQ  = dZ W1
//   M   = W0^T dW1 + dW1^T W0             (symmetric)
//   dK  = beta (V dW1 - K M)
//   dV  = beta K dW1^T
//   dW0 = sum_b dW1 (I - beta A),  deta = -sum_b <dW1, G>.
// Three launches (plus the forward's Gram pass when A and G were not saved):
//   pass 1   per (slice, split): dQ for its tokens and its share of dW1;
//   reduce   per slice: dW1, M, the slice's dW0 and deta terms;
//   pass 2   per (slice, split): dK, dV for its tokens; its first H x 16
//            workgroups also sum dW0 and deta over b in ascending order
//            (a fourth launch, batch, when the grid is smaller).
// Every reduction has a fixed order, so results are bitwise reproducible.
//
// Products on the matrix cores (16x16 tiles, lane l = 16 g + m):
//  * per-token products (dQ, dK, dV) take the 64x64 operator as the A
//    operand with output rows permuted by perm_row, and the token rows as
//    the B operand straight from memory; a lane then stores 8 contiguous
//    channels of its token.
//  * dW1 = dZ^T Q contracts over tokens: each wave writes its 32-token rows
//    of dZ and Q to a private LDS area and reads them back transposed with
//    ds_read_b64_tr_b16 (bf16) or single-element reads (fp32).
// bf16 inputs use 16x16x32 bf16 products with fp32 accumulation; fp32
// inputs use 16x16x4 fp32 products throughout.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace ttt {
namespace {

constexpr int MB = 68;     // pitch (floats) of 64x64 fp32 matrices in LDS
constexpr int kRowB = 72;  // pitch (bf16) of a staged bf16 token row (144 bytes)
constexpr int kRowF = 68;  // pitch (floats) of a staged fp32 token row (272 bytes)


struct BwdArgs {
    View4 X0, X1;     // pass 1: dZ, Q.   pass 2: K, V
    View4 O0, O1;     // pass 1: dQ.      pass 2: dK, dV
    const float* W0;
    const float* eta;
    const float* saved; // [slices][2][64][64]: A then G
    float* part;        // [slices][S][64][64]: dW1 shares
    float* dm;          // [slices][2][64][64]: dW1 then M
    float* dW0s;        // [slices][64][64]
    float* detas;       // [slices]
    float* dW0;         // [H][64][64]
    float* deta;        // [H]
    u32x4* fr;          // [slices][3][8][64]: bf16 fragments of beta dW1^T, -beta M, beta dW1
    int B, H, N, S, per, xcd;
    int S2, per2;       // bf16 pass 2: splits per slice, tokens per split (<= kP2Tok)
    int dot;            // dot-product loss: beta = eta / N, M = 0, dW0 = sum_b dW1
    int batch_in_pass2; // bf16 pass 2 forms the batch sums (its grid has >= H x 16 workgroups)
};

// beta of the loss: L2 G = (2/N)(W0 A - C); dot-product G = -(1/N) C.
__device__ __forceinline__ float bwd_beta(const BwdArgs& a, int h) {
    return (a.dot ? 1.0f : 2.0f) * a.eta[h] / (float)a.N;
}
constexpr int kP2Tok = 256; // bf16 pass 2: tokens per workgroup, resident in LDS
constexpr int kP1Tok = 256; // bf16 pass 1: tokens per workgroup, resident in LDS (64 KB: two per CU)

// ------------------------------------------------------------ fragments --
template <bool BF> struct Frags;
template <> struct Frags<true> {
    v8bf f[4][2];
};
template <> struct Frags<false> {
    float f[4][16];
};
template <bool BF> struct Row;
template <> struct Row<true> {
    u32x4 x[2]; // channels 32 kb + 8 g .. +7
};
template <> struct Row<false> {
    u32x4 x[4]; // channels 16 hh + 4 g .. +3
};

// A operand of Wt[o][k] = s * (tr ? M[k][o] : M[o][k]) with output rows
// o = perm_row(rb, m); M is 64x64 fp32 in LDS (pitch MB).
template <bool BF>
__device__ __forceinline__ Frags<BF> make_frags(const float* M, bool tr, float s, int g, int m) {
    Frags<BF> F;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int o = perm_row(rb, m);
        auto at = [&](int k) { return s * (tr ? M[k * MB + o] : M[o * MB + k]); };
        if constexpr (BF) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int k0 = 32 * kb + 8 * g;
                u32x4 u{pack_bf2(at(k0), at(k0 + 1)), pack_bf2(at(k0 + 2), at(k0 + 3)),
                        pack_bf2(at(k0 + 4), at(k0 + 5)), pack_bf2(at(k0 + 6), at(k0 + 7))};
                F.f[rb][kb] = as_v8bf(u);
            }
        } else {
#pragma unroll
            for (int hh = 0; hh < 4; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i) F.f[rb][4 * hh + i] = at(16 * hh + 4 * g + i);
        }
    }
    return F;
}

template <bool BF>
__device__ __forceinline__ Row<BF> load_row(const char* row, int g) {
    Row<BF> r;
    if constexpr (BF) {
        r.x[0] = *reinterpret_cast<const u32x4*>(row + (8 * g) * 2);
        r.x[1] = *reinterpret_cast<const u32x4*>(row + (32 + 8 * g) * 2);
    } else {
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) r.x[hh] = *reinterpret_cast<const u32x4*>(row + (16 * hh + 4 * g) * 4);
    }
    return r;
}
template <bool BF> __device__ __forceinline__ void zero_row(Row<BF>& r) {
#pragma unroll
    for (int i = 0; i < (BF ? 2 : 4); ++i) r.x[i] = u32x4{0u, 0u, 0u, 0u};
}

// d[rb] += Wt x  for the lane's token row x
template <bool BF>
__device__ __forceinline__ void mac(const Frags<BF>& F, const Row<BF>& x, v4f* d) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        if constexpr (BF) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) d[rb] = mfma32(F.f[rb][kb], as_v8bf(x.x[kb]), d[rb]);
        } else {
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                const f32x4 xv = __builtin_bit_cast(f32x4, x.x[hh]);
#pragma unroll
                for (int i = 0; i < 4; ++i) d[rb] = mfma4(F.f[rb][4 * hh + i], xv[i], d[rb]);
            }
        }
    }
}

// lane (g, m) holds out[token m][perm_row(rb, 4g+i)]: channels 8g..8g+7 and
// 32+8g..32+8g+7
template <bool BF> __device__ __forceinline__ void store_row(char* row, const v4f* d, int g) {
    if constexpr (BF) {
        const u32x4 o0{pack_bf2(d[0][0], d[0][1]), pack_bf2(d[0][2], d[0][3]), pack_bf2(d[1][0], d[1][1]),
                       pack_bf2(d[1][2], d[1][3])};
        const u32x4 o1{pack_bf2(d[2][0], d[2][1]), pack_bf2(d[2][2], d[2][3]), pack_bf2(d[3][0], d[3][1]),
                       pack_bf2(d[3][2], d[3][3])};
        // streaming stores: the gradients are not read again here
        __builtin_nontemporal_store(o0, reinterpret_cast<u32x4*>(row + (8 * g) * 2));
        __builtin_nontemporal_store(o1, reinterpret_cast<u32x4*>(row + (32 + 8 * g) * 2));
    } else {
        float* r = reinterpret_cast<float*>(row);
        __builtin_nontemporal_store(f32x4{d[0][0], d[0][1], d[0][2], d[0][3]}, reinterpret_cast<f32x4*>(r + 8 * g));
        __builtin_nontemporal_store(f32x4{d[1][0], d[1][1], d[1][2], d[1][3]}, reinterpret_cast<f32x4*>(r + 8 * g + 4));
        __builtin_nontemporal_store(f32x4{d[2][0], d[2][1], d[2][2], d[2][3]}, reinterpret_cast<f32x4*>(r + 32 + 8 * g));
        __builtin_nontemporal_store(f32x4{d[3][0], d[3][1], d[3][2], d[3][3]}, reinterpret_cast<f32x4*>(r + 36 + 8 * g));
    }
}

struct Ctx {
    int slice, split, b, h, t0, t1;
};
__device__ __forceinline__ Ctx ctx_of(const BwdArgs& a) {
    Ctx c;
    const SliceSplit ss = map_block(blockIdx.x, a.S, a.xcd);
    c.slice = ss.slice;
    c.split = ss.split;
    c.b = c.slice / a.H;
    c.h = c.slice % a.H;
    c.t0 = min(a.N, c.split * a.per);
    c.t1 = min(a.N, c.t0 + a.per);
    return c;
}
template <int ESZ> __device__ __forceinline__ const char* base_of(const View4& v, const Ctx& c) {
    return (const char*)v.ptr + (c.b * v.sb + c.h * v.sh) * (long long)ESZ;
}

// ---------------------------------------------------------------- pass 1 --
// dQ = dZ W1 for the workgroup's tokens and its share of dW1 = dZ^T Q.
template <bool BF>
__global__ __launch_bounds__(kThreads, 1) void bwd_pass1(BwdArgs a) {
    constexpr int ESZ = BF ? 2 : 4;
    constexpr int WAVE_BYTES = BF ? 2 * 32 * kRowB * 2 : 2 * 32 * kRowF * 4; // dZ + Q rows
    constexpr int LDS_BYTES = 4 * 64 * 64 * 4 > 4 * WAVE_BYTES ? 4 * 64 * 64 * 4 : 4 * WAVE_BYTES;
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    float* ldsf = reinterpret_cast<float*>(lds);

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Ctx c = ctx_of(a);
    if (c.slice >= a.B * a.H) return; // padding block of the XCD-aware grid

    // W1 = W0 - eta G in LDS, then the A operand of dQ^T = W1^T dZ^T
    {
        const float eta = a.eta[c.h];
        const float* W0 = a.W0 + (long long)c.h * 4096;
        const float* G = a.saved + (long long)c.slice * 8192 + 4096;
        for (int e = tid; e < 4096; e += kThreads) ldsf[(e >> 6) * MB + (e & 63)] = W0[e] - eta * G[e];
    }
    __syncthreads();
    const Frags<BF> F = make_frags<BF>(ldsf, true, 1.0f, g, m);
    __syncthreads();

    const char* dZp = base_of<ESZ>(a.X0, c);
    const char* Qp = base_of<ESZ>(a.X1, c);
    char* dQp = (char*)base_of<ESZ>(a.O0, c);
    const long long sz = a.X0.sn * ESZ, sq = a.X1.sn * ESZ, so = a.O0.sn * ESZ;
    char* wz = lds + w * WAVE_BYTES;       // this wave's 32 dZ rows
    char* wq = wz + WAVE_BYTES / 2;        // and 32 Q rows

    v4f acc[16]; // dW1 tile (rb, cb) = acc[4 rb + cb]: [16rb + 4g + i][16cb + m]
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    // wave steps of 32 tokens: wave w takes tokens t0 + 128 s + 32 w + [0, 32)
    const int nst = (c.t1 - c.t0 + 127) / 128;
    for (int s = 0; s < nst; ++s) {
        const int tb = c.t0 + 128 * s + 32 * w;
        Row<BF> z[2], q[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = tb + 16 * h + m;
            const int tc = min(t, c.t1 - 1);
            z[h] = load_row<BF>(dZp + tc * sz, g);
            q[h] = load_row<BF>(Qp + tc * sq, g);
            if (t >= c.t1) {
                zero_row<BF>(z[h]);
                zero_row<BF>(q[h]);
            }
        }
        // dQ for both halves
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4f d[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) d[rb] = v4f{0.f, 0.f, 0.f, 0.f};
            mac<BF>(F, z[h], d);
            const int t = tb + 16 * h + m;
            if (t < c.t1) store_row<BF>(dQp + t * so, d, g);
        }
        // dW1 += dZ^T Q over these 32 tokens
        if constexpr (BF) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int off = ((16 * h + m) * kRowB + 32 * kb + 8 * g) * 2;
                    *reinterpret_cast<u32x4*>(wz + off) = z[h].x[kb];
                    *reinterpret_cast<u32x4*>(wq + off) = q[h].x[kb];
                }
            // transposed operand reads: lane (g, 4e + a) points at token
            // 8g + e (+4), channels 16 blk + 4a .. +3
            const int e = (lane & 15) >> 2, aa = lane & 3;
            v8bf A[4], Bq[4];
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const int o0 = ((8 * g + e) * kRowB + 16 * blk + 4 * aa) * 2;
                const int o1 = o0 + 4 * kRowB * 2;
                const v4s_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(wz + o0));
                const v4s_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(wz + o1));
                const v4s_t b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(wq + o0));
                const v4s_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(wq + o1));
                A[blk] = __builtin_bit_cast(v8bf, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
                Bq[blk] = __builtin_bit_cast(v8bf, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) acc[4 * rb + cb] = mfma32(A[rb], Bq[cb], acc[4 * rb + cb]);
        } else {
            float* fz = reinterpret_cast<float*>(wz);
            float* fq = reinterpret_cast<float*>(wq);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) {
                    const int off = (16 * h + m) * kRowF + 16 * hh + 4 * g;
                    *reinterpret_cast<u32x4*>(fz + off) = z[h].x[hh];
                    *reinterpret_cast<u32x4*>(fq + off) = q[h].x[hh];
                }
#pragma unroll 2
            for (int kk = 0; kk < 8; ++kk) {
                const int t = 4 * kk + g;
                float av[4], bv[4];
#pragma unroll
                for (int blk = 0; blk < 4; ++blk) {
                    av[blk] = fz[t * kRowF + 16 * blk + m];
                    bv[blk] = fq[t * kRowF + 16 * blk + m];
                }
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) acc[4 * rb + cb] = mfma4(av[rb], bv[cb], acc[4 * rb + cb]);
            }
        }
    }

    // sum the four waves' shares (fixed order) and publish this split's dW1
    __syncthreads();
    float* red = ldsf + w * 4096;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(16 * rb + 4 * g + i) * 64 + 16 * cb + m] = acc[4 * rb + cb][i];
    __syncthreads();
    float* dst = a.part + ((long long)c.slice * a.S + c.split) * 4096;
#pragma unroll 4
    for (int e = tid; e < 4096; e += kThreads)
        dst[e] = ((ldsf[e] + ldsf[4096 + e]) + ldsf[8192 + e]) + ldsf[12288 + e];
}

// ------------------------------------------------------ pass 1 (bf16) --
// dQ = dZ W1 and the split's dW1 = dZ^T Q with the split's dZ and Q rows
// staged in LDS chunk by chunk (kP1Tok tokens each) by direct-to-LDS loads
// with the swz_tr swizzle; in each chunk the first half is processed while
// the second lands.  dW1 by row ownership: wave w accumulates rows 16w..
// over every token of the split (dZ block w against all Q blocks,
// transposed reads), so the waves add nothing up; each stores its rows of
// the split's share.  Several chunks per split keep the shares (and the
// reduce's reads of them) few.
__global__ __launch_bounds__(kThreads, 2) void bwd_pass1_bf(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[2 * kP1Tok * 128];
    static_assert(kP1Tok * 64 >= 4096 * 4, "W1 fits in the upper half of the dZ rows");
    char* Zs = lds;
    char* Qs = lds + kP1Tok * 128;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = blockIdx.x / a.S, split = blockIdx.x % a.S;
    if (slice >= a.B * a.H) return;
    const int b = slice / a.H, h = slice % a.H;
    const int s0 = min(a.N, split * a.per), s1 = min(a.N, s0 + a.per);
    const char* Zp = (const char*)a.X0.ptr + (b * a.X0.sb + h * a.X0.sh) * 2LL;
    const char* Qp = (const char*)a.X1.ptr + (b * a.X1.sb + h * a.X1.sh) * 2LL;
    char* dQp = (char*)a.O0.ptr + (b * a.O0.sb + h * a.O0.sh) * 2LL;
    const long long sz = a.X0.sn * 2, sq = a.X1.sn * 2, so = a.O0.sn * 2;

    // rows [q_begin, q_end) x 8 of the chunk at token t0 (T tokens; rows
    // past T load clamped copies); returns the instructions this wave issued
    auto issue = [&](int t0, int T, int q_begin, int q_end) __attribute__((always_inline)) {
        int n = 0;
        for (int q = q_begin + w; q < q_end; q += 4, ++n) {
            const int p = q * 64 + lane, row = p >> 3;
            const int off = ((p & 7) ^ swz_tr(row)) * 16;
            const long long tk = t0 + min(row, T - 1);
            dma16(Zp + tk * sz + off, Zs + q * 1024);
            dma16(Qp + tk * sq + off, Qs + q * 1024);
        }
        return 2 * n;
    };
    v4f acc[4], unused[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = unused[cb] = v4f{0.f, 0.f, 0.f, 0.f};
    v8bf F[4][2];
    for (int t0 = s0; t0 < s1; t0 += kP1Tok) {
        const int T = min(kP1Tok, s1 - t0);
        const int rows = (T + 31) & ~31, ninstr = rows / 8;
        const int half = min(ninstr, kP1Tok / 16); // rows < kP1Tok / 2
        if (t0 == s0) {
            issue(t0, T, 0, half);
            // W1 = W0 - eta G (the forward's G) staged in fp32 in the upper
            // half of the dZ rows, which only the second half's loads fill;
            // row k's columns are XOR-swizzled by sw(k) = 4 ((k >> 3) & 1) +
            // 32 ((k >> 4) & 1) so that the fragment reads below spread over
            // all banks
            float* w1s = reinterpret_cast<float*>(Zs + kP1Tok * 64);
            {
                const float eta = a.eta[h];
                const f32x4* W04 = reinterpret_cast<const f32x4*>(a.W0 + (long long)h * 4096);
                const f32x4* G4 = reinterpret_cast<const f32x4*>(a.saved + (long long)slice * 8192 + 4096);
                f32x4 wv[4], gv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wv[i] = W04[tid + kThreads * i];
                    gv[i] = G4[tid + kThreads * i];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e4 = tid + kThreads * i, k = e4 >> 4;
                    const int col = ((e4 & 15) * 4) ^ (4 * ((k >> 3) & 1) + 32 * ((k >> 4) & 1));
                    *reinterpret_cast<f32x4*>(w1s + k * 64 + col) =
                        f32x4{wv[i][0] - eta * gv[i][0], wv[i][1] - eta * gv[i][1], wv[i][2] - eta * gv[i][2],
                              wv[i][3] - eta * gv[i][3]};
                }
            }
            // W1 is staged; this wave's first-half rows, loaded before W0
            // and G, have landed too (a wave's loads return in order)
            __syncthreads();
            // W1^T as bf16 A-operand fragments: piece (rb, kb) of lane (g, m)
            // holds W1[k][o], o = perm_row(rb, m), k = 32 kb + 8 g + (0..7)
            // (sw(k) = 4 (g & 1) + 32 (g >> 1) for all eight)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int o = perm_row(rb, m) ^ (4 * (g & 1) + 32 * (g >> 1));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const float* col = w1s + (32 * kb + 8 * g) * 64 + o;
                    F[rb][kb] = as_v8bf(u32x4{pack_bf2(col[0], col[64]), pack_bf2(col[128], col[192]),
                                              pack_bf2(col[256], col[320]), pack_bf2(col[384], col[448])});
                }
            }
            __syncthreads(); // every wave has its fragments before the second half overwrites W1
            issue(t0, T, half, ninstr);
        } else {
            __syncthreads(); // every wave is done with the previous chunk's rows
            issue(t0, T, 0, half);
            vmcnt_at_most(issue(t0, T, half, ninstr)); // this wave's first-half rows have landed
        }

        // rows [r0, r1): dQ of its 16-token steps (wave w: steps = w mod 4),
        // then dW1 rows 16w.. over the rows
        auto process = [&](int r0, int r1) __attribute__((always_inline)) {
            for (int st = r0 / 16 + w; st < r1 / 16; st += 4) {
                const int row = 16 * st + m;
                u32x4 zx[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    zx[kb] = *reinterpret_cast<const u32x4*>(Zs + (row * 8 + ((4 * kb + g) ^ swz_tr(row))) * 16);
                v4f d[4];
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    d[rb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) d[rb] = mfma32(F[rb][kb], as_v8bf(zx[kb]), d[rb]);
                }
                if (row < T) store_row<true>(dQp + (t0 + row) * so, d, g);
            }
            switch (w) {
            case 0: gram_owned_bf<0, true, false>(Qs, Zs, r0, r1, lane, acc, unused); break;
            case 1: gram_owned_bf<1, true, false>(Qs, Zs, r0, r1, lane, acc, unused); break;
            case 2: gram_owned_bf<2, true, false>(Qs, Zs, r0, r1, lane, acc, unused); break;
            default: gram_owned_bf<3, true, false>(Qs, Zs, r0, r1, lane, acc, unused); break;
            }
        };
        // rows past T hold clamped copies: zeroed (after their loads) so the
        // Gram adds nothing for them
        auto zero_tail = [&]() __attribute__((always_inline)) {
            for (int e = tid; e < (rows - T) * 8; e += kThreads) {
                const int off = (T + (e >> 3)) * 128 + (e & 7) * 16;
                *reinterpret_cast<u32x4*>(Zs + off) = u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(Qs + off) = u32x4{0u, 0u, 0u, 0u};
            }
        };
        const int rh = min(rows, kP1Tok / 2);
        __syncthreads(); // every wave's first-half rows have landed
        if (rows == rh && T < rows) {
            zero_tail();
            __syncthreads();
        }
        process(0, rh);
        drain_vmem();
        __syncthreads();
        if (rows > rh) {
            if (T < rows) {
                zero_tail();
                __syncthreads();
            }
            process(rh, rows);
        }
    }
    // this split's share of dW1, rows 16w.. (row-major)
    float* dst = a.part + ((long long)slice * a.S + split) * 4096;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * w + 4 * g + i) * 64 + 16 * cb + m] = acc[cb][i];
}

// ---------------------------------------------------------------- reduce --
// Per slice: dW1 (splits summed in order), M = P + P^T with P = W0^T dW1,
// the slice's dW0 term dW1 - beta dW1 A and deta term -<dW1, G>.
constexpr int kRT = 512; // reduce: threads per workgroup (8 waves)
__global__ __launch_bounds__(kRT, 1) void bwd_reduce(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float D[64 * MB];
    __shared__ __attribute__((aligned(16))) float W[64 * MB];
    __shared__ __attribute__((aligned(16))) float Am[64 * MB];
    __shared__ float red[kRT];
    const int tid = threadIdx.x;
    const int slice = blockIdx.x;
    const int h = slice % a.H;
    const float beta = bwd_beta(a, h);
    const float wa = a.dot ? 0.f : 1.f; // the dot-product loss has no A or M terms
    const float* W0 = a.W0 + (long long)h * 4096;
    const float* A = a.saved + (long long)slice * 8192;
    const float* G = A + 4096;
    const float* part = a.part + (long long)slice * a.S * 4096;
    // thread t owns float4s t + 512 k (k < 2); every load of a chunk of
    // eight splits is in flight at once, the splits are added in order
    const f32x4* p4 = reinterpret_cast<const f32x4*>(part);
    f32x4 w0v[2], av[2], gv[2], acc[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int q = tid + kRT * k;
        w0v[k] = reinterpret_cast<const f32x4*>(W0)[q];
        av[k] = reinterpret_cast<const f32x4*>(A)[q];
        gv[k] = reinterpret_cast<const f32x4*>(G)[q];
        acc[k] = p4[q];
    }
    for (int s0 = 1; s0 < a.S; s0 += 8) {
        f32x4 v[8][2];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int k = 0; k < 2; ++k) v[j][k] = p4[(long long)min(s0 + j, a.S - 1) * 1024 + tid + kRT * k];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s0 + j < a.S) {
#pragma unroll
                for (int k = 0; k < 2; ++k) acc[k] += v[j][k];
            }
    }
    float dsum = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e = 4 * (tid + kRT * k), r = e >> 6, cc = e & 63;
        *reinterpret_cast<f32x4*>(D + r * MB + cc) = acc[k];
        *reinterpret_cast<f32x4*>(W + r * MB + cc) = w0v[k];
        *reinterpret_cast<f32x4*>(Am + r * MB + cc) = av[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) dsum += acc[k][i] * gv[k][i];
    }
    red[tid] = dsum;
    __syncthreads();
    // P = W0^T dW1 (waves 0-3) and Q2 = dW1 A (waves 4-7) on fp32 matrix
    // cores (16x16x4 tiles): wave w owns the 16-row block w mod 4 of its
    // product, four 16-column tiles
    const int lane = tid & 63, g = lane >> 4, m = lane & 15, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int R0 = 16 * (w & 3);
    const bool isP = w < 4;
    const float* Bm = isP ? D : Am; // B operand: dW1 (P) or A (Q2), rows k
    v4f X[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) X[cb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k0 = 0; k0 < 64; k0 += 4) {
        // A operand: W0^T[R0+m][k0+g] (P) or dW1[R0+m][k0+g] (Q2)
        const float xa = isP ? W[(k0 + g) * MB + R0 + m] : D[(R0 + m) * MB + k0 + g];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) X[cb] = mfma4(xa, Bm[(k0 + g) * MB + 16 * cb + m], X[cb]);
    }
    // lane (g, m) holds rows R0 + 4g + i, column 16 cb + m
    float* dm = a.dm + (long long)slice * 8192;
    float* dW0s = a.dW0s + (long long)slice * 4096;
    if (!isP) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = R0 + 4 * g + i, c = 16 * cb + m;
                dW0s[r * 64 + c] = D[r * MB + c] - wa * beta * X[cb][i];
            }
    }
    for (int e = tid; e < 1024; e += kRT) {
        const int r = e >> 4, c4 = (e & 15) * 4;
        *reinterpret_cast<f32x4*>(dm + r * 64 + c4) = *reinterpret_cast<const f32x4*>(D + r * MB + c4);
    }
    __syncthreads(); // every thread has read W
    // M = P + P^T through LDS (W's space is free now)
    if (isP) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) W[(R0 + 4 * g + i) * MB + 16 * cb + m] = X[cb][i];
    }
    __syncthreads();
    if (tid < 256) {
        const int r0 = (tid >> 4) * 4, c0 = (tid & 15) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + i;
            f32x4 mv;
#pragma unroll
            for (int j = 0; j < 4; ++j) mv[j] = wa * (W[r * MB + c0 + j] + W[(c0 + j) * MB + r]);
            *reinterpret_cast<f32x4*>(dm + 4096 + r * 64 + c0) = mv;
            *reinterpret_cast<f32x4*>(Am + r * MB + c0) = mv; // A's space is free now
        }
    }
    __syncthreads();
    // bf16 operator fragments for pass 2 (A operand of Wt[o][k] with output
    // rows o = perm_row(rb, m)): piece (f, rb, kb, lane) holds
    // k = 32 kb + 8 g + (0..7); f = 0: beta dW1^T, 1: -beta M, 2: beta dW1.
    // Each piece is eight consecutive floats of a row of dW1^T, M or dW1:
    // dW1^T is first written to W (free again), so all three are read as
    // two 16-byte LDS reads per piece.
    if (a.fr) {
        if (tid < 256) {
            const int r0 = (tid >> 4) * 4, c0 = (tid & 15) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 dv = *reinterpret_cast<const f32x4*>(D + (r0 + i) * MB + c0);
#pragma unroll
                for (int j = 0; j < 4; ++j) W[(c0 + j) * MB + r0 + i] = dv[j];
            }
        }
        __syncthreads();
        u32x4* fr = a.fr + (long long)slice * 1536;
        static_assert(kRT == 512, "one fragment piece of each of the three operators per thread");
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const int pc = tid, rb = pc >> 7, kb = (pc >> 6) & 1, ln = pc & 63;
            const int o = perm_row(rb, ln & 15), k0 = 32 * kb + 8 * (ln >> 4);
            const float* src = (f == 0 ? W : (f == 1 ? Am : D)) + o * MB + k0;
            const float sc = f == 1 ? -beta : beta;
            const f32x4 x = *reinterpret_cast<const f32x4*>(src), y = *reinterpret_cast<const f32x4*>(src + 4);
            fr[f * 512 + pc] = u32x4{pack_bf2(sc * x[0], sc * x[1]), pack_bf2(sc * x[2], sc * x[3]),
                                     pack_bf2(sc * y[0], sc * y[1]), pack_bf2(sc * y[2], sc * y[3])};
        }
    }
    // deta term: fixed-order tree over the threads' partial sums
    for (int st = kRT / 2; st > 0; st >>= 1) {
        if (tid < st) red[tid] += red[tid + st];
        __syncthreads();
    }
    if (tid == 0) a.detas[slice] = -red[0];
}

// ------------------------------------------------------------ batch sums --
// 16 workgroups per head, one dW0 element per thread; the B terms of an
// element are loaded together and added in ascending b.  blk: the
// workgroup's index among the H x 16.
__device__ __forceinline__ void batch_sums(const BwdArgs& a, int blk) {
    const int h = blk >> 4, tid = threadIdx.x;
    const int e = (blk & 15) * kThreads + tid;
    const float* src = a.dW0s + (long long)h * 4096 + e;
    const long long step = (long long)a.H * 4096;
    float v = 0.f;
    for (int b0 = 0; b0 < a.B; b0 += 8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = src[min(b0 + i, a.B - 1) * step];
            t[i] = b0 + i < a.B ? x : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) v += t[i];
    }
    a.dW0[(long long)h * 4096 + e] = v;
    if ((blk & 15) == 0 && tid == 0) {
        // eight loads at a time before their adds (one past the end adds 0)
        float d = 0.f;
        for (int b0 = 0; b0 < a.B; b0 += 8) {
            float t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = a.detas[(long long)min(b0 + i, a.B - 1) * a.H + h];
                t[i] = b0 + i < a.B ? x : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) d += t[i];
        }
        a.deta[h] = d;
    }
}
__global__ __launch_bounds__(kThreads, 1) void bwd_batch(BwdArgs a) { batch_sums(a, (int)blockIdx.x); }

// ---------------------------------------------------------------- pass 2 --
// dK = beta (V dW1 - K M), dV = beta K dW1^T for the workgroup's tokens.
template <bool BF>
__global__ __launch_bounds__(kThreads, 1) void bwd_pass2(BwdArgs a) {
    constexpr int ESZ = BF ? 2 : 4;
    __shared__ __attribute__((aligned(16))) float mats[2 * 64 * MB];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Ctx c = ctx_of(a);
    if (c.slice >= a.B * a.H) return; // padding block of the XCD-aware grid

    const float beta = bwd_beta(a, c.h);
    {
        const float* src = a.dm + (long long)c.slice * 8192;
        for (int e = tid; e < 8192; e += kThreads) mats[(e >> 6) * MB + (e & 63)] = src[e];
    }
    __syncthreads();
    const float* dW1 = mats;
    const float* Mm = mats + 64 * MB;
    const Frags<BF> F1 = make_frags<BF>(dW1, true, beta, g, m);  // beta dW1^T
    const Frags<BF> F2 = make_frags<BF>(Mm, false, -beta, g, m); // -beta M
    const Frags<BF> F3 = make_frags<BF>(dW1, false, beta, g, m); // beta dW1

    const char* Kp = base_of<ESZ>(a.X0, c);
    const char* Vp = base_of<ESZ>(a.X1, c);
    char* dKp = (char*)base_of<ESZ>(a.O0, c);
    char* dVp = (char*)base_of<ESZ>(a.O1, c);
    const long long sk = a.X0.sn * ESZ, sv = a.X1.sn * ESZ, sdk = a.O0.sn * ESZ, sdv = a.O1.sn * ESZ;

    // 16-token steps, wave w takes steps w, w + 4, ...: four steps per
    // round, their K and V rows loaded together (rows past the range are
    // clamped copies, loaded unconditionally and not stored)
    const int nst = (c.t1 - c.t0 + 15) / 16;
    for (int s0 = w; s0 < nst; s0 += 16) {
        Row<BF> k[4], v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tc = min(c.t0 + 16 * (s0 + 4 * u) + m, c.t1 - 1);
            k[u] = load_row<BF>(Kp + tc * sk, g);
            v[u] = load_row<BF>(Vp + tc * sv, g);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v4f dk[4], dv[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) dk[rb] = dv[rb] = v4f{0.f, 0.f, 0.f, 0.f};
            mac<BF>(F1, v[u], dk);
            mac<BF>(F2, k[u], dk);
            mac<BF>(F3, k[u], dv);
            const int t = c.t0 + 16 * (s0 + 4 * u) + m;
            if (t < c.t1) {
                store_row<BF>(dKp + t * sdk, dk, g);
                store_row<BF>(dVp + t * sdv, dv, g);
            }
        }
    }
}

// ------------------------------------------------------- pass 2 (bf16) --
// The same products with the workgroup's K and V rows (kP2Tok tokens)
// resident in LDS: every row is issued at once as direct-to-LDS loads, and
// the operators come as ready bf16 fragments from the reduce.  Two
// workgroups per CU, and the first 128 rows are processed while the rest
// land.  Rows
// are 128 bytes, 16-byte slots XOR-swizzled by (row / 2) % 8 so the 16
// rows one operand read covers touch different banks.
__global__ __launch_bounds__(kThreads, 2) void bwd_pass2_bf(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[2 * kP2Tok * 128];
    char* Ks = lds;
    char* Vs = lds + kP2Tok * 128;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = blockIdx.x / a.S2, split = blockIdx.x % a.S2;
    // the first H x 16 workgroups also form dW0 and deta over the batch
    // (the reduce has written every slice's terms)
    if (a.batch_in_pass2 && (int)blockIdx.x < a.H * 16) batch_sums(a, (int)blockIdx.x);
    if (slice >= a.B * a.H) return;
    const int b = slice / a.H, h = slice % a.H;
    const int t0 = min(a.N, split * a.per2), t1 = min(a.N, t0 + a.per2), T = t1 - t0;
    const char* Kp = (const char*)a.X0.ptr + (b * a.X0.sb + h * a.X0.sh) * 2LL;
    const char* Vp = (const char*)a.X1.ptr + (b * a.X1.sb + h * a.X1.sh) * 2LL;
    char* dKp = (char*)a.O0.ptr + (b * a.O0.sb + h * a.O0.sh) * 2LL;
    char* dVp = (char*)a.O1.ptr + (b * a.O1.sb + h * a.O1.sh) * 2LL;
    const long long sk = a.X0.sn * 2, sv = a.X1.sn * 2, sdk = a.O0.sn * 2, sdv = a.O1.sn * 2;
    auto swz = [](int row) { return (row >> 1) & 7; };

    // rows: instruction q covers rows 8q .. 8q + 7 (clamped into the range);
    // q < 16 is the first half (rows < 128)
    const int rows = (T + 15) & ~15, ninstr = rows / 8;
    auto issue = [&](int q_begin, int q_end) __attribute__((always_inline)) {
        for (int q = q_begin + w; q < q_end; q += 4) {
            const int p = q * 64 + lane, row = p >> 3;
            const int off = ((p & 7) ^ swz(row)) * 16;
            const long long tk = t0 + min(row, T - 1);
            dma16(Kp + tk * sk + off, Ks + q * 1024);
            dma16(Vp + tk * sv + off, Vs + q * 1024);
        }
    };
    issue(0, min(ninstr, 16));
    // operator fragments; the asm operand makes the compiler wait for them
    // here (together with the first half's rows), so no wait at their use
    // covers the second half's loads, issued next
    const u32x4* fr = a.fr + (long long)slice * 1536 + lane;
    v8bf F[3][4][2];
#pragma unroll
    for (int f = 0; f < 3; ++f)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) F[f][rb][kb] = as_v8bf(fr[(f * 8 + rb * 2 + kb) * 64]);
    drain_vmem();
#pragma unroll
    for (int f = 0; f < 3; ++f)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+v"(F[f][rb][kb]));
    issue(16, ninstr);
    const int nst = rows / 16;
    auto steps = [&](int s_begin, int s_end) __attribute__((always_inline)) {
        for (int st = s_begin + w; st < s_end; st += 4) {
            const int row = 16 * st + m;
            u32x4 kx[2], vx[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int off = (row * 8 + ((4 * kb + g) ^ swz(row))) * 16;
                kx[kb] = *reinterpret_cast<const u32x4*>(Ks + off);
                vx[kb] = *reinterpret_cast<const u32x4*>(Vs + off);
            }
            v4f dk[4], dv[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                dk[rb] = dv[rb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    dk[rb] = mfma32(F[0][rb][kb], as_v8bf(vx[kb]), dk[rb]);
                    dk[rb] = mfma32(F[1][rb][kb], as_v8bf(kx[kb]), dk[rb]);
                    dv[rb] = mfma32(F[2][rb][kb], as_v8bf(kx[kb]), dv[rb]);
                }
            }
            const int t = t0 + row;
            if (row < T) {
                store_row<true>(dKp + t * sdk, dk, g);
                store_row<true>(dVp + t * sdv, dv, g);
            }
        }
    };
    __syncthreads(); // every wave's first-half rows have landed
    steps(0, min(nst, 8));
    drain_vmem();
    __syncthreads();
    steps(8, nst);
}

// Workgroups per slice: at least 1024 workgroups in all (several rounds
// of the device's 512 resident slots: two per CU), each with at least 128
// tokens; among split counts up to twice that minimum, the one whose grid
// fills its last round of slots best (a partly filled last round costs a
// whole round).
int bwd_splits(int B, int H, int N) {
    const long long slices = (long long)B * H;
    constexpr long long kSlots = 512;
    long long maxs = (N + 127) / 128;
    if (maxs > 64) maxs = 64;
    if (maxs < 1) maxs = 1;
    long long s0 = (1024 + slices - 1) / slices;
    if (s0 > maxs) s0 = maxs;
    if (s0 < 1) s0 = 1;
    long long best = s0;
    double best_fill = 0.0;
    for (long long s = s0; s <= 2 * s0 && s <= maxs; ++s) {
        const long long wgs = slices * s;
        const long long rounds = (wgs + kSlots - 1) / kSlots;
        const double fill = (double)wgs / (double)(rounds * kSlots);
        if (fill > best_fill + 1e-9) {
            best_fill = fill;
            best = s;
        }
    }
    return (int)best;
}

// bf16 pass 1: the split count of bwd_splits (the grid fills whole rounds
// of resident slots), each split walking its tokens in chunks of kP1Tok
int bwd_splits_bf(int B, int H, int N) { return bwd_splits(B, H, N); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

} // namespace

// Workspace: [forward's workspace | A, G per slice (when not saved)] then
// [dW1 shares | dW1, M | dW0 terms | deta terms].
size_t lin_bwd_ws_bytes(int B, int H, int N) {
    const size_t slices = (size_t)B * H;
    const size_t S = bwd_splits(B, H, N);
    // (the forward's workspace, at least its counter block: the workspace
    // query reads the failure words there)
    size_t bytes = align256(std::max(lin_fwd_ws_bytes(B, H, N), kCounterBytes));
    bytes += align256(slices * 8192 * 4);     // recomputed A, G
    bytes += align256(slices * S * 4096 * 4); // dW1 shares
    bytes += align256(slices * 8192 * 4);     // dW1, M
    bytes += align256(slices * 4096 * 4);     // dW0 terms
    bytes += align256(slices * 4);            // deta terms
    bytes += align256(slices * 1536 * 16);    // bf16 operator fragments
    return bytes;
}

float* lin_bwd_saved_region(void* ws, int B, int H, int N) {
    return (float*)((char*)ws + align256(std::max(lin_fwd_ws_bytes(B, H, N), kCounterBytes)));
}

hipError_t launch_lin_bwd(LinBwdLaunch s, hipStream_t stream) {
    BwdArgs a{};
    a.W0 = s.W0;
    a.eta = s.eta;
    a.saved = s.saved;
    a.dW0 = s.dW0;
    a.deta = s.deta;
    a.B = s.B; a.H = s.H; a.N = s.N;
    a.dot = s.dot;
    // pass 1 splits (bf16: walked in chunks of kP1Tok tokens resident in LDS)
    a.S = s.bf16 ? bwd_splits_bf(s.B, s.H, s.N) : bwd_splits(s.B, s.H, s.N);
    a.per = (((s.N + a.S - 1) / a.S) + 15) & ~15;
    a.xcd = 1;
    const size_t slices = (size_t)s.B * s.H;
    const size_t Smax = bwd_splits(s.B, s.H, s.N);
    char* p = (char*)lin_bwd_saved_region(s.ws, s.B, s.H, s.N) + align256(slices * 8192 * 4);
    a.part = (float*)p;
    p += align256(slices * Smax * 4096 * 4);
    a.dm = (float*)p;
    p += align256(slices * 8192 * 4);
    a.dW0s = (float*)p;
    p += align256(slices * 4096 * 4);
    a.detas = (float*)p;
    p += align256(slices * 4);
    a.fr = s.bf16 ? (u32x4*)p : nullptr;
    a.S2 = (s.N + kP2Tok - 1) / kP2Tok;
    if (a.S2 < 1) a.S2 = 1;
    a.per2 = (((s.N + a.S2 - 1) / a.S2) + 15) & ~15; // <= kP2Tok

    const long long padded = ((long long)slices + 7) / 8 * 8;
    const dim3 grid((unsigned)(padded * a.S)), block(kThreads);
    a.X0 = s.dZ; a.X1 = s.Q; a.O0 = s.dQ;
    if (s.bf16) {
        hipLaunchKernelGGL(bwd_pass1_bf, dim3((unsigned)(slices * a.S)), block, 0, stream, a);
    } else {
        hipLaunchKernelGGL(bwd_pass1<false>, grid, block, 0, stream, a);
    }
    hipLaunchKernelGGL(bwd_reduce, dim3((unsigned)slices), dim3(kRT), 0, stream, a);
    a.X0 = s.K; a.X1 = s.V; a.O0 = s.dK; a.O1 = s.dV;
    a.batch_in_pass2 = s.bf16 && (long long)slices * a.S2 >= (long long)s.H * 16 ? 1 : 0;
    if (s.bf16) hipLaunchKernelGGL(bwd_pass2_bf, dim3((unsigned)(slices * a.S2)), block, 0, stream, a);
    else hipLaunchKernelGGL(bwd_pass2<false>, grid, block, 0, stream, a);
    if (!a.batch_in_pass2) hipLaunchKernelGGL(bwd_batch, dim3((unsigned)s.H * 16), block, 0, stream, a);
    return hipGetLastError();
}

} // namespace ttt
