// mlp_fullbatch.hip -- one full-batch L2 step of the two-layer SiLU MLP
// inner model, then apply (ViT3 article, observation 4: a wider inner model,
// hidden = r d with r = 1..4, keeps improving the layer).
//
// f(k) = W2 silu(W1 k), W1 [hid][64], W2 [64][hid].  Per slice, the mean L2
// loss over the N tokens and its gradient by backpropagation per token:
//   h = W1 k,  a = silu(h),  e = W2 a - v,
//   dW2 = (2/N) sum e a^T,   g = (W2^T e) * silu'(h),   dW1 = (2/N) sum g k^T,
//   W1' = W1 - eta dW1,  W2' = W2 - eta dW2,  z = W2' silu(W1' q).
// Every product runs on the matrix cores (bf16 operands, fp32 accumulation):
//   train   per (slice, token split), 64 tokens per step, eight waves: wave
//           (t, half) takes token tile t (16 tokens) through
//             h, a, silu'(h) for its half of the hidden units -> LDS rows,
//             o = W2 a and e = o - v for its two 16-channel output blocks,
//             u = W2^T e and g = u * silu'(h) for its hidden half -> LDS,
//           and then owns a quarter of dW2 (half 0) or of dW1 (half 1) for
//           the whole split, contracting over the step's tokens with
//           transposing LDS reads of the staged rows.  Accumulator tiles
//           (features 4g+i, token m) feed the next product as B operands;
//           the token-major rows give the A/B operands that need the
//           token or the feature as the contracted index.  One fp32
//           partial per split;
//   update  per slice, the split partials summed in split order, then
//           W' = W - eta (2/N) sum, stored as bf16;
//   apply   z = W2' silu(W1' q), 64 tokens per wave so that each weight
//           fragment read from LDS feeds four products.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace ttt {
namespace {

constexpr int kMT = 256;      // 4 waves
constexpr int kChunk = 64;    // tokens per train step (16 per wave)
constexpr int kW1P = 72;      // LDS pitch of W1 rows (bf16)

// sigma(x) with the hardware reciprocal (about 1 ulp; the results are
// rounded to bf16): silu(x) = x sigma(x), silu'(x) = sigma(x)(1 + x(1 - sigma(x))).
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigm(x); }

// Transposing read of a 4 x 16 bf16 block: in each 16-lane group, lane
// 4e + a gives the address of row e, columns 4a..4a+3; lane m receives
// column m of the four rows.
__device__ __forceinline__ v4s_t tr4(const bf16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
}
__device__ __forceinline__ v8bf cat8(v4s_t lo, v4s_t hi) {
    return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ v8bf cat8u(u32x2 lo, u32x2 hi) {
    return __builtin_bit_cast(v8bf, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

struct MlpArgs {
    View4 K, Q, V, Z;
    const float* W1;  // [H][hid][64]
    const float* W2;  // [H][64][hid]
    const float* eta;
    bf16_t* Wn;       // [slices][2][64 hid]: W1', W2' in bf16
    float* part;      // [slices][S][2][64 hid]: dW1 [hid][64], dW2 [64][hid] sums
    int B, H, N, S, per;
};

template <int NHB> struct Mlp {
    static constexpr int HID = 16 * NHB;
    static constexpr int W2P = HID + 16;               // LDS pitch of W2 rows (swizzled)
    static constexpr int KO = 0, EO = 64, AO = 128, GO = 128 + HID;
    static constexpr int SP = 128 + 2 * HID + 16;      // stage row pitch (swizzled)
    static constexpr int WLDS = HID * kW1P + 64 * W2P; // bf16 elements
};

// The W2 rows and the staged token rows have a pitch of 32 words + 8 and
// swap the two 16-byte halves of every 32-byte group in rows whose bit 2
// is set (column bit 3 flipped).  The four rows of a transposing read
// (rows 4j .. 4j+3, 32 bytes each) then cover all 32 banks, and so do eight
// consecutive rows read at one 16-byte column (the pitch alone would put
// rows r and r+4 on the same banks).
__device__ __forceinline__ int sw(int r, int c) { return c ^ (((r >> 2) & 1) << 3); }

// W1 rows (pitch kW1P) and W2 rows (pitch W2P) in LDS as bf16, from bf16
// [2][64 hid] (T = bf16_t) or from the fp32 W1, W2 of a head (T = float).
template <int NHB, int NT>
__device__ __forceinline__ void load_weights(const bf16_t* src, bf16_t* w1s, bf16_t* w2s) {
    constexpr int HID = Mlp<NHB>::HID, W2P = Mlp<NHB>::W2P;
    for (int q = threadIdx.x; q < HID * 8; q += NT) {
        const int r = q >> 3, s = q & 7;
        *reinterpret_cast<u32x4*>(w1s + r * kW1P + 8 * s) = *reinterpret_cast<const u32x4*>(src + r * 64 + 8 * s);
    }
    const bf16_t* w2 = src + 64 * HID;
    for (int q = threadIdx.x; q < 64 * (HID / 8); q += NT) {
        const int r = q / (HID / 8), s = q % (HID / 8);
        *reinterpret_cast<u32x4*>(w2s + r * W2P + sw(r, 8 * s)) =
            *reinterpret_cast<const u32x4*>(w2 + r * HID + 8 * s);
    }
}
template <int NHB, int NT>
__device__ __forceinline__ void load_weights_f32(const float* W1, const float* W2, bf16_t* w1s, bf16_t* w2s) {
    constexpr int HID = Mlp<NHB>::HID, W2P = Mlp<NHB>::W2P;
    for (int q = threadIdx.x; q < HID * 8; q += NT) {
        const int r = q >> 3, s = q & 7;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(W1 + r * 64 + 8 * s);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(W1 + r * 64 + 8 * s + 4);
        *reinterpret_cast<u32x4*>(w1s + r * kW1P + 8 * s) =
            u32x4{pack_bf2(x0[0], x0[1]), pack_bf2(x0[2], x0[3]), pack_bf2(x1[0], x1[1]), pack_bf2(x1[2], x1[3])};
    }
    for (int q = threadIdx.x; q < 64 * (HID / 8); q += NT) {
        const int r = q / (HID / 8), s = q % (HID / 8);
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(W2 + r * HID + 8 * s);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(W2 + r * HID + 8 * s + 4);
        *reinterpret_cast<u32x4*>(w2s + r * W2P + sw(r, 8 * s)) =
            u32x4{pack_bf2(x0[0], x0[1]), pack_bf2(x0[2], x0[3]), pack_bf2(x1[0], x1[1]), pack_bf2(x1[2], x1[3])};
    }
}

// h = W1 x for hidden block hb; lane (g, m): h[16 hb + 4g + i][token m].
__device__ __forceinline__ v4f hidden_block(const bf16_t* w1s, const u32x4* xf, int hb, int g, int m) {
    v4f acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const u32x4 wf = *reinterpret_cast<const u32x4*>(w1s + (16 * hb + m) * kW1P + 32 * kb + 8 * g);
        acc = mfma32(as_v8bf(wf), as_v8bf(xf[kb]), acc);
    }
    return acc;
}

constexpr int kTT = 512; // train: 8 waves
typedef __fp16 h2_t __attribute__((ext_vector_type(2)));

template <int NHB>
__global__ __launch_bounds__(kTT) void mlp_train(MlpArgs a) {
    using M = Mlp<NHB>;
    constexpr int HID = M::HID, SP = M::SP, W2P = M::W2P, NH2 = NHB / 2, NQ = NHB / 4;
    __shared__ __attribute__((aligned(16))) bf16_t smem[M::WLDS + kChunk * SP];
    bf16_t* w1s = smem;
    bf16_t* w2s = smem + HID * kW1P;
    bf16_t* st = smem + M::WLDS;
    const int slice = blockIdx.x / a.S, split = blockIdx.x % a.S;
    const int bb = slice / a.H, h = slice % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform
    const int tt = w & 3, hh = w >> 2;                      // token tile, hidden half (and Gram kind)
    const int e4 = m >> 2, a4 = m & 3;              // transposing-read roles
    const int t0 = min(a.N, split * a.per), t1 = min(a.N, t0 + a.per);
    load_weights_f32<NHB, kTT>(a.W1 + (long long)h * 64 * HID, a.W2 + (long long)h * 64 * HID, w1s, w2s);
    const char* Kp = (const char*)a.K.ptr + ((long long)bb * a.K.sb + (long long)h * a.K.sh) * 2;
    const char* Vp = (const char*)a.V.ptr + ((long long)bb * a.V.sb + (long long)h * a.V.sh) * 2;
    // Gram tiles of this wave: hidden blocks tt*NQ + l, 16-column blocks x;
    // half 0: dW2[16x + 4g+i][16hb + m], half 1: dW1[16hb + 4g+i][16x + m]
    v4f acc[NQ][4];
#pragma unroll
    for (int l = 0; l < NQ; ++l)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[l][x] = v4f{0.f, 0.f, 0.f, 0.f};
    // the lane's token r0 + 16 tt + m, clamped to a valid row for the loads
    // (rows past the split contribute zero a and g); V for its two output
    // blocks 2 hh, 2 hh + 1
    u32x4 xf[2];
    u32x2 vv[2];
    auto fetch_k = [&](int r0) __attribute__((always_inline)) {
        const char* kr = Kp + (long long)min(r0 + 16 * tt + m, a.N - 1) * a.K.sn * 2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xf[kb] = *reinterpret_cast<const u32x4*>(kr + (32 * kb + 8 * g) * 2);
    };
    auto fetch_v = [&](int r0) __attribute__((always_inline)) {
        const char* vr = Vp + (long long)min(r0 + 16 * tt + m, a.N - 1) * a.V.sn * 2;
#pragma unroll
        for (int j = 0; j < 2; ++j) vv[j] = *reinterpret_cast<const u32x2*>(vr + (16 * (2 * hh + j) + 4 * g) * 2);
    };
    fetch_k(t0);
    fetch_v(t0);
    __syncthreads();
    const int rr = 16 * tt + m;              // the lane's stage row
    bf16_t* srow = st + rr * SP;
    for (int r0 = t0; r0 < t1; r0 += kChunk) {
        const bool ok = r0 + 16 * tt + m < t1;
        // 1. h, a = silu(h), silu'(h) for hidden blocks hh*NH2 + l
        if (hh == 0) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) *reinterpret_cast<u32x4*>(srow + sw(rr, M::KO + 32 * kb + 8 * g)) = xf[kb];
        }
        // silu'(h) waits for phase 3 as fp16 pairs (10-bit mantissa; g is
        // rounded to bf16 anyway), which keeps the wave within 256 VGPRs
        h2_t sp[NH2][2];
#pragma unroll
        for (int l = 0; l < NH2; ++l) {
            const int hb = hh * NH2 + l;
            const v4f hv = hidden_block(w1s, xf, hb, g, m);
            float av[4], dv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sg = sigm(hv[i]);
                av[i] = hv[i] * sg;
                dv[i] = sg * (1.f + hv[i] * (1.f - sg));
            }
            sp[l][0] = __builtin_amdgcn_cvt_pkrtz(dv[0], dv[1]);
            sp[l][1] = __builtin_amdgcn_cvt_pkrtz(dv[2], dv[3]);
            const u32x2 ap{pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3])};
            *reinterpret_cast<u32x2*>(srow + sw(rr, M::AO + 16 * hb + 4 * g)) = ok ? ap : u32x2{0u, 0u};
        }
        // the next step's K is in flight across phases 2-4 (its V across 3-4)
        if (r0 + kChunk < t1) fetch_k(r0 + kChunk);
        lds_barrier();
        // 2. o = W2 a over every hidden unit for output blocks 2 hh + j, e = o - v
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ob = 2 * hh + j;
            v4f o{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < NHB / 2; ++p) {
                const int wr = 16 * ob + m;
                const u32x4 wf = *reinterpret_cast<const u32x4*>(w2s + wr * W2P + sw(wr, 32 * p + 8 * g));
                const u32x4 af = *reinterpret_cast<const u32x4*>(srow + sw(rr, M::AO + 32 * p + 8 * g));
                o = mfma32(as_v8bf(wf), as_v8bf(af), o);
            }
            *reinterpret_cast<u32x2*>(srow + sw(rr, M::EO + 16 * ob + 4 * g)) =
                u32x2{pack_bf2(o[0] - bflo(vv[j][0]), o[1] - bfhi(vv[j][0])),
                      pack_bf2(o[2] - bflo(vv[j][1]), o[3] - bfhi(vv[j][1]))};
        }
        if (r0 + kChunk < t1) fetch_v(r0 + kChunk);
        lds_barrier();
        // 3. u = W2^T e, g = u * silu'(h) for hidden blocks hh*NH2 + l
        u32x4 ef[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) ef[q] = *reinterpret_cast<const u32x4*>(srow + sw(rr, M::EO + 32 * q + 8 * g));
#pragma unroll
        for (int l = 0; l < NH2; ++l) {
            const int hb = hh * NH2 + l;
            v4f u{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int r0 = 32 * q + 8 * g + e4, c = 16 * hb + 4 * a4;
                u = mfma32(cat8(tr4(w2s + r0 * W2P + sw(r0, c)), tr4(w2s + (r0 + 4) * W2P + sw(r0 + 4, c))),
                           as_v8bf(ef[q]), u);
            }
            const u32x2 gv{pack_bf2(u[0] * (float)sp[l][0][0], u[1] * (float)sp[l][0][1]),
                           pack_bf2(u[2] * (float)sp[l][1][0], u[3] * (float)sp[l][1][1])};
            *reinterpret_cast<u32x2*>(srow + sw(rr, M::GO + 16 * hb + 4 * g)) = ok ? gv : u32x2{0u, 0u};
        }
        lds_barrier();
        // 4. contraction over the step's 64 tokens, 32 at a time: lane (g, m)
        //    reads tokens 32 s + 8g + e4 (and + 4) at columns c + 4 a4
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int r0 = 32 * s + 8 * g + e4;
            const bf16_t* lo = st + r0 * SP;
            const bf16_t* hi = st + (r0 + 4) * SP;
            const int xo = (hh == 0 ? M::EO : M::KO) + 4 * a4, yo = (hh == 0 ? M::AO : M::GO) + 4 * a4;
            v8bf X[4], Y[NQ];
#pragma unroll
            for (int x = 0; x < 4; ++x) X[x] = cat8(tr4(lo + sw(r0, xo + 16 * x)), tr4(hi + sw(r0 + 4, xo + 16 * x)));
#pragma unroll
            for (int l = 0; l < NQ; ++l) {
                const int c = yo + 16 * (tt * NQ + l);
                Y[l] = cat8(tr4(lo + sw(r0, c)), tr4(hi + sw(r0 + 4, c)));
            }
            if (hh == 0) {
#pragma unroll
                for (int l = 0; l < NQ; ++l)
#pragma unroll
                    for (int x = 0; x < 4; ++x) acc[l][x] = mfma32(X[x], Y[l], acc[l][x]);
            } else {
#pragma unroll
                for (int l = 0; l < NQ; ++l)
#pragma unroll
                    for (int x = 0; x < 4; ++x) acc[l][x] = mfma32(Y[l], X[x], acc[l][x]);
            }
        }
        lds_barrier();
    }
    // partial: dW1 [hid][64] then dW2 [64][hid]
    float* p1 = a.part + ((long long)slice * a.S + split) * 2 * 64 * HID;
    float* p2 = p1 + 64 * HID;
    if (hh == 0) {
#pragma unroll
        for (int l = 0; l < NQ; ++l)
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) p2[(16 * x + 4 * g + i) * HID + 16 * (tt * NQ + l) + m] = acc[l][x][i];
    } else {
#pragma unroll
        for (int l = 0; l < NQ; ++l)
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) p1[(16 * (tt * NQ + l) + 4 * g + i) * 64 + 16 * x + m] = acc[l][x][i];
    }
}

// W' = W - eta (2/N) (sum of the split partials, in split order), bf16.
__global__ __launch_bounds__(kMT) void mlp_update(MlpArgs a, int hid) {
    const int n2 = 2 * 64 * hid;
    const int chunks = (n2 + kMT - 1) / kMT;
    const int slice = blockIdx.x / chunks, e = (blockIdx.x % chunks) * kMT + threadIdx.x;
    if (e >= n2) return;
    const int h = slice % a.H;
    const float* p = a.part + (long long)slice * a.S * n2 + e;
    const float W = e < n2 / 2 ? a.W1[(long long)h * (n2 / 2) + e] : a.W2[(long long)h * (n2 / 2) + e - n2 / 2];
    // the split partials in order, eight loads in flight before their adds
    // (one past the last split adds 0)
    float s = 0.f;
    for (int s0 = 0; s0 < a.S; s0 += 8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = p[(long long)min(s0 + i, a.S - 1) * n2];
            t[i] = s0 + i < a.S ? x : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) s += t[i];
    }
    a.Wn[(long long)slice * n2 + e] = f2bf(W - a.eta[h] * ((2.f / (float)a.N) * s));
}

// z = W2' silu(W1' q): eight waves of 32 tokens (two 16-token tiles) per
// block, so each weight fragment read from LDS feeds two products; two
// blocks per CU (the weights fill the LDS) of up to 128 VGPRs per lane keep
// four waves on every SIMD.
constexpr int kAT = 512, kATile = 2, kABlk = 8 * 16 * kATile; // tokens per block
template <int NHB>
__global__ __launch_bounds__(kAT, 2) void mlp_apply(MlpArgs a) {
    using M = Mlp<NHB>;
    constexpr int W2P = M::W2P;
    __shared__ __attribute__((aligned(16))) bf16_t smem[M::WLDS];
    bf16_t* w1s = smem;
    bf16_t* w2s = smem + M::HID * kW1P;
    const int nb = (a.N + kABlk - 1) / kABlk;
    const int slice = blockIdx.x / nb, tb = blockIdx.x % nb;
    const int bb = slice / a.H, h = slice % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15, w = tid >> 6;
    const char* Qp = (const char*)a.Q.ptr + ((long long)bb * a.Q.sb + (long long)h * a.Q.sh) * 2;
    char* Zp = (char*)a.Z.ptr + ((long long)bb * a.Z.sb + (long long)h * a.Z.sh) * 2;
    const int row0 = tb * kABlk + 16 * kATile * w + m; // tile tt: row0 + 16 tt
    u32x4 xf[kATile][2];
#pragma unroll
    for (int tt = 0; tt < kATile; ++tt) {
        const char* qr = Qp + (long long)min(row0 + 16 * tt, a.N - 1) * a.Q.sn * 2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xf[tt][kb] = *reinterpret_cast<const u32x4*>(qr + (32 * kb + 8 * g) * 2);
    }
    load_weights<NHB, kAT>(a.Wn + (long long)slice * 2 * 64 * M::HID, w1s, w2s);
    __syncthreads();
    u32x2 af[kATile][NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        u32x4 wf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            wf[kb] = *reinterpret_cast<const u32x4*>(w1s + (16 * hb + m) * kW1P + 32 * kb + 8 * g);
#pragma unroll
        for (int tt = 0; tt < kATile; ++tt) {
            v4f hv{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) hv = mfma32(as_v8bf(wf[kb]), as_v8bf(xf[tt][kb]), hv);
            af[tt][hb] = u32x2{pack_bf2(silu_f(hv[0]), silu_f(hv[1])), pack_bf2(silu_f(hv[2]), silu_f(hv[3]))};
        }
    }
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
        v4f o[kATile];
#pragma unroll
        for (int tt = 0; tt < kATile; ++tt) o[tt] = v4f{0.f, 0.f, 0.f, 0.f};
        const int wr = 16 * ob + m;
        const bf16_t* wrow = w2s + wr * W2P;
#pragma unroll
        for (int p = 0; p < NHB / 2; ++p) {
            const v8bf wf = cat8u(*reinterpret_cast<const u32x2*>(wrow + sw(wr, 32 * p + 4 * g)),
                                  *reinterpret_cast<const u32x2*>(wrow + sw(wr, 32 * p + 16 + 4 * g)));
#pragma unroll
            for (int tt = 0; tt < kATile; ++tt) o[tt] = mfma32(wf, cat8u(af[tt][2 * p], af[tt][2 * p + 1]), o[tt]);
        }
#pragma unroll
        for (int tt = 0; tt < kATile; ++tt) {
            const int row = row0 + 16 * tt;
            if (row < a.N)
                *reinterpret_cast<u32x2*>(Zp + (long long)row * a.Z.sn * 2 + (16 * ob + 4 * g) * 2) =
                    u32x2{pack_bf2(o[tt][0], o[tt][1]), pack_bf2(o[tt][2], o[tt][3])};
        }
    }
}

size_t a256m(size_t x) { return (x + 255) & ~(size_t)255; }

struct MlpPlan {
    int S, per;
};
// Splits per slice: about one train block per CU over all slices, each a
// multiple of 64 tokens.
MlpPlan mlp_plan(int B, int H, int N) {
    const long long slices = (long long)B * H;
    const long long steps = (N + kChunk - 1) / kChunk;
    long long S = std::max<long long>(1, std::min<long long>(steps, 256 / std::max<long long>(slices, 1)));
    const long long per = (steps + S - 1) / S * kChunk;
    S = (N + per - 1) / per;
    return MlpPlan{(int)std::max<long long>(S, 1), (int)per};
}

template <int NHB> hipError_t launch_nhb(const MlpArgs& a, int slices, hipStream_t stream) {
    const dim3 block(kMT);
    hipLaunchKernelGGL(mlp_train<NHB>, dim3((unsigned)(slices * a.S)), dim3(kTT), 0, stream, a);
    const int n2 = 2 * 64 * Mlp<NHB>::HID;
    hipLaunchKernelGGL(mlp_update, dim3((unsigned)(slices * ((n2 + kMT - 1) / kMT))), block, 0, stream, a,
                       Mlp<NHB>::HID);
    hipLaunchKernelGGL(mlp_apply<NHB>, dim3((unsigned)(slices * ((a.N + kABlk - 1) / kABlk))), dim3(kAT), 0, stream,
                       a);
    return hipGetLastError();
}

} // namespace

bool mlp_hidden_supported(int hid) { return hid == 64 || hid == 128 || hid == 192 || hid == 256; }

size_t mlp_ws_bytes(int B, int H, int N, int hid) {
    const size_t slices = (size_t)B * H;
    if (slices == 0 || N <= 0 || !mlp_hidden_supported(hid)) return 0;
    const MlpPlan p = mlp_plan(B, H, N);
    const size_t n2 = 2 * 64 * (size_t)hid;
    return a256m(slices * n2 * 2) + a256m(slices * p.S * n2 * 4);
}

hipError_t launch_mlp(const MlpLaunch& l, hipStream_t stream) {
    MlpArgs a{};
    a.K = l.K; a.Q = l.Q; a.V = l.V; a.Z = l.Z;
    a.W1 = l.W1; a.W2 = l.W2; a.eta = l.eta;
    a.B = l.B; a.H = l.H; a.N = l.N;
    const MlpPlan p = mlp_plan(l.B, l.H, l.N);
    a.S = p.S;
    a.per = p.per;
    const int slices = l.B * l.H;
    const size_t n2 = 2 * 64 * (size_t)l.hid;
    char* w = (char*)l.ws;
    a.Wn = (bf16_t*)w;
    w += a256m((size_t)slices * n2 * 2);
    a.part = (float*)w;
    switch (l.hid) {
    case 64: return launch_nhb<4>(a, slices, stream);
    case 128: return launch_nhb<8>(a, slices, stream);
    case 192: return launch_nhb<12>(a, slices, stream);
    default: return launch_nhb<16>(a, slices, stream);
    }
}

} // namespace ttt
