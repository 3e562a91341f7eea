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
//   prep    W1, W2 of each head to bf16 once;
//   train   per (slice, token split), 64 tokens per step.  Each wave takes
//           16 tokens through h -> a -> e -> g in registers: a product's
//           accumulator tile (features 4g+i, token m) is the next product's
//           B operand, two 16-row blocks making one 32-deep operand whose k
//           order (4g+i, then 16+4g+i) the A fragment follows.  The step's
//           K, e, a and g go to LDS as token rows, and the four waves then
//           contract over the 64 tokens (dW2 = E^T A, dW1 = G^T K) with
//           transposing LDS reads, each wave owning 16 rows of dW2 and 16
//           columns of dW1 for the whole split.  One fp32 partial per split;
//   update  per slice, the split partials summed in split order, then
//           W' = W - eta (2/N) sum, stored as bf16;
//   apply   z = W2' silu(W1' q), 16-token tiles as in the train pass.
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
    bf16_t* Wb;       // [H][2][64 hid]: W1, W2 in bf16
    bf16_t* Wn;       // [slices][2][64 hid]: W1', W2' in bf16
    float* part;      // [slices][S][2][64 hid]: dW1 [hid][64], dW2 [64][hid] sums
    int B, H, N, S, per;
};

template <int NHB> struct Mlp {
    static constexpr int HID = 16 * NHB;
    static constexpr int W2P = HID + 8;                // LDS pitch of W2 rows
    static constexpr int KO = 0, EO = 64, AO = 128, GO = 128 + HID;
    static constexpr int SP = 128 + 2 * HID + 16;      // stage row pitch
    static constexpr int WLDS = HID * kW1P + 64 * W2P; // bf16 elements
};

// W1 rows (pitch kW1P) and W2 rows (pitch W2P) from bf16 [2][64 hid].
template <int NHB>
__device__ __forceinline__ void load_weights(const bf16_t* src, bf16_t* w1s, bf16_t* w2s) {
    constexpr int HID = Mlp<NHB>::HID, W2P = Mlp<NHB>::W2P;
    for (int q = threadIdx.x; q < HID * 8; q += kMT) {
        const int r = q >> 3, s = q & 7;
        *reinterpret_cast<u32x4*>(w1s + r * kW1P + 8 * s) = *reinterpret_cast<const u32x4*>(src + r * 64 + 8 * s);
    }
    const bf16_t* w2 = src + 64 * HID;
    for (int q = threadIdx.x; q < 64 * (HID / 8); q += kMT) {
        const int r = q / (HID / 8), s = q % (HID / 8);
        *reinterpret_cast<u32x4*>(w2s + r * W2P + 8 * s) = *reinterpret_cast<const u32x4*>(w2 + r * HID + 8 * s);
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

// o = W2 a for output block ob from the packed a blocks.
template <int NHB>
__device__ __forceinline__ v4f out_block(const bf16_t* w2s, const u32x2* af, int ob, int g, int m) {
    constexpr int W2P = Mlp<NHB>::W2P;
    v4f acc{0.f, 0.f, 0.f, 0.f};
    const bf16_t* row = w2s + (16 * ob + m) * W2P + 4 * g;
#pragma unroll
    for (int p = 0; p < NHB / 2; ++p) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 32 * p);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 32 * p + 16);
        acc = mfma32(cat8u(lo, hi), cat8u(af[2 * p], af[2 * p + 1]), acc);
    }
    return acc;
}

__global__ __launch_bounds__(kMT) void mlp_prep(const float* W1, const float* W2, bf16_t* Wb, int hid) {
    const int n = 64 * hid, h = blockIdx.y;
    const int e = blockIdx.x * kMT + threadIdx.x;
    if (e >= n) return;
    Wb[(long long)h * 2 * n + e] = f2bf(W1[(long long)h * n + e]);
    Wb[(long long)h * 2 * n + n + e] = f2bf(W2[(long long)h * n + e]);
}

template <int NHB>
__global__ __launch_bounds__(kMT) void mlp_train(MlpArgs a) {
    using M = Mlp<NHB>;
    constexpr int HID = M::HID, SP = M::SP, W2P = M::W2P;
    __shared__ __attribute__((aligned(16))) bf16_t smem[M::WLDS + kChunk * SP];
    bf16_t* w1s = smem;
    bf16_t* w2s = smem + HID * kW1P;
    bf16_t* st = smem + M::WLDS;
    const int slice = blockIdx.x / a.S, split = blockIdx.x % a.S;
    const int bb = slice / a.H, h = slice % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15, w = tid >> 6;
    const int e4 = m >> 2, a4 = m & 3; // transposing-read roles
    const int t0 = min(a.N, split * a.per), t1 = min(a.N, t0 + a.per);
    load_weights<NHB>(a.Wb + (long long)h * 2 * 64 * HID, w1s, w2s);
    const char* Kp = (const char*)a.K.ptr + ((long long)bb * a.K.sb + (long long)h * a.K.sh) * 2;
    const char* Vp = (const char*)a.V.ptr + ((long long)bb * a.V.sb + (long long)h * a.V.sh) * 2;
    v4f dw2[NHB], dw1[NHB]; // dW2[16w + 4g+i][16hb + m], dW1[16hb + 4g+i][16w + m]
#pragma unroll
    for (int i = 0; i < NHB; ++i) dw2[i] = dw1[i] = v4f{0.f, 0.f, 0.f, 0.f};
    // this lane's token in the step: r0 + 16 w + m, clamped to a valid row
    // for the loads (rows past the split contribute zero a and g)
    u32x4 xf[2];
    u32x2 vv[4];
    auto fetch = [&](int r0) __attribute__((always_inline)) {
        const int tok = min(r0 + 16 * w + m, a.N - 1);
        const char* kr = Kp + (long long)tok * a.K.sn * 2;
        const char* vr = Vp + (long long)tok * a.V.sn * 2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xf[kb] = *reinterpret_cast<const u32x4*>(kr + (32 * kb + 8 * g) * 2);
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) vv[ob] = *reinterpret_cast<const u32x2*>(vr + (16 * ob + 4 * g) * 2);
    };
    fetch(t0);
    __syncthreads();
    bf16_t* srow = st + (16 * w + m) * SP; // this lane's stage row
    for (int r0 = t0; r0 < t1; r0 += kChunk) {
        const bool ok = r0 + 16 * w + m < t1;
        // h, a = silu(h), silu'(h)
        u32x2 af[NHB];
        float sp[NHB][4];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const v4f hv = hidden_block(w1s, xf, hb, g, m);
            float av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sg = sigm(hv[i]);
                av[i] = hv[i] * sg;
                sp[hb][i] = sg * (1.f + hv[i] * (1.f - sg));
            }
            af[hb] = u32x2{pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3])};
        }
        // e = W2 a - v
        u32x2 ef[4];
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
            const v4f o = out_block<NHB>(w2s, af, ob, g, m);
            ef[ob] = u32x2{pack_bf2(o[0] - bflo(vv[ob][0]), o[1] - bfhi(vv[ob][0])),
                           pack_bf2(o[2] - bflo(vv[ob][1]), o[3] - bfhi(vv[ob][1]))};
        }
        // stage K, e, a (a is dead afterwards)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) *reinterpret_cast<u32x4*>(srow + M::KO + 32 * kb + 8 * g) = xf[kb];
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) *reinterpret_cast<u32x2*>(srow + M::EO + 16 * ob + 4 * g) = ef[ob];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
            *reinterpret_cast<u32x2*>(srow + M::AO + 16 * hb + 4 * g) = ok ? af[hb] : u32x2{0u, 0u};
        // g = (W2^T e) * silu'(h); the A fragment is W2[32q + 4g+i | 32q+16 + 4g+i][16 hb + m]
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            v4f u{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const bf16_t* p = w2s + (32 * q + 4 * g + e4) * W2P + 16 * hb + 4 * a4;
                u = mfma32(cat8(tr4(p), tr4(p + 16 * W2P)), cat8u(ef[2 * q], ef[2 * q + 1]), u);
            }
            const u32x2 gv{pack_bf2(u[0] * sp[hb][0], u[1] * sp[hb][1]),
                           pack_bf2(u[2] * sp[hb][2], u[3] * sp[hb][3])};
            *reinterpret_cast<u32x2*>(srow + M::GO + 16 * hb + 4 * g) = ok ? gv : u32x2{0u, 0u};
        }
        // the next step's K and V stay in flight across the contraction
        if (r0 + kChunk < t1) fetch(r0 + kChunk);
        lds_barrier();
        // contraction over the step's 64 tokens, 32 at a time: lane (g, m)
        // reads tokens 32 s + 8g + e4 (and + 4) at columns c + 4 a4
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const bf16_t* base = st + (32 * s + 8 * g + e4) * SP + 4 * a4;
            const v8bf eT = cat8(tr4(base + M::EO + 16 * w), tr4(base + 4 * SP + M::EO + 16 * w));
            const v8bf kT = cat8(tr4(base + M::KO + 16 * w), tr4(base + 4 * SP + M::KO + 16 * w));
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
                const v8bf aT = cat8(tr4(base + M::AO + 16 * hb), tr4(base + 4 * SP + M::AO + 16 * hb));
                const v8bf gT = cat8(tr4(base + M::GO + 16 * hb), tr4(base + 4 * SP + M::GO + 16 * hb));
                dw2[hb] = mfma32(eT, aT, dw2[hb]);
                dw1[hb] = mfma32(gT, kT, dw1[hb]);
            }
        }
        lds_barrier();
    }
    // partial: dW1 [hid][64] then dW2 [64][hid]
    float* p1 = a.part + ((long long)slice * a.S + split) * 2 * 64 * HID;
    float* p2 = p1 + 64 * HID;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p1[(16 * hb + 4 * g + i) * 64 + 16 * w + m] = dw1[hb][i];
            p2[(16 * w + 4 * g + i) * HID + 16 * hb + m] = dw2[hb][i];
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
    float s = 0.f;
    for (int sp = 0; sp < a.S; ++sp) s += p[(long long)sp * n2];
    const float W = e < n2 / 2 ? a.W1[(long long)h * (n2 / 2) + e] : a.W2[(long long)h * (n2 / 2) + e - n2 / 2];
    a.Wn[(long long)slice * n2 + e] = f2bf(W - a.eta[h] * ((2.f / (float)a.N) * s));
}

// z = W2' silu(W1' q): 256 tokens per block, 64 per wave as four 16-token
// tiles, so each weight fragment read from LDS feeds four products.
template <int NHB>
__global__ __launch_bounds__(kMT) void mlp_apply(MlpArgs a) {
    using M = Mlp<NHB>;
    constexpr int W2P = M::W2P;
    __shared__ __attribute__((aligned(16))) bf16_t smem[M::WLDS];
    bf16_t* w1s = smem;
    bf16_t* w2s = smem + M::HID * kW1P;
    const int nb = (a.N + 255) / 256;
    const int slice = blockIdx.x / nb, tb = blockIdx.x % nb;
    const int bb = slice / a.H, h = slice % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15, w = tid >> 6;
    load_weights<NHB>(a.Wn + (long long)slice * 2 * 64 * M::HID, w1s, w2s);
    const char* Qp = (const char*)a.Q.ptr + ((long long)bb * a.Q.sb + (long long)h * a.Q.sh) * 2;
    char* Zp = (char*)a.Z.ptr + ((long long)bb * a.Z.sb + (long long)h * a.Z.sh) * 2;
    const int row0 = tb * 256 + 64 * w + m; // tile tt: row0 + 16 tt
    u32x4 xf[4][2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const char* qr = Qp + (long long)min(row0 + 16 * tt, a.N - 1) * a.Q.sn * 2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xf[tt][kb] = *reinterpret_cast<const u32x4*>(qr + (32 * kb + 8 * g) * 2);
    }
    __syncthreads();
    u32x2 af[4][NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        u32x4 wf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            wf[kb] = *reinterpret_cast<const u32x4*>(w1s + (16 * hb + m) * kW1P + 32 * kb + 8 * g);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            v4f hv{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) hv = mfma32(as_v8bf(wf[kb]), as_v8bf(xf[tt][kb]), hv);
            af[tt][hb] = u32x2{pack_bf2(silu_f(hv[0]), silu_f(hv[1])), pack_bf2(silu_f(hv[2]), silu_f(hv[3]))};
        }
    }
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
        v4f o[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) o[tt] = v4f{0.f, 0.f, 0.f, 0.f};
        const bf16_t* wrow = w2s + (16 * ob + m) * W2P + 4 * g;
#pragma unroll
        for (int p = 0; p < NHB / 2; ++p) {
            const v8bf wf = cat8u(*reinterpret_cast<const u32x2*>(wrow + 32 * p),
                                  *reinterpret_cast<const u32x2*>(wrow + 32 * p + 16));
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) o[tt] = mfma32(wf, cat8u(af[tt][2 * p], af[tt][2 * p + 1]), o[tt]);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
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
    hipLaunchKernelGGL(mlp_train<NHB>, dim3((unsigned)(slices * a.S)), block, 0, stream, a);
    const int n2 = 2 * 64 * Mlp<NHB>::HID;
    hipLaunchKernelGGL(mlp_update, dim3((unsigned)(slices * ((n2 + kMT - 1) / kMT))), block, 0, stream, a,
                       Mlp<NHB>::HID);
    hipLaunchKernelGGL(mlp_apply<NHB>, dim3((unsigned)(slices * ((a.N + 255) / 256))), block, 0, stream, a);
    return hipGetLastError();
}

} // namespace

bool mlp_hidden_supported(int hid) { return hid == 64 || hid == 128 || hid == 192 || hid == 256; }

size_t mlp_ws_bytes(int B, int H, int N, int hid) {
    const size_t slices = (size_t)B * H;
    if (slices == 0 || N <= 0 || !mlp_hidden_supported(hid)) return 0;
    const MlpPlan p = mlp_plan(B, H, N);
    const size_t n2 = 2 * 64 * (size_t)hid;
    return a256m((size_t)H * n2 * 2) + a256m(slices * n2 * 2) + a256m(slices * p.S * n2 * 4);
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
    a.Wb = (bf16_t*)w;
    w += a256m((size_t)l.H * n2 * 2);
    a.Wn = (bf16_t*)w;
    w += a256m((size_t)slices * n2 * 2);
    a.part = (float*)w;
    hipLaunchKernelGGL(mlp_prep, dim3((unsigned)((64 * l.hid + kMT - 1) / kMT), (unsigned)l.H), dim3(kMT), 0, stream,
                       l.W1, l.W2, a.Wb, l.hid);
    switch (l.hid) {
    case 64: return launch_nhb<4>(a, slices, stream);
    case 128: return launch_nhb<8>(a, slices, stream);
    case 192: return launch_nhb<12>(a, slices, stream);
    default: return launch_nhb<16>(a, slices, stream);
    }
}

} // namespace ttt
