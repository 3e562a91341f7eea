// linear_fullbatch.hip -- one full-batch L2 gradient step of the linear
// d x d inner model, then apply (ViT3 article, observation 2; Vision-TTT
// notes, "关键设计" item 1 for the loss, the per-token gradient and
// z_t = W_t x_t^Q).
//
// Per slice (image b, head h) the gradient is rewritten with the Gram
// blocks A = sum_i k_i k_i^T and C = sum_i v_i k_i^T:
//     G = (2/N) (W0 A - C),   W1 = W0 - eta G,   z_i = W1 q_i.
// A and C stream K and V once; the update is d x d work; the apply streams Q
// once and writes Z once.  The layer is HBM-bound (48 flop/byte in bf16).
//
// One launch does everything.  A slice is split over S workgroups along
// the tokens (the grid is slices x S, every workgroup resident):
//   phase 1  each workgroup streams 128-token K/V tiles through registers
//            (3 tiles in flight) into double-buffered LDS and accumulates
//            its partial [A; C] with 16x16x32 bf16 MFMAs, 4 waves over
//            disjoint tokens, then sums the 4 waves in a fixed order;
//            Q tiles for the apply are prefetched into registers;
//   phase 2  (S > 1) partials go to the workspace, a per-slice barrier,
//            each workgroup reduces 64/S columns of [A; C] over the S
//            partials in split order, forms those columns of G and W1,
//            a second barrier, every workgroup reads W1;
//            (S == 1) the workgroup forms G and W1 itself;
//   phase 3  Z^T = W1 Q^T with W1 rows as the MFMA A operand, so each
//            lane's outputs are 8 contiguous channels of one token.
// fp32 inputs take the same path with 16x16x4 fp32 MFMAs.
#include "common.hpp"
#include "internal.hpp"

#include <atomic>

namespace ttt {
namespace {

template <bool BF> struct LinCfg;
template <> struct LinCfg<true> {
    static constexpr int esz = 2;
    static constexpr int tile = 128;     // tokens per LDS stage
    static constexpr int row_slots = 8;  // 16-byte slots per token row
    static constexpr int qpre = 2;       // apply steps prefetched per wave
};
template <> struct LinCfg<false> {
    static constexpr int esz = 4;
    static constexpr int tile = 64;
    static constexpr int row_slots = 16;
    static constexpr int qpre = 2;
};

constexpr int kStages = 3;                          // tiles in flight (registers)
constexpr int kStageBytes = 32768;                  // K tile + V tile
constexpr int kLdsFloats = 2 * kStageBytes / 4;     // double-buffered: 64 KB
constexpr int MP = 68;                              // pitch of 64x64 fp32 matrices in LDS
// float offsets of the phase-2 LDS regions (the staging buffers are dead by then)
constexpr int RED = 0;        // 26 tiles x 256 floats
constexpr int MAT_A = 6656;
constexpr int MAT_C = MAT_A + 64 * MP;
// After the wave reduction: W0 is staged over the dead reduction buffer and
// W1 overwrites C in place (each W1 element is written by the thread that
// last reads the C element at the same position; A stays intact).
constexpr int MAT_W = MAT_C;
constexpr int W0S = 0;
static_assert(MAT_C + 64 * MP <= kLdsFloats, "LDS layout");
static_assert(W0S + 64 * MP <= MAT_A, "W0 staging must not overlap A");

// XOR swizzle of the 16-byte slots of a staged row: keeps the transposed
// (token-major per lane) fragment reads free of bank conflicts.
template <bool BF> __device__ __forceinline__ int swz(int row);
template <> __device__ __forceinline__ int swz<true>(int row) { return ((row >> 2) & 3) << 1; }
template <> __device__ __forceinline__ int swz<false>(int row) { return (row & 3) << 2; }

__device__ __forceinline__ int perm_row(int rb, int m) {
    // MFMA row m of output block rb -> output channel; lane (g, .) then owns
    // channels [8g, 8g+8) (blocks 0,1) and [32+8g, 32+8g+8) (blocks 2,3).
    return 32 * (rb >> 1) + 8 * (m >> 2) + 4 * (rb & 1) + (m & 3);
}

template <bool BF>
__global__ __launch_bounds__(kThreads, 1) void lin_fwd_kernel(LinFwdLaunch a) {
    using Cfg = LinCfg<BF>;
    __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
    char* ldsb = reinterpret_cast<char*>(lds);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, m = lane & 15;
    const SliceSplit ss = map_block(blockIdx.x, a.S, a.xcd);
    const int slice = ss.slice, split = ss.split;
    const int b = slice / a.H, h = slice % a.H;
    const int N = a.N;
    const int per = (((N + a.S - 1) / a.S) + 15) & ~15;
    const int t0 = min(N, split * per), t1 = min(N, t0 + per);

    const char* Kp = (const char*)a.K.ptr + (b * a.K.sb + h * a.K.sh) * (long long)Cfg::esz;
    const char* Vp = (const char*)a.V.ptr + (b * a.V.sb + h * a.V.sh) * (long long)Cfg::esz;
    const char* Qp = (const char*)a.Q.ptr + (b * a.Q.sb + h * a.Q.sh) * (long long)Cfg::esz;
    char* Zp = (char*)a.Z.ptr + (b * a.Z.sb + h * a.Z.sh) * (long long)Cfg::esz;
    const long long Ksn = a.K.sn * Cfg::esz, Vsn = a.V.sn * Cfg::esz;
    const long long Qsn = a.Q.sn * Cfg::esz, Zsn = a.Z.sn * Cfg::esz;

    // ------------------------------------------------------------ phase 1
    v4f accC[16], accA[10];
#pragma unroll
    for (int t = 0; t < 16; ++t) accC[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 10; ++t) accA[t] = v4f{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (t1 - t0 + Cfg::tile - 1) / Cfg::tile;

    // Tile `it` -> 8 x 16-byte loads per thread (4 of K, 4 of V); chunk
    // p = j*256 + tid covers token row p / row_slots, slot p % row_slots.
    u32x4 R[kStages][8];
    auto load_tile = [&](int it, u32x4* r) __attribute__((always_inline)) {
        const int tb = t0 + it * Cfg::tile;
        const int nvalid = t1 - tb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = j * kThreads + tid;
            const int row = min(p / Cfg::row_slots, nvalid - 1);
            const int off = (p % Cfg::row_slots) * 16;
            r[j] = *reinterpret_cast<const u32x4*>(Kp + (long long)(tb + row) * Ksn + off);
            r[4 + j] = *reinterpret_cast<const u32x4*>(Vp + (long long)(tb + row) * Vsn + off);
        }
    };
    auto store_tile = [&](const u32x4* r, char* st) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = j * kThreads + tid;
            const int row = p / Cfg::row_slots;
            const int slot = row * Cfg::row_slots + ((p % Cfg::row_slots) ^ swz<BF>(row));
            *reinterpret_cast<u32x4*>(st + slot * 16) = r[j];
            *reinterpret_cast<u32x4*>(st + 16384 + slot * 16) = r[4 + j];
        }
    };
    auto compute_tile = [&](int it, const char* sK) __attribute__((always_inline)) {
        const char* sV = sK + 16384;
        const int nvalid = t1 - (t0 + it * Cfg::tile);
        if constexpr (BF) {
            // lane (g, m) gathers tokens 32w + 8g + j (j = 0..7) of channel
            // 16cb + m: the k-major operand layout of the 16x16x32 MFMA
            v8bf kf[4], vf[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int c = 16 * cb + m;
                v8s kv, vv;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int row = 32 * w + 8 * g + j;
                    const int addr = (row * 8 + ((c >> 3) ^ swz<true>(row))) * 16 + (c & 7) * 2;
                    const bool ok = row < nvalid;
                    kv[j] = ok ? *reinterpret_cast<const short*>(sK + addr) : (short)0;
                    vv[j] = ok ? *reinterpret_cast<const short*>(sV + addr) : (short)0;
                }
                kf[cb] = __builtin_bit_cast(v8bf, kv);
                vf[cb] = __builtin_bit_cast(v8bf, vv);
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) accC[rb * 4 + cb] = mfma32(vf[rb], kf[cb], accC[rb * 4 + cb]);
            int t = 0;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = rb; cb < 4; ++cb, ++t) accA[t] = mfma32(kf[rb], kf[cb], accA[t]);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = 16 * w + 4 * s + g;
                float kf[4], vf[4];
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int c = 16 * cb + m;
                    const int addr = (row * 16 + ((c >> 2) ^ swz<false>(row))) * 16 + (c & 3) * 4;
                    kf[cb] = row < nvalid ? *reinterpret_cast<const float*>(sK + addr) : 0.f;
                    vf[cb] = row < nvalid ? *reinterpret_cast<const float*>(sV + addr) : 0.f;
                }
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) accC[rb * 4 + cb] = mfma4(vf[rb], kf[cb], accC[rb * 4 + cb]);
                int t = 0;
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int cb = rb; cb < 4; ++cb, ++t) accA[t] = mfma4(kf[rb], kf[cb], accA[t]);
            }
        }
    };

    if (ntiles > 0) {
#pragma unroll
        for (int s = 0; s < kStages; ++s) load_tile(min(s, ntiles - 1), R[s]);
    }

    // Prefetch this wave's first Q tiles for the apply (16 tokens per step,
    // steps w, w+4, ...).  Token rows are clamped into the range (a clamped
    // step is never applied), so the loads are unconditional.
    const int nsteps = (t1 - t0 + 15) / 16;
    constexpr int QV = BF ? 2 : 4; // 16-byte loads per lane per step
    u32x4 qpre[Cfg::qpre][QV];
    if (ntiles > 0) {
#pragma unroll
        for (int k = 0; k < Cfg::qpre; ++k) {
            const int tok = min(t0 + (w + 4 * k) * 16 + m, t1 - 1);
#pragma unroll
            for (int hh = 0; hh < QV; ++hh) {
                const int ch = BF ? (32 * hh + 8 * g) : (16 * hh + 4 * g);
                qpre[k][hh] = *reinterpret_cast<const u32x4*>(Qp + tok * Qsn + ch * Cfg::esz);
            }
        }
    }

    // Pipelined tile loop: tile it is written from its registers into LDS
    // buffer it&1, the registers are refilled with tile it+3, then the
    // waves consume the buffer (one LDS barrier per tile).  Every load is
    // unconditional inside the main loop and the first loads are clamped
    // duplicates for short ranges, so the compiler's load counters stay
    // exact and three tiles remain in flight.
    auto step = [&](int it, u32x4* r, bool reload) __attribute__((always_inline)) {
        char* st = ldsb + (it & 1) * kStageBytes;
        store_tile(r, st);
        lds_barrier();
        if (reload) load_tile(it + kStages, r);
        compute_tile(it, st);
    };
    if (ntiles > 0) {
        int it = 0;
        for (; it + 2 * kStages <= ntiles; it += kStages) {
            step(it, R[0], true);
            step(it + 1, R[1], true);
            step(it + 2, R[2], true);
        }
#pragma unroll
        for (int s = 0; s < 2 * kStages - 1; ++s) {
            const int t = it + s;
            if (t < ntiles) step(t, R[s % kStages], t + kStages < ntiles);
        }
    }
    lds_barrier();

    // ------------------------------------------------ wave reduction of [A;C]
    // Fixed order ((w3 + w2) + w1) + w0 through one 26-tile LDS buffer.
    {
        float* red = lds + RED;
        auto tile_ref = [&](int t) -> v4f& { return t < 16 ? accC[t] : accA[t - 16]; };
#pragma unroll
        for (int src = 3; src >= 1; --src) {
            if (w == src) {
#pragma unroll
                for (int t = 0; t < 26; ++t) {
                    if (src < 3) tile_ref(t) += *reinterpret_cast<const v4f*>(red + t * 256 + lane * 4);
                    *reinterpret_cast<v4f*>(red + t * 256 + lane * 4) = tile_ref(t);
                }
            }
            lds_barrier();
        }
        if (w == 0) {
            float* mA = lds + MAT_A;
            float* mC = lds + MAT_C;
#pragma unroll
            for (int t = 0; t < 26; ++t)
                tile_ref(t) += *reinterpret_cast<const v4f*>(red + t * 256 + lane * 4);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        mC[(16 * rb + 4 * g + i) * MP + 16 * cb + m] = accC[rb * 4 + cb][i];
            int t = 0;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = rb; cb < 4; ++cb, ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = accA[t][i];
                        mA[(16 * rb + 4 * g + i) * MP + 16 * cb + m] = v;
                        if (rb < cb) mA[(16 * cb + m) * MP + 16 * rb + 4 * g + i] = v;
                    }
        }
        lds_barrier();
    }

    // ----------------------------------------------- phase 2: G and W1
    const float* W0h = a.W0 + (long long)h * 4096;
    const float eta = a.eta[h];
    const float scale = 2.0f / (float)N;
    float* mA = lds + MAT_A;
    float* mC = lds + MAT_C;
    float* mW = lds + MAT_W;
    float* W0s = lds + W0S;
    auto stage_w0 = [&]() {
        for (int e = tid; e < 1024; e += kThreads) {
            const int r = e >> 4, c4 = (e & 15) * 4;
            *reinterpret_cast<f32x4*>(W0s + r * MP + c4) = *reinterpret_cast<const f32x4*>(W0h + r * 64 + c4);
        }
    };
    if (a.S == 1) {
        stage_w0();
        lds_barrier();
        const int r0 = (tid >> 4) * 4, c0 = (tid & 15) * 4;
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[i][k] = 0.f;
        for (int j = 0; j < 64; ++j) {
            float av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = W0s[(r0 + i) * MP + j];
            const f32x4 bv = *reinterpret_cast<const f32x4*>(mA + j * MP + c0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i][0] += av[i] * bv.x;
                acc[i][1] += av[i] * bv.y;
                acc[i][2] += av[i] * bv.z;
                acc[i][3] += av[i] * bv.w;
            }
        }
        float* sv = a.saved ? a.saved + (long long)slice * 8192 : nullptr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = r0 + i, c = c0 + k;
                const float gv = scale * (acc[i][k] - mC[r * MP + c]);
                mW[r * MP + c] = W0s[r * MP + c] - eta * gv;
                if (sv) {
                    sv[r * 64 + c] = mA[r * MP + c];
                    sv[4096 + r * 64 + c] = gv;
                }
            }
        lds_barrier();
    } else {
        float* P = a.part + ((long long)slice * a.S + split) * 8192;
        for (int e = tid; e < 2048; e += kThreads) {
            const int mat = e >> 10, idx = e & 1023, r = idx >> 4, c4 = (idx & 15) * 4;
            const float* src = (mat ? mC : mA) + r * MP + c4;
            *reinterpret_cast<f32x4*>(P + mat * 4096 + r * 64 + c4) = *reinterpret_cast<const f32x4*>(src);
        }
        slice_barrier(a.cnt + slice, (unsigned)a.S);
        const int c0 = (64 * split) / a.S, c1 = (64 * (split + 1)) / a.S, nc = c1 - c0;
        const float* P0 = a.part + (long long)slice * a.S * 8192;
        for (int e = tid; e < 2 * 64 * nc; e += kThreads) {
            const int mat = e / (64 * nc), rem = e % (64 * nc), r = rem / nc, c = c0 + rem % nc;
            const float* src = P0 + mat * 4096 + r * 64 + c;
            float s = 0.f;
            for (int sp = 0; sp < a.S; ++sp) s += src[(long long)sp * 8192];
            (mat ? mC : mA)[r * MP + c] = s;
        }
        stage_w0();
        lds_barrier();
        float* sv = a.saved ? a.saved + (long long)slice * 8192 : nullptr;
        float* w1g = a.w1 + (long long)slice * 4096;
        for (int e = tid; e < 64 * nc; e += kThreads) {
            const int r = e / nc, c = c0 + e % nc;
            float acc = 0.f;
            for (int j = 0; j < 64; ++j) acc += W0s[r * MP + j] * mA[j * MP + c];
            const float gv = scale * (acc - mC[r * MP + c]);
            w1g[r * 64 + c] = W0s[r * MP + c] - eta * gv;
            if (sv) {
                sv[r * 64 + c] = mA[r * MP + c];
                sv[4096 + r * 64 + c] = gv;
            }
        }
        slice_barrier(a.cnt + slice, 2u * a.S);
        for (int e = tid; e < 1024; e += kThreads) {
            const int r = e >> 4, c4 = (e & 15) * 4;
            *reinterpret_cast<f32x4*>(mW + r * MP + c4) = *reinterpret_cast<const f32x4*>(w1g + r * 64 + c4);
        }
        slice_barrier_release(a.cnt + slice, 3u * a.S);
        lds_barrier();
    }

    // ------------------------------------------------------ phase 3: apply
    if constexpr (BF) {
        v8bf wf[4][2];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int r = perm_row(rb, m);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const float* src = mW + r * MP + 32 * hh + 8 * g;
                u32x4 u;
                u.x = pack_bf2(src[0], src[1]);
                u.y = pack_bf2(src[2], src[3]);
                u.z = pack_bf2(src[4], src[5]);
                u.w = pack_bf2(src[6], src[7]);
                wf[rb][hh] = as_v8bf(u);
            }
        }
        auto apply = [&](int step, const u32x4* q) {
            v4f d[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                d[rb] = v4f{0.f, 0.f, 0.f, 0.f};
                d[rb] = mfma32(wf[rb][0], as_v8bf(q[0]), d[rb]);
                d[rb] = mfma32(wf[rb][1], as_v8bf(q[1]), d[rb]);
            }
            const int tok = t0 + step * 16 + m;
            if (tok < t1) {
                u32x4 o0{pack_bf2(d[0][0], d[0][1]), pack_bf2(d[0][2], d[0][3]),
                         pack_bf2(d[1][0], d[1][1]), pack_bf2(d[1][2], d[1][3])};
                u32x4 o1{pack_bf2(d[2][0], d[2][1]), pack_bf2(d[2][2], d[2][3]),
                         pack_bf2(d[3][0], d[3][1]), pack_bf2(d[3][2], d[3][3])};
                *reinterpret_cast<u32x4*>(Zp + tok * Zsn + (8 * g) * 2) = o0;
                *reinterpret_cast<u32x4*>(Zp + tok * Zsn + (32 + 8 * g) * 2) = o1;
            }
        };
#pragma unroll
        for (int k = 0; k < Cfg::qpre; ++k) {
            const int step = w + 4 * k;
            if (step < nsteps) apply(step, qpre[k]);
        }
        for (int step = w + 4 * Cfg::qpre; step < nsteps; step += 4) {
            const int tok = min(t0 + step * 16 + m, t1 - 1);
            u32x4 q[2];
            q[0] = *reinterpret_cast<const u32x4*>(Qp + tok * Qsn + (8 * g) * 2);
            q[1] = *reinterpret_cast<const u32x4*>(Qp + tok * Qsn + (32 + 8 * g) * 2);
            apply(step, q);
        }
    } else {
        float wf[4][16];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int r = perm_row(rb, m);
#pragma unroll
            for (int hh = 0; hh < 4; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i) wf[rb][hh * 4 + i] = mW[r * MP + 16 * hh + 4 * g + i];
        }
        auto apply = [&](int step, const u32x4* q) {
            v4f d[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                d[rb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) {
                    const f32x4 qv = __builtin_bit_cast(f32x4, q[hh]);
                    d[rb] = mfma4(wf[rb][hh * 4 + 0], qv.x, d[rb]);
                    d[rb] = mfma4(wf[rb][hh * 4 + 1], qv.y, d[rb]);
                    d[rb] = mfma4(wf[rb][hh * 4 + 2], qv.z, d[rb]);
                    d[rb] = mfma4(wf[rb][hh * 4 + 3], qv.w, d[rb]);
                }
            }
            const int tok = t0 + step * 16 + m;
            if (tok < t1) {
                float* zr = reinterpret_cast<float*>(Zp + tok * Zsn);
                *reinterpret_cast<f32x4*>(zr + 8 * g) = f32x4{d[0][0], d[0][1], d[0][2], d[0][3]};
                *reinterpret_cast<f32x4*>(zr + 8 * g + 4) = f32x4{d[1][0], d[1][1], d[1][2], d[1][3]};
                *reinterpret_cast<f32x4*>(zr + 32 + 8 * g) = f32x4{d[2][0], d[2][1], d[2][2], d[2][3]};
                *reinterpret_cast<f32x4*>(zr + 36 + 8 * g) = f32x4{d[3][0], d[3][1], d[3][2], d[3][3]};
            }
        };
#pragma unroll
        for (int k = 0; k < Cfg::qpre; ++k) {
            const int step = w + 4 * k;
            if (step < nsteps) apply(step, qpre[k]);
        }
        for (int step = w + 4 * Cfg::qpre; step < nsteps; step += 4) {
            const int tok = min(t0 + step * 16 + m, t1 - 1);
            u32x4 q[4];
#pragma unroll
            for (int hh = 0; hh < 4; ++hh)
                q[hh] = *reinterpret_cast<const u32x4*>(Qp + tok * Qsn + (16 * hh + 4 * g) * 4);
            apply(step, q);
        }
    }
}

} // namespace

int lin_fwd_max_splits(int B, int H, int N) {
    const long long slices = (long long)B * H;
    if (slices <= 0 || N <= 0) return 1;
    // at most 64 splits, at least ~128 tokens each, and no more workgroups
    // than one MI355X keeps resident (256 CUs x 1)
    long long s = (N + 127) / 128;
    if (s > 64) s = 64;
    const long long cap = 256 / slices;
    if (s > cap) s = cap;
    return s < 1 ? 1 : (int)s;
}

size_t lin_fwd_ws_bytes(int B, int H, int N) {
    const long long slices = (long long)B * H;
    const int S = lin_fwd_max_splits(B, H, N);
    if (S <= 1) return 0;
    const size_t cnt = ((size_t)slices * 4 + 255) & ~(size_t)255;
    return cnt + (size_t)slices * S * 8192 * 4 + (size_t)slices * 4096 * 4;
}

int lin_fwd_resident_per_cu(int bf16) {
    static std::atomic<int> cached[2];
    int n = cached[bf16 ? 1 : 0].load(std::memory_order_relaxed);
    if (n > 0) return n;
    hipError_t e = bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lin_fwd_kernel<true>, kThreads, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lin_fwd_kernel<false>, kThreads, 0);
    if (e != hipSuccess || n < 0) return 0;
    cached[bf16 ? 1 : 0].store(n, std::memory_order_relaxed);
    return n;
}

hipError_t launch_lin_fwd(LinFwdLaunch a, hipStream_t stream, int resident_wgs) {
    const long long slices = (long long)a.B * a.H;
    (void)resident_wgs;
    const dim3 grid((unsigned)(slices * a.S)), block(kThreads);
    void* args[] = {&a};
    const void* fn = a.bf16 ? (const void*)lin_fwd_kernel<true> : (const void*)lin_fwd_kernel<false>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

} // namespace ttt
