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
//   phase 1  partial [A; C] of the workgroup's tokens with 16x16x32 bf16
//            MFMAs (4 waves over disjoint tokens, summed in a fixed order);
//   phase 2  (S > 1) partials meet in the workspace at a per-slice barrier,
//            each workgroup reduces 64/S columns over the S partials in
//            split order and forms those columns of G and W1, a second
//            barrier, every workgroup reads W1; (S == 1) the workgroup
//            forms G and W1 itself;
//   phase 3  Z^T = W1 Q^T with W1 rows as the MFMA A operand, so each
//            lane's outputs are 8 contiguous channels of one token.
// Two variants of phase 1 / 3:
//   resident  (a workgroup owns <= 384 bf16 tokens): every K, V and Q byte
//             of the workgroup is requested at kernel start with direct
//             global->LDS loads and W0 is prefetched into registers, so no
//             load is issued after the start -- the latency of the whole
//             range overlaps, and the exchange in phase 2 never queues
//             behind streaming traffic;
//   streaming (longer ranges): 128-token K/V tiles flow through registers
//             (3 in flight) into double-buffered LDS; Q is loaded per
//             apply step with a short prefetch.
// fp32 inputs take the same paths with 16x16x4 fp32 MFMAs.
#include "common.hpp"
#include "conv_body.hpp"
#include "internal.hpp"

#include <atomic>

namespace ttt {
namespace {

constexpr int MP = 68; // pitch (floats) of 64x64 fp32 matrices in LDS

// G = scale (w_A W0 A - C): the L2 loss has scale 2/N and w_A = 1; the
// dot-product loss (l = -<W k, v>) has scale 1/N and no W0 A term.
__device__ __forceinline__ float grad_scale(const LinFwdLaunch& a) {
    return (a.dot ? 1.0f : 2.0f) / (float)a.N;
}

template <bool BF> struct LinCfg;
template <> struct LinCfg<true> {
    static constexpr int esz = 2;
    static constexpr int row_slots = 8;  // 16-byte slots per token row
    static constexpr int tile = 128;     // streaming: tokens per LDS stage
    static constexpr int qpre = 2;       // streaming: apply steps prefetched per wave
    static constexpr int tmax = 384;     // resident: tokens per workgroup
};
template <> struct LinCfg<false> {
    static constexpr int esz = 4;
    static constexpr int row_slots = 16;
    static constexpr int tile = 64;
    static constexpr int qpre = 2;
    static constexpr int tmax = 192;
};

// XOR swizzles of the 16-byte slots of a staged token row.
// K and V (Gram reads: the 4 lane groups read rows 8 apart inside a 32-row
// step): bf16 flips slot bits 1-2 by (row / 8) % 4, so each group reads a
// different 32-byte band, and a lane's addresses are 4 fixed bases plus
// row offsets.  Q (apply reads: 16 consecutive rows, one slot each):
// slot ^ (row % 8) (bf16) / (row % 16) (fp32).
template <bool BF> __device__ __forceinline__ int swz_kv(int row);
template <> __device__ __forceinline__ int swz_kv<true>(int row) { return ((row >> 3) & 3) << 1; }
template <> __device__ __forceinline__ int swz_kv<false>(int row) { return (row & 3) << 2; }
template <bool BF> __device__ __forceinline__ int swz_q(int row);
template <> __device__ __forceinline__ int swz_q<true>(int row) { return (row >> 1) & 7; }
template <> __device__ __forceinline__ int swz_q<false>(int row) { return row & 15; }


typedef __attribute__((address_space(3))) void lds_void;

// ------------------------------------------------------------- Gram step --
// One k-step of [A; C] from a swizzled row-major K/V region in LDS whose
// rows past the valid range hold zeros.
// bf16: the wave takes token rows [r0, r0+32) (r0 % 32 == 0); lane (g, m)
// gathers rows r0 + 8g + j (j = 0..7) of channel 16cb + m -- the k-major
// operand layout of the 16x16x32 MFMA.  With the K/V swizzle that element
// sits at byte (r0 + j)*128 + kb[cb], kb[cb] = 1024g + 32(cb ^ g) + 2m.
// fp32: rows [r0, r0+16) as 4 sub-steps of the 16x16x4 MFMA.
struct GramLanes {
    int kb[4];
};
__device__ __forceinline__ GramLanes gram_lanes(int g, int m) {
    GramLanes l;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) l.kb[cb] = 1024 * g + 32 * (cb ^ g) + 2 * m;
    return l;
}
template <bool BF>
__device__ __forceinline__ void gram_step(const char* sK, const char* sV, int r0, const GramLanes& gl,
                                          v4f* accC, v4f* accA, int g, int m) {
    if constexpr (BF) {
        v8bf kf[4], vf[4];
        const char* k0 = sK + r0 * 128;
        const char* v0 = sV + r0 * 128;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            v8s kv, vv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                kv[j] = *reinterpret_cast<const short*>(k0 + gl.kb[cb] + j * 128);
                vv[j] = *reinterpret_cast<const short*>(v0 + gl.kb[cb] + j * 128);
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
        (void)gl;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int row = r0 + 4 * s + g;
            float kf[4], vf[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int c = 16 * cb + m;
                const int addr = (row * 16 + ((c >> 2) ^ swz_kv<false>(row))) * 16 + (c & 3) * 4;
                kf[cb] = *reinterpret_cast<const float*>(sK + addr);
                vf[cb] = *reinterpret_cast<const float*>(sV + addr);
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
}

// Tile t of [A; C] in MFMA layout: t < 16 is C block (t/4, t%4); t >= 16 the
// upper-triangle A blocks (0,0),(0,1),(0,2),(0,3),(1,1),...,(3,3).
__device__ __forceinline__ void tile_blocks(int t, int& mat, int& rb, int& cb) {
    if (t < 16) {
        mat = 1; rb = t >> 2; cb = t & 3;
    } else {
        const int u = t - 16; // 0..9
        mat = 0;
        rb = u < 4 ? 0 : (u < 7 ? 1 : (u < 9 ? 2 : 3));
        const int first = rb == 0 ? 0 : (rb == 1 ? 4 : (rb == 2 ? 7 : 9));
        cb = rb + (u - first);
    }
}
// Write one final tile as row-major 64x64 (A blocks also mirrored).
__device__ __forceinline__ void write_tile(const v4f& v, int t, float* mA, float* mC, int g, int m) {
    int mat, rb, cb;
    tile_blocks(t, mat, rb, cb);
    float* M = mat ? mC : mA;
#pragma unroll
    for (int i = 0; i < 4; ++i) M[(16 * rb + 4 * g + i) * MP + 16 * cb + m] = v[i];
    if (!mat && rb < cb) *reinterpret_cast<f32x4*>(mA + (16 * cb + m) * MP + 16 * rb + 4 * g) = v;
}

// ------------------------------------------------------------- phase 2 --
// A store from one CU to a line that is not in its XCD's L2 goes on to
// memory without allocating the line there, so a later load of it from
// another CU of the XCD misses too (measured on MI355X: about 0.6 us for
// 32 KB, against 0.3 us for L2 hits).  A store to a line that is present
// updates it in place.  Each workgroup therefore touches one word of every
// line it will read after the slice barriers -- its gather block of the
// partials and its share of W1 -- before the writers store them, with
// device-scope loads: those fill the XCD's L2 but not the CU's L1 (plain
// loads would leave a copy in L1 that the post-barrier reads would hit,
// stale).  Touching a line after its writer stored it is harmless: the
// load then fetches the new contents.  The returned values only keep the
// loads alive (keep_alive(), placed after the last barrier: nothing waits
// for them before).
struct Prefetch {
    float blk, w1;
};
template <bool BF, bool XC>
__device__ __forceinline__ Prefetch exchange_prefetch(const LinFwdLaunch& a, int slice, int split, bool gx) {
    if constexpr (!XC) return Prefetch{0.f, 0.f}; // device-wide protocol: atomics at the coherence point
    const int tid = threadIdx.x;
    // gather block: [A; C] exchange S * 128 * (64 / S) floats = 256 lines
    // of 32 floats; G exchange 4096 floats = 128 lines
    const float* blk = gx ? a.part + (long long)slice * a.S * 4096 + (long long)split * 4096 + min(tid, 127) * 32
                          : a.part + (long long)slice * a.S * 8192 + (long long)split * 8192 + tid * 32;
    // W1 (bf16 fragments: 64 lines; fp32: 128 lines), spread over the
    // slice's S workgroups; threads past the share repeat its last line
    const int per = (BF ? 64 : 128) >> __builtin_ctz(a.S);
    const int line = split * per + min(tid, per - 1);
    return Prefetch{xload(blk), xload(a.w1 + (long long)slice * 4096 + line * 32)};
}
__device__ __forceinline__ void keep_alive(const Prefetch& p) { asm volatile("" ::"v"(p.blk), "v"(p.w1)); }

// From the workgroup's [A; C] (mA, mC: full 64x64, pitch MP) to W1 in LDS.
// w0r: this thread's 4 x 16 bytes of W0[h] (floats 4*tid + 1024*k).
// LDS use, S == 1: W0 staged at w0s_one (disjoint from mA, mC); W1 written
//   over mC in place (each element read, then written, by one thread).
// LDS use, S > 1: scratch [0, 8192) floats (may overlap mA / mC: they are
//   consumed before the first barrier), W0 at w0s_split >= 8192.
// Returns W1 in LDS (pitch MP) when S == 1; nullptr when S > 1, where W1 is
// complete in the workspace at a.w1 + slice*4096 on return.
// Sum this workgroup's block of the S partials over the splits, in split
// order, straight from memory: the block is contiguous, split sp's part at
// blk[sp * 8192 / S ...] (2048 / S float4s).  Every load of a thread is in
// flight at once; res receives the reduced block (same layout).
template <int S, bool XC>
__device__ __forceinline__ void gather_sum(const float* blk, float* res) {
    constexpr int n4 = 2048 / S;
    const int tid = threadIdx.x;
    const f32x4* b4 = reinterpret_cast<const f32x4*>(blk);
    auto ld = [&](int i) {
        if constexpr (XC) return b4[i];
        const float* p = blk + 4 * i;
        return f32x4{xload(p), xload(p + 1), xload(p + 2), xload(p + 3)};
    };
    if constexpr (n4 >= kThreads) {
        constexpr int per = n4 / kThreads;
        f32x4 v[per][S];
#pragma unroll
        for (int k = 0; k < per; ++k)
#pragma unroll
            for (int sp = 0; sp < S; ++sp) v[k][sp] = ld(sp * n4 + k * kThreads + tid);
#pragma unroll
        for (int k = 0; k < per; ++k) {
            f32x4 acc = v[k][0];
#pragma unroll
            for (int sp = 1; sp < S; ++sp) acc += v[k][sp];
            reinterpret_cast<f32x4*>(res)[k * kThreads + tid] = acc;
        }
    } else if (tid < n4) {
        f32x4 v[S];
#pragma unroll
        for (int sp = 0; sp < S; ++sp) v[sp] = ld(sp * n4 + tid);
        f32x4 acc = v[0];
#pragma unroll
        for (int sp = 1; sp < S; ++sp) acc += v[sp];
        reinterpret_cast<f32x4*>(res)[tid] = acc;
    }
}

// Index of W1[r][c] in the bf16 fragment copy of W1 that the XCD-local
// exchange hands to the apply phase: 16-byte piece (rb, hh, lane) holds
// W1[perm_row(rb, m)][32 hh + 8 g + j], j = 0..7, lane = 16 g + m, at
// piece index (rb * 2 + hh) * 64 + lane -- so a lane's eight operand
// registers are eight 16-byte loads, each wave instruction one contiguous
// kilobyte.
__device__ __forceinline__ int w1_frag_index(int r, int c) {
    const int rb = 2 * (r >> 5) + ((r >> 2) & 1), m = 4 * ((r >> 3) & 3) + (r & 3);
    const int hh = c >> 5, g = (c >> 3) & 3;
    return ((rb * 2 + hh) * 64 + 16 * g + m) * 8 + (c & 7);
}

template <bool BF, bool XC>
__device__ float* lin_update(const LinFwdLaunch& a, int slice, int split, int h, float* lds,
                             float* mA, float* mC, float* w0s_one, float* w0s_split, const f32x4* w0r,
                             SliceWords* sw, bool published = false, Prefetch pf = Prefetch{0.f, 0.f}) {
    const int tid = threadIdx.x;
    const float eta = a.eta[h];
    const float scale = grad_scale(a);
    const float wa = a.dot ? 0.f : 1.f; // weight of the W0 A term
    auto stage_w0 = [&](float* dst) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = 4 * tid + 1024 * k, r = e >> 6, c = e & 63;
            *reinterpret_cast<f32x4*>(dst + r * MP + c) = w0r[k];
        }
    };
    if (a.S == 1) {
        static_assert(kThreads == 256, "four waves: one 16-row block of W0 A each");
        stage_w0(w0s_one);
        lds_barrier();
        // W0 A on the fp32 matrix cores (16x16x4 tiles): wave w forms rows
        // 16 w.., lane (g, m) then holds rows 16 w + 4 g + i, columns
        // 16 cb + m
        const int lane = tid & 63, g = lane >> 4, m = lane & 15, w = tid >> 6;
        v4f acc[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k0 = 0; k0 < 64; k0 += 4) {
            const float av = w0s_one[(16 * w + m) * MP + k0 + g]; // W0[16w+m][k0+g]
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc[cb] = mfma4(av, mA[(k0 + g) * MP + 16 * cb + m], acc[cb]);
        }
        float* sv = a.saved ? a.saved + (long long)slice * 8192 : nullptr;
        lds_barrier(); // every thread has read mA / W0 rows before W1 replaces C
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * g + i, c = 16 * cb + m;
                const float gv = scale * (wa * acc[cb][i] - mC[r * MP + c]);
                mC[r * MP + c] = w0s_one[r * MP + c] - eta * gv;
                if (sv) {
                    sv[r * 64 + c] = mA[r * MP + c];
                    sv[4096 + r * 64 + c] = gv;
                }
            }
        lds_barrier();
        return mC;
    }

    // S > 1: publish this workgroup's partial in reducer-major order,
    // part[slice][j][sp][mat][cc][r] with column c = j*nc + cc: the block a
    // reducer j gathers is then one contiguous run of S*128*nc floats, and
    // four consecutive rows of one column are one 16-byte store.
    const int lgnc = 6 - __builtin_ctz(a.S); // S is a power of two
    const int nc = 1 << lgnc, c0 = split * nc;
    const long long sb = (long long)slice * a.S * 8192;
    unsigned* cnt = counter_at(a.cnt, slice);
    auto pidx = [&](int j, int sp, int mat, int cc, int r) {
        return sb + ((long long)(j * a.S + sp) * 2 + mat) * 64 * nc + cc * 64 + r;
    };
    if (published) {
        // the caller stored this workgroup's partial from its registers
    } else if constexpr (XC) {
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const int q = f * kThreads + tid, mat = q >> 10, c = (q >> 4) & 63, r4 = (q & 15) * 4;
            const float* M = mat ? mC : mA;
            *reinterpret_cast<f32x4*>(a.part + pidx(c >> lgnc, split, mat, c & (nc - 1), r4)) =
                f32x4{M[r4 * MP + c], M[(r4 + 1) * MP + c], M[(r4 + 2) * MP + c], M[(r4 + 3) * MP + c]};
        }
    } else {
#pragma unroll 8
        for (int f = 0; f < 32; ++f) {
            const int e = f * kThreads + tid, mat = e >> 12, r = (e >> 6) & 63, c = e & 63;
            xstore(a.part + pidx(c >> lgnc, split, mat, c & (nc - 1), r), (mat ? mC : mA)[r * MP + c]);
        }
    }
    slice_barrier(cnt, (unsigned)a.S + a.tbias, true, a.spin);

    const float* blk = a.part + pidx(split, 0, 0, 0, 0);
    float* res = lds; // [mat][nc][64] reduced block
    switch (a.S) {
    case 2: gather_sum<2, XC>(blk, res); break;
    case 4: gather_sum<4, XC>(blk, res); break;
    case 8: gather_sum<8, XC>(blk, res); break;
    case 16: gather_sum<16, XC>(blk, res); break;
    default: gather_sum<32, XC>(blk, res); break;
    }
    stage_w0(w0s_split);
    lds_barrier();
    float* sv = a.saved ? a.saved + (long long)slice * 8192 : nullptr;
    float* w1g = a.w1 + (long long)slice * 4096;
    for (int e = tid; e < 64 * nc; e += kThreads) {
        const int r = e >> lgnc, cc = e & (nc - 1), c = c0 + cc;
        const float* acol = res + cc * 64; // A[.][c]
        float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll 4
        for (int j = 0; j < 64; j += 4) {
            const f32x4 wv = *reinterpret_cast<const f32x4*>(w0s_split + r * MP + j);
            const f32x4 av = *reinterpret_cast<const f32x4*>(acol + j);
            acc0 += wv[0] * av[0];
            acc1 += wv[1] * av[1];
            acc2 += wv[2] * av[2];
            acc3 += wv[3] * av[3];
        }
        const float gv = scale * (wa * ((acc0 + acc1) + (acc2 + acc3)) - res[(nc + cc) * 64 + r]);
        const float w1v = w0s_split[r * MP + c] - eta * gv;
        if constexpr (BF && XC) reinterpret_cast<bf16_t*>(w1g)[w1_frag_index(r, c)] = f2bf(w1v);
        else if constexpr (XC) w1g[r * 64 + c] = w1v;
        else xstore(w1g + r * 64 + c, w1v);
        if (sv) {
            sv[r * 64 + c] = acol[r];
            sv[4096 + r * 64 + c] = gv;
        }
    }
    slice_barrier(cnt, 2u * a.S + a.tbias, true, a.spin);
    if (tid == 0) *sw = slice_words(cnt);
    keep_alive(pf);
    // W1 is complete in the workspace at a.w1 + slice*4096 (bf16 fragments
    // for BF && XC, else row-major fp32)
    return nullptr;
}

// Counter release after the last barrier: the increment's result is only
// needed at the very end of the kernel (reset by the last workgroup).
__device__ __forceinline__ unsigned release_begin(const LinFwdLaunch& a, int slice) {
    unsigned old = 0;
    if (a.S > 1 && threadIdx.x == 0)
        old = __hip_atomic_fetch_add(counter_at(a.cnt, slice), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return old;
}
__device__ __forceinline__ void release_end(const LinFwdLaunch& a, int slice, unsigned old) {
    const unsigned steps = a.steps > 1 ? (unsigned)a.steps : 1u; // two barriers per step, one release
    if (a.S > 1 && threadIdx.x == 0 && old == (2u * steps + 1u) * a.S - 1) slice_reset(counter_at(a.cnt, slice));
}

// After the slice's last waiting barrier, with the loads the apply needs
// (W1) already issued: waits for every load of the workgroup, then thread
// 0's slice words (loaded right after that barrier, before any release)
// decide through LDS whether the slice's outputs are NaN -- Z by the
// caller, A and G (this workgroup's columns) here.
template <bool XC>
__device__ __forceinline__ bool exchange_outcome(const LinFwdLaunch& a, int slice, int split,
                                                 const SliceWords& sw, int* chk, int nthreads) {
    drain_vmem();
    if (a.S > 1 && threadIdx.x == 0) *chk = slice_bad(sw, XC ? a.S : 0) ? 1 : 0;
    __syncthreads();
    const bool bad = a.S > 1 && *chk != 0;
    if (bad && a.saved) {
        const int lgnc = 6 - __builtin_ctz(a.S), nc = 1 << lgnc, c0 = split * nc;
        float* sv = a.saved + (long long)slice * 8192;
        for (int e = threadIdx.x; e < 64 * nc; e += nthreads) {
            const int r = e >> lgnc, c = c0 + (e & (nc - 1));
            sv[r * 64 + c] = sv[4096 + r * 64 + c] = __builtin_nanf("");
        }
    }
    return bad;
}

// ------------------------------------------------------------- phase 3 --
// W1 fragments: A operand rows perm_row(rb, m) of W1 (LDS, pitch MP).
struct W1FragsBF {
    v8bf f[4][2];
};
__device__ __forceinline__ W1FragsBF w1_frags_bf(const float* mW, int g, int m) {
    W1FragsBF w;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int r = perm_row(rb, m);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float* src = mW + r * MP + 32 * hh + 8 * g;
            u32x4 u;
            u[0] = pack_bf2(src[0], src[1]);
            u[1] = pack_bf2(src[2], src[3]);
            u[2] = pack_bf2(src[4], src[5]);
            u[3] = pack_bf2(src[6], src[7]);
            w.f[rb][hh] = as_v8bf(u);
        }
    }
    return w;
}
// The same fragments loaded straight from the workspace copy of W1
// (row-major 64x64 fp32; plain loads in the XCD-local protocol).
template <bool XC>
__device__ __forceinline__ W1FragsBF w1_frags_bf_global(const float* w1g, int g, int m) {
    W1FragsBF w;
    f32x4 v[4][2][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float* src = w1g + perm_row(rb, m) * 64 + 32 * hh + 8 * g + 4 * k;
                if constexpr (XC) v[rb][hh][k] = *reinterpret_cast<const f32x4*>(src);
                else v[rb][hh][k] = f32x4{xload(src), xload(src + 1), xload(src + 2), xload(src + 3)};
            }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const f32x4 lo = v[rb][hh][0], hi = v[rb][hh][1];
            u32x4 u{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3])};
            w.f[rb][hh] = as_v8bf(u);
        }
    return w;
}
// The fragments from the bf16 fragment copy (w1_frag_index).
__device__ __forceinline__ W1FragsBF w1_frags_bf_packed(const float* w1g, int lane) {
    W1FragsBF w;
    const u32x4* src = reinterpret_cast<const u32x4*>(w1g) + lane;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) w.f[rb][hh] = as_v8bf(src[(rb * 2 + hh) * 64]);
    return w;
}
struct W1FragsF32 {
    float f[4][16];
};
template <bool XC>
__device__ __forceinline__ W1FragsF32 w1_frags_f32_global(const float* w1g, int g, int m) {
    W1FragsF32 w;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            const float* src = w1g + perm_row(rb, m) * 64 + 16 * hh + 4 * g;
            f32x4 v;
            if constexpr (XC) v = *reinterpret_cast<const f32x4*>(src);
            else v = f32x4{xload(src), xload(src + 1), xload(src + 2), xload(src + 3)};
#pragma unroll
            for (int i = 0; i < 4; ++i) w.f[rb][hh * 4 + i] = v[i];
        }
    return w;
}
__device__ __forceinline__ W1FragsF32 w1_frags_f32(const float* mW, int g, int m) {
    W1FragsF32 w;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int r = perm_row(rb, m);
#pragma unroll
        for (int hh = 0; hh < 4; ++hh)
#pragma unroll
            for (int i = 0; i < 4; ++i) w.f[rb][hh * 4 + i] = mW[r * MP + 16 * hh + 4 * g + i];
    }
    return w;
}

// 16 tokens of Z from the lane's Q fragment q (bf16: channels 32h+8g..+8 of
// token row m for h = 0,1; fp32: channels 16h+4g..+4 for h = 0..3).
__device__ __forceinline__ void apply_bf(const W1FragsBF& w, const u32x4* q, char* zrow, bool ok, int g,
                                         bool poison) {
    v4f d[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        d[rb] = v4f{0.f, 0.f, 0.f, 0.f};
        d[rb] = mfma32(w.f[rb][0], as_v8bf(q[0]), d[rb]);
        d[rb] = mfma32(w.f[rb][1], as_v8bf(q[1]), d[rb]);
        if (poison) d[rb] = v4f{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
    if (ok) {
        u32x4 o0{pack_bf2(d[0][0], d[0][1]), pack_bf2(d[0][2], d[0][3]), pack_bf2(d[1][0], d[1][1]),
                 pack_bf2(d[1][2], d[1][3])};
        u32x4 o1{pack_bf2(d[2][0], d[2][1]), pack_bf2(d[2][2], d[2][3]), pack_bf2(d[3][0], d[3][1]),
                 pack_bf2(d[3][2], d[3][3])};
        // streaming stores: Z is not read again by this kernel
        __builtin_nontemporal_store(o0, reinterpret_cast<u32x4*>(zrow + (8 * g) * 2));
        __builtin_nontemporal_store(o1, reinterpret_cast<u32x4*>(zrow + (32 + 8 * g) * 2));
    }
}
__device__ __forceinline__ void apply_f32(const W1FragsF32& w, const u32x4* q, char* zrow, bool ok, int g,
                                          bool poison) {
    v4f d[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        d[rb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            const f32x4 qv = __builtin_bit_cast(f32x4, q[hh]);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[rb] = mfma4(w.f[rb][hh * 4 + i], qv[i], d[rb]);
        }
        if (poison) d[rb] = v4f{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
    if (ok) {
        float* zr = reinterpret_cast<float*>(zrow);
        __builtin_nontemporal_store(f32x4{d[0][0], d[0][1], d[0][2], d[0][3]}, reinterpret_cast<f32x4*>(zr + 8 * g));
        __builtin_nontemporal_store(f32x4{d[1][0], d[1][1], d[1][2], d[1][3]}, reinterpret_cast<f32x4*>(zr + 8 * g + 4));
        __builtin_nontemporal_store(f32x4{d[2][0], d[2][1], d[2][2], d[2][3]}, reinterpret_cast<f32x4*>(zr + 32 + 8 * g));
        __builtin_nontemporal_store(f32x4{d[3][0], d[3][1], d[3][2], d[3][3]}, reinterpret_cast<f32x4*>(zr + 36 + 8 * g));
    }
}

struct SliceCtx {
    int slice, split, b, h, t0, t1;
    const char *Kp, *Vp, *Qp;
    char* Zp;
    long long Ksn, Vsn, Qsn, Zsn;
};
template <bool BF, bool XC> __device__ __forceinline__ SliceCtx slice_ctx(const LinFwdLaunch& a) {
    constexpr int esz = LinCfg<BF>::esz;
    SliceCtx c;
    const SliceSplit ss = XC ? map_block_xcc(blockIdx.x, a.S, xcc_id()) : map_block(blockIdx.x, a.S, 0);
    c.slice = ss.slice;
    c.split = ss.split;
    c.b = c.slice / a.H;
    c.h = c.slice % a.H;
    const int per = (((a.N + a.S - 1) / a.S) + 15) & ~15;
    c.t0 = min(a.N, c.split * per);
    c.t1 = min(a.N, c.t0 + per);
    c.Kp = (const char*)a.K.ptr + (c.b * a.K.sb + c.h * a.K.sh) * (long long)esz;
    c.Vp = (const char*)a.V.ptr + (c.b * a.V.sb + c.h * a.V.sh) * (long long)esz;
    c.Qp = (const char*)a.Q.ptr + (c.b * a.Q.sb + c.h * a.Q.sh) * (long long)esz;
    c.Zp = (char*)a.Z.ptr + (c.b * a.Z.sb + c.h * a.Z.sh) * (long long)esz;
    c.Ksn = a.K.sn * esz;
    c.Vsn = a.V.sn * esz;
    c.Qsn = a.Q.sn * esz;
    c.Zsn = a.Z.sn * esz;
    return c;
}

__device__ __forceinline__ void load_w0(const LinFwdLaunch& a, int h, f32x4* w0r) {
    const float* W0h = a.W0 + (long long)h * 4096;
#pragma unroll
    for (int k = 0; k < 4; ++k) w0r[k] = *reinterpret_cast<const f32x4*>(W0h + 4 * threadIdx.x + 1024 * k);
}

// Sum the four waves' 26 tiles.  Wave (t % 4) owns tile t: the other
// waves leave their copy in `red` (3 slots per tile, 78 KB), the owner adds
// them to its own in the fixed order ((w0 + w1) + w2) + w3 and writes the
// result as row-major matrices mA / mC (which may overlap `red`: they are
// written after a barrier).
__device__ __forceinline__ void reduce_waves(v4f* accC, v4f* accA, float* red, float* mA, float* mC,
                                             int w, int lane, int g, int m, bool overlap) {
    auto tile_ref = [&](int t) -> v4f& { return t < 16 ? accC[t] : accA[t - 16]; };
    auto slot = [&](int t, int src) { return (t * 3 + (src < (t & 3) ? src : src - 1)) * 256 + lane * 4; };
#pragma unroll
    for (int t = 0; t < 26; ++t)
        if ((t & 3) != w) *reinterpret_cast<v4f*>(red + slot(t, w)) = tile_ref(t);
    lds_barrier();
#pragma unroll
    for (int t = 0; t < 26; ++t) {
        if ((t & 3) == w) {
            v4f parts[4];
#pragma unroll
            for (int src = 0; src < 4; ++src)
                parts[src] = src == w ? tile_ref(t) : *reinterpret_cast<const v4f*>(red + slot(t, src));
            tile_ref(t) = ((parts[0] + parts[1]) + parts[2]) + parts[3];
        }
    }
    if (overlap) lds_barrier(); // mA / mC overlap `red`
#pragma unroll
    for (int t = 0; t < 26; ++t)
        if ((t & 3) == w) write_tile(tile_ref(t), t, mA, mC, g, m);
    lds_barrier();
}

// The owned rows into full row-major [A; C] in LDS (pitch MP).
__device__ __forceinline__ void write_owned(const v4f* accC, const v4f* accA, int w, int lane, float* mA, float* mC) {
    lds_barrier(); // mA / mC overlap the K and V regions other waves read
    const int g = lane >> 4, m = lane & 15;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * g + i, c = 16 * cb + m;
            mC[r * MP + c] = accC[cb][i];
            mA[r * MP + c] = accA[cb][i];
        }
    lds_barrier();
}
// The owned rows straight into this split's partial in the exchange layout
// of lin_update (reducer-major: part[slice][j][split][mat][cc][r] with
// column c = j*nc + cc): a lane's four rows of one column are one 16-byte
// store.
template <bool XC>
__device__ __forceinline__ void publish_owned(const LinFwdLaunch& a, int slice, int split, const v4f* accC,
                                              const v4f* accA, int w, int lane) {
    const int lgnc = 6 - __builtin_ctz(a.S), nc = 1 << lgnc; // S is a power of two
    const long long sb = (long long)slice * a.S * 8192;
    const int g = lane >> 4, m = lane & 15;
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int c = 16 * cb + m, r0 = 16 * w + 4 * g;
            float* dst =
                a.part + sb + ((long long)((c >> lgnc) * a.S + split) * 2 + mat) * 64 * nc + (c & (nc - 1)) * 64 + r0;
            const v4f v = mat ? accC[cb] : accA[cb];
            if constexpr (XC) {
                *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) xstore(dst + i, v[i]);
            }
        }
}


// ------------------------------------------------------- G exchange --
// bf16, XCD-local, when A and G are not wanted: each split publishes
// G_s = W0 A_s - C_s (16 KB) instead of [A_s; C_s] (32 KB), so the
// reducers only add the S partials and apply W1 = W0 - eta (2/N) G
// elementwise.  (G is linear in A and C, so the sum of the G_s is G.)
//
// Publish order of the 4096 entries P = 256 q + e: chunk q = 4 rb + 2 hh
// + jh holds rows perm_row(rb, m') (m' = 0..15) x columns 32 hh + 16 jh +
// cl (cl = 0..15); inside a chunk e = 128 p + 64 gh + 4 cl + i stands for
// m' = 8 p + 4 gh + i.  Wave w's lanes (g, m) hold G rows 16 w + 4 g + i,
// column 16 cb + m, i.e. chunk 8 (w>>1) + 4 (g&1) + cb, p = w&1, gh = g>>1,
// cl = m: one store instruction writes two runs of 512 contiguous bytes
// (whole cache lines, no partial-line traffic).  The W1 fragment pieces of
// chunk q are pieces 32 q .. 32 q + 31.  With R = 4096 / S, reducer j sums
// entries [j R, (j+1) R); split sp stores its part of them at
// part[slice][j][sp][R].
__device__ __forceinline__ void split_bf(const float* v, v8bf& hi, v8bf& lo) {
    u32x4 h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        h[k] = pack_bf2(v[2 * k], v[2 * k + 1]);
        l[k] = pack_bf2(v[2 * k] - bflo(h[k]), v[2 * k + 1] - bfhi(h[k]));
    }
    hi = as_v8bf(h);
    lo = as_v8bf(l);
}
constexpr int kAP = 72; // pitch (bf16) of the A planes
// Byte offset in a kernel's LDS of the exchange outcome (slice_bad),
// written after the last slice barrier: above the phase-2 regions of
// lin_update (gather staging, W0) and the G-phase regions, below the end
// of the K/V regions and of the streaming kernel's LDS.
constexpr int kChkByte = (8192 + 128 + 64 * MP) * 4;
// Group sums of reduce_g (4 KB), right above the G-phase regions.
constexpr int kGSumByte = 4 * 64 * kAP + 64 * MP * 4;
static_assert(kGSumByte + 4096 <= kChkByte, "reduce_g group sums below the exchange outcome");
static_assert(kChkByte >= 4 * 64 * kAP + 64 * MP * 4, "exchange outcome above the G-phase regions");
static_assert(kChkByte + 4 <= 20480 * 4, "exchange outcome inside the streaming kernel's LDS");
// Wave w's rows of G_s from its owned rows of A_s and C_s.  The product
// W0 A runs in bf16 with both factors split hi + lo (the lo x lo term is
// below fp32 rounding) and fp32 accumulation.  A's planes go through LDS:
// lane (g, m) stores its A[16 w + 4 g + i][16 cb + m] as row 16 cb + m,
// columns 16 w + 4 g + i of the planes (A is symmetric); W0 is staged from
// the registers w0r (floats 4 tid + 1024 k of W0[h]).
// LDS layout of the G phase (inside the K and V regions, free after the
// Gram): A's hi and lo planes (bf16, pitch kAP), then W0 (fp32, pitch MP).
struct GLds {
    bf16_t *ahi, *alo;
    float* w0s;
};
__device__ __forceinline__ GLds g_lds(char* lds) {
    GLds L;
    L.ahi = reinterpret_cast<bf16_t*>(lds);
    L.alo = L.ahi + 64 * kAP;
    L.w0s = reinterpret_cast<float*>(lds + 4 * 64 * kAP);
    return L;
}
// Lane (g, m) of wave w (w < 4) stores its A[16 w + 4 g + i][16 cb + m] as
// row 16 cb + m, columns 16 w + 4 g + i of the planes (A is symmetric).
__device__ __forceinline__ void g_write_a(const GLds& L, const v4f* oA, int w, int lane) {
    const int g = lane >> 4, m = lane & 15;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const v4f v = oA[cb];
        const uint32_t h01 = pack_bf2(v[0], v[1]), h23 = pack_bf2(v[2], v[3]);
        const uint32_t l01 = pack_bf2(v[0] - bflo(h01), v[1] - bfhi(h01));
        const uint32_t l23 = pack_bf2(v[2] - bflo(h23), v[3] - bfhi(h23));
        const int off = (16 * cb + m) * kAP + 16 * w + 4 * g;
        *reinterpret_cast<u32x2*>(L.ahi + off) = u32x2{h01, h23};
        *reinterpret_cast<u32x2*>(L.alo + off) = u32x2{l01, l23};
    }
}
// Wave w's rows of G_s = W0 A_s - C_s from the staged planes and W0, stored
// in publish order.
__device__ __forceinline__ void g_rows_store(const LinFwdLaunch& a, int slice, int split, const v4f* oC,
                                             const GLds& L, int w, int lane) {
    const int g = lane >> 4, m = lane & 15;
    v8bf wh[2], wl[2]; // A operand: W0[16 w + m][32 kk + 8 g + (0..7)]
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const float* src = L.w0s + (16 * w + m) * MP + 32 * kk + 8 * g;
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(src), a1 = *reinterpret_cast<const f32x4*>(src + 4);
        const float wv[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        split_bf(wv, wh[kk], wl[kk]);
    }
    v4f G[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) G[cb] = v4f{0.f, 0.f, 0.f, 0.f};
    if (!a.dot) { // (the dot-product loss has no W0 A term)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                // B operand A[32 kk + 8 g + j][16 cb + m] = A[16 cb + m][32 kk + 8 g + j]
                const int off = (16 * cb + m) * kAP + 32 * kk + 8 * g;
                const v8bf bh = as_v8bf(*reinterpret_cast<const u32x4*>(L.ahi + off));
                const v8bf bl = as_v8bf(*reinterpret_cast<const u32x4*>(L.alo + off));
                G[cb] = mfma32(wh[kk], bh, G[cb]);
                G[cb] = mfma32(wh[kk], bl, G[cb]);
                G[cb] = mfma32(wl[kk], bh, G[cb]);
            }
    }
    const int lgS = __builtin_ctz(a.S), lgR = 12 - lgS, R = 1 << lgR;
    const long long sb = (long long)slice * a.S * 4096;
    const int e = 128 * (w & 1) + 64 * (g >> 1) + 4 * m;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const v4f gv = G[cb] - oC[cb];
        const int P = (8 * (w >> 1) + 4 * (g & 1) + cb) * 256 + e;
        float* dst = a.part + sb + (long long)(((P >> lgR) << lgS) + split) * R + (P & (R - 1));
        *reinterpret_cast<f32x4*>(dst) = f32x4{gv[0], gv[1], gv[2], gv[3]};
    }
}
// Four-wave form: w0r holds floats 4 tid + 1024 k of W0[h].
__device__ __forceinline__ void publish_g(const LinFwdLaunch& a, int slice, int split, const v4f* oC,
                                          const v4f* oA, const f32x4* w0r, char* lds, int w, int lane) {
    const int tid = threadIdx.x;
    const GLds L = g_lds(lds);
    lds_barrier(); // the planes overlap the K and V regions other waves read
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = 4 * tid + 1024 * k, r = e >> 6, c = e & 63;
        *reinterpret_cast<f32x4*>(L.w0s + r * MP + c) = w0r[k];
    }
    g_write_a(L, oA, w, lane);
    lds_barrier();
    g_rows_store(a, slice, split, oC, L, w, lane);
}
// Reducer `split`: sum its R = 4096/S entries over the S splits, form
// W1 = W0 - eta (2/N) G and store them as bf16 fragments (w1_frag_index).
// The 256 threads of waves 0-3 (`active`) load: with S >= 8 thread t sums
// float4 t % n4 of the reducer's block over the four splits of group
// t / n4 (split order), and the S/4 group sums meet in LDS (group order);
// with S <= 4 every thread sums its float4s over all splits.  W0 is read
// from w0src (pitch w0p: its staged copy, g_lds, or global memory); the
// group sums use 4 KB of LDS at lds + gsum_byte.  Every wave of the
// workgroup calls this (with S >= 8 it holds one workgroup barrier).
template <int S>
__device__ __forceinline__ void reduce_g(const LinFwdLaunch& a, int slice, int split, int h, char* lds,
                                         bool active, const float* w0src, int w0p, int gsum_byte,
                                         bool reread = false) {
    constexpr int R = 4096 / S, n4 = R / 4;
    constexpr int NG = S >= 8 ? S / 4 : 1; // split groups
    constexpr int SG = S / NG;             // splits per group
    const int tid = threadIdx.x;
    const float eta = a.eta[h];
    const float scale = grad_scale(a);
    const f32x4* blk = reinterpret_cast<const f32x4*>(a.part + (long long)slice * S * 4096 + (long long)split * S * R);
    bf16_t* w1b = reinterpret_cast<bf16_t*>(a.w1 + (long long)slice * 4096);
    // several steps: the new state in fp32 too (row-major), read by every
    // split of the slice for the next step
    float* wk = a.steps > 1 ? a.wk + (long long)slice * 4096 : nullptr;
    auto finish = [&](int t4, const f32x4& acc) __attribute__((always_inline)) {
        const int P = split * R + 4 * t4, q = P >> 8, e = P & 255;
        const int mq = 8 * (e >> 7) + 4 * ((e >> 6) & 1); // m' of the first of four rows
        const int rb = q >> 2, c = 32 * ((q >> 1) & 1) + 16 * (q & 1) + ((e >> 2) & 15), r0 = perm_row(rb, mq);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float wn = w0src[(r0 + i) * w0p + c] - eta * (scale * acc[i]);
            w1b[w1_frag_index(r0 + i, c)] = f2bf(wn);
            if (wk) wk[(r0 + i) * 64 + c] = wn;
        }
    };
    // The partials of a later step sit at the addresses an earlier step's
    // reduce read, whose lines this CU's L1 may still hold: device-scope
    // loads (L2, not L1) for those.
    auto ld = [&](int i) __attribute__((always_inline)) -> f32x4 {
        if (!reread) return blk[i];
        const float* p = reinterpret_cast<const float*>(blk + i);
        return f32x4{xload(p), xload(p + 1), xload(p + 2), xload(p + 3)};
    };
    if constexpr (NG == 1) {
        if (active) {
#pragma unroll
            for (int t4 = tid; t4 < n4; t4 += 256) {
                f32x4 v[S];
#pragma unroll
                for (int sp = 0; sp < S; ++sp) v[sp] = ld(sp * n4 + t4);
                f32x4 acc = v[0];
#pragma unroll
                for (int sp = 1; sp < S; ++sp) acc += v[sp];
                finish(t4, acc);
            }
        }
    } else {
        f32x4* gs = reinterpret_cast<f32x4*>(lds + gsum_byte); // [NG][n4]
        if (active) {
            const int t4 = tid % n4, gq = tid / n4;
            f32x4 v[SG];
#pragma unroll
            for (int k = 0; k < SG; ++k) v[k] = ld((gq * SG + k) * n4 + t4);
            f32x4 acc = v[0];
#pragma unroll
            for (int k = 1; k < SG; ++k) acc += v[k];
            gs[gq * n4 + t4] = acc;
        }
        lds_barrier(); // (waits for no global load: waves 4-7 keep their Q loads in flight)
        if (active && tid < n4) {
            f32x4 acc = gs[tid];
#pragma unroll
            for (int gq = 1; gq < NG; ++gq) acc += gs[gq * n4 + tid];
            finish(tid, acc);
        }
    }
}

// ------------------------------------------------------ resident kernel --
template <bool BF, bool XC>
__global__ __launch_bounds__(kThreads, 1) void lin_fwd_resident(LinFwdLaunch a) {
    using Cfg = LinCfg<BF>;
    constexpr int RS = Cfg::row_slots;
    constexpr int TB = Cfg::tmax * RS * 16; // bytes of one tensor region
    constexpr int SPARE = 16384;            // lets [A; C] sit beside the wave sums
    __shared__ __attribute__((aligned(16))) char lds[3 * TB + SPARE];
    float* ldsf = reinterpret_cast<float*>(lds);
    char* Ks = lds;
    char* Vs = lds + TB;
    char* Qs = lds + 2 * TB + SPARE;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6); // wave index, uniform
    int* const chk = reinterpret_cast<int*>(lds + kChkByte);
    const SliceCtx c = slice_ctx<BF, XC>(a);
    if (c.slice >= a.B * a.H) return; // padding block of the XCD-aware grid
    if (XC && a.S > 1 && tid == 0) placement_note(counter_at(a.cnt, c.slice), c.split);
    const int T = c.t1 - c.t0;

    // ---- every load of the workgroup, issued up front: all of K and V,
    // then all of Q, so K and V land first and Q streams in during the Gram
    // phase.  The Gram phase waits for K and V only.
    f32x4 w0r[4];
    load_w0(a, c.h, w0r);
    int nq = 0; // Q loads of this wave still allowed in flight
    if (T > 0) {
        const int rows = (T + 31) & ~31;
        const int ninstr = rows * RS / 64; // 1 KB per wave instruction
        for (int q = w; q < ninstr; q += 4) {
            const int p = q * 64 + lane;
            const int row = p / RS;
            const int okv = ((p % RS) ^ (BF ? swz_tr(row) : swz_kv<BF>(row))) * 16;
            const long long tok = c.t0 + min(row, T - 1);
            dma16(c.Kp + tok * c.Ksn + okv, Ks + q * 1024);
            dma16(c.Vp + tok * c.Vsn + okv, Vs + q * 1024);
        }
        if (a.Z.ptr) {
            for (int q = w; q < ninstr; q += 4) {
                const int p = q * 64 + lane;
                const int row = p / RS;
                const int oq = ((p % RS) ^ swz_q<BF>(row)) * 16;
                const long long tok = c.t0 + min(row, T - 1);
                dma16(c.Qp + tok * c.Qsn + oq, Qs + q * 1024);
                ++nq;
            }
        }
    }
    vmcnt_at_most(nq); // this wave's K, V (and W0) loads have landed
    __syncthreads();   // ... and every wave's
    // G exchange: bf16, XCD-local, S > 1, A and G not wanted
    const bool gx = BF && XC && a.S > 1 && !a.saved;
    // lines read after the slice barriers, into L2 while the Gram runs
    Prefetch pf{0.f, 0.f};
    if (a.S > 1) pf = exchange_prefetch<BF, XC>(a, c.slice, c.split, gx);
    // rows past the range hold clamped copies: zero them in K and V so the
    // Gram fragments need no masking
    {
        const int rows = (T + 31) & ~31;
        for (int e = tid; e < (rows - T) * RS; e += kThreads) {
            const int off = (T + e / RS) * RS * 16 + (e % RS) * 16;
            *reinterpret_cast<u32x4*>(Ks + off) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(Vs + off) = u32x4{0u, 0u, 0u, 0u};
        }
        lds_barrier();
    }

    // ---- phase 1: Gram blocks.  K/V regions are free afterwards: (fp32)
    // 3 x 26 tiles of wave sums at the bottom, [A; C] right above them; the
    // Q region stays intact for phase 3
    float* mA = ldsf + 3 * 26 * 256;
    float* mC = mA + 64 * MP;
    bool published = false;
    if constexpr (BF) {
        v4f oC[4], oA[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) oC[cb] = oA[cb] = v4f{0.f, 0.f, 0.f, 0.f};
        switch (w) {
        case 0: gram_owned_bf<0>(Ks, Vs, 0, (T + 31) & ~31, lane, oC, oA); break;
        case 1: gram_owned_bf<1>(Ks, Vs, 0, (T + 31) & ~31, lane, oC, oA); break;
        case 2: gram_owned_bf<2>(Ks, Vs, 0, (T + 31) & ~31, lane, oC, oA); break;
        default: gram_owned_bf<3>(Ks, Vs, 0, (T + 31) & ~31, lane, oC, oA); break;
        }
        if (gx) {
            publish_g(a, c.slice, c.split, oC, oA, w0r, lds, w, lane);
            published = true;
        } else if (a.S > 1) {
            publish_owned<XC>(a, c.slice, c.split, oC, oA, w, lane);
            published = true;
        } else {
            write_owned(oC, oA, w, lane, mA, mC);
        }
    } else {
        v4f accC[16], accA[10];
#pragma unroll
        for (int t = 0; t < 16; ++t) accC[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 10; ++t) accA[t] = v4f{0.f, 0.f, 0.f, 0.f};
        constexpr int KS = 16; // tokens per wave k-step
        const GramLanes gl = gram_lanes(g, m);
        for (int r0 = w * KS; r0 < T; r0 += 4 * KS) gram_step<BF>(Ks, Vs, r0, gl, accC, accA, g, m);
        lds_barrier();
        reduce_waves(accC, accA, ldsf, mA, mC, w, lane, g, m, false);
    }

    // ---- phase 2
    float* W1 = nullptr;
    SliceWords sw{}; // thread 0, after the last slice barrier
    if (gx) {
        unsigned* cnt = counter_at(a.cnt, c.slice);
        slice_barrier(cnt, (unsigned)a.S + a.tbias, true, a.spin);
        const float* w0g = g_lds(lds).w0s;
        switch (a.S) {
        case 2: reduce_g<2>(a, c.slice, c.split, c.h, lds, true, w0g, MP, kGSumByte); break;
        case 4: reduce_g<4>(a, c.slice, c.split, c.h, lds, true, w0g, MP, kGSumByte); break;
        case 8: reduce_g<8>(a, c.slice, c.split, c.h, lds, true, w0g, MP, kGSumByte); break;
        case 16: reduce_g<16>(a, c.slice, c.split, c.h, lds, true, w0g, MP, kGSumByte); break;
        default: reduce_g<32>(a, c.slice, c.split, c.h, lds, true, w0g, MP, kGSumByte); break;
        }
        slice_barrier(cnt, 2u * a.S + a.tbias, true, a.spin);
        if (tid == 0) sw = slice_words(cnt);
        keep_alive(pf);
    } else {
        W1 = lin_update<BF, XC>(a, c.slice, c.split, c.h, ldsf, mA, mC, ldsf, ldsf + 8192 + 128, w0r, &sw,
                                published, pf);
    }

    // ---- phase 3: Z from the resident Q region (skipped when only A and G
    // are wanted); W1's fragments are loaded while the exchange outcome and
    // every wave's Q loads (normally long since landed) are waited for
    const int nsteps = (T + 15) / 16;
    const float* w1g = a.w1 + (long long)c.slice * 4096;
    if constexpr (BF) {
        const W1FragsBF wf = W1   ? w1_frags_bf(W1, g, m)
                             : XC ? w1_frags_bf_packed(w1g, lane)
                                  : w1_frags_bf_global<XC>(w1g, g, m);
        const bool poison = exchange_outcome<XC>(a, c.slice, c.split, sw, chk, kThreads);
        if (!a.Z.ptr) {
            release_end(a, c.slice, release_begin(a, c.slice));
            return;
        }
        const unsigned rel = release_begin(a, c.slice);
#pragma unroll 2
        for (int step = w; step < nsteps; step += 4) {
            const int row = step * 16 + m;
            u32x4 q[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                q[hh] = *reinterpret_cast<const u32x4*>(Qs + (row * 8 + ((4 * hh + g) ^ swz_q<true>(row))) * 16);
            apply_bf(wf, q, c.Zp + (long long)(c.t0 + row) * c.Zsn, row < T, g, poison);
        }
        release_end(a, c.slice, rel);
    } else {
        const W1FragsF32 wf = W1 ? w1_frags_f32(W1, g, m) : w1_frags_f32_global<XC>(w1g, g, m);
        const bool poison = exchange_outcome<XC>(a, c.slice, c.split, sw, chk, kThreads);
        if (!a.Z.ptr) {
            release_end(a, c.slice, release_begin(a, c.slice));
            return;
        }
        const unsigned rel = release_begin(a, c.slice);
        for (int step = w; step < nsteps; step += 4) {
            const int row = step * 16 + m;
            u32x4 q[4];
#pragma unroll
            for (int hh = 0; hh < 4; ++hh)
                q[hh] = *reinterpret_cast<const u32x4*>(Qs + (row * 16 + ((4 * hh + g) ^ swz_q<false>(row))) * 16);
            apply_f32(wf, q, c.Zp + (long long)(c.t0 + row) * c.Zsn, row < T, g, poison);
        }
        release_end(a, c.slice, rel);
    }
}

// ------------------------------------- resident kernel, G exchange --
// The bf16 XCD-local case without saved A and G (the common one) with 8
// waves, two per SIMD, so one wave's LDS reads overlap the other's matrix
// products.  Waves 0-3 accumulate C_s, waves 4-7 A_s (rows 16 (w % 4)..
// each); the first four form and publish G_s, and all eight share the
// apply.
constexpr int kThreads8 = 512;
constexpr int kGxLds = 3 * LinCfg<true>::tmax * 8 * 16 + 16384; // K, V, spare, Q

// LDS map of the body: K [0, TB), V [TB, 2 TB), Q [2 TB + 16 KB, 3 TB + 16 KB);
// the G phase in [0, 35840) (g_lds); the reduce's group sums (4 KB) at
// gsum_byte and the exchange outcome at chk_byte, both outside Q and the
// G phase.  w0_lds: the reduce reads W0 from its staged copy (else from
// global memory).
template <bool STEPS> // STEPS: the launch may take several full-batch steps (a.steps > 1)
__device__ __forceinline__ void lin_gx_body(const LinFwdLaunch& a, char* lds, int gsum_byte, int chk_byte,
                                            bool w0_lds) {
    using Cfg = LinCfg<true>;
    constexpr int RS = Cfg::row_slots;
    constexpr int TB = Cfg::tmax * RS * 16;
    constexpr int SPARE = 16384;
    char* Ks = lds;
    char* Vs = lds + TB;
    char* Qs = lds + 2 * TB + SPARE;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6); // wave index 0..7, uniform
    int* const chk = reinterpret_cast<int*>(lds + chk_byte);
    const SliceCtx c = slice_ctx<true, true>(a);
    if (c.slice >= a.B * a.H) return; // padding block of the XCD-aware grid
    if (tid == 0) placement_note(counter_at(a.cnt, c.slice), c.split);
    const int T = c.t1 - c.t0;

    // ---- loads: W0 (floats 4 tid + 2048 k) and all of K and V now; Q is
    // loaded by waves 4-7 after the Gram, while the exchange leaves HBM idle
    f32x4 w0r[2];
    {
        const float* W0h = a.W0 + (long long)c.h * 4096;
#pragma unroll
        for (int k = 0; k < 2; ++k) w0r[k] = *reinterpret_cast<const f32x4*>(W0h + 4 * tid + 2048 * k);
    }
    const int rows = (T + 31) & ~31;
    const int ninstr = rows * RS / 64; // 1 KB per wave instruction
    for (int q = w; q < ninstr; q += 8) {
        const int p = q * 64 + lane;
        const int row = p / RS;
        const int okv = ((p % RS) ^ swz_tr(row)) * 16;
        const long long tok = c.t0 + min(row, T - 1);
        dma16(c.Kp + tok * c.Ksn + okv, Ks + q * 1024);
        dma16(c.Vp + tok * c.Vsn + okv, Vs + q * 1024);
    }
    drain_vmem(); // this wave's K, V (and W0) loads have landed
    // W0 counts as arrived from here on: no later wait for it (which would
    // also wait for the Q loads issued after the Gram)
    asm volatile("" ::"v"(w0r[0]), "v"(w0r[1]));
    __syncthreads(); // ... and every wave's loads have landed
    Prefetch pf{0.f, 0.f};
    if (w < 4) pf = exchange_prefetch<true, true>(a, c.slice, c.split, true);
    for (int e = tid; e < (rows - T) * RS; e += kThreads8) { // zero the clamped rows
        const int off = (T + e / RS) * RS * 16 + (e % RS) * 16;
        *reinterpret_cast<u32x4*>(Ks + off) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(Vs + off) = u32x4{0u, 0u, 0u, 0u};
    }
    lds_barrier();

    // ---- phase 1: waves 0-3 accumulate rows 16 w.. of C and of A over all
    // of the split's tokens (each K fragment read serves both products:
    // fewer LDS reads than C and A on separate waves); waves 4-7 wait
    v4f oC[4], oA[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) oC[cb] = oA[cb] = v4f{0.f, 0.f, 0.f, 0.f};
    if (w >= 4 && a.Z.ptr) {
        // Q, by the waves that neither take part in the Gram nor publish or
        // reduce (their loads stay in flight across the slice barriers),
        // issued as the Gram starts: HBM is idle from here to the apply
        for (int q = w - 4; q < ninstr; q += 4) {
            const int p = q * 64 + lane;
            const int row = p / RS;
            const int oq = ((p % RS) ^ swz_q<true>(row)) * 16;
            const long long tok = c.t0 + min(row, T - 1);
            dma16(c.Qp + tok * c.Qsn + oq, Qs + q * 1024);
        }
    }
    switch (w) {
    case 0: gram_owned_bf<0>(Ks, Vs, 0, rows, lane, oC, oA); break;
    case 1: gram_owned_bf<1>(Ks, Vs, 0, rows, lane, oC, oA); break;
    case 2: gram_owned_bf<2>(Ks, Vs, 0, rows, lane, oC, oA); break;
    case 3: gram_owned_bf<3>(Ks, Vs, 0, rows, lane, oC, oA); break;
    default: break;
    }
    // A's owners write its planes, W0 is staged, then the same waves form
    // and publish their rows of G_s
    const GLds L = g_lds(lds);
    lds_barrier(); // every Gram is done with K and V
    if (w < 4) g_write_a(L, oA, w, lane);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e = 4 * tid + 2048 * k, r = e >> 6, cc = e & 63;
        *reinterpret_cast<f32x4*>(L.w0s + r * MP + cc) = w0r[k];
    }
    lds_barrier();
    if (w < 4) g_rows_store(a, c.slice, c.split, oC, L, w, lane);

    // ---- phase 2: reduce this workgroup's block of G, W1 as bf16 fragments
    unsigned* cnt = counter_at(a.cnt, c.slice);
    slice_barrier(cnt, (unsigned)a.S + a.tbias, w < 4, a.spin);
    // waves 0-3 reduce (waves 4-7 have Q loads in flight, which a gather of
    // theirs would queue behind)
    const float* w0src = w0_lds ? L.w0s : a.W0 + (long long)c.h * 4096;
    const int w0p = w0_lds ? MP : 64;
    auto reduce = [&](const float* wsrc, int wp, bool reread) __attribute__((always_inline)) {
        switch (a.S) {
        case 2: reduce_g<2>(a, c.slice, c.split, c.h, lds, w < 4, wsrc, wp, gsum_byte, reread); break;
        case 4: reduce_g<4>(a, c.slice, c.split, c.h, lds, w < 4, wsrc, wp, gsum_byte, reread); break;
        case 8: reduce_g<8>(a, c.slice, c.split, c.h, lds, w < 4, wsrc, wp, gsum_byte, reread); break;
        case 16: reduce_g<16>(a, c.slice, c.split, c.h, lds, w < 4, wsrc, wp, gsum_byte, reread); break;
        default: reduce_g<32>(a, c.slice, c.split, c.h, lds, w < 4, wsrc, wp, gsum_byte, reread); break;
        }
    };
    reduce(w0src, w0p, false);
    slice_barrier(cnt, 2u * a.S + a.tbias, w < 4, a.spin);
    // ---- further full-batch steps (the epochs of the inner training):
    // W_{k+1} = W_k - eta (2/N) (W_k A - C).  A_s (its planes in LDS) and
    // C_s (oC) of the split stay where the first step left them, so each
    // step is one more exchange: stage W_k over W0, publish
    // G_s = W_k A_s - C_s, reduce into W_{k+1}.  Lines read again within
    // the launch (W_k, the partials) are read with device-scope loads.
    for (int k = 1; STEPS && k < a.steps; ++k) {
        lds_barrier(); // the reduce is done with the staged state
        const float* wsrc = a.wk + (long long)c.slice * 4096;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int e = 4 * tid + 2048 * k2, r = e >> 6, cc = e & 63;
            const f32x4 v{xload(wsrc + e), xload(wsrc + e + 1), xload(wsrc + e + 2), xload(wsrc + e + 3)};
            *reinterpret_cast<f32x4*>(L.w0s + r * MP + cc) = v;
        }
        lds_barrier();
        if (w < 4) g_rows_store(a, c.slice, c.split, oC, L, w, lane);
        slice_barrier(cnt, (2u * k + 1u) * a.S + a.tbias, w < 4, a.spin);
        reduce(L.w0s, MP, true);
        slice_barrier(cnt, (2u * k + 2u) * a.S + a.tbias, w < 4, a.spin);
    }
    keep_alive(pf);
    // W1's fragments load while every wave's Q loads (normally long since
    // landed) and the exchange outcome are waited for; the counter line's
    // words after them (results return in issue order, and that line is
    // still contended by the slice's polls and releases)
    const W1FragsBF wf = w1_frags_bf_packed(a.w1 + (long long)c.slice * 4096, lane);
    SliceWords sw{};
    if (tid == 0) sw = slice_words(cnt);
    const bool poison = exchange_outcome<true>(a, c.slice, c.split, sw, chk, kThreads8);

    // ---- phase 3: Z from the resident Q region
    if (!a.Z.ptr) {
        release_end(a, c.slice, release_begin(a, c.slice));
        return;
    }
    const int nsteps = (T + 15) / 16;
    const unsigned rel = release_begin(a, c.slice);
    for (int step = w; step < nsteps; step += 8) {
        const int row = step * 16 + m;
        u32x4 q[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            q[hh] = *reinterpret_cast<const u32x4*>(Qs + (row * 8 + ((4 * hh + g) ^ swz_q<true>(row))) * 16);
        apply_bf(wf, q, c.Zp + (long long)(c.t0 + row) * c.Zsn, row < T, g, poison);
    }
    release_end(a, c.slice, rel);
}
static_assert(4 * 64 * kAP + 64 * MP * 4 <= 2 * LinCfg<true>::tmax * 8 * 16, "G-phase LDS inside the K/V regions");

template <bool STEPS>
__global__ __launch_bounds__(kThreads8, 1) void lin_fwd_resident_gx(LinFwdLaunch a) {
    __shared__ __attribute__((aligned(16))) char lds[kGxLds];
    lin_gx_body<STEPS>(a, lds, kGSumByte, kChkByte, true);
}

// ------------------------------------------------------ fused layer --
// The linear heads (lin_gx_body) and the depthwise-conv heads (conv_body,
// one tile per workgroup) of one layer in one launch.  Workgroup i does
// the linear split of virtual block i, then the conv split of the same
// block (both XCD-local exchanges): one launch instead of two, and a
// workgroup's conv work starts as soon as its linear work is done.  (Its
// conv loads cannot usefully start earlier: issued during the linear
// exchange they held up its barrier polls and gathers, whose results
// return behind them; issued during the linear apply, their issue stalled
// it.  Both measured slower than this order.)  LDS map: the linear
// kernel's, then conv w0 + K + V [0, ckv); at ckv the linear reduce's
// group sums and exchange outcome, later the conv's wave sums, w1 and
// outcome; the conv Q halo at the top once the linear apply is done.
struct LayerArgs {
    LinFwdLaunch lin;
    ConvArgs conv;
    int ckv; // conv_kv_bytes of the conv tile
};
constexpr int kLayerScratch = (kRedFloats + 576) * 4 + 256; // conv wave sums, w1, outcome
static_assert(4096 + 256 <= kLayerScratch, "linear group sums and outcome inside the layer scratch");

__global__ __launch_bounds__(kThreads8, 1) void layer_fused(LayerArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kGxLds];
    const int ckv = a.ckv;
    float* scratch = reinterpret_cast<float*>(lds + ckv);
    const ConvLds CL{lds, lds + kGxLds - conv_q_bytes<true>(a.conv.R, a.conv.TW), scratch, scratch + kRedFloats,
                     reinterpret_cast<int*>(scratch + kRedFloats + 576)};
    lin_gx_body<false>(a.lin, lds, ckv, ckv + 4096, true);
    lds_barrier(); // the linear apply is done with its Q rows
    conv_body<true, true>(a.conv, CL);
}

// Fusable: the linear heads take lin_fwd_resident_gx, the conv heads one
// tile per workgroup over an XCD-local exchange, and the LDS map fits.
bool layer_fusable(const LinFwdLaunch& l, int resident, const ConvArgs& c, int cbf16) {
    using Cfg = LinCfg<true>;
    constexpr int lin_q = 2 * Cfg::tmax * 8 * 16 + 16384; // start of the linear Q rows
    if (!(resident && l.xcd && l.bf16 && l.S > 1 && !l.saved && l.Z.ptr)) return false;
    if (!(cbf16 && c.xcd && c.S > 1 && c.tpw == 1 && c.Z.ptr)) return false;
    const int ckv = conv_kv_bytes<true>(c.R, c.TW), cq = conv_q_bytes<true>(c.R, c.TW);
    return ckv % 16 == 0 && ckv + kLayerScratch <= lin_q && ckv + kLayerScratch <= kGxLds - cq;
}

// resident kernel, floats below the Q region: wave sums + [A; C] (phase 1),
// gather staging / W0 / W1 (phase 2)
static_assert(3 * 26 * 256 + 2 * 64 * MP <= (2 * LinCfg<true>::tmax * 8 * 16 + 16384) / 4, "resident LDS (bf16)");
static_assert(3 * 26 * 256 + 2 * 64 * MP <= (2 * LinCfg<false>::tmax * 16 * 16 + 16384) / 4, "resident LDS (fp32)");
static_assert(8192 + 128 + 64 * MP <= 3 * 26 * 256, "phase-2 regions below [A; C]");

// ----------------------------------------------------- streaming kernel --
constexpr int kStages = 3;         // K/V tiles in flight (registers)
constexpr int kQRing = 8;          // apply steps whose Q rows are in flight per wave
constexpr int kStageBytes = 32768; // K tile + V tile

template <bool BF, bool XC>
__global__ __launch_bounds__(kThreads, 1) void lin_fwd_stream(LinFwdLaunch a) {
    using Cfg = LinCfg<BF>;
    // 64 KB of double-buffered K/V tiles during phase 1; the 78 KB of wave
    // sums need the rest afterwards
    __shared__ __attribute__((aligned(16))) float lds[20480]; // 80 KB
    char* ldsb = reinterpret_cast<char*>(lds);

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6); // wave index, uniform
    int* const chk = reinterpret_cast<int*>(ldsb + kChkByte);
    const SliceCtx c = slice_ctx<BF, XC>(a);
    if (c.slice >= a.B * a.H) return; // padding block of the XCD-aware grid
    if (XC && a.S > 1 && tid == 0) placement_note(counter_at(a.cnt, c.slice), c.split);
    const int t0 = c.t0, t1 = c.t1;

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
            r[j] = *reinterpret_cast<const u32x4*>(c.Kp + (long long)(tb + row) * c.Ksn + off);
            r[4 + j] = *reinterpret_cast<const u32x4*>(c.Vp + (long long)(tb + row) * c.Vsn + off);
        }
    };
    // rows past the range (clamped copies) are stored as zeros
    auto store_tile = [&](const u32x4* r, char* st, int nvalid) __attribute__((always_inline)) {
        const u32x4 z{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = j * kThreads + tid;
            const int row = p / Cfg::row_slots;
            const int slot = row * Cfg::row_slots + ((p % Cfg::row_slots) ^ swz_kv<BF>(row));
            const bool ok = row < nvalid;
            *reinterpret_cast<u32x4*>(st + slot * 16) = ok ? r[j] : z;
            *reinterpret_cast<u32x4*>(st + 16384 + slot * 16) = ok ? r[4 + j] : z;
        }
    };

    if (ntiles > 0) {
#pragma unroll
        for (int s = 0; s < kStages; ++s) load_tile(min(s, ntiles - 1), R[s]);
    }
    // Prefetch this wave's first Q steps (16 tokens each, steps w, w+4, ...);
    // rows are clamped into the range, so the loads are unconditional.
    const int nsteps = (t1 - t0 + 15) / 16;
    constexpr int QV = BF ? 2 : 4; // 16-byte loads per lane per step
    // this wave's k-th apply step (tokens t0 + 16 (w + 4 k) ..), clamped
    // into the range so that the load is unconditional
    auto qload = [&](int k, u32x4* q) __attribute__((always_inline)) {
        const int tok = min(t0 + (w + 4 * k) * 16 + m, t1 - 1);
#pragma unroll
        for (int hh = 0; hh < QV; ++hh) {
            const int ch = BF ? (32 * hh + 8 * g) : (16 * hh + 4 * g);
            q[hh] = *reinterpret_cast<const u32x4*>(c.Qp + tok * c.Qsn + ch * Cfg::esz);
        }
    };
    u32x4 qpre[Cfg::qpre][QV];
    if (ntiles > 0 && a.Z.ptr) {
#pragma unroll
        for (int k = 0; k < Cfg::qpre; ++k) qload(k, qpre[k]);
    }
    f32x4 w0r[4];
    load_w0(a, c.h, w0r);

    // Pipelined tile loop: tile it is written from its registers into LDS
    // buffer it&1, the registers are refilled with tile it+3, then the
    // waves consume the buffer (one LDS barrier per tile).  Every load is
    // unconditional inside the main loop and the first loads are clamped
    // duplicates for short ranges, so the compiler's load counters stay
    // exact and three tiles remain in flight.
    const GramLanes gl = gram_lanes(g, m);
    auto step = [&](int it, u32x4* r, bool reload) __attribute__((always_inline)) {
        char* st = ldsb + (it & 1) * kStageBytes;
        store_tile(r, st, t1 - (t0 + it * Cfg::tile));
        lds_barrier();
        if (reload) load_tile(it + kStages, r);
        constexpr int KS = BF ? 32 : 16;
        gram_step<BF>(st, st + 16384, w * KS, gl, accC, accA, g, m);
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
    // the apply's first Q rows load during the update, while HBM is idle
    // (Q is a valid view even when no Z is wanted)
    u32x4 qr[kQRing][QV];
#pragma unroll
    for (int u = 0; u < kQRing; ++u) qload(Cfg::qpre + u, qr[u]);
    lds_barrier();
    // staging buffers are free: wave sums, then [A; C] over them (wave 0
    // reads every sum before it writes the matrices)
    float* mA = lds;
    float* mC = lds + 64 * MP;
    reduce_waves(accC, accA, lds, mA, mC, w, lane, g, m, true);

    SliceWords sw{}; // thread 0, after the last slice barrier
    float* W1 = lin_update<BF, XC>(a, c.slice, c.split, c.h, lds, mA, mC, lds + 128 * MP, lds + 8192 + 128, w0r, &sw);

    const float* w1g = a.w1 + (long long)c.slice * 4096;
    if constexpr (BF) {
        const W1FragsBF wf = W1   ? w1_frags_bf(W1, g, m)
                             : XC ? w1_frags_bf_packed(w1g, lane)
                                  : w1_frags_bf_global<XC>(w1g, g, m);
        // (one split: no exchange, and every load here is the compiler's,
        // so there is nothing to drain)
        const bool poison = a.S > 1 ? exchange_outcome<XC>(a, c.slice, c.split, sw, chk, kThreads) : false;
        if (!a.Z.ptr) { // only A and G wanted
            release_end(a, c.slice, release_begin(a, c.slice));
            return;
        }
        const unsigned rel = release_begin(a, c.slice);
#pragma unroll
        for (int k = 0; k < Cfg::qpre; ++k) {
            const int st = w + 4 * k;
            const int tok = t0 + st * 16 + m;
            if (st < nsteps) apply_bf(wf, qpre[k], c.Zp + (long long)tok * c.Zsn, tok < t1, g, poison);
        }
        for (int k0 = Cfg::qpre; w + 4 * k0 < nsteps; k0 += kQRing) {
#pragma unroll
            for (int u = 0; u < kQRing; ++u) {
                const int st = w + 4 * (k0 + u);
                const int tok = t0 + st * 16 + m;
                if (st < nsteps) apply_bf(wf, qr[u], c.Zp + (long long)tok * c.Zsn, tok < t1, g, poison);
                qload(k0 + u + kQRing, qr[u]);
            }
        }
        release_end(a, c.slice, rel);
    } else {
        const W1FragsF32 wf = W1 ? w1_frags_f32(W1, g, m) : w1_frags_f32_global<XC>(w1g, g, m);
        // (one split: no exchange, and every load here is the compiler's,
        // so there is nothing to drain)
        const bool poison = a.S > 1 ? exchange_outcome<XC>(a, c.slice, c.split, sw, chk, kThreads) : false;
        if (!a.Z.ptr) { // only A and G wanted
            release_end(a, c.slice, release_begin(a, c.slice));
            return;
        }
        const unsigned rel = release_begin(a, c.slice);
#pragma unroll
        for (int k = 0; k < Cfg::qpre; ++k) {
            const int st = w + 4 * k;
            const int tok = t0 + st * 16 + m;
            if (st < nsteps) apply_f32(wf, qpre[k], c.Zp + (long long)tok * c.Zsn, tok < t1, g, poison);
        }
        for (int k0 = Cfg::qpre; w + 4 * k0 < nsteps; k0 += kQRing) {
#pragma unroll
            for (int u = 0; u < kQRing; ++u) {
                const int st = w + 4 * (k0 + u);
                const int tok = t0 + st * 16 + m;
                if (st < nsteps) apply_f32(wf, qr[u], c.Zp + (long long)tok * c.Zsn, tok < t1, g, poison);
                qload(k0 + u + kQRing, qr[u]);
            }
        }
        release_end(a, c.slice, rel);
    }
}

// ------------------------------------------------ several full-batch steps --
// E gradient steps over the whole token set (the ViT3 article, observation
// 2: more inner epochs).  A and C do not change between steps, so with
// G0 = G(W0) the gradient at any W is G0 + (2/N) (W - W0) A (L2), or G0
// (dot-product loss).  Per slice, from A and G0 saved by the forward's Gram
// pass: W_1 = W0 - eta G0, W_{e+1} = W_e - eta (G0 + (2/N)(W_e - W0) A).
// fp32 throughout; thread t owns rows 4 (t / 16).., columns 4 (t % 16)...
__global__ __launch_bounds__(kThreads) void lin_epochs(LinEpochArgs a) {
    __shared__ __attribute__((aligned(16))) float W0s[64 * MP];
    __shared__ __attribute__((aligned(16))) float As[64 * MP];
    __shared__ __attribute__((aligned(16))) float Ds[64 * MP]; // W_e - W0
    const int slice = blockIdx.x, tid = threadIdx.x, h = slice % a.H;
    const float eta = a.eta[h];
    const float beta = 2.0f * eta / (float)a.N;
    const float* A = a.saved + (long long)slice * 8192;
    const float* G0 = A + 4096;
    const float* W0 = a.W0 + (long long)h * 4096;
    const int r0 = (tid >> 4) * 4, c0 = (tid & 15) * 4;
    // every load (W0, A and this thread's G0 block, as float4s) in flight
    // before the first use
    static_assert(1024 % kThreads == 0, "whole float4s per thread");
    constexpr int n4 = 1024 / kThreads;
    f32x4 wv[n4], av[n4], gq[4];
#pragma unroll
    for (int k = 0; k < n4; ++k) {
        const int q = tid + kThreads * k;
        wv[k] = reinterpret_cast<const f32x4*>(W0)[q];
        av[k] = reinterpret_cast<const f32x4*>(A)[q];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) gq[i] = *reinterpret_cast<const f32x4*>(G0 + (r0 + i) * 64 + c0);
#pragma unroll
    for (int k = 0; k < n4; ++k) {
        const int q = tid + kThreads * k, r = q >> 4, c4 = (q & 15) * 4;
        *reinterpret_cast<f32x4*>(W0s + r * MP + c4) = wv[k];
        *reinterpret_cast<f32x4*>(As + r * MP + c4) = av[k];
    }
    float g0[4][4], w[4][4];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            g0[i][k] = gq[i][k];
            w[i][k] = W0s[(r0 + i) * MP + c0 + k] - eta * g0[i][k];
        }
    for (int e = 1; e < a.steps; ++e) {
        if (a.dot) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k) w[i][k] -= eta * g0[i][k];
            continue;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) Ds[(r0 + i) * MP + c0 + k] = w[i][k] - W0s[(r0 + i) * MP + c0 + k];
        __syncthreads();
        float t[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) t[i][k] = 0.f;
#pragma unroll 4
        for (int j = 0; j < 64; ++j) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(As + j * MP + c0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float dv = Ds[(r0 + i) * MP + j];
#pragma unroll
                for (int k = 0; k < 4; ++k) t[i][k] = fmaf(dv, av[k], t[i][k]);
            }
        }
        __syncthreads(); // Ds is rewritten by the next step
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) w[i][k] -= eta * g0[i][k] + beta * t[i][k];
    }
    float* out = a.WE + (long long)slice * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(out + (r0 + i) * 64 + c0) = f32x4{w[i][0], w[i][1], w[i][2], w[i][3]};
}

// Per-slice 64x64 weights staged into LDS (pitch MP) for the fragment helpers.
__device__ __forceinline__ void stage_mat(float* dst, const float* src) {
    static_assert(1024 % kThreads == 0, "whole float4s per thread");
    constexpr int n = 1024 / kThreads;
    f32x4 v[n]; // every load in flight before the first LDS store
#pragma unroll
    for (int k = 0; k < n; ++k) {
        const int e = threadIdx.x + kThreads * k, r = e >> 4, c4 = (e & 15) * 4;
        v[k] = *reinterpret_cast<const f32x4*>(src + r * 64 + c4);
    }
#pragma unroll
    for (int k = 0; k < n; ++k) {
        const int e = threadIdx.x + kThreads * k, r = e >> 4, c4 = (e & 15) * 4;
        *reinterpret_cast<f32x4*>(dst + r * MP + c4) = v[k];
    }
}

// The lane's operand fragment of token row `row` (bf16: channels 32 h + 8 g
// .. +8 for h = 0, 1; fp32: channels 16 h + 4 g .. +4 for h = 0..3), zeros
// past the last token: loaded unconditionally from a row clamped into the
// range and zeroed after the load (a branch around the load would make the
// compiler wait for every load in flight at the join, so the loads of
// several steps could not be in flight together).
template <bool BF>
__device__ __forceinline__ void row_frags_masked(const char* base, long long sn, int row, int N, int g, u32x4* q) {
    constexpr int nh = BF ? 2 : 4;
    const unsigned keep = row < N ? ~0u : 0u;
    const char* r = base + (long long)min(row, N - 1) * sn;
#pragma unroll
    for (int hh = 0; hh < nh; ++hh) {
        const int ch = BF ? 32 * hh + 8 * g : 16 * hh + 4 * g;
        const u32x4 x = *reinterpret_cast<const u32x4*>(r + ch * (BF ? 2 : 4));
        q[hh] = u32x4{x[0] & keep, x[1] & keep, x[2] & keep, x[3] & keep};
    }
}

// Z = Q W^T for per-slice weights W (fp32 [slices][64][64]): 256 tokens per
// workgroup, 16-token steps per wave on the matrix cores.
template <bool BF>
__global__ __launch_bounds__(kThreads) void lin_apply(LinApplyArgs a) {
    __shared__ __attribute__((aligned(16))) float mW[64 * MP];
    constexpr int esz = BF ? 2 : 4;
    const int nb = (a.N + 255) / 256;
    const int slice = blockIdx.x / nb, tb = blockIdx.x % nb;
    const int b = slice / a.H, h = slice % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15, w = tid >> 6;
    const char* Qp = (const char*)a.Q.ptr + (b * a.Q.sb + h * a.Q.sh) * (long long)esz;
    char* Zp = (char*)a.Z.ptr + (b * a.Z.sb + h * a.Z.sh) * (long long)esz;
    const long long Qsn = a.Q.sn * esz, Zsn = a.Z.sn * esz;
    // every step's Q rows are loaded first, W while they are in flight
    constexpr int nh = BF ? 2 : 4;
    u32x4 q[4][nh];
#pragma unroll
    for (int st = 0; st < 4; ++st) row_frags_masked<BF>(Qp, Qsn, tb * 256 + w * 64 + st * 16 + m, a.N, g, q[st]);
    stage_mat(mW, a.W + (long long)slice * 4096);
    __syncthreads();
    if constexpr (BF) {
        const W1FragsBF wf = w1_frags_bf(mW, g, m);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int row = tb * 256 + w * 64 + st * 16 + m;
            apply_bf(wf, q[st], Zp + (long long)row * Zsn, row < a.N, g, false);
        }
    } else {
        const W1FragsF32 wf = w1_frags_f32(mW, g, m);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int row = tb * 256 + w * 64 + st * 16 + m;
            apply_f32(wf, q[st], Zp + (long long)row * Zsn, row < a.N, g, false);
        }
    }
}

// ------------------------------------------------ gradient magnitude map --
// Per token, the Frobenius norm of its own gradient at W0 (the Vision-TTT
// notes' gradient magnitude map).  The gradient is rank one, so
// ||G_t||_F = 2 ||W0 k_t - v_t|| ||k_t|| (L2) or ||v_t|| ||k_t|| (dot-
// product loss).  W0 k_t on the matrix cores (bf16 inputs: W0 rounded to
// bf16 like the apply's W1; fp32 inputs: fp32 products); lane (g, m) holds
// 16 of token m's channels, the four lane groups add their squares.
// tokens per workgroup (four waves, kGmmSt 16-token steps each).  Many
// small workgroups spread evenly over the CUs: on the 1248x1248 linear heads
// 64 tokens (1536 workgroups) took 7.1 us, 128 tokens 7.5 us, 256 tokens
// (384 workgroups, half the CUs holding two) 8.4-10.8 us.
constexpr int kGmmSt = 1, kGmmTok = 4 * 16 * kGmmSt;
template <bool BF>
__global__ __launch_bounds__(kThreads) void lin_gmm(LinGmmArgs a) {
    __shared__ __attribute__((aligned(16))) float mW[64 * MP];
    constexpr int esz = BF ? 2 : 4;
    const int nb = (a.N + kGmmTok - 1) / kGmmTok;
    const int slice = blockIdx.x / nb, tb = blockIdx.x % nb;
    const int b = slice / a.H, h = slice % a.H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, m = lane & 15, w = tid >> 6;
    const char* Kp = (const char*)a.K.ptr + (b * a.K.sb + h * a.K.sh) * (long long)esz;
    const char* Vp = (const char*)a.V.ptr + (b * a.V.sb + h * a.V.sh) * (long long)esz;
    const long long Ksn = a.K.sn * esz, Vsn = a.V.sn * esz;
    float* out = a.out + (long long)slice * a.N;
    auto finish = [&](int row, float kk, float rr) __attribute__((always_inline)) {
        kk += __shfl_xor(kk, 16);
        kk += __shfl_xor(kk, 32);
        rr += __shfl_xor(rr, 16);
        rr += __shfl_xor(rr, 32);
        if (g == 0 && row < a.N) out[row] = (a.dot ? 1.0f : 2.0f) * sqrtf(rr) * sqrtf(kk);
    };
    // every step's K and V rows are loaded first, W0 while they are in flight
    // (branch-free: clamped rows, zeroed past N)
    constexpr int nh = BF ? 2 : 4;
    u32x4 kq[kGmmSt][nh], vq[kGmmSt][nh];
#pragma unroll
    for (int st = 0; st < kGmmSt; ++st) {
        const int row = tb * kGmmTok + w * (16 * kGmmSt) + st * 16 + m;
        row_frags_masked<BF>(Kp, Ksn, row, a.N, g, kq[st]);
        // v at the lane's output channels 8 g .. 8 g + 7 and 32 + 8 g .. +7
        const unsigned keep = row < a.N ? ~0u : 0u;
        const char* vr = Vp + (long long)min(row, a.N - 1) * Vsn;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int ch = 32 * half + 8 * g;
#pragma unroll
            for (int p = 0; p < nh / 2; ++p) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(vr + (ch + 4 * p) * (BF ? 2 : 4));
                vq[st][half * (nh / 2) + p] = u32x4{x[0] & keep, x[1] & keep, x[2] & keep, x[3] & keep};
            }
        }
    }
    stage_mat(mW, a.W0 + (long long)h * 4096); // while the rows are in flight
    __syncthreads();
#pragma unroll
    for (int st = 0; st < kGmmSt; ++st) {
        const int row = tb * kGmmTok + w * (16 * kGmmSt) + st * 16 + m;
        float vv[16];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if constexpr (BF) {
                const u32x4 u = vq[st][half];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    vv[8 * half + 2 * k] = bflo(u[k]);
                    vv[8 * half + 2 * k + 1] = bfhi(u[k]);
                }
            } else {
                const f32x4 u0 = __builtin_bit_cast(f32x4, vq[st][2 * half]);
                const f32x4 u1 = __builtin_bit_cast(f32x4, vq[st][2 * half + 1]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    vv[8 * half + k] = u0[k];
                    vv[8 * half + 4 + k] = u1[k];
                }
            }
        }
        const u32x4* q = kq[st];
        float kk = 0.f;
#pragma unroll
        for (int hh = 0; hh < nh; ++hh)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (BF) {
                    kk = fmaf(bflo(q[hh][k]), bflo(q[hh][k]), kk);
                    kk = fmaf(bfhi(q[hh][k]), bfhi(q[hh][k]), kk);
                } else {
                    const float x = __uint_as_float(q[hh][k]);
                    kk = fmaf(x, x, kk);
                }
            }
        // r = W0 k - v (L2) or -v (dot); d[rb][i] is output channel
        // 32 (rb >> 1) + 8 g + 4 (rb & 1) + i (perm_row)
        v4f d[4];
        if constexpr (BF) {
            const W1FragsBF wf = w1_frags_bf(mW, g, m);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                d[rb] = v4f{0.f, 0.f, 0.f, 0.f};
                d[rb] = mfma32(wf.f[rb][0], as_v8bf(q[0]), d[rb]);
                d[rb] = mfma32(wf.f[rb][1], as_v8bf(q[1]), d[rb]);
            }
        } else {
            const W1FragsF32 wf = w1_frags_f32(mW, g, m);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                d[rb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) {
                    const f32x4 qv = __builtin_bit_cast(f32x4, q[hh]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) d[rb] = mfma4(wf.f[rb][hh * 4 + i], qv[i], d[rb]);
                }
            }
        }
        float rr = 0.f;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = (a.dot ? 0.f : d[rb][i]) - vv[8 * (rb >> 1) + 4 * (rb & 1) + i];
                rr = fmaf(x, x, rr);
            }
        finish(row, kk, rr);
    }
}

int pow2_floor(long long s) {
    int p = 1;
    while (2LL * p <= s) p *= 2;
    return p;
}

int occupancy(const void* fn, std::atomic<int>& cache, int threads = kThreads) {
    int n = cache.load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess || n < 0) return 0;
    cache.store(n, std::memory_order_relaxed);
    return n;
}

} // namespace

int lin_fwd_max_splits(int B, int H, int N) {
    // a power of two (the reduction gathers 64/S columns), at most 64, about
    // 128 tokens per split, and no more workgroups than one MI355X keeps
    // resident (256 CUs x 1)
    const long long slices = (long long)B * H;
    if (slices <= 0 || N <= 0) return 1;
    const long long padded = (slices + 7) / 8 * 8; // XCD-aware grids round slices up to 8
    long long s = (N + 127) / 128;
    if (s > 32) s = 32; // the reduction sums 32/S elements per thread
    int p = pow2_floor(s);
    if (p < s) p *= 2;
    while (p > 1 && p * padded > 256) p /= 2;
    return p;
}

size_t lin_fwd_ws_bytes(int B, int H, int N) {
    const long long slices = (long long)B * H;
    const int S = lin_fwd_max_splits(B, H, N);
    if (S <= 1) return 0;
    return kCounterBytes + (size_t)slices * S * 8192 * 4 + (size_t)slices * 4096 * 4;
}

int lin_fwd_resident_per_cu(int bf16) {
    static std::atomic<int> cache[5];
    // the kernels of both exchange protocols have the same LDS footprint
    int r = bf16 ? occupancy((const void*)lin_fwd_resident<true, true>, cache[0])
                 : occupancy((const void*)lin_fwd_resident<false, true>, cache[1]);
    const int s = bf16 ? occupancy((const void*)lin_fwd_stream<true, true>, cache[2])
                       : occupancy((const void*)lin_fwd_stream<false, true>, cache[3]);
    if (bf16) {
        const int x = occupancy((const void*)lin_fwd_resident_gx<false>, cache[4], kThreads8);
        r = r < x ? r : x;
    }
    return r < s ? r : s;
}

bool lin_fwd_is_resident(int N, int S, int bf16) {
    const int per = (((N + S - 1) / S) + 15) & ~15;
    return per <= (bf16 ? LinCfg<true>::tmax : LinCfg<false>::tmax);
}

int lin_fwd_kernel(const LinFwdLaunch& a, int resident) {
    if (resident && a.xcd && a.bf16 && a.S > 1 && !a.saved) return kLinResidentGx;
    return resident ? kLinResident : kLinStream;
}

hipError_t launch_lin_fwd(LinFwdLaunch a, hipStream_t stream, int resident) {
    const long long slices = (long long)a.B * a.H;
    const long long gslices = a.xcd ? (slices + 7) / 8 * 8 : slices;
    const dim3 grid((unsigned)(gslices * a.S));
    dim3 block(kThreads);
    void* args[] = {&a};
    const void* fn;
    const int kind = lin_fwd_kernel(a, resident);
    if (kind == kLinResidentGx) {
        fn = a.steps > 1 ? (const void*)lin_fwd_resident_gx<true> : (const void*)lin_fwd_resident_gx<false>;
        block = dim3(kThreads8);
    } else if (kind == kLinResident) {
        if (a.xcd) fn = a.bf16 ? (const void*)lin_fwd_resident<true, true> : (const void*)lin_fwd_resident<false, true>;
        else fn = a.bf16 ? (const void*)lin_fwd_resident<true, false> : (const void*)lin_fwd_resident<false, false>;
    } else {
        if (a.xcd) fn = a.bf16 ? (const void*)lin_fwd_stream<true, true> : (const void*)lin_fwd_stream<false, true>;
        else fn = a.bf16 ? (const void*)lin_fwd_stream<true, false> : (const void*)lin_fwd_stream<false, false>;
    }
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

bool layer_would_fuse(const LinFwdLaunch& l, int resident, const ConvLaunch& cl) {
    if ((long long)l.B * l.H <= 0 || (long long)cl.B * cl.H <= 0) return false;
    ConvArgs c;
    unsigned cgrid = 0;
    conv_prepare(cl, c, cgrid);
    return layer_fusable(l, resident, c, cl.bf16);
}

hipError_t launch_lin_epochs(const LinEpochArgs& e, hipStream_t stream) {
    hipLaunchKernelGGL(lin_epochs, dim3((unsigned)e.slices), dim3(kThreads), 0, stream, e);
    return hipGetLastError();
}

hipError_t launch_lin_apply(const LinApplyArgs& a, int bf16, hipStream_t stream) {
    const long long blocks = (long long)a.B * a.H * ((a.N + 255) / 256);
    if (bf16) hipLaunchKernelGGL(lin_apply<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(lin_apply<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_lin_gmm(const LinGmmArgs& a, int bf16, hipStream_t stream) {
    const long long blocks = (long long)a.B * a.H * ((a.N + kGmmTok - 1) / kGmmTok);
    if (bf16) hipLaunchKernelGGL(lin_gmm<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(lin_gmm<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_layer(LinFwdLaunch l, int resident, ConvLaunch cl, hipStream_t stream) {
    ConvArgs c;
    unsigned cgrid = 0;
    const bool conv_on = (long long)cl.B * cl.H > 0;
    const bool lin_on = (long long)l.B * l.H > 0;
    if (conv_on) conv_prepare(cl, c, cgrid);
    if (lin_on && conv_on && layer_fusable(l, resident, c, cl.bf16)) {
        LayerArgs a{l, c, conv_kv_bytes<true>(c.R, c.TW)};
        const long long lgrid = (((long long)l.B * l.H + 7) / 8 * 8) * l.S;
        const unsigned grid = (unsigned)(lgrid > cgrid ? lgrid : cgrid);
        void* args[] = {&a};
        return hipLaunchKernel((const void*)layer_fused, dim3(grid), dim3(kThreads8), args, 0, stream);
    }
    if (lin_on) {
        const hipError_t e = launch_lin_fwd(l, stream, resident);
        if (e != hipSuccess) return e;
    }
    return conv_on ? conv_launch_prepared(c, cgrid, cl.bf16, stream) : hipSuccess;
}

} // namespace ttt
