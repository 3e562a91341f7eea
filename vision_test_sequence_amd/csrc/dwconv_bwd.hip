// dwconv_bwd.hip -- gradient of the full-batch step of the 3x3 depthwise-
// convolution inner model (ViT3 article: observation 6 for the conv inner
// model, observation 1 for end-to-end training through the inner gradient).
//
// Forward, per channel of a slice, t over the 9 taps, zero padding:
//   P[p] = sum_t w0[t] K[p+t],  R = P - V,  g[t] = (2/N) sum_p R[p] K[p+t],
//   w1 = w0 - eta g,  Z[p] = sum_t w1[t] Q[p+t].
// Backward of L = <dZ, Z>:
//   dw1[t] = sum_p dZ[p] Q[p+t]              (reduction over pixels)
//   dg = -eta dw1,  deta = -sum <dw1, g>
//   dQ[q]  = sum_t w1[t] dZ[q-t]
//   dR[p]  = (2/N) sum_t dg[t] K[p+t],  dV = -dR
//   dK[q]  = sum_t ((2/N) dg[t] R[q-t] + w0[t] dR[q-t])   (R, dR zero off-grid)
//   dw0[t] = dw1[t] + sum_p dR[p] K[p+t]     (reduction over pixels)
// dw0 and deta are also summed over the batch.
//
// Element-wise stencil work on the vector ALUs (no dense contraction): one
// channel per lane, so every load or store of a wave is one contiguous
// token row (128 bytes bf16, 256 bytes fp32).  A wave walks one grid row
// over a segment of at most 16 columns with sliding register windows, the
// loads of the next kPD columns in flight (a ring of registers, so the
// walk waits on memory once, not per column).  Four launches, all
// reductions in a fixed order (bitwise reproducible):
//   pass 1  per (slice, 4-row group, column segment): partial g (unless the
//           forward's g is supplied) and dw1, summed over the 4 waves;
//   reduce  per (slice, 64 of its 576 (channel, tap) entries): g, dw1 over
//           the partials in order; w1, dg, the entries' deta terms;
//   pass 2  per (slice, 4-row group, segment): dQ, dV, dK and the partial
//           sum_p dR[p] K[p+t];
//   sums    per (slice, 64 entries): the dw0 term dw1 + the pass-2 partials
//           in order; the last of a head's workgroups to finish (a counter
//           per head) sums dw0 and deta over the batch in b order.
#include "common.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kCbSeg = 16;     // columns per segment (at most)
constexpr int kCbRows = 4;     // grid rows per workgroup: one per wave
constexpr int kPD = 4;         // columns whose loads are in flight ahead of the walk
constexpr uint32_t kOffOut = 0x80000000u; // an offset past every slice span

struct CbArgs {
    View4 K, Q, V, dZ, dK, dQ, dV;
    const float* w0;    // [H][64][9]
    const float* eta;   // [H]
    const float* gsv;   // nullable: the forward's g [slices][64][9]
    float* part1;       // [slices][P][64][18]: g (0..8), dw1 (9..17)
    float* part2;       // [slices][P][64][9]
    float* sl;          // [slices][5][64][9]: w1, (2/N) dg, dw1, g, dw0 term
    float* deta_s;      // [slices][9]: deta terms of the reduce's entry blocks
    unsigned* cnt;      // [H]: finished sums workgroups per head (zeroed by the reduce)
    float* dw0;         // [H][64][9]
    float* deta;        // [H]
    int B, H, gh, gw;
    int nseg, seglen, ngrp; // column segments, columns per segment, row groups
    int dot;                // dot-product loss: g = -(1/N) sum V K-shifted
};

template <bool BF> struct Elt;
template <> struct Elt<true> {
    static constexpr int esz = 2;
    __device__ static float ld(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
        return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0) << 16);
    }
    __device__ static void st(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(f2bf(v), rs, off, 0, 2 /* nontemporal */);
    }
};
template <> struct Elt<false> {
    static constexpr int esz = 4;
    __device__ static float ld(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    }
    __device__ static void st(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, off, 0, 2 /* nontemporal */);
    }
};

// One slice's token map of a view, read and written through a buffer
// descriptor over the slice's span (the host bounds it below 2^31 bytes).
// A token's byte offset is wave-uniform and formed on the scalar unit; a
// lane adds its channel's offset.  Positions off the grid read 0 from past
// the descriptor's range: a column off the grid takes the offset kOffOut,
// and a row off the grid needs nothing, its offset being negative (2^31 or
// more as unsigned) or at least N tokens.  No clamp, no select per load and
// no branch (a branch around a load would make the compiler wait for every
// load in flight at the join).
template <bool BF> struct Map {
    __amdgpu_buffer_rsrc_t rs;
    int sn;     // bytes between tokens (at least 64 elements)
    int gw;
    uint32_t lo; // the lane's channel offset in bytes
    __device__ uint32_t off(int y, int x) const {
        // both arms formed first, so the choice is a select, not a branch
        const uint32_t tok = (uint32_t)((y * gw + x) * sn);
        const bool on = (unsigned)x < (unsigned)gw;
        return (on ? tok : kOffOut) + lo;
    }
    __device__ float at(int y, int x) const { return Elt<BF>::ld(rs, off(y, x)); }
    __device__ void put(int y, int x, float v) const { Elt<BF>::st(rs, off(y, x), v); }
};
template <bool BF>
__device__ __forceinline__ Map<BF> map_of(const View4& v, int b, int h, int gh, int gw, int lane) {
    constexpr int es = Elt<BF>::esz;
    Map<BF> m;
    const char* base = (const char*)v.ptr + ((long long)b * v.sb + (long long)h * v.sh) * es;
    m.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0,
                                              (int)(((long long)gh * gw - 1) * v.sn * es + 64 * es), 0x00020000);
    // (a one-token slice may have any stride; 64 elements keep its
    // neighbours' offsets outside the span)
    m.sn = (int)max(v.sn * es, 64LL * es);
    m.gw = gw;
    m.lo = (uint32_t)(lane * es);
    return m;
}

struct Task {
    int slice, b, h, grp, seg, y, x0, x1, pidx;
};
__device__ __forceinline__ Task task_of(const CbArgs& a, int w) {
    Task t;
    const int per = a.ngrp * a.nseg;
    t.slice = blockIdx.x / per;
    const int r = blockIdx.x % per;
    t.grp = r / a.nseg;
    t.seg = r % a.nseg;
    t.pidx = r;
    t.b = t.slice / a.H;
    t.h = t.slice % a.H;
    t.y = t.grp * kCbRows + w;
    t.x0 = t.seg * a.seglen;
    t.x1 = min(a.gw, t.x0 + a.seglen);
    return t;
}

// Sum NV per-lane values of the 4 waves in wave order and store them as
// this workgroup's partial, [64][NV] floats at dst.
template <int NV>
__device__ __forceinline__ void wave_sum_store(const float* v, float* red, float* dst) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int k = 0; k < NV; ++k) red[(w * 64 + lane) * NV + k] = v[k];
    __syncthreads();
    for (int e = tid; e < 64 * NV; e += 256) {
        const float s = ((red[e] + red[64 * NV + e]) + red[128 * NV + e]) + red[192 * NV + e];
        dst[e] = s;
    }
}

// ---- pass 1: partial g and dw1 ----------------------------------------
template <bool BF, bool HAS_G>
__global__ __launch_bounds__(256) void cbwd_pass1(CbArgs a) {
    __shared__ float red[4 * 64 * 18];
    // the wave index is uniform: the row, and with it every address but the
    // lane's channel offset, is formed on the scalar unit
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Task t = task_of(a, w);
    float acc[18];
#pragma unroll
    for (int k = 0; k < 18; ++k) acc[k] = 0.f;
    if (t.y < a.gh && t.x0 < t.x1) {
        const Map<BF> Km = map_of<BF>(a.K, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> Qm = map_of<BF>(a.Q, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> Vm = map_of<BF>(a.V, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> Dm = map_of<BF>(a.dZ, t.b, t.h, a.gh, a.gw, lane);
        // taps of P = conv(K, w0) in R = P - V (none under the dot-product loss)
        float wt[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) wt[k] = a.dot ? 0.f : a.w0[((long long)t.h * 64 + lane) * 9 + k];
        const int y = t.y;
        // windows: columns x-1, x, x+1 of rows y-1..y+1 (index 3 i + j)
        float kw[9], qw[9];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if constexpr (!HAS_G) kw[3 * i + j + 1] = Km.at(y + i - 1, t.x0 + j - 1);
                qw[3 * i + j + 1] = Qm.at(y + i - 1, t.x0 + j - 1);
            }
        }
        // ring slot u holds the loads of step x0 + u (+ kPD after each use):
        // K and Q column x+1, V and dZ at (y, x)
        float kn[kPD][3], qn[kPD][3], vn[kPD], dn[kPD];
        auto fetch = [&](int u, int x) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                if constexpr (!HAS_G) kn[u][i] = Km.at(y + i - 1, x + 1);
                qn[u][i] = Qm.at(y + i - 1, x + 1);
            }
            if constexpr (!HAS_G) vn[u] = Vm.at(y, x);
            dn[u] = Dm.at(y, x);
        };
#pragma unroll
        for (int u = 0; u < kPD; ++u) fetch(u, t.x0 + u);
        // a whole segment (at most kCbSeg columns) unrolled: the loads of
        // later columns are not held back at a loop edge
#pragma unroll
        for (int xb = 0; xb < kCbSeg; xb += kPD) {
#pragma unroll
            for (int u = 0; u < kPD; ++u) {
                const int x = t.x0 + xb + u;
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    if constexpr (!HAS_G) {
                        kw[3 * i] = kw[3 * i + 1];
                        kw[3 * i + 1] = kw[3 * i + 2];
                        kw[3 * i + 2] = kn[u][i];
                    }
                    qw[3 * i] = qw[3 * i + 1];
                    qw[3 * i + 1] = qw[3 * i + 2];
                    qw[3 * i + 2] = qn[u][i];
                }
                float vc = 0.f;
                if constexpr (!HAS_G) vc = vn[u];
                const float dz = dn[u];
                fetch(u, x + kPD);
                if (x < t.x1) {
                    if constexpr (!HAS_G) {
                        float r = -vc;
#pragma unroll
                        for (int k = 0; k < 9; ++k) r = fmaf(wt[k], kw[k], r);
#pragma unroll
                        for (int k = 0; k < 9; ++k) acc[k] = fmaf(r, kw[k], acc[k]);
                    }
#pragma unroll
                    for (int k = 0; k < 9; ++k) acc[9 + k] = fmaf(dz, qw[k], acc[9 + k]);
                }
            }
        }
    }
    float* dst = a.part1 + ((long long)t.slice * a.ngrp * a.nseg + t.pidx) * 64 * 18;
    wave_sum_store<18>(acc, red, dst);
}

// ---- per-slice reduce ---------------------------------------------------
// Workgroup (slice, j) takes entries e = 64 j + lane of the slice's 576
// (channel e / 9, tap e % 9) and sums their P partials: wave q of kCbSumW
// adds partials [q per, (q+1) per) in order, eight loads issued before
// their adds (a slot past the range adds 0), and the waves' sums are added
// in wave order.
constexpr int kCbEnt = 64;                          // entries per reduce / sums workgroup
constexpr int kCbBlk = (576 + kCbEnt - 1) / kCbEnt; // such workgroups per slice
constexpr int kCbSumW = 4;                          // waves per reduce / sums workgroup
template <int NV, int STRIDE>
__device__ __forceinline__ void part_sums(const float* src, int P, const int* off, float* qs, float* out) {
    const int lane = threadIdx.x & 63, q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per = (P + kCbSumW - 1) / kCbSumW, p0 = q * per, p1 = min(P, p0 + per);
    float s[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) s[v] = 0.f;
    for (int p = p0; p < p1; p += 8) {
        float t[8][NV];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int pc = min(p + i, p1 - 1);
#pragma unroll
            for (int v = 0; v < NV; ++v) t[i][v] = src[(long long)pc * STRIDE + off[v]];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int v = 0; v < NV; ++v) s[v] += p + i < p1 ? t[i][v] : 0.f;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) qs[(v * kCbSumW + q) * 64 + lane] = s[v];
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float x = qs[(v * kCbSumW) * 64 + lane];
#pragma unroll
        for (int w = 1; w < kCbSumW; ++w) x += qs[(v * kCbSumW + w) * 64 + lane];
        out[v] = x;
    }
}

__global__ __launch_bounds__(64 * kCbSumW) void cbwd_reduce(CbArgs a) {
    __shared__ float qs[2 * kCbSumW * 64];
    const int slice = blockIdx.x / kCbBlk, j = blockIdx.x % kCbBlk, tid = threadIdx.x, lane = tid & 63;
    const int h = slice % a.H;
    const int P = a.ngrp * a.nseg;
    if (blockIdx.x == 0) // the sums' counters, for this call
        for (int i = tid; i < a.H; i += 64 * kCbSumW) a.cnt[i] = 0u;
    const int e = j * kCbEnt + lane, ec = min(e, 575);
    const int c = ec / 9, k = ec % 9;
    const int off[2] = {c * 18 + k, c * 18 + 9 + k};
    float sums[2];
    part_sums<2, 1152>(a.part1 + (long long)slice * P * 1152, P, off, qs, sums);
    if (tid >= 64) return;
    const float eta = a.eta[h];
    const float scale = (a.dot ? 1.0f : 2.0f) / (float)(a.gh * a.gw);
    float* sl = a.sl + (long long)slice * 5 * 576;
    float d = 0.f;
    if (e < 576) {
        const float gs = sums[0], ds = sums[1];
        const float g = a.gsv ? a.gsv[(long long)slice * 576 + e] : scale * gs;
        sl[e] = a.w0[(long long)h * 576 + e] - eta * g; // w1
        sl[576 + e] = scale * (-eta * ds);              // (2/N) dg
        sl[1152 + e] = ds;                              // dw1
        sl[1728 + e] = g;
        d = -ds * g;
    }
    // the 64 entries' deta terms, summed in a fixed tree over the wave
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) d += __shfl_xor(d, m);
    if (lane == 0) a.deta_s[(long long)slice * kCbBlk + j] = d;
}

// ---- pass 2: dQ, dV, dK and the partial sum_p dR[p] K[p+t] -------------
template <bool BF>
__global__ __launch_bounds__(256) void cbwd_pass2(CbArgs a) {
    __shared__ float red[4 * 64 * 9];
    // the wave index is uniform: the row, and with it every address but the
    // lane's channel offset, is formed on the scalar unit
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Task t = task_of(a, w);
    float acc[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) acc[k] = 0.f;
    if (t.y < a.gh && t.x0 < t.x1) {
        const Map<BF> Km = map_of<BF>(a.K, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> Vm = map_of<BF>(a.V, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> Dm = map_of<BF>(a.dZ, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> dKm = map_of<BF>(a.dK, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> dQm = map_of<BF>(a.dQ, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> dVm = map_of<BF>(a.dV, t.b, t.h, a.gh, a.gw, lane);
        const float* sl = a.sl + (long long)t.slice * 5 * 576 + lane * 9;
        float wt[9], w1[9], dgs[9];
        // Under the dot-product loss g = -(1/N) sum_p V[p] K[p+t] has no
        // P = conv(K, w0) term: R = -V, dK gets no w0 dR term and dw0 no
        // sum_p dR[p] K[p+t] term (wt = 0, wd = 0).
        const float wd = a.dot ? 0.f : 1.f;
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            wt[k] = wd * a.w0[((long long)t.h * 64 + lane) * 9 + k];
            w1[k] = sl[k];
            dgs[k] = sl[576 + k];
        }
        const int y = t.y;
        // K window: rows y-2..y+2 (index 5 col + row) over columns x-1..x+2
        // (cols 0..3); R, dR windows: rows y-1..y+1 over columns x-1..x+1;
        // dZ window: rows y-1..y+1 over columns x-1..x+1.
        float kw[4][5], rw[3][3], drw[3][3], dzw[3][3];
        // R and dR of grid position (yy = y-1..y+1, xx) from the K window
        // column cc (columns cc-1..cc+1 around it) and V at (yy, xx); zero
        // off the grid.
        auto rcol = [&](int xx, int cc, const float* vv, float* rr, float* dr) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int yy = y + i - 1;
                float p = 0.f, q = 0.f;
#pragma unroll
                for (int ii = 0; ii < 3; ++ii)
#pragma unroll
                    for (int jj = 0; jj < 3; ++jj) {
                        const float kv = kw[cc + jj - 1][i + ii];
                        p = fmaf(wt[3 * ii + jj], kv, p);
                        q = fmaf(dgs[3 * ii + jj], kv, q);
                    }
                // a 0/1 factor, not a branch, zeroes positions off the grid
                const float in = yy >= 0 && yy < a.gh && xx >= 0 && xx < a.gw ? 1.f : 0.f;
                rr[i] = in * (p - vv[i]);
                dr[i] = in * q;
            }
        };
        // initial windows for x = x0: K columns x0-2..x0+1 into kw[0..3]
        // (kw[c] holds column x - 2 + c before the first shift)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 5; ++r) kw[c][r] = Km.at(y + r - 2, t.x0 - 2 + c);
        // R, dR at columns x0-1 and x0 (window columns 1 and 2)
        {
            float rr[3], dr[3], vv[3];
#pragma unroll
            for (int i = 0; i < 3; ++i) vv[i] = Vm.at(y + i - 1, t.x0 - 1);
            rcol(t.x0 - 1, 1, vv, rr, dr);
#pragma unroll
            for (int i = 0; i < 3; ++i) { rw[1][i] = rr[i]; drw[1][i] = dr[i]; }
#pragma unroll
            for (int i = 0; i < 3; ++i) vv[i] = Vm.at(y + i - 1, t.x0);
            rcol(t.x0, 2, vv, rr, dr);
#pragma unroll
            for (int i = 0; i < 3; ++i) { rw[2][i] = rr[i]; drw[2][i] = dr[i]; }
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            dzw[1][i] = Dm.at(y + i - 1, t.x0 - 1);
            dzw[2][i] = Dm.at(y + i - 1, t.x0);
        }
        // ring slot u holds the loads of step x0 + u (+ kPD after each use):
        // K column x+2 (5 rows), dZ and V column x+1 (3 rows each)
        float kn[kPD][5], dn[kPD][3], vn[kPD][3];
        auto fetch = [&](int u, int x) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < 5; ++r) kn[u][r] = Km.at(y + r - 2, x + 2);
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                dn[u][i] = Dm.at(y + i - 1, x + 1);
                vn[u][i] = Vm.at(y + i - 1, x + 1);
            }
        };
#pragma unroll
        for (int u = 0; u < kPD; ++u) fetch(u, t.x0 + u);
        // a whole segment (at most kCbSeg columns) unrolled: the loads of
        // later columns are not held back at a loop edge
#pragma unroll
        for (int xb = 0; xb < kCbSeg; xb += kPD) {
#pragma unroll
            for (int u = 0; u < kPD; ++u) {
                const int x = t.x0 + xb + u;
                // shift: K columns x-1..x+2, dZ columns x-1..x+1
#pragma unroll
                for (int r = 0; r < 5; ++r) {
                    kw[0][r] = kw[1][r];
                    kw[1][r] = kw[2][r];
                    kw[2][r] = kw[3][r];
                    kw[3][r] = kn[u][r];
                }
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    rw[0][i] = rw[1][i];
                    rw[1][i] = rw[2][i];
                    drw[0][i] = drw[1][i];
                    drw[1][i] = drw[2][i];
                    dzw[0][i] = dzw[1][i];
                    dzw[1][i] = dzw[2][i];
                    dzw[2][i] = dn[u][i];
                }
                // R, dR at column x+1 (K window column 2 = x+1)
                {
                    float rr[3], dr[3];
                    rcol(x + 1, 2, vn[u], rr, dr);
#pragma unroll
                    for (int i = 0; i < 3; ++i) { rw[2][i] = rr[i]; drw[2][i] = dr[i]; }
                }
                fetch(u, x + kPD);
                if (x < t.x1) {
                    // outputs at (y, x): window index [col][row], q - t with t = (i-1, j-1)
                    float dq = 0.f, dk = 0.f;
#pragma unroll
                    for (int i = 0; i < 3; ++i)
#pragma unroll
                        for (int j = 0; j < 3; ++j) {
                            const int tt = 3 * i + j;
                            dq = fmaf(w1[tt], dzw[2 - j][2 - i], dq);
                            dk = fmaf(dgs[tt], rw[2 - j][2 - i], dk);
                            dk = fmaf(wt[tt], drw[2 - j][2 - i], dk);
                        }
                    const float drc = drw[1][1];
#pragma unroll
                    for (int i = 0; i < 3; ++i)
#pragma unroll
                        for (int j = 0; j < 3; ++j) acc[3 * i + j] = fmaf(wd * drc, kw[j][i + 1], acc[3 * i + j]);
                    dQm.put(y, x, dq);
                    dKm.put(y, x, dk);
                    dVm.put(y, x, -drc);
                }
            }
        }
    }
    float* dst = a.part2 + ((long long)t.slice * a.ngrp * a.nseg + t.pidx) * 576;
    wave_sum_store<9>(acc, red, dst);
}

// ---- per-slice dw0 term, then the batch sums --------------------------
// Workgroup (slice, j): the dw0 term dw1 + the pass-2 partials (in order) of
// its 64 entries.  Each workgroup then counts itself done on its head's
// counter (release: its terms are visible device-wide first); the last of
// the head's B x kCbBlk workgroups (acquire) adds dw0 and deta over b in
// order.  Which workgroup is last varies; the sums' order does not.
__global__ __launch_bounds__(64 * kCbSumW) void cbwd_sums(CbArgs a) {
    __shared__ float qs[kCbSumW * 64];
    __shared__ int last;
    const int slice = blockIdx.x / kCbBlk, j = blockIdx.x % kCbBlk, tid = threadIdx.x, lane = tid & 63;
    const int h = slice % a.H;
    const int P = a.ngrp * a.nseg;
    const int e = j * kCbEnt + lane, ec = min(e, 575);
    const int off[1] = {ec};
    float s2[1];
    part_sums<1, 576>(a.part2 + (long long)slice * P * 576, P, off, qs, s2);
    float* sl = a.sl + (long long)slice * 5 * 576;
    if (tid < 64 && e < 576) sl[2304 + e] = sl[1152 + e] + s2[0];
    // the stores have reached L2 before the barrier; one release fence (an
    // L2 write-back, costly per wave) then publishes them device-wide
    drain_vmem();
    __syncthreads();
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned done = __hip_atomic_fetch_add(a.cnt + h, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = done == (unsigned)(a.B * kCbBlk - 1);
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (!last) return;
    // dw0: a thread per entry, the B terms loaded eight at a time
    for (int ee = tid; ee < 576; ee += 64 * kCbSumW) {
        const float* src = a.sl + (long long)h * 5 * 576 + 2304 + ee;
        const long long step = (long long)a.H * 5 * 576;
        float v = 0.f;
        int b = 0;
        for (; b + 8 <= a.B; b += 8) {
            float t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = src[(b + i) * step];
#pragma unroll
            for (int i = 0; i < 8; ++i) v += t[i];
        }
        for (; b < a.B; ++b) v += src[b * step];
        a.dw0[(long long)h * 576 + ee] = v;
    }
    // deta: image b's term (its kCbBlk entry blocks in order) by thread b
    // mod the block size, then the images in order
    float d = 0.f;
    for (int b0 = 0; b0 < a.B; b0 += 64 * kCbSumW) {
        const int b = b0 + tid;
        if (b < a.B) {
            const float* ds = a.deta_s + ((long long)b * a.H + h) * kCbBlk;
            float t[kCbBlk];
#pragma unroll
            for (int jj = 0; jj < kCbBlk; ++jj) t[jj] = ds[jj];
            float u = 0.f;
#pragma unroll
            for (int jj = 0; jj < kCbBlk; ++jj) u += t[jj];
            qs[tid] = u;
        }
        __syncthreads();
        if (tid == 0)
            for (int i = 0; i < min(64 * kCbSumW, a.B - b0); ++i) d += qs[i];
        __syncthreads();
    }
    if (tid == 0) a.deta[h] = d;
}

struct CbPlan {
    int nseg, seglen, ngrp;
};
CbPlan cb_plan(int gh, int gw) {
    CbPlan p; // segments of at most kCbSeg columns: the walks are unrolled for that many
    p.nseg = (gw + kCbSeg - 1) / kCbSeg;
    p.seglen = (gw + p.nseg - 1) / p.nseg;
    p.ngrp = (gh + kCbRows - 1) / kCbRows;
    return p;
}
size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

} // namespace

size_t conv_bwd_ws_bytes(int B, int H, int gh, int gw) {
    const size_t slices = (size_t)B * H;
    if (slices == 0 || gh <= 0 || gw <= 0) return 0;
    const CbPlan p = cb_plan(gh, gw);
    const size_t P = (size_t)p.ngrp * p.nseg;
    return a256(slices * P * 64 * 18 * 4) + a256(slices * P * 576 * 4) + a256(slices * 5 * 576 * 4) +
           a256(slices * kCbBlk * 4) + a256((size_t)H * 4);
}

hipError_t launch_conv_bwd(const ConvBwdLaunch& s, hipStream_t stream) {
    CbArgs a{};
    a.K = s.K; a.Q = s.Q; a.V = s.V; a.dZ = s.dZ;
    a.dK = s.dK; a.dQ = s.dQ; a.dV = s.dV;
    a.w0 = s.w0; a.eta = s.eta; a.gsv = s.saved;
    a.dw0 = s.dw0; a.deta = s.deta;
    a.B = s.B; a.H = s.H; a.gh = s.gh; a.gw = s.gw;
    a.dot = s.dot;
    const CbPlan p = cb_plan(s.gh, s.gw);
    a.nseg = p.nseg; a.seglen = p.seglen; a.ngrp = p.ngrp;
    const size_t slices = (size_t)s.B * s.H;
    const size_t P = (size_t)p.ngrp * p.nseg;
    char* w = (char*)s.ws;
    a.part1 = (float*)w;
    w += a256(slices * P * 64 * 18 * 4);
    a.part2 = (float*)w;
    w += a256(slices * P * 576 * 4);
    a.sl = (float*)w;
    w += a256(slices * 5 * 576 * 4);
    a.deta_s = (float*)w;
    w += a256(slices * kCbBlk * 4);
    a.cnt = (unsigned*)w;
    const dim3 grid((unsigned)(slices * P)), block(256);
    if (s.bf16) {
        if (s.saved) hipLaunchKernelGGL((cbwd_pass1<true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((cbwd_pass1<true, false>), grid, block, 0, stream, a);
    } else {
        if (s.saved) hipLaunchKernelGGL((cbwd_pass1<false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((cbwd_pass1<false, false>), grid, block, 0, stream, a);
    }
    const dim3 sgrid((unsigned)(slices * kCbBlk));
    hipLaunchKernelGGL(cbwd_reduce, sgrid, dim3(64 * kCbSumW), 0, stream, a);
    if (s.bf16) hipLaunchKernelGGL((cbwd_pass2<true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((cbwd_pass2<false>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(cbwd_sums, sgrid, dim3(64 * kCbSumW), 0, stream, a);
    return hipGetLastError();
}

} // namespace ttt
