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
// walk waits on memory once, not per column).  Seven launches, all
// reductions in a fixed order (bitwise reproducible):
//   pass 1  per (slice, 4-row group, column segment): partial g (unless the
//           forward's g is supplied) and dw1, summed over the 4 waves;
//   reduce  per slice: g, dw1 over the partials in order; w1, dg, the deta
//           term;
//   pass 2  per (slice, 4-row group, segment): dQ, dV, dK and the partial
//           sum_p dR[p] K[p+t];
//   sum     per slice: the dw0 term dw1 + the pass-2 partials in order;
//   batch   per head: dw0 and deta summed over the batch in b order.
#include "common.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kCbSeg = 16;     // columns per segment (at most)
constexpr int kCbRows = 4;     // grid rows per workgroup: one per wave
constexpr int kPD = 4;         // columns whose loads are in flight ahead of the walk

struct CbArgs {
    View4 K, Q, V, dZ, dK, dQ, dV;
    const float* w0;    // [H][64][9]
    const float* eta;   // [H]
    const float* gsv;   // nullable: the forward's g [slices][64][9]
    float* part1;       // [slices][P][64][18]: g (0..8), dw1 (9..17)
    float* part2;       // [slices][P][64][9]
    float* sl;          // [slices][5][64][9]: w1, (2/N) dg, dw1, g, dw0 term
    float* sum1;        // [slices][64][18]: part1 summed over the partials
    float* sum2;        // [slices][64][9]: part2 summed over the partials
    float* deta_s;      // [slices]
    float* dw0;         // [H][64][9]
    float* deta;        // [H]
    int B, H, gh, gw;
    int nseg, seglen, ngrp; // column segments, columns per segment, row groups
    int dot;                // dot-product loss: g = -(1/N) sum V K-shifted
};

template <bool BF> struct Elt;
template <> struct Elt<true> {
    static constexpr int esz = 2;
    __device__ static float ld(const char* p) { return __uint_as_float((uint32_t)(*(const uint16_t*)p) << 16); }
    __device__ static void st(char* p, float v) { __builtin_nontemporal_store(f2bf(v), (uint16_t*)p); }
};
template <> struct Elt<false> {
    static constexpr int esz = 4;
    __device__ static float ld(const char* p) { return *(const float*)p; }
    __device__ static void st(char* p, float v) { __builtin_nontemporal_store(v, (float*)p); }
};

// Channel `lane` of one slice's token map; positions off the grid read 0.
// Branch-free: the load goes to the clamped position and the value is
// selected afterwards, so a load in flight is waited for only where its
// value is used (a branch around the load would wait for every load at the
// join).
template <bool BF> struct Map {
    const char* base;
    long long sn; // bytes between tokens
    int gh, gw;
    __device__ float at(int y, int x) const {
        const bool in = y >= 0 && y < gh && x >= 0 && x < gw;
        const int yc = min(max(y, 0), gh - 1), xc = min(max(x, 0), gw - 1);
        const float v = Elt<BF>::ld(base + (long long)(yc * gw + xc) * sn);
        return in ? v : 0.f;
    }
};
template <bool BF>
__device__ __forceinline__ Map<BF> map_of(const View4& v, int b, int h, int gh, int gw, int lane) {
    constexpr int es = Elt<BF>::esz;
    Map<BF> m;
    m.base = (const char*)v.ptr + ((long long)b * v.sb + (long long)h * v.sh + lane) * es;
    m.sn = v.sn * es;
    m.gh = gh;
    m.gw = gw;
    return m;
}
template <bool BF>
__device__ __forceinline__ char* out_of(const View4& v, int b, int h, int lane) {
    constexpr int es = Elt<BF>::esz;
    return (char*)v.ptr + ((long long)b * v.sb + (long long)h * v.sh + lane) * es;
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
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
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
__global__ __launch_bounds__(256) void cbwd_reduce(CbArgs a) {
    __shared__ float de[256];
    const int slice = blockIdx.x, tid = threadIdx.x;
    const int h = slice % a.H;
    const int P = a.ngrp * a.nseg;
    const float eta = a.eta[h];
    const float scale = (a.dot ? 1.0f : 2.0f) / (float)(a.gh * a.gw);
    const float* src = a.sum1 + (long long)slice * 64 * 18;
    float* sl = a.sl + (long long)slice * 5 * 576;
    float dsum = 0.f;
    (void)P;
    for (int e = tid; e < 576; e += 256) {
        const int c = e / 9, k = e % 9;
        const float gs = src[c * 18 + k], ds = src[c * 18 + 9 + k];
        const float g = a.gsv ? a.gsv[(long long)slice * 576 + e] : scale * gs;
        const float w1 = a.w0[(long long)h * 576 + e] - eta * g;
        sl[e] = w1;
        sl[576 + e] = scale * (-eta * ds); // (2/N) dg
        sl[1152 + e] = ds;                 // dw1
        sl[1728 + e] = g;
        dsum -= ds * g;
    }
    de[tid] = dsum;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) de[tid] += de[tid + s];
        __syncthreads();
    }
    if (tid == 0) a.deta_s[slice] = de[0];
}

// ---- pass 2: dQ, dV, dK and the partial sum_p dR[p] K[p+t] -------------
template <bool BF>
__global__ __launch_bounds__(256) void cbwd_pass2(CbArgs a) {
    __shared__ float red[4 * 64 * 9];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const Task t = task_of(a, w);
    float acc[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) acc[k] = 0.f;
    if (t.y < a.gh && t.x0 < t.x1) {
        const Map<BF> Km = map_of<BF>(a.K, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> Vm = map_of<BF>(a.V, t.b, t.h, a.gh, a.gw, lane);
        const Map<BF> Dm = map_of<BF>(a.dZ, t.b, t.h, a.gh, a.gw, lane);
        char* dKp = out_of<BF>(a.dK, t.b, t.h, lane);
        char* dQp = out_of<BF>(a.dQ, t.b, t.h, lane);
        char* dVp = out_of<BF>(a.dV, t.b, t.h, lane);
        constexpr int es = Elt<BF>::esz;
        const long long sK = a.dK.sn * es, sQ = a.dQ.sn * es, sV = a.dV.sn * es;
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
                const bool in = yy >= 0 && yy < a.gh && xx >= 0 && xx < a.gw;
                rr[i] = in ? p - vv[i] : 0.f;
                dr[i] = in ? q : 0.f;
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
                    const long long n = (long long)y * a.gw + x;
                    Elt<BF>::st(dQp + n * sQ, dq);
                    Elt<BF>::st(dKp + n * sK, dk);
                    Elt<BF>::st(dVp + n * sV, -drc);
                }
            }
        }
    }
    float* dst = a.part2 + ((long long)t.slice * a.ngrp * a.nseg + t.pidx) * 576;
    wave_sum_store<9>(acc, red, dst);
}

// ---- per-slice dw0 term: dw1 + the pass-2 partials in order -------------
__global__ __launch_bounds__(256) void cbwd_slice_sum(CbArgs a) {
    const int slice = blockIdx.x, tid = threadIdx.x;
    float* sl = a.sl + (long long)slice * 5 * 576;
    const float* s2 = a.sum2 + (long long)slice * 576;
    for (int e = tid; e < 576; e += 256) sl[2304 + e] = sl[1152 + e] + s2[e];
}

// ---- sum of per-workgroup partials, [slices][P][E] -> [slices][E] --------
// Block (slice, 64-element chunk); its four waves each add a quarter of the
// partials in order, then the four quarter sums are added in order: the
// same order on every run.
__global__ __launch_bounds__(256) void cbwd_sum_partials(const float* part, float* out, int P, int E) {
    __shared__ float qs[4][64];
    const int nchunk = (E + 63) / 64;
    const int slice = blockIdx.x / nchunk, e = (blockIdx.x % nchunk) * 64 + (threadIdx.x & 63);
    const int q = threadIdx.x >> 6, per = (P + 3) / 4, p0 = q * per, p1 = min(P, p0 + per);
    float s = 0.f;
    if (e < E) {
        const float* src = part + (long long)slice * P * E + e;
#pragma unroll 8
        for (int p = p0; p < p1; ++p) s += src[(long long)p * E];
    }
    qs[q][threadIdx.x & 63] = s;
    __syncthreads();
    if (q == 0 && e < E) {
        const int l = threadIdx.x;
        out[(long long)slice * E + e] = ((qs[0][l] + qs[1][l]) + qs[2][l]) + qs[3][l];
    }
}

// ---- per-head batch sums -------------------------------------------------
__global__ __launch_bounds__(256) void cbwd_batch(CbArgs a) {
    const int h = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < 576; e += 256) {
        float s = 0.f;
        for (int b = 0; b < a.B; ++b) s += a.sl[((long long)b * a.H + h) * 5 * 576 + 2304 + e];
        a.dw0[(long long)h * 576 + e] = s;
    }
    if (tid == 0) {
        float s = 0.f;
        for (int b = 0; b < a.B; ++b) s += a.deta_s[(long long)b * a.H + h];
        a.deta[h] = s;
    }
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
           a256(slices * 4) + a256(slices * 1152 * 4) + a256(slices * 576 * 4);
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
    w += a256(slices * 4);
    a.sum1 = (float*)w;
    w += a256(slices * 1152 * 4);
    a.sum2 = (float*)w;
    const dim3 grid((unsigned)(slices * P)), block(256);
    if (s.bf16) {
        if (s.saved) hipLaunchKernelGGL((cbwd_pass1<true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((cbwd_pass1<true, false>), grid, block, 0, stream, a);
    } else {
        if (s.saved) hipLaunchKernelGGL((cbwd_pass1<false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((cbwd_pass1<false, false>), grid, block, 0, stream, a);
    }
    hipLaunchKernelGGL(cbwd_sum_partials, dim3((unsigned)(slices * 18)), block, 0, stream, (const float*)a.part1,
                       a.sum1, (int)P, 1152);
    hipLaunchKernelGGL(cbwd_reduce, dim3((unsigned)slices), block, 0, stream, a);
    if (s.bf16) hipLaunchKernelGGL((cbwd_pass2<true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((cbwd_pass2<false>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(cbwd_sum_partials, dim3((unsigned)(slices * 9)), block, 0, stream, (const float*)a.part2,
                       a.sum2, (int)P, 576);
    hipLaunchKernelGGL(cbwd_slice_sum, dim3((unsigned)slices), block, 0, stream, a);
    hipLaunchKernelGGL(cbwd_batch, dim3((unsigned)s.H), block, 0, stream, a);
    return hipGetLastError();
}

} // namespace ttt
