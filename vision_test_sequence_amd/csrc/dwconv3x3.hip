// dwconv3x3.hip -- one full-batch L2 gradient step of the 3x3 depthwise-
// convolution inner model, then apply (ViT3 article, observation 6: a conv
// inner model keeps the global K/V information in its kernel; the layer
// recipe uses one depthwise 3x3 head).
//
// Per slice and channel c, on the row-major token grid with zero padding:
//   P = conv(K, w0), R = P - V,
//   g[c][i][j] = (2/N) sum_{y,x} R[y][x] K[y+i-1][x+j-1],
//   w1 = w0 - eta g,  Z = conv(Q, w1).
// The work is HBM-bound element-wise stencil arithmetic on the vector ALUs
// (no dense contraction): one channel per lane (d = 64 = wavefront width),
// so every LDS access of a wave is one contiguous 128-byte (bf16) pixel.
//
// A slice's grid is cut into rectangular tiles of R rows x TW columns; a
// workgroup owns one or more consecutive tiles of one slice.
//   phase 1  the K halo tile ((R+2) x (TW+2) pixels), the V tile and (for
//            single-tile workgroups) the Q halo tile are staged into LDS
//            with direct global->LDS 16-byte loads (positions outside the
//            grid load a zero pixel); each wave slides a 3x3 window along x
//            over its row segments, forms P and R, and accumulates its
//            lane's 9 tap sums; the 8 waves are summed in a fixed order;
//   phase 2  with S > 1 workgroups per slice the 64 x 9 partials meet in the
//            workspace (one per-slice barrier) and every workgroup sums all
//            S of them in split order into w1 (so all form the same w1);
//   phase 3  the same sliding window over Q with w1 writes Z.
#include "conv_body.hpp"

#include <atomic>

namespace ttt {
namespace {

template <bool BF, bool XC>
__global__ __launch_bounds__(kCT, 1) void conv_kernel(ConvArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kW0Bytes + kTileBytes];
    __shared__ float red[kRedFloats];
    __shared__ float w1s[64 * 9];
    __shared__ int s_chk; // outcome of the exchange (slice_bad)
    conv_body<BF, XC>(a, ConvLds{lds, nullptr, red, w1s, &s_chk});
}

struct ConvPlan {
    int R, TW, ny, nx, S, tpw;
};

// Tile the grid so that the slices x S workgroups fill (but do not exceed)
// one MI355X (256 resident workgroups) and a tile's staging fits in LDS.
ConvPlan plan_conv(int nslices, int gh, int gw, int esz, int cap) {
    const long long slices = (nslices + 7) / 8 * 8; // XCD-aware grids round slices up to 8
    const int pb = 64 * esz;
    auto fits = [&](int R, int TW) {
        const int TWp = TW > kSeg ? TW : kSeg; // LDS rows hold at least one segment
        const long long KP = esz == 2 ? conv_pitch<true>(TWp + 2) : conv_pitch<false>(TWp + 2);
        const long long VP = esz == 2 ? conv_pitch<true>(TWp) : conv_pitch<false>(TWp);
        return (2 * (R + 2) * KP + (long long)R * VP) * pb <= kTileBytes;
    };
    ConvPlan p{};
    long long target = cap > 0 ? cap / slices : 1;
    if (target < 1) target = 1;
    // widest tiles first: full rows when they fit, else column bands
    int TW = gw;
    while (!fits(1, TW)) TW = (TW + 1) / 2;
    int nx = (gw + TW - 1) / TW;
    TW = (gw + nx - 1) / nx;
    long long ny = target / nx;
    if (ny < 1) ny = 1;
    if (ny > gh) ny = gh;
    int R = (int)((gh + ny - 1) / ny);
    while (!fits(R, TW)) --R;
    ny = (gh + R - 1) / R;
    const long long ntile = ny * (long long)nx;
    // one workgroup per tile when that stays resident, else as many
    // workgroups per slice as stay resident, each taking consecutive tiles
    long long S = ntile;
    const long long room = (cap > 0 ? cap : 1) / slices;
    if (S > room) S = room > 1 ? room : 1;
    const long long tpw = (ntile + S - 1) / S;
    S = (ntile + tpw - 1) / tpw;
    (void)nslices;
    p.R = R; p.TW = TW; p.ny = (int)ny; p.nx = nx; p.S = (int)S;
    p.tpw = (int)tpw;
    return p;
}

} // namespace

size_t conv_ws_bytes(int B, int H, int gh, int gw) {
    const long long slices = (long long)B * H;
    if (slices <= 0 || gh <= 0 || gw <= 0) return 0;
    // sized for the largest split the planner can choose on a 256-CU device
    const ConvPlan p = plan_conv((int)slices, gh, gw, 2, 256);
    const ConvPlan q = plan_conv((int)slices, gh, gw, 4, 256);
    const int S = p.S > q.S ? p.S : q.S;
    if (S <= 1) return 0;
    return kCounterBytes + (size_t)slices * S * 576 * 4;
}

int conv_resident_per_cu(int bf16) {
    static std::atomic<int> cached[2];
    int n = cached[bf16 ? 1 : 0].load(std::memory_order_relaxed);
    if (n > 0) return n;
    hipError_t e = bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, conv_kernel<true, true>, kCT, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, conv_kernel<false, true>, kCT, 0);
    if (e != hipSuccess || n < 0) return 0;
    cached[bf16 ? 1 : 0].store(n, std::memory_order_relaxed);
    return n;
}

void conv_prepare(const ConvLaunch& l, ConvArgs& a, unsigned& grid) {
    const long long slices = (long long)l.B * l.H;
    const int esz = l.bf16 ? 2 : 4;
    const int cap = l.cap < 256 ? l.cap : 256; // the workspace is sized for 256
    ConvPlan p = plan_conv((int)slices, l.gh, l.gw, esz, cap);
    a = ConvArgs{};
    a.K = l.K; a.Q = l.Q; a.V = l.V; a.Z = l.Z;
    a.w0 = l.w0; a.eta = l.eta; a.saved = l.saved;
    a.H = l.H; a.gh = l.gh; a.gw = l.gw;
    a.R = p.R; a.TW = p.TW; a.ny = p.ny; a.nx = p.nx; a.S = p.S; a.tpw = p.tpw;
    a.slices = (int)slices;
    a.xcd = (p.S > 1 && l.xcd_ok) ? 1 : 0;
    a.spin = l.spin;
    a.tbias = l.tbias;
    a.dot = l.dot;
    if (p.S > 1) {
        // workspace layout as conv_ws_bytes: fixed counter block, partials
        char* base = (char*)l.ws;
        a.cnt = (unsigned*)base;
        a.part = l.part ? (float*)l.part : (float*)(base + kCounterBytes);
    }
    const long long gslices = a.xcd ? (slices + 7) / 8 * 8 : slices;
    grid = (unsigned)(gslices * p.S);
}

void conv_plan_info(const ConvLaunch& l, int* S, int* xcd) {
    ConvArgs a;
    unsigned grid = 0;
    conv_prepare(l, a, grid);
    *S = a.S;
    *xcd = a.xcd;
}

hipError_t conv_launch_prepared(const ConvArgs& a0, unsigned grid, int bf16, hipStream_t stream) {
    ConvArgs a = a0;
    void* args[] = {&a};
    const void* fn = a.xcd ? (bf16 ? (const void*)conv_kernel<true, true> : (const void*)conv_kernel<false, true>)
                           : (bf16 ? (const void*)conv_kernel<true, false> : (const void*)conv_kernel<false, false>);
    return hipLaunchKernel(fn, dim3(grid), dim3(kCT), args, 0, stream);
}

hipError_t launch_conv(ConvLaunch l, hipStream_t stream) {
    const long long slices = (long long)l.B * l.H;
    ConvArgs a;
    unsigned grid = 0;
    conv_prepare(l, a, grid);
    if (a.S > 1 && slices > kMaxBarrierSlices) return hipErrorInvalidValue; // unreachable: S > 1
    return conv_launch_prepared(a, grid, l.bf16, stream);
}

} // namespace ttt
