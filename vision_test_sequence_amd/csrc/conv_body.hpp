// conv_body.hpp -- device code of the full-batch step of the 3x3
// depthwise-convolution inner model (ViT3 article, observation 6), shared by
// the conv kernel and the fused layer kernel.  The method and the phases
// are described in dwconv3x3.hip.
#pragma once

#include "common.hpp"
#include "internal.hpp"

#include <type_traits>

namespace ttt {

struct ConvArgs {
    View4 K, Q, V, Z;
    const float* w0;
    const float* eta;
    float* saved;
    float* part;       // [slices][S][64][9]
    unsigned* cnt;     // [slices]
    int H, gh, gw;
    int R, TW;         // tile rows / columns
    int ny, nx;        // tiles per slice along y / x
    int S;             // workgroups per slice
    int tpw;           // tiles per workgroup
    int slices;        // B * H
    int xcd;           // XCD-aware grid and XCD-local exchange
    unsigned spin;     // slice barrier: poll limit
    unsigned tbias;    // slice barrier: added to every target (0)
    int dot;           // dot-product loss: R = -V (no w0 term), scale 1/N
};

// Plan of a conv call (tiles, splits, the exchange protocol) as kernel
// arguments and grid size; defined with the conv kernel.
void conv_prepare(const ConvLaunch& l, ConvArgs& a, unsigned& grid);
hipError_t conv_launch_prepared(const ConvArgs& a, unsigned grid, int bf16, hipStream_t stream);

namespace {

constexpr int kTileBytes = 147456;           // K halo + V + Q halo regions
constexpr int kW0Bytes = 3 * 1024;           // w0 of the head, 576 floats (3 staging instructions)
constexpr int kCT = 512;                     // threads per workgroup: 8 waves, 2 per SIMD
constexpr int kCW = kCT / 64;
constexpr int kRedFloats = 4 * 64 * 9;       // tap sums of 4 waves (the 8 are paired first)
constexpr int kSeg = 16;                     // pixels per row segment


template <bool BF> struct ConvT;
template <> struct ConvT<true> {
    static constexpr int esz = 2;
    typedef uint16_t raw_t;
    __device__ static raw_t raw(const char* p) { return *(const uint16_t*)p; }
    __device__ static float cvt(raw_t v) { return __uint_as_float((uint32_t)v << 16); }
    __device__ static float ld(const char* p) { return __uint_as_float((uint32_t)*(const uint16_t*)p << 16); }
    __device__ static void st(char* p, float v) { __builtin_nontemporal_store(f2bf(v), (uint16_t*)p); }
};
template <> struct ConvT<false> {
    static constexpr int esz = 4;
    typedef float raw_t;
    __device__ static raw_t raw(const char* p) { return *(const float*)p; }
    __device__ static float cvt(raw_t v) { return v; }
    __device__ static float ld(const char* p) { return *(const float*)p; }
    __device__ static void st(char* p, float v) { __builtin_nontemporal_store(v, (float*)p); }
};

// Zero pixel: the source of every staged position outside the grid, so
// the halo reads zero padding with no masks and no clearing pass.
__device__ __attribute__((aligned(256))) u32x4 conv_zero_px[16];

// Pixels per direct-to-LDS instruction (64 lanes x 16 bytes): LDS row
// pitches are multiples of it, so every row is whole instructions.
template <bool BF> constexpr int px_per_instr() { return 64 * 16 / (64 * ConvT<BF>::esz); }
template <bool BF> __host__ __device__ constexpr int conv_pitch(int px) {
    return (px + px_per_instr<BF>() - 1) / px_per_instr<BF>() * px_per_instr<BF>();
}

// Stage `rows` rows of `pitch` pixels whose top-left grid position is
// (ya, xa) into LDS at dst (row-major, pixel-contiguous), as direct
// global->LDS loads hidden from the compiler: instruction i of the block
// (1 KB of LDS) is issued by wave i mod 8.  Positions outside the grid
// load the zero pixel.  Returns the number of instructions this wave
// issued; the caller waits for them with vmcnt_at_most().
template <bool BF>
__device__ __forceinline__ int stage_rows(char* dst, const char* src, long long sn, int ya, int xa,
                                          int rows, int pitch, int gh, int gw) {
    constexpr int cpp = 64 * ConvT<BF>::esz / 16; // 16-byte chunks per pixel
    const int ninstr = rows * pitch * cpp / 64;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const char* zero = reinterpret_cast<const char*>(conv_zero_px);
    int n = 0;
    for (int i = w; i < ninstr; i += kCW, ++n) {
        const int q = i * 64 + lane;
        const int px = q / cpp, sub = q % cpp;
        const int y = ya + px / pitch, x = xa + px % pitch;
        const bool in = y >= 0 && y < gh && x >= 0 && x < gw;
        const char* g = in ? src + ((long long)y * gw + x) * sn + sub * 16 : zero + sub * 16;
        dma16(g, dst + i * 1024);
    }
    return n;
}

// w0 of one head (576 floats) into LDS: three instructions, by waves 0-2.
__device__ __forceinline__ int stage_w0(char* dst, const float* w0h) {
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= 3) return 0;
    const int q = w * 64 + lane; // 16-byte chunk
    const char* g = q < 144 ? reinterpret_cast<const char*>(w0h) + q * 16
                            : reinterpret_cast<const char*>(conv_zero_px);
    dma16(g, dst + w * 1024);
    return 1;
}

// bf16 -> fp32 without conversion instructions: ds_read_u16_d16_hi writes a
// register's high half and keeps its low half, so a register whose low half
// is zero holds the exact fp32 value of the bf16 it receives.  The callers'
// registers start at zero and receive nothing else.  Each asm block issues
// its loads and waits for them itself, so every output is complete when the
// block ends.  Rows are LDS addresses of 18 consecutive pixels (128-byte
// pitch: one bf16 per lane of 64 channels).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
// three rows of 18 pixels (K halo) and 16 pixels of one row (V)
__device__ __forceinline__ void lds_window_kv(float (&k)[3][kSeg + 2], float (&v)[kSeg], const char* k0,
                                              const char* k1, const char* k2, const char* v0) {
    static_assert(kSeg == 16, "the asm below is written for 16-pixel segments");
    asm volatile(
        "ds_read_u16_d16_hi %0, %70 offset:0\n\t" "ds_read_u16_d16_hi %1, %70 offset:128\n\t" "ds_read_u16_d16_hi %2, %70 offset:256\n\t"
        "ds_read_u16_d16_hi %3, %70 offset:384\n\t" "ds_read_u16_d16_hi %4, %70 offset:512\n\t" "ds_read_u16_d16_hi %5, %70 offset:640\n\t"
        "ds_read_u16_d16_hi %6, %70 offset:768\n\t" "ds_read_u16_d16_hi %7, %70 offset:896\n\t" "ds_read_u16_d16_hi %8, %70 offset:1024\n\t"
        "ds_read_u16_d16_hi %9, %70 offset:1152\n\t" "ds_read_u16_d16_hi %10, %70 offset:1280\n\t" "ds_read_u16_d16_hi %11, %70 offset:1408\n\t"
        "ds_read_u16_d16_hi %12, %70 offset:1536\n\t" "ds_read_u16_d16_hi %13, %70 offset:1664\n\t" "ds_read_u16_d16_hi %14, %70 offset:1792\n\t"
        "ds_read_u16_d16_hi %15, %70 offset:1920\n\t" "ds_read_u16_d16_hi %16, %70 offset:2048\n\t" "ds_read_u16_d16_hi %17, %70 offset:2176\n\t"
        "ds_read_u16_d16_hi %18, %71 offset:0\n\t" "ds_read_u16_d16_hi %19, %71 offset:128\n\t" "ds_read_u16_d16_hi %20, %71 offset:256\n\t"
        "ds_read_u16_d16_hi %21, %71 offset:384\n\t" "ds_read_u16_d16_hi %22, %71 offset:512\n\t" "ds_read_u16_d16_hi %23, %71 offset:640\n\t"
        "ds_read_u16_d16_hi %24, %71 offset:768\n\t" "ds_read_u16_d16_hi %25, %71 offset:896\n\t" "ds_read_u16_d16_hi %26, %71 offset:1024\n\t"
        "ds_read_u16_d16_hi %27, %71 offset:1152\n\t" "ds_read_u16_d16_hi %28, %71 offset:1280\n\t" "ds_read_u16_d16_hi %29, %71 offset:1408\n\t"
        "ds_read_u16_d16_hi %30, %71 offset:1536\n\t" "ds_read_u16_d16_hi %31, %71 offset:1664\n\t" "ds_read_u16_d16_hi %32, %71 offset:1792\n\t"
        "ds_read_u16_d16_hi %33, %71 offset:1920\n\t" "ds_read_u16_d16_hi %34, %71 offset:2048\n\t" "ds_read_u16_d16_hi %35, %71 offset:2176\n\t"
        "ds_read_u16_d16_hi %36, %72 offset:0\n\t" "ds_read_u16_d16_hi %37, %72 offset:128\n\t" "ds_read_u16_d16_hi %38, %72 offset:256\n\t"
        "ds_read_u16_d16_hi %39, %72 offset:384\n\t" "ds_read_u16_d16_hi %40, %72 offset:512\n\t" "ds_read_u16_d16_hi %41, %72 offset:640\n\t"
        "ds_read_u16_d16_hi %42, %72 offset:768\n\t" "ds_read_u16_d16_hi %43, %72 offset:896\n\t" "ds_read_u16_d16_hi %44, %72 offset:1024\n\t"
        "ds_read_u16_d16_hi %45, %72 offset:1152\n\t" "ds_read_u16_d16_hi %46, %72 offset:1280\n\t" "ds_read_u16_d16_hi %47, %72 offset:1408\n\t"
        "ds_read_u16_d16_hi %48, %72 offset:1536\n\t" "ds_read_u16_d16_hi %49, %72 offset:1664\n\t" "ds_read_u16_d16_hi %50, %72 offset:1792\n\t"
        "ds_read_u16_d16_hi %51, %72 offset:1920\n\t" "ds_read_u16_d16_hi %52, %72 offset:2048\n\t" "ds_read_u16_d16_hi %53, %72 offset:2176\n\t"
        "ds_read_u16_d16_hi %54, %73 offset:0\n\t" "ds_read_u16_d16_hi %55, %73 offset:128\n\t" "ds_read_u16_d16_hi %56, %73 offset:256\n\t"
        "ds_read_u16_d16_hi %57, %73 offset:384\n\t" "ds_read_u16_d16_hi %58, %73 offset:512\n\t" "ds_read_u16_d16_hi %59, %73 offset:640\n\t"
        "ds_read_u16_d16_hi %60, %73 offset:768\n\t" "ds_read_u16_d16_hi %61, %73 offset:896\n\t" "ds_read_u16_d16_hi %62, %73 offset:1024\n\t"
        "ds_read_u16_d16_hi %63, %73 offset:1152\n\t" "ds_read_u16_d16_hi %64, %73 offset:1280\n\t" "ds_read_u16_d16_hi %65, %73 offset:1408\n\t"
        "ds_read_u16_d16_hi %66, %73 offset:1536\n\t" "ds_read_u16_d16_hi %67, %73 offset:1664\n\t" "ds_read_u16_d16_hi %68, %73 offset:1792\n\t"
        "ds_read_u16_d16_hi %69, %73 offset:1920\n\t" "s_waitcnt lgkmcnt(0)"
        : "+v"(k[0][0]), "+v"(k[0][1]), "+v"(k[0][2]), "+v"(k[0][3]), "+v"(k[0][4]), "+v"(k[0][5]),
          "+v"(k[0][6]), "+v"(k[0][7]), "+v"(k[0][8]), "+v"(k[0][9]), "+v"(k[0][10]), "+v"(k[0][11]),
          "+v"(k[0][12]), "+v"(k[0][13]), "+v"(k[0][14]), "+v"(k[0][15]), "+v"(k[0][16]), "+v"(k[0][17]),
          "+v"(k[1][0]), "+v"(k[1][1]), "+v"(k[1][2]), "+v"(k[1][3]), "+v"(k[1][4]), "+v"(k[1][5]),
          "+v"(k[1][6]), "+v"(k[1][7]), "+v"(k[1][8]), "+v"(k[1][9]), "+v"(k[1][10]), "+v"(k[1][11]),
          "+v"(k[1][12]), "+v"(k[1][13]), "+v"(k[1][14]), "+v"(k[1][15]), "+v"(k[1][16]), "+v"(k[1][17]),
          "+v"(k[2][0]), "+v"(k[2][1]), "+v"(k[2][2]), "+v"(k[2][3]), "+v"(k[2][4]), "+v"(k[2][5]),
          "+v"(k[2][6]), "+v"(k[2][7]), "+v"(k[2][8]), "+v"(k[2][9]), "+v"(k[2][10]), "+v"(k[2][11]),
          "+v"(k[2][12]), "+v"(k[2][13]), "+v"(k[2][14]), "+v"(k[2][15]), "+v"(k[2][16]), "+v"(k[2][17]),
          "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
          "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
        : "v"(lds_addr(k0)), "v"(lds_addr(k1)), "v"(lds_addr(k2)), "v"(lds_addr(v0))
        : "memory");
}
// three rows of 18 pixels (Q halo)
__device__ __forceinline__ void lds_window_q(float (&q)[3][kSeg + 2], const char* q0, const char* q1,
                                             const char* q2) {
    static_assert(kSeg == 16, "the asm below is written for 16-pixel segments");
    asm volatile(
        "ds_read_u16_d16_hi %0, %54 offset:0\n\t" "ds_read_u16_d16_hi %1, %54 offset:128\n\t" "ds_read_u16_d16_hi %2, %54 offset:256\n\t"
        "ds_read_u16_d16_hi %3, %54 offset:384\n\t" "ds_read_u16_d16_hi %4, %54 offset:512\n\t" "ds_read_u16_d16_hi %5, %54 offset:640\n\t"
        "ds_read_u16_d16_hi %6, %54 offset:768\n\t" "ds_read_u16_d16_hi %7, %54 offset:896\n\t" "ds_read_u16_d16_hi %8, %54 offset:1024\n\t"
        "ds_read_u16_d16_hi %9, %54 offset:1152\n\t" "ds_read_u16_d16_hi %10, %54 offset:1280\n\t" "ds_read_u16_d16_hi %11, %54 offset:1408\n\t"
        "ds_read_u16_d16_hi %12, %54 offset:1536\n\t" "ds_read_u16_d16_hi %13, %54 offset:1664\n\t" "ds_read_u16_d16_hi %14, %54 offset:1792\n\t"
        "ds_read_u16_d16_hi %15, %54 offset:1920\n\t" "ds_read_u16_d16_hi %16, %54 offset:2048\n\t" "ds_read_u16_d16_hi %17, %54 offset:2176\n\t"
        "ds_read_u16_d16_hi %18, %55 offset:0\n\t" "ds_read_u16_d16_hi %19, %55 offset:128\n\t" "ds_read_u16_d16_hi %20, %55 offset:256\n\t"
        "ds_read_u16_d16_hi %21, %55 offset:384\n\t" "ds_read_u16_d16_hi %22, %55 offset:512\n\t" "ds_read_u16_d16_hi %23, %55 offset:640\n\t"
        "ds_read_u16_d16_hi %24, %55 offset:768\n\t" "ds_read_u16_d16_hi %25, %55 offset:896\n\t" "ds_read_u16_d16_hi %26, %55 offset:1024\n\t"
        "ds_read_u16_d16_hi %27, %55 offset:1152\n\t" "ds_read_u16_d16_hi %28, %55 offset:1280\n\t" "ds_read_u16_d16_hi %29, %55 offset:1408\n\t"
        "ds_read_u16_d16_hi %30, %55 offset:1536\n\t" "ds_read_u16_d16_hi %31, %55 offset:1664\n\t" "ds_read_u16_d16_hi %32, %55 offset:1792\n\t"
        "ds_read_u16_d16_hi %33, %55 offset:1920\n\t" "ds_read_u16_d16_hi %34, %55 offset:2048\n\t" "ds_read_u16_d16_hi %35, %55 offset:2176\n\t"
        "ds_read_u16_d16_hi %36, %56 offset:0\n\t" "ds_read_u16_d16_hi %37, %56 offset:128\n\t" "ds_read_u16_d16_hi %38, %56 offset:256\n\t"
        "ds_read_u16_d16_hi %39, %56 offset:384\n\t" "ds_read_u16_d16_hi %40, %56 offset:512\n\t" "ds_read_u16_d16_hi %41, %56 offset:640\n\t"
        "ds_read_u16_d16_hi %42, %56 offset:768\n\t" "ds_read_u16_d16_hi %43, %56 offset:896\n\t" "ds_read_u16_d16_hi %44, %56 offset:1024\n\t"
        "ds_read_u16_d16_hi %45, %56 offset:1152\n\t" "ds_read_u16_d16_hi %46, %56 offset:1280\n\t" "ds_read_u16_d16_hi %47, %56 offset:1408\n\t"
        "ds_read_u16_d16_hi %48, %56 offset:1536\n\t" "ds_read_u16_d16_hi %49, %56 offset:1664\n\t" "ds_read_u16_d16_hi %50, %56 offset:1792\n\t"
        "ds_read_u16_d16_hi %51, %56 offset:1920\n\t" "ds_read_u16_d16_hi %52, %56 offset:2048\n\t" "ds_read_u16_d16_hi %53, %56 offset:2176\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "+v"(q[0][0]), "+v"(q[0][1]), "+v"(q[0][2]), "+v"(q[0][3]), "+v"(q[0][4]), "+v"(q[0][5]),
          "+v"(q[0][6]), "+v"(q[0][7]), "+v"(q[0][8]), "+v"(q[0][9]), "+v"(q[0][10]), "+v"(q[0][11]),
          "+v"(q[0][12]), "+v"(q[0][13]), "+v"(q[0][14]), "+v"(q[0][15]), "+v"(q[0][16]), "+v"(q[0][17]),
          "+v"(q[1][0]), "+v"(q[1][1]), "+v"(q[1][2]), "+v"(q[1][3]), "+v"(q[1][4]), "+v"(q[1][5]),
          "+v"(q[1][6]), "+v"(q[1][7]), "+v"(q[1][8]), "+v"(q[1][9]), "+v"(q[1][10]), "+v"(q[1][11]),
          "+v"(q[1][12]), "+v"(q[1][13]), "+v"(q[1][14]), "+v"(q[1][15]), "+v"(q[1][16]), "+v"(q[1][17]),
          "+v"(q[2][0]), "+v"(q[2][1]), "+v"(q[2][2]), "+v"(q[2][3]), "+v"(q[2][4]), "+v"(q[2][5]),
          "+v"(q[2][6]), "+v"(q[2][7]), "+v"(q[2][8]), "+v"(q[2][9]), "+v"(q[2][10]), "+v"(q[2][11]),
          "+v"(q[2][12]), "+v"(q[2][13]), "+v"(q[2][14]), "+v"(q[2][15]), "+v"(q[2][16]), "+v"(q[2][17])
        : "v"(lds_addr(q0)), "v"(lds_addr(q1)), "v"(lds_addr(q2))
        : "memory");
}

// The workgroup's (slice, split): XCD-aware grids place by the XCD the
// workgroup runs on (map_block_xcc).
template <bool XC> __device__ __forceinline__ SliceSplit conv_slice_split(const ConvArgs& a) {
    return XC ? map_block_xcc(blockIdx.x, a.S, xcc_id()) : map_block(blockIdx.x, a.S, 0);
}

// LDS of one workgroup: `tile` holds w0 (kW0Bytes), the K halo rows and
// the V rows of a tile; `qs` the Q halo rows (null: right after V);
// red (kRedFloats), w1s (576 floats) and chk are small scratch.
struct ConvLds {
    char* tile;
    char* qs;
    float* red;
    float* w1s;
    int* chk;
};
template <bool BF> __host__ __device__ constexpr int conv_kv_bytes(int R, int TW) {
    return kW0Bytes + ((R + 2) * conv_pitch<BF>((TW > kSeg ? TW : kSeg) + 2) + R * conv_pitch<BF>(TW > kSeg ? TW : kSeg)) *
                          64 * ConvT<BF>::esz;
}
template <bool BF> __host__ __device__ constexpr int conv_q_bytes(int R, int TW) {
    return (R + 2) * conv_pitch<BF>((TW > kSeg ? TW : kSeg) + 2) * 64 * ConvT<BF>::esz;
}

// The whole step for one workgroup, 8 waves (two per SIMD: while one waits
// for its LDS reads the other computes).
template <bool BF, bool XC>
__device__ __forceinline__ void conv_body(const ConvArgs& a, const ConvLds& L) {
    using T = ConvT<BF>;
    constexpr int pb = 64 * T::esz; // bytes per pixel
    float* red = L.red;
    float* w1s = L.w1s;
    int& s_chk = *L.chk;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6); // wave index, uniform
    const SliceSplit ss = conv_slice_split<XC>(a);
    const int slice = ss.slice, split = ss.split;
    if (slice >= a.slices) return; // padding block of the XCD-aware grid
    if (XC && a.S > 1 && tid == 0) placement_note(counter_at(a.cnt, slice), split);
    bool poison = false; // NaN output for a failed exchange
    const int b = slice / a.H, h = slice % a.H;
    const int gh = a.gh, gw = a.gw, N = gh * gw;
    const int ntile = a.ny * a.nx;
    const int tb = split * a.tpw, te = min(ntile, tb + a.tpw);

    const char* Kp = (const char*)a.K.ptr + (b * a.K.sb + h * a.K.sh) * (long long)T::esz;
    const char* Vp = (const char*)a.V.ptr + (b * a.V.sb + h * a.V.sh) * (long long)T::esz;
    const char* Qp = (const char*)a.Q.ptr + (b * a.Q.sb + h * a.Q.sh) * (long long)T::esz;
    char* Zp = (char*)a.Z.ptr + (b * a.Z.sb + h * a.Z.sh) * (long long)T::esz;
    const long long Ksn = a.K.sn * T::esz, Vsn = a.V.sn * T::esz;
    const long long Qsn = a.Q.sn * T::esz, Zsn = a.Z.sn * T::esz;

    // LDS rows are at least kSeg pixels wide (plus the halo), so a row
    // segment of kSeg pixels never reads past its row; pitches are whole
    // staging instructions; positions outside the grid hold zeros (K, Q) or
    // are masked (V)
    const int KP = conv_pitch<BF>(max(a.TW, kSeg) + 2), VP = conv_pitch<BF>(max(a.TW, kSeg));
    char* W0s = L.tile;
    char* Ks = L.tile + kW0Bytes;
    char* Vs = Ks + (a.R + 2) * KP * pb;
    char* Qs = L.qs ? L.qs : Vs + a.R * VP * pb;
    const bool q_early = (te - tb) == 1;

    float gacc[9];
#pragma unroll
    for (int t = 0; t < 9; ++t) gacc[t] = 0.f;
    float wt[9];
#pragma unroll
    for (int t = 0; t < 9; ++t) wt[t] = 0.f;
    float pf = 0.f; // L2 prefetch of this workgroup's partial (see below)
    // the 3x3 window's registers (bf16: low halves stay zero, lds_window_*)
    float kr[3][kSeg + 2], vv[kSeg];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < kSeg + 2; ++j) kr[i][j] = 0.f;
#pragma unroll
    for (int j = 0; j < kSeg; ++j) vv[j] = 0.f;
    unsigned rel = 0; // thread 0: the counter before this workgroup's release

    // ------------------------------------------------------------ phase 1
    for (int tile = tb; tile < te; ++tile) {
        const int y0 = (tile / a.nx) * a.R, x0 = (tile % a.nx) * a.TW;
        const int rr = min(a.R, gh - y0), tw = min(a.TW, gw - x0);
        // always the nominal tile shape, so the LDS pitches are fixed; the
        // part of an edge tile outside the grid is zero or masked.  (The
        // whole chip issues its loads at once and the memory system does
        // not serve them in issue order, so staging the rows in the order
        // they are needed and starting on the first ones measured no
        // earlier start.)
        if (tile == tb) stage_w0(W0s, a.w0 + (long long)h * 576);
        stage_rows<BF>(Ks, Kp, Ksn, y0 - 1, x0 - 1, a.R + 2, KP, gh, gw);
        stage_rows<BF>(Vs, Vp, Vsn, y0, x0, a.R, VP, gh, gw);
        int nq = 0;
        if (q_early) nq = stage_rows<BF>(Qs, Qp, Qsn, y0 - 1, x0 - 1, a.R + 2, KP, gh, gw);
        vmcnt_at_most(nq); // this wave's K and V (and w0) loads have landed
        lds_barrier();     // ... and every wave's
        if (tile == tb) {
#pragma unroll
            for (int t = 0; t < 9; ++t) wt[t] = a.dot ? 0.f : reinterpret_cast<const float*>(W0s)[lane * 9 + t];
            // A store to a line that is not in the XCD's L2 goes on to
            // memory without allocating it, and the slice's other
            // workgroups would then read the partial from memory: a
            // device-scope load of each of its 18 lines (it fills L2, not
            // L1) makes the later stores and reads hit L2.
            if (XC && a.S > 1 && w == 0)
                pf = xload(a.part + ((long long)slice * a.S + split) * 576 + min(lane, 17) * 32);
        }

        const int nsx = (tw + kSeg - 1) / kSeg;
        {
            for (int sgi = w; sgi < rr * nsx; sgi += kCW) {
                const int r = sgi / nsx;
                // Segment k of a row covers pixels [16k, 16k+16); the last one is
                // shifted left to end at the row's end (its first pixels, done by
                // the previous segment, are masked) -- or, in a row narrower than
                // a segment, starts at 0 and masks the pixels past the row.  Every
                // LDS value a segment needs is read up front at fixed offsets
                // from one base, then the 3x3 window slides in registers.
                const int k = sgi % nsx;
                const int xs = min(k * kSeg, max(tw - kSeg, 0));
                const int lo = k * kSeg - xs, hi = min(kSeg, tw - xs);
                const char* kb = Ks + ((r * KP + xs) * 64 + lane) * T::esz;
                const char* vb = Vs + ((r * VP + xs) * 64 + lane) * T::esz;
                if constexpr (BF) {
                    lds_window_kv(kr, vv, kb, kb + KP * pb, kb + 2 * KP * pb, vb);
                } else {
                    typename T::raw_t kraw[3][kSeg + 2], vraw[kSeg];
#pragma unroll
                    for (int i = 0; i < 3; ++i)
#pragma unroll
                        for (int j = 0; j < kSeg + 2; ++j) kraw[i][j] = T::raw(kb + ((i * KP + j) * 64) * T::esz);
#pragma unroll
                    for (int j = 0; j < kSeg; ++j) vraw[j] = T::raw(vb + (j * 64) * T::esz);
                    __builtin_amdgcn_sched_barrier(0); // all reads in flight before the arithmetic
#pragma unroll
                    for (int i = 0; i < 3; ++i)
#pragma unroll
                        for (int j = 0; j < kSeg + 2; ++j) kr[i][j] = T::cvt(kraw[i][j]);
#pragma unroll
                    for (int j = 0; j < kSeg; ++j) vv[j] = T::cvt(vraw[j]);
                }
                // R = P - V as one fused multiply-add chain from -V per
                // pixel, branch-free, so the 16 pixels' chains interleave.
                // A segment with masked pixels (the last of a row) gives
                // them R = 0 through a 0/1 factor (their values are finite:
                // in-grid or zero pixels).
                auto grad = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
                    for (int x = 0; x < kSeg; ++x) {
                        float rv = -vv[x];
#pragma unroll
                        for (int i = 0; i < 3; ++i)
#pragma unroll
                            for (int jj = 0; jj < 3; ++jj) rv = __builtin_fmaf(wt[i * 3 + jj], kr[i][x + jj], rv);
                        if constexpr (decltype(masked)::value) rv *= (x >= lo && x < hi) ? 1.f : 0.f;
#pragma unroll
                        for (int i = 0; i < 3; ++i)
#pragma unroll
                            for (int jj = 0; jj < 3; ++jj) gacc[i * 3 + jj] = __builtin_fmaf(rv, kr[i][x + jj], gacc[i * 3 + jj]);
                    }
                };
                if (lo == 0 && hi == kSeg) grad(std::false_type{});
                else grad(std::true_type{});
            }
        }
        lds_barrier(); // every wave is done with this tile's K and V
    }

    // fixed-order sum of the 8 waves' tap sums: waves w and w + 4 first,
    // then the four pair sums
    if (w >= 4) {
#pragma unroll
        for (int t = 0; t < 9; ++t) red[((w - 4) * 64 + lane) * 9 + t] = gacc[t];
    }
    __syncthreads();
    if (w < 4) {
#pragma unroll
        for (int t = 0; t < 9; ++t) red[(w * 64 + lane) * 9 + t] = gacc[t] + red[(w * 64 + lane) * 9 + t];
    }
    __syncthreads();
    const float eta = a.eta[h];
    const float scale = (a.dot ? 1.0f : 2.0f) / (float)N;
    if (a.S == 1) {
        if (w == 0) {
            for (int t = 0; t < 9; ++t) {
                const float s = ((red[lane * 9 + t] + red[(64 + lane) * 9 + t]) + red[(128 + lane) * 9 + t]) +
                                red[(192 + lane) * 9 + t];
                const float gv = scale * s;
                w1s[lane * 9 + t] = reinterpret_cast<const float*>(W0s)[lane * 9 + t] - eta * gv;
                if (a.saved) a.saved[((long long)slice * 64 + lane) * 9 + t] = gv;
            }
        }
        __syncthreads();
    } else {
        float* P = a.part + ((long long)slice * a.S + split) * 576;
        unsigned* cnt = counter_at(a.cnt, slice);
        asm volatile("" ::"v"(pf)); // the prefetch has completed before the stores
        for (int e = tid; e < 576; e += kCT) {
            const int c = e / 9, t = e % 9;
            const float v = ((red[c * 9 + t] + red[(64 + c) * 9 + t]) + red[(128 + c) * 9 + t]) +
                            red[(192 + c) * 9 + t];
            if constexpr (XC) P[e] = v;
            else xstore(P + e, v);
        }
        slice_barrier(cnt, (unsigned)a.S + a.tbias, true, a.spin);
        SliceWords sw{}; // thread 0; loaded after the partials (see below)
        float gv[4];
        // Every workgroup sums all S partials itself (576 floats each, in
        // a fixed order, so all of them form the same w1): one barrier, and
        // no second round trip for w1.  Threads t < 432 share the loads:
        // element group e4 = t % 144 (floats 4 e4..4 e4+3) of the splits in
        // group t / 144 of three (consecutive runs of ceil(S/3) <= 11
        // splits, S <= 32: the grid holds at most 256 workgroups of >= 8
        // slices); the three group sums meet in LDS.
        float* gsum = red; // [3][576], free once the partial is published
        if (tid < 432) {
            const int e4 = tid % 144, q = tid / 144;
            const int G = (a.S + 2) / 3, s0 = q * G, s1 = min(a.S, s0 + G);
            const float* src = a.part + (long long)slice * a.S * 576 + 4 * e4;
            f32x4 v[11];
#pragma unroll
            for (int k = 0; k < 11; ++k) {
                if (k < G) { // uniform
                    const float* p = src + min(s0 + k, s1 - 1) * 576;
                    if constexpr (XC) v[k] = *reinterpret_cast<const f32x4*>(p);
                    else v[k] = f32x4{xload(p), xload(p + 1), xload(p + 2), xload(p + 3)};
                }
            }
            // the counter line's words after the partials: the CU returns
            // vector-memory results in issue order, and that line is still
            // contended by the slice's polls and releases
            if (tid == 0) sw = slice_words(cnt);
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 11; ++k)
                if (k < G && s0 + k < s1) acc += v[k];
            *reinterpret_cast<f32x4*>(gsum + q * 576 + 4 * e4) = acc;
        }
        __syncthreads();
        if (tid < 144) {
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(gsum + 4 * tid);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(gsum + 576 + 4 * tid);
            const f32x4 g2 = *reinterpret_cast<const f32x4*>(gsum + 1152 + 4 * tid);
            const f32x4 acc = (g0 + g1) + g2;
            const float* w0e = reinterpret_cast<const float*>(W0s) + 4 * tid; // w0 of the head, staged
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                gv[k] = scale * acc[k];
                w1s[4 * tid + k] = w0e[k] - eta * gv[k];
            }
        }
        if (tid == 0) s_chk = slice_bad(sw, XC ? a.S : 0) ? 1 : 0;
        __syncthreads();
        poison = s_chk != 0;
        if (a.saved && split == 0 && tid < 144) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                a.saved[(long long)slice * 576 + 4 * tid + k] = poison ? __builtin_nanf("") : gv[k];
        }
        // The counter's release, once the partials are read (vector-memory
        // results return in issue order across the CU's waves, so an
        // atomic on the slice's contended counter line issued earlier
        // would hold up their loads); its result (does this workgroup
        // complete the count and reset it?) is used at the end.
        if (tid == 0) rel = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (q_early && a.S == 1) { // (with S > 1 the slice barrier drained every wave)
        drain_vmem();           // this wave's Q loads have landed
        __syncthreads();        // ... and every wave's
    }
    float wq[9];
#pragma unroll
    for (int t = 0; t < 9; ++t) wq[t] = w1s[lane * 9 + t];

    // ------------------------------------------------------------ phase 3
    for (int tile = tb; tile < te; ++tile) {
        const int y0 = (tile / a.nx) * a.R, x0 = (tile % a.nx) * a.TW;
        const int rr = min(a.R, gh - y0), tw = min(a.TW, gw - x0);
        if (!q_early) {
            stage_rows<BF>(Qs, Qp, Qsn, y0 - 1, x0 - 1, a.R + 2, KP, gh, gw);
            drain_vmem();
            __syncthreads();
        }
        const int nsx = (tw + kSeg - 1) / kSeg;
        for (int sgi = w; sgi < rr * nsx; sgi += kCW) {
            const int r = sgi / nsx, k = sgi % nsx; // segments as in phase 1
            const int xs = min(k * kSeg, max(tw - kSeg, 0));
            const int lo = k * kSeg - xs, hi = min(kSeg, tw - xs);
            const int y = y0 + r;
            const char* qb = Qs + ((r * KP + xs) * 64 + lane) * T::esz;
            char* zrow = Zp + ((long long)y * gw + x0 + xs) * Zsn + lane * T::esz;
            float (&qr)[3][kSeg + 2] = kr; // the window's registers again (low halves zero)
            if constexpr (BF) {
                lds_window_q(qr, qb, qb + KP * pb, qb + 2 * KP * pb);
            } else {
                typename T::raw_t qraw[3][kSeg + 2];
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int j = 0; j < kSeg + 2; ++j) qraw[i][j] = T::raw(qb + ((i * KP + j) * 64) * T::esz);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int j = 0; j < kSeg + 2; ++j) qr[i][j] = T::cvt(qraw[i][j]);
            }
            auto zpix = [&](int x) __attribute__((always_inline)) {
                float z = wq[0] * qr[0][x];
#pragma unroll
                for (int t = 1; t < 9; ++t) z = __builtin_fmaf(wq[t], qr[t / 3][x + t % 3], z);
                return poison ? __builtin_nanf("") : z;
            };
            if constexpr (BF) {
                // Eight pixels at a time through 1 KB of LDS private to the
                // wave (in the K/V region, free after phase 1): each lane
                // writes its channel, then stores 16 contiguous bytes (8
                // channels of one pixel) -- one 1 KB store instruction
                // instead of eight of 128 bytes.  (The K region holds at
                // least 3 rows of 24 pixels: 9 KB >= 8 waves x 1 KB.)
                char* zs = Ks + w * 1024;
#pragma unroll
                for (int h8 = 0; h8 < kSeg / 8; ++h8) {
#pragma unroll
                    for (int x8 = 0; x8 < 8; ++x8)
                        *reinterpret_cast<bf16_t*>(zs + x8 * 128 + lane * 2) = f2bf(zpix(8 * h8 + x8));
                    const u32x4 v = *reinterpret_cast<const u32x4*>(zs + lane * 16);
                    const int px = 8 * h8 + (lane >> 3);
                    if (px >= lo && px < hi)
                        __builtin_nontemporal_store(
                            v, reinterpret_cast<u32x4*>(Zp + ((long long)y * gw + x0 + xs + px) * Zsn + (lane & 7) * 16));
                }
            } else {
#pragma unroll
                for (int x = 0; x < kSeg; ++x)
                    if (x >= lo && x < hi) T::st(zrow + x * Zsn, zpix(x));
            }
        }
        if (!q_early) __syncthreads();
    }
    if (a.S > 1 && tid == 0 && rel == 2u * a.S - 1) slice_reset(counter_at(a.cnt, slice));
}


} // namespace
} // namespace ttt
