// internal.hpp -- host-side launch plans shared between the C-ABI entry
// points (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ttt {

struct View4 {
    void* ptr;
    long long sb, sh, sn; // element strides
};

// ---- full-batch linear step ------------------------------------------
struct LinFwdLaunch {
    View4 K, Q, V, Z;
    const float* W0;
    const float* eta;
    float* saved;     // nullable [slices][2][64][64]: A then G
    float* part;      // [slices][S][2][64][64]  (S > 1)
    float* w1;        // [slices][64][64]        (S > 1)
    unsigned* cnt;    // [slices]                (S > 1)
    int B, H, N;
    int S;            // workgroups per slice
    int xcd;          // XCD-aware block mapping
    int bf16;
};
size_t lin_fwd_ws_bytes(int B, int H, int N);
int lin_fwd_max_splits(int B, int H, int N);
hipError_t launch_lin_fwd(LinFwdLaunch a, hipStream_t stream, int resident);
int lin_fwd_resident_per_cu(int bf16);
bool lin_fwd_is_resident(int N, int S, int bf16);

// ---- depthwise 3x3 ----------------------------------------------------
struct ConvLaunch {
    View4 K, Q, V, Z;
    const float* w0;
    const float* eta;
    float* saved;     // nullable [slices][64][9]
    int B, H, gh, gw;
    int bf16;
    void* ws;         // conv_ws_bytes(...) bytes, zero-filled before first use
    void* part;       // null: the partials follow the counters in ws; else their own region
    int cap;          // resident workgroups of the device for the conv kernel
    int xcd_ok;       // the device is an MI355X in whole-device (SPX) mode
};
size_t conv_ws_bytes(int B, int H, int gh, int gw);
hipError_t launch_conv(ConvLaunch a, hipStream_t stream);
int conv_resident_per_cu(int bf16);

// ---- one layer: linear heads and conv heads (one launch when they fit)
hipError_t launch_layer(LinFwdLaunch l, int resident, ConvLaunch c, hipStream_t stream);

// ---- mini-batch scans -------------------------------------------------
struct ScanLaunch {
    View4 K, Q, V, Z;
    const float* W0;
    const float* eta;
    int B, H, N, b, mode;
    int bf16;
    void* ws;         // scan_ws_bytes(...) bytes
    int cus;          // compute units of the device
};
size_t scan_ws_bytes(int B, int H, int N, int mode);
hipError_t launch_scan(ScanLaunch a, hipStream_t stream);

// ---- backward of the full-batch linear step ----------------------------
struct LinBwdLaunch {
    View4 K, Q, V, dZ, dK, dQ, dV;
    const float* W0;
    const float* eta;
    const float* saved; // nullable
    float* dW0;
    float* deta;
    int B, H, N;
    int bf16;
    void* ws;         // lin_bwd_ws_bytes(...) bytes
};
size_t lin_bwd_ws_bytes(int B, int H, int N);
// A and G recomputed by the forward's Gram pass when the caller saved none
float* lin_bwd_saved_region(void* ws, int B, int H, int N);
hipError_t launch_lin_bwd(LinBwdLaunch a, hipStream_t stream);

} // namespace ttt
