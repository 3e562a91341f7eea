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
    unsigned spin;    // slice barrier: poll limit before giving up
    unsigned tbias;   // slice barrier: added to every target (0 in normal use)
    int dot;          // dot-product loss: G = -(1/N) C
    int steps;        // full-batch steps (0 or 1: one); > 1 only for the G-exchange kernel
    float* wk;        // [slices][64][64] fp32 state between steps (steps > 1)
};

// Kernel a full-batch linear plan launches (plan queries of the C ABI).
enum LinKernel { kLinResident = 1, kLinResidentGx = 2, kLinStream = 3 };
int lin_fwd_kernel(const LinFwdLaunch& a, int resident);
size_t lin_fwd_ws_bytes(int B, int H, int N);
int lin_fwd_max_splits(int B, int H, int N);
hipError_t launch_lin_fwd(LinFwdLaunch a, hipStream_t stream, int resident);
int lin_fwd_resident_per_cu(int bf16);
bool lin_fwd_is_resident(int N, int S, int bf16);

// ---- several full-batch steps, apply, gradient magnitude map -----------
struct LinEpochArgs {
    const float* W0;
    const float* eta;
    const float* saved; // [slices][2][64][64]: A, G at W0
    float* WE;          // [slices][64][64]: the weights after `steps` steps
    int H, N, slices, steps, dot;
};
hipError_t launch_lin_epochs(const LinEpochArgs& e, hipStream_t stream);
struct LinApplyArgs {
    View4 Q, Z;
    const float* W; // [slices][64][64]
    int B, H, N;
};
hipError_t launch_lin_apply(const LinApplyArgs& a, int bf16, hipStream_t stream);
struct LinGmmArgs {
    View4 K, V;
    const float* W0;
    float* out;     // [slices][N]
    int B, H, N, dot;
};
hipError_t launch_lin_gmm(const LinGmmArgs& a, int bf16, hipStream_t stream);

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
    unsigned spin;    // slice barrier: poll limit before giving up
    unsigned tbias;   // slice barrier: added to every target (0 in normal use)
    int dot;          // dot-product loss: g = -(1/N) sum V K-shifted
};
size_t conv_ws_bytes(int B, int H, int gh, int gw);
// Splits per slice and exchange protocol a conv plan uses (plan queries).
void conv_plan_info(const ConvLaunch& l, int* S, int* xcd);
hipError_t launch_conv(ConvLaunch a, hipStream_t stream);
int conv_resident_per_cu(int bf16);

// ---- backward of the depthwise 3x3 step ----------------------------------
struct ConvBwdLaunch {
    View4 K, Q, V, dZ, dK, dQ, dV;
    const float* w0;
    const float* eta;
    const float* saved; // nullable: the forward's g [slices][64][9]
    float* dw0;
    float* deta;
    int B, H, gh, gw;
    int bf16;
    void* ws;           // conv_bwd_ws_bytes(...) bytes
    int dot;            // dot-product loss
};
size_t conv_bwd_ws_bytes(int B, int H, int gh, int gw);
hipError_t launch_conv_bwd(const ConvBwdLaunch& a, hipStream_t stream);

// ---- one layer: linear heads and conv heads (one launch when they fit)
hipError_t launch_layer(LinFwdLaunch l, int resident, ConvLaunch c, hipStream_t stream);
bool layer_would_fuse(const LinFwdLaunch& l, int resident, const ConvLaunch& c);

// ---- mini-batch scans -------------------------------------------------
struct ScanLaunch {
    View4 K, Q, V, Z;
    const float* W0;
    const float* eta;
    int B, H, N, b, mode;
    int bf16;
    void* ws;         // scan_ws_bytes(...) bytes
    int cus;          // compute units of the device
    int w0dir;        // W0 is [2][H][64][64]: forward, then reverse scan
    int segs;         // chunk-parallel segments per chain: 0 = planned
};
size_t scan_ws_bytes(int B, int H, int N, int mode);
// Mini-batch sizes the scan takes (any b >= 1).
bool scan_minibatch_supported(int b, int N);
hipError_t launch_scan(ScanLaunch a, hipStream_t stream);
// fp32 views: the vector-ALU scan (minibatch_scan_f32.hip), same workspace.
hipError_t launch_scan_f32(const ScanLaunch& a, hipStream_t stream);

// ---- backward of the mini-batch scans --------------------------------------
struct ScanBwdLaunch {
    View4 K, Q, V, dZ, dK, dQ, dV;
    const float* W0;
    const float* eta;
    float* dW0;
    float* deta;
    int B, H, N, b, mode, w0dir, bf16;
    int walks;        // the serial walks on the matrix cores (bf16, b <= 16, 32-bit row offsets)
    int cus;          // compute units of the device
    void* ws;         // scan_bwd_ws_bytes(...) bytes
};
// The backward's two serial walks on the matrix cores (bf16 views, b <= 16):
// every mini-batch's forward start state (bf16), then the gradient walk (dwn in bf16,
// dR by walk position, each chain's dW0 term), in the layouts of the scan
// backward's workspace.
struct ScanBwdWalks {
    View4 K, Q, V, dZ;
    const float* W0;
    const float* eta;
    uint16_t* states; // [chains][nch][64][64] bf16
    uint16_t* dwn;    // [chains][nch][64][64] bf16
    float* dRp;       // [chains][N][64]
    float* dW0c;      // [chains][64][64]
    int B, H, N, b, mode, w0dir;
    int cus;          // compute units of the device
};
hipError_t launch_scan_bwd_walks(const ScanBwdWalks& l, hipStream_t stream);
bool scan_bwd_supported(int b);
size_t scan_bwd_ws_bytes(int B, int H, int N, int b, int mode);
hipError_t launch_scan_bwd(const ScanBwdLaunch& a, hipStream_t stream);

// ---- two-layer SiLU MLP inner model, one full-batch L2 step --------------
struct MlpLaunch {
    View4 K, Q, V, Z;  // bf16
    const float* W1;   // [H][hid][64]
    const float* W2;   // [H][64][hid]
    const float* eta;
    int B, H, N, hid;
    void* ws;          // mlp_ws_bytes(...) bytes
};
bool mlp_hidden_supported(int hid);
size_t mlp_ws_bytes(int B, int H, int N, int hid);
hipError_t launch_mlp(const MlpLaunch& a, hipStream_t stream);

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
    int dot;          // dot-product loss
};
size_t lin_bwd_ws_bytes(int B, int H, int N);
// A and G recomputed by the forward's Gram pass when the caller saved none
float* lin_bwd_saved_region(void* ws, int B, int H, int N);
hipError_t launch_lin_bwd(LinBwdLaunch a, hipStream_t stream);

} // namespace ttt
