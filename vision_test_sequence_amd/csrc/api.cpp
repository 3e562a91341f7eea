// api.cpp -- the C ABI of ttt.h: argument validation (before any HIP call),
// workspace sizing, launch planning and dispatch to the gfx950 kernels.
#include "ttt.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <atomic>
#include <mutex>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "internal.hpp"
#include "common.hpp"

using namespace ttt;

namespace {

struct Span {
    uintptr_t lo = 0, hi = 0;
    bool valid = false;
};

bool overlap(const Span& a, const Span& b) {
    return a.valid && b.valid && a.lo < b.hi && b.lo < a.hi;
}

size_t esize(ttt_dtype t) { return t == TTT_BF16 ? 2 : 4; }

// Shape checks common to every op.  *noop is set when B or H is zero.
ttt_status check_problem(const ttt_problem* p, bool* noop) {
    *noop = false;
    if (!p) return TTT_ERR_NULL_POINTER;
    if (p->B < 0 || p->H < 0 || p->N <= 0 || p->d <= 0) return TTT_ERR_BAD_SHAPE;
    if (p->dtype != TTT_F32 && p->dtype != TTT_BF16) return TTT_ERR_UNSUPPORTED;
    if (p->d != 64) return TTT_ERR_UNSUPPORTED;
    if ((int64_t)p->B * p->H > (int64_t)1 << 24) return TTT_ERR_UNSUPPORTED;
    if (p->loss != TTT_LOSS_L2 && p->loss != TTT_LOSS_DOT) return TTT_ERR_UNSUPPORTED;
    if (p->steps < 0) return TTT_ERR_BAD_SHAPE;
    if (p->w0_per_direction != 0 && p->w0_per_direction != 1) return TTT_ERR_UNSUPPORTED;
    if (p->B == 0 || p->H == 0) *noop = true;
    return TTT_OK;
}

// The options an operation does not take: more than one step (all but the
// full-batch linear forward), a W0 per direction (all but the scan).
ttt_status check_single_step(const ttt_problem* p) {
    if (p->steps > 1 || p->w0_per_direction) return TTT_ERR_UNSUPPORTED;
    return TTT_OK;
}

size_t align256z(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of ttt_linear_fullbatch.  More than one step: [the one-step
// workspace, at least its counter block][A, G(W0) per slice][W_E per slice].
size_t lin_ws_bytes(const ttt_problem* p) {
    const size_t one = lin_fwd_ws_bytes(p->B, p->H, p->N);
    if (p->steps <= 1) return one;
    const size_t slices = (size_t)p->B * p->H;
    return align256z(std::max(one, kCounterBytes)) + align256z(slices * 8192 * 4) + slices * 4096 * 4;
}

// A [B,H,N,d] view: non-null, non-negative strides, no two elements at one
// address (strides sorted ascending must each clear the span of the smaller
// dimensions), 16-byte alignment of the pointer and of each stride.
ttt_status check_view(const ttt_view& v, const ttt_problem& p, Span* sp) {
    if (!v.ptr) return TTT_ERR_NULL_POINTER;
    if (v.stride_b < 0 || v.stride_h < 0 || v.stride_n < 0) return TTT_ERR_BAD_STRIDE;
    struct Dim {
        int64_t ext, st;
    } dims[3] = {{p.B, v.stride_b}, {p.H, v.stride_h}, {p.N, v.stride_n}};
    std::sort(dims, dims + 3, [](const Dim& x, const Dim& y) { return x.st < y.st; });
    const int64_t lim = (int64_t)1 << 60;
    int64_t span = p.d;
    for (const Dim& dm : dims) {
        if (dm.ext <= 1) continue;
        if (dm.st < span) return TTT_ERR_BAD_STRIDE;
        if (dm.st > lim / dm.ext) return TTT_ERR_BAD_STRIDE;
        span += dm.st * (dm.ext - 1);
        if (span > lim) return TTT_ERR_BAD_STRIDE;
    }
    const size_t es = esize(p.dtype);
    if ((uintptr_t)v.ptr % 16) return TTT_ERR_MISALIGNED;
    for (const Dim& dm : dims)
        if (dm.ext > 1 && (dm.st * (int64_t)es) % 16) return TTT_ERR_MISALIGNED;
    sp->lo = (uintptr_t)v.ptr;
    sp->hi = sp->lo + (uintptr_t)(span * (int64_t)es);
    sp->valid = true;
    return TTT_OK;
}

ttt_status check_buf(const void* ptr, size_t bytes, size_t align, Span* sp) {
    if (!ptr) return TTT_ERR_NULL_POINTER;
    if ((uintptr_t)ptr % align) return TTT_ERR_MISALIGNED;
    sp->lo = (uintptr_t)ptr;
    sp->hi = sp->lo + bytes;
    sp->valid = true;
    return TTT_OK;
}

// Every output span must be disjoint from every input span and from every
// other output span.
ttt_status check_aliasing(const Span* in, int nin, const Span* out, int nout) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(out[i], in[j])) return TTT_ERR_ALIASING;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return TTT_ERR_ALIASING;
    }
    return TTT_OK;
}

// Two views with the same strides and batch size that are head ranges of
// one larger view (the second starts k whole heads from the first, and the
// union of the two head ranges is itself a view without coinciding
// elements): disjoint exactly when the head ranges are.  Returns false when
// the two do not have this form (the caller then compares address spans).
bool head_ranges_disjoint(const ttt_view& a, int Ha, const ttt_view& b, int Hb, const ttt_problem& p) {
    if (a.stride_b != b.stride_b || a.stride_h != b.stride_h || a.stride_n != b.stride_n) return false;
    const int64_t es = (int64_t)esize(p.dtype);
    const int64_t delta = ((int64_t)(uintptr_t)b.ptr - (int64_t)(uintptr_t)a.ptr);
    if (a.stride_h <= 0 || delta % (es * a.stride_h)) return false;
    const int64_t k = delta / (es * a.stride_h);
    const int64_t h0 = k < 0 ? k : 0, h1 = std::max<int64_t>(Ha, k + Hb);
    if (h1 - h0 > (int64_t)1 << 24) return false;
    ttt_problem u = p;
    u.H = (int32_t)(h1 - h0);
    ttt_view uv = a;
    uv.ptr = (char*)a.ptr + h0 * a.stride_h * es;
    Span sp;
    if (check_view(uv, u, &sp) != TTT_OK) return false;
    return k >= Ha || k + Hb <= 0;
}

ttt_status check_ws(void* ws, size_t ws_bytes, size_t need, Span* sp) {
    if (ws_bytes < need) return TTT_ERR_WORKSPACE_TOO_SMALL;
    if (need == 0) return TTT_OK;
    return check_buf(ws, need, 256, sp);
}

View4 v4(const ttt_view& v) { return View4{v.ptr, v.stride_b, v.stride_h, v.stride_n}; }

// Resident-workgroup capacity of the current device for a kernel, cached
// per device.  Slices that are split over several workgroups meet at a
// barrier, so their grid must not exceed this.
constexpr int kMaxDev = 64;
std::atomic<int> g_cus[kMaxDev];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        g_cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

ttt_status hip_status(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_ERR_HIP; }

// Diagnostic switches, read from the environment at every call (the library
// keeps no state of its own for them):
//  * TTT_EXCHANGE=device -- split slices exchange through device-scope
//    atomics with the plain block mapping even on a 256-CU MI355X (the
//    protocol any other part or partition mode gets);
//  * TTT_TEST_EXCHANGE_GIVEUP=1 -- every slice barrier waits for an
//    unreachable count and gives up after a few polls: the failure path of
//    the exchange, with every kernel still ending normally;
//  * TTT_CONV_CAP=n -- the depthwise planner sees at most n resident
//    workgroups, so a slice's tiles are shared out several to a workgroup
//    (the multi-tile splits of devices with fewer CUs);
//  * TTT_SPLIT_STEPS=1 -- several full-batch linear steps take the
//    three-launch path (Gram pass, steps, apply) even where the G-exchange
//    kernel could run them in one launch.
struct Knobs {
    unsigned spin, tbias;
    bool device_exchange;
    int conv_cap; // TTT_CONV_CAP: fewer resident conv workgroups (0: none)
    bool split_steps;
};
Knobs knobs() {
    Knobs k{kSpinLimit, 0u, false, 0, false};
    const char* cc = getenv("TTT_CONV_CAP");
    if (cc) k.conv_cap = atoi(cc);
    const char* ss = getenv("TTT_SPLIT_STEPS");
    if (ss && strcmp(ss, "1") == 0) k.split_steps = true;
    const char* e = getenv("TTT_EXCHANGE");
    if (e && strcmp(e, "device") == 0) k.device_exchange = true;
    const char* g = getenv("TTT_TEST_EXCHANGE_GIVEUP");
    if (g && strcmp(g, "1") == 0) {
        k.spin = 64;
        k.tbias = 1u << 24;
    }
    return k;
}

// The XCD-local exchange relies on MI355X's whole-device (SPX) layout: 256
// CUs in 8 XCDs, workgroup i on XCD i % 8.  The kernels also check the XCC
// id of every workgroup and poison their outputs with NaN if it differs.
bool xcd_local_ok(const Knobs& k) { return device_cus() == 256 && !k.device_exchange; }

// ---- scratch of the allocation-free entry point ----------------------
// The full-batch linear workspace (counter block, [A; C] or G partials,
// W1) for any problem: the planner keeps slices x splits <= 256 with
// splits >= 2 only for <= 128 slices, so the workspace never exceeds
// 64 KB + 256 x 32 KB + 128 x 16 KB = 10.06 MiB.  Each device that runs the
// entry point holds its own copy until the process ends; its address is
// taken once per device with hipGetSymbolAddress (the array's name in host
// code is not a device address).
constexpr size_t kScratchBytes = (size_t)21 << 19; // 10.5 MiB
static __device__ __align__(256) char scratch[kScratchBytes];
void* g_scratch_ptr[kMaxDev];
hipError_t g_scratch_err[kMaxDev];
std::once_flag g_scratch_once[kMaxDev];

// This device's copy of `scratch` (the device must be current), or null.
void* scratch_for_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    return g_scratch_ptr[dev];
}

// Zero n 16-byte words (the scratch's counter block before each call: the
// previous call may have left a failed slice line).  A kernel, not a
// memset node, so that callers may capture the call in a HIP graph.
__global__ void zero_words16(uint4* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

} // namespace

extern "C" {

const char* ttt_status_string(ttt_status s) {
    switch (s) {
    case TTT_OK: return "TTT_OK";
    case TTT_ERR_NULL_POINTER: return "TTT_ERR_NULL_POINTER";
    case TTT_ERR_BAD_SHAPE: return "TTT_ERR_BAD_SHAPE";
    case TTT_ERR_BAD_STRIDE: return "TTT_ERR_BAD_STRIDE";
    case TTT_ERR_MISALIGNED: return "TTT_ERR_MISALIGNED";
    case TTT_ERR_UNSUPPORTED: return "TTT_ERR_UNSUPPORTED";
    case TTT_ERR_ALIASING: return "TTT_ERR_ALIASING";
    case TTT_ERR_WORKSPACE_TOO_SMALL: return "TTT_ERR_WORKSPACE_TOO_SMALL";
    case TTT_ERR_HIP: return "TTT_ERR_HIP";
    }
    return "TTT_ERR_UNKNOWN";
}

size_t ttt_workspace_size(ttt_op op, const ttt_problem* p) {
    bool noop = false;
    if (check_problem(p, &noop) != TTT_OK || noop) return 0;
    switch (op) {
    case TTT_OP_LINEAR_FULLBATCH: return lin_ws_bytes(p);
    case TTT_OP_DWCONV3X3_FULLBATCH:
        if (p->grid_h <= 0 || p->grid_w <= 0 || (int64_t)p->grid_h * p->grid_w != p->N) return 0;
        return conv_ws_bytes(p->B, p->H, p->grid_h, p->grid_w);
    case TTT_OP_LINEAR_MINIBATCH_BIDIR: return scan_ws_bytes(p->B, p->H, p->N, (int)p->mode);
    case TTT_OP_LINEAR_FULLBATCH_BWD: return lin_bwd_ws_bytes(p->B, p->H, p->N);
    case TTT_OP_LAYER_FULLBATCH: return 0; // two problems: ttt_layer_workspace_size
    case TTT_OP_DWCONV3X3_FULLBATCH_BWD:
        if (p->grid_h <= 0 || p->grid_w <= 0 || (int64_t)p->grid_h * p->grid_w != p->N) return 0;
        return conv_bwd_ws_bytes(p->B, p->H, p->grid_h, p->grid_w);
    case TTT_OP_LINEAR_MINIBATCH_BIDIR_BWD:
        if (!scan_bwd_supported(p->minibatch)) return 0;
        return scan_bwd_ws_bytes(p->B, p->H, p->N, p->minibatch, (int)p->mode);
    case TTT_OP_MLP_FULLBATCH: return mlp_ws_bytes(p->B, p->H, p->N, p->hidden);
    }
    return 0;
}

// Plan the full-batch forward (validated arguments).  A null Z computes
// only A and G into `saved`.
static ttt_status plan_fullbatch(const ttt_problem* p, View4 K, View4 Q, View4 V, View4 Z, const float* W0,
                                 const float* eta, float* saved, void* ws, LinFwdLaunch& a, int& resident) {
    a = LinFwdLaunch{};
    const Knobs kn = knobs();
    a.spin = kn.spin;
    a.tbias = kn.tbias;
    a.K = K; a.Q = Q; a.V = V; a.Z = Z;
    a.W0 = W0; a.eta = eta; a.saved = saved;
    a.B = p->B; a.H = p->H; a.N = p->N;
    a.bf16 = p->dtype == TTT_BF16;
    a.dot = p->loss == TTT_LOSS_DOT ? 1 : 0;
    const long long slices = (long long)p->B * p->H;
    int S = lin_fwd_max_splits(p->B, p->H, p->N);
    const long long padded = (slices + 7) / 8 * 8;
    if (S > 1) {
        const int cap = device_cus() * lin_fwd_resident_per_cu(a.bf16);
        while (S > 1 && (long long)S * padded > cap) S /= 2; // stays a power of two
    }
    a.S = S;
    a.xcd = (S > 1 && xcd_local_ok(kn)) ? 1 : 0;
    if (S > 1) {
        // workspace: [fixed counter block][partials, Smax per slice][W1 per slice]
        char* base = (char*)ws;
        const int Smax = lin_fwd_max_splits(p->B, p->H, p->N);
        if (slices > kMaxBarrierSlices) return TTT_ERR_UNSUPPORTED; // unreachable: S > 1 => slices <= 128
        a.cnt = (unsigned*)base;
        a.part = (float*)(base + kCounterBytes);
        a.w1 = (float*)(base + kCounterBytes + (size_t)slices * Smax * 8192 * 4);
    }
    resident = lin_fwd_is_resident(p->N, S, a.bf16) ? 1 : 0;
    return TTT_OK;
}

static ttt_status launch_fullbatch(const ttt_problem* p, View4 K, View4 Q, View4 V, View4 Z, const float* W0,
                                   const float* eta, float* saved, void* ws, hipStream_t stream) {
    LinFwdLaunch a;
    int resident = 0;
    if (p->steps > 1) {
        // the Gram pass saves A and G(W0) in the workspace (no apply), the
        // steps run per slice, then Z = Q W_E^T
        const size_t slices = (size_t)p->B * p->H;
        char* base = (char*)ws + align256z(std::max(lin_fwd_ws_bytes(p->B, p->H, p->N), kCounterBytes));
        float* sv = (float*)base;
        float* WE = (float*)(base + align256z(slices * 8192 * 4));
        const View4 none{nullptr, 0, 0, 0};
        ttt_problem one = *p;
        one.steps = 1;
        // One launch when the splits exchange G: each split keeps its A_s
        // and C_s and the steps are further exchange rounds, the state
        // between them in W_E
        ttt_status st = plan_fullbatch(&one, K, Q, V, Z, W0, eta, nullptr, ws, a, resident);
        if (st != TTT_OK) return st;
        if (lin_fwd_kernel(a, resident) == kLinResidentGx && !knobs().split_steps) {
            a.steps = p->steps;
            a.wk = WE;
            return hip_status(launch_lin_fwd(a, stream, resident));
        }
        st = plan_fullbatch(&one, K, K, V, none, W0, eta, sv, ws, a, resident);
        if (st != TTT_OK) return st;
        hipError_t e = launch_lin_fwd(a, stream, resident);
        if (e != hipSuccess) return TTT_ERR_HIP;
        LinEpochArgs ea{W0, eta, sv, WE, p->H, p->N, (int)slices, p->steps, p->loss == TTT_LOSS_DOT ? 1 : 0};
        if ((e = launch_lin_epochs(ea, stream)) != hipSuccess) return TTT_ERR_HIP;
        LinApplyArgs aa{Q, Z, WE, p->B, p->H, p->N};
        return hip_status(launch_lin_apply(aa, p->dtype == TTT_BF16, stream));
    }
    const ttt_status st = plan_fullbatch(p, K, Q, V, Z, W0, eta, saved, ws, a, resident);
    if (st != TTT_OK) return st;
    return hip_status(launch_lin_fwd(a, stream, resident));
}

// The conv call's launch description (validated arguments).
static ConvLaunch plan_conv_call(const ttt_problem* p, View4 K, View4 Q, View4 V, View4 Z, const float* w0,
                                 const float* eta, float* saved, void* ws) {
    ConvLaunch a{};
    a.K = K; a.Q = Q; a.V = V; a.Z = Z;
    a.w0 = w0; a.eta = eta; a.saved = saved;
    a.B = p->B; a.H = p->H; a.gh = p->grid_h; a.gw = p->grid_w;
    a.bf16 = p->dtype == TTT_BF16;
    a.ws = ws;
    a.cap = device_cus() * conv_resident_per_cu(a.bf16);
    a.dot = p->loss == TTT_LOSS_DOT ? 1 : 0;
    const Knobs kn = knobs();
    if (kn.conv_cap > 0 && kn.conv_cap < a.cap) a.cap = kn.conv_cap;
    a.xcd_ok = xcd_local_ok(kn) ? 1 : 0;
    a.spin = kn.spin;
    a.tbias = kn.tbias;
    return a;
}

ttt_status ttt_linear_fullbatch(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                const float* W0, const float* eta, ttt_view Z, float* saved,
                                void* ws, size_t ws_bytes, ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if (p->w0_per_direction || (p->steps > 1 && saved)) return TTT_ERR_UNSUPPORTED;
    if (noop) return TTT_OK;
    Span in[5], out[3];
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(Q, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[2])) != TTT_OK) return st;
    if ((st = check_buf(W0, (size_t)p->H * p->d * p->d * 4, 16, &in[3])) != TTT_OK) return st;
    if ((st = check_buf(eta, (size_t)p->H * 4, 4, &in[4])) != TTT_OK) return st;
    if ((st = check_view(Z, *p, &out[0])) != TTT_OK) return st;
    if (saved && (st = check_buf(saved, (size_t)p->B * p->H * 2 * p->d * p->d * 4, 4, &out[1])) != TTT_OK)
        return st;
    const size_t need = lin_ws_bytes(p);
    if ((st = check_ws(ws, ws_bytes, need, &out[2])) != TTT_OK) return st;
    if ((st = check_aliasing(in, 5, out, 3)) != TTT_OK) return st;

    return launch_fullbatch(p, v4(K), v4(Q), v4(V), v4(Z), W0, eta, saved, ws, (hipStream_t)stream);
}

ttt_status ttt_linear_fullbatch_noalloc(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                        const float* W0, const float* eta, ttt_view Z, float* saved,
                                        ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if ((st = check_single_step(p)) != TTT_OK) return st; // the scratch holds one step's workspace
    if (noop) return TTT_OK;
    Span in[5], out[2];
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(Q, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[2])) != TTT_OK) return st;
    if ((st = check_buf(W0, (size_t)p->H * p->d * p->d * 4, 16, &in[3])) != TTT_OK) return st;
    if ((st = check_buf(eta, (size_t)p->H * 4, 4, &in[4])) != TTT_OK) return st;
    if ((st = check_view(Z, *p, &out[0])) != TTT_OK) return st;
    if (saved && (st = check_buf(saved, (size_t)p->B * p->H * 2 * p->d * p->d * 4, 4, &out[1])) != TTT_OK)
        return st;
    if ((st = check_aliasing(in, 5, out, 2)) != TTT_OK) return st;
    const size_t need = lin_fwd_ws_bytes(p->B, p->H, p->N);
    if (need > kScratchBytes) return TTT_ERR_WORKSPACE_TOO_SMALL; // beyond the fixed scratch
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_for_current_device();
        if (!ws) return TTT_ERR_HIP;
        const int n16 = (int)(kCounterBytes / 16);
        hipLaunchKernelGGL(zero_words16, dim3((n16 + 255) / 256), dim3(256), 0, (hipStream_t)stream, (uint4*)ws,
                           n16);
        if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
    }
    return launch_fullbatch(p, v4(K), v4(Q), v4(V), v4(Z), W0, eta, saved, ws, (hipStream_t)stream);
}

ttt_status ttt_dwconv3x3_fullbatch(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                   const float* w0, const float* eta, ttt_view Z, float* saved,
                                   void* ws, size_t ws_bytes, ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if ((st = check_single_step(p)) != TTT_OK) return st;
    if (p->grid_h <= 0 || p->grid_w <= 0 || (int64_t)p->grid_h * p->grid_w != p->N)
        return TTT_ERR_BAD_SHAPE;
    if (noop) return TTT_OK;
    Span in[5], out[3];
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(Q, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[2])) != TTT_OK) return st;
    if ((st = check_buf(w0, (size_t)p->H * p->d * 9 * 4, 16, &in[3])) != TTT_OK) return st;
    if ((st = check_buf(eta, (size_t)p->H * 4, 4, &in[4])) != TTT_OK) return st;
    if ((st = check_view(Z, *p, &out[0])) != TTT_OK) return st;
    if (saved && (st = check_buf(saved, (size_t)p->B * p->H * p->d * 9 * 4, 4, &out[1])) != TTT_OK)
        return st;
    const size_t need = conv_ws_bytes(p->B, p->H, p->grid_h, p->grid_w);
    if ((st = check_ws(ws, ws_bytes, need, &out[2])) != TTT_OK) return st;
    if ((st = check_aliasing(in, 5, out, 3)) != TTT_OK) return st;

    const ConvLaunch a = plan_conv_call(p, v4(K), v4(Q), v4(V), v4(Z), w0, eta, saved, ws);
    return hip_status(launch_conv(a, (hipStream_t)stream));
}

ttt_status ttt_dwconv3x3_fullbatch_bwd(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                       const float* w0, const float* eta, ttt_view dZ, const float* saved,
                                       ttt_view dK, ttt_view dQ, ttt_view dV, float* dw0, float* deta,
                                       void* ws, size_t ws_bytes, ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if ((st = check_single_step(p)) != TTT_OK) return st;
    if (p->grid_h <= 0 || p->grid_w <= 0 || (int64_t)p->grid_h * p->grid_w != p->N)
        return TTT_ERR_BAD_SHAPE;
    if (noop) return TTT_OK;
    Span in[7], out[6];
    int nin = 6;
    if ((st = check_buf(dw0, (size_t)p->H * p->d * 9 * 4, 4, &out[3])) != TTT_OK) return st;
    if ((st = check_buf(deta, (size_t)p->H * 4, 4, &out[4])) != TTT_OK) return st;
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(Q, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[2])) != TTT_OK) return st;
    if ((st = check_buf(w0, (size_t)p->H * p->d * 9 * 4, 16, &in[3])) != TTT_OK) return st;
    if ((st = check_buf(eta, (size_t)p->H * 4, 4, &in[4])) != TTT_OK) return st;
    if ((st = check_view(dZ, *p, &in[5])) != TTT_OK) return st;
    if (saved) {
        if ((st = check_buf(saved, (size_t)p->B * p->H * p->d * 9 * 4, 4, &in[6])) != TTT_OK) return st;
        nin = 7;
    }
    if ((st = check_view(dK, *p, &out[0])) != TTT_OK) return st;
    if ((st = check_view(dQ, *p, &out[1])) != TTT_OK) return st;
    if ((st = check_view(dV, *p, &out[2])) != TTT_OK) return st;
    // the kernels address a slice of each view with 32-bit offsets, the
    // stencil's rows two past either edge included
    for (const ttt_view* v : {&K, &Q, &V, &dZ, &dK, &dQ, &dV})
        if (p->N > 1 && (int64_t)p->N * v->stride_n * (int64_t)esize(p->dtype) >= ((int64_t)1 << 29))
            return TTT_ERR_UNSUPPORTED;
    const size_t need = conv_bwd_ws_bytes(p->B, p->H, p->grid_h, p->grid_w);
    if ((st = check_ws(ws, ws_bytes, need, &out[5])) != TTT_OK) return st;
    if ((st = check_aliasing(in, nin, out, 6)) != TTT_OK) return st;

    ConvBwdLaunch a{};
    a.K = v4(K); a.Q = v4(Q); a.V = v4(V); a.dZ = v4(dZ);
    a.dK = v4(dK); a.dQ = v4(dQ); a.dV = v4(dV);
    a.w0 = w0; a.eta = eta; a.saved = saved; a.dw0 = dw0; a.deta = deta;
    a.B = p->B; a.H = p->H; a.gh = p->grid_h; a.gw = p->grid_w;
    a.bf16 = p->dtype == TTT_BF16;
    a.ws = ws;
    a.dot = p->loss == TTT_LOSS_DOT ? 1 : 0;
    return hip_status(launch_conv_bwd(a, (hipStream_t)stream));
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Layer workspace: [conv counters][linear workspace, at least a counter
// block][conv partials].  Both counter blocks sit at fixed offsets for
// every shape, so calls of any shapes can share one zeroed workspace (a
// counter block never lands where another call left data).
struct LayerWs {
    size_t lin_off, conv_part_off, total;
};
static LayerWs layer_ws(size_t lws, size_t cws) {
    LayerWs w{};
    if (lws == 0 && cws == 0) return w;
    w.lin_off = kCounterBytes;
    w.conv_part_off = kCounterBytes + align256(std::max(lws, kCounterBytes));
    w.total = w.conv_part_off + (cws > kCounterBytes ? cws - kCounterBytes : 0);
    return w;
}

size_t ttt_layer_workspace_size(const ttt_problem* lin, const ttt_problem* conv) {
    return layer_ws(ttt_workspace_size(TTT_OP_LINEAR_FULLBATCH, lin),
                    ttt_workspace_size(TTT_OP_DWCONV3X3_FULLBATCH, conv)).total;
}

ttt_status ttt_layer_fullbatch(const ttt_problem* lin, ttt_view Kl, ttt_view Ql, ttt_view Vl, const float* W0,
                               const float* eta_l, ttt_view Zl, const ttt_problem* conv, ttt_view Kc,
                               ttt_view Qc, ttt_view Vc, const float* w0, const float* eta_c, ttt_view Zc,
                               void* ws, size_t ws_bytes, ttt_stream_t stream) {
    bool lnoop = false, cnoop = false;
    ttt_status st = check_problem(lin, &lnoop);
    if (st != TTT_OK) return st;
    if ((st = check_problem(conv, &cnoop)) != TTT_OK) return st;
    if ((st = check_single_step(lin)) != TTT_OK || (st = check_single_step(conv)) != TTT_OK) return st;
    if (conv->grid_h <= 0 || conv->grid_w <= 0 || (int64_t)conv->grid_h * conv->grid_w != conv->N)
        return TTT_ERR_BAD_SHAPE;
    Span in[10], out[3];
    if (!lnoop) {
        if ((st = check_view(Kl, *lin, &in[0])) != TTT_OK) return st;
        if ((st = check_view(Ql, *lin, &in[1])) != TTT_OK) return st;
        if ((st = check_view(Vl, *lin, &in[2])) != TTT_OK) return st;
        if ((st = check_buf(W0, (size_t)lin->H * lin->d * lin->d * 4, 16, &in[3])) != TTT_OK) return st;
        if ((st = check_buf(eta_l, (size_t)lin->H * 4, 4, &in[4])) != TTT_OK) return st;
        if ((st = check_view(Zl, *lin, &out[0])) != TTT_OK) return st;
    }
    if (!cnoop) {
        if ((st = check_view(Kc, *conv, &in[5])) != TTT_OK) return st;
        if ((st = check_view(Qc, *conv, &in[6])) != TTT_OK) return st;
        if ((st = check_view(Vc, *conv, &in[7])) != TTT_OK) return st;
        if ((st = check_buf(w0, (size_t)conv->H * conv->d * 9 * 4, 16, &in[8])) != TTT_OK) return st;
        if ((st = check_buf(eta_c, (size_t)conv->H * 4, 4, &in[9])) != TTT_OK) return st;
        if ((st = check_view(Zc, *conv, &out[1])) != TTT_OK) return st;
    }
    const size_t lws = lnoop ? 0 : lin_fwd_ws_bytes(lin->B, lin->H, lin->N);
    const size_t cws = cnoop ? 0 : conv_ws_bytes(conv->B, conv->H, conv->grid_h, conv->grid_w);
    const LayerWs lw = layer_ws(lws, cws);
    const size_t need = lw.total;
    if ((st = check_ws(ws, ws_bytes, need, &out[2])) != TTT_OK) return st;
    // The two outputs may be head ranges of one tensor (the layer's heads
    // split between the two inner models): compared exactly, not by span.
    if (!lnoop && !cnoop && lin->B == conv->B && lin->N == conv->N && lin->dtype == conv->dtype &&
        head_ranges_disjoint(Zl, lin->H, Zc, conv->H, *lin)) {
        Span zc = out[1];
        out[1].valid = false;
        if ((st = check_aliasing(in, 10, out, 3)) != TTT_OK) return st;
        Span o2[2] = {zc, out[2]};
        if ((st = check_aliasing(in, 10, o2, 2)) != TTT_OK) return st;
    } else if ((st = check_aliasing(in, 10, out, 3)) != TTT_OK) {
        return st;
    }
    if (lnoop && cnoop) return TTT_OK;

    char* wsb = (char*)ws;
    LinFwdLaunch l{};
    int resident = 0;
    if (!lnoop &&
        (st = plan_fullbatch(lin, v4(Kl), v4(Ql), v4(Vl), v4(Zl), W0, eta_l, nullptr,
                             lws ? wsb + lw.lin_off : nullptr, l, resident)) != TTT_OK)
        return st;
    ConvLaunch c{};
    if (!cnoop) {
        c = plan_conv_call(conv, v4(Kc), v4(Qc), v4(Vc), v4(Zc), w0, eta_c, nullptr, cws ? wsb : nullptr);
        c.part = cws ? wsb + lw.conv_part_off : nullptr;
    }
    return hip_status(launch_layer(l, resident, c, (hipStream_t)stream));
}

ttt_status ttt_linear_minibatch_bidir(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                      const float* W0, const float* eta, ttt_view Z, void* ws,
                                      size_t ws_bytes, ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if (p->minibatch < 1) return TTT_ERR_BAD_SHAPE;
    if (p->mode != TTT_BIDIR_AVG && p->mode != TTT_FORWARD_ONLY && p->mode != TTT_BACKWARD_ONLY)
        return TTT_ERR_UNSUPPORTED;
    if (!scan_minibatch_supported(p->minibatch, p->N)) return TTT_ERR_UNSUPPORTED;
    if (p->loss != TTT_LOSS_L2 || p->steps > 1) return TTT_ERR_UNSUPPORTED;
    if (noop) return TTT_OK;
    Span in[5], out[2];
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(Q, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[2])) != TTT_OK) return st;
    const size_t nw0 = p->w0_per_direction ? 2 : 1;
    if ((st = check_buf(W0, nw0 * p->H * p->d * p->d * 4, 16, &in[3])) != TTT_OK) return st;
    if ((st = check_buf(eta, (size_t)p->H * 4, 4, &in[4])) != TTT_OK) return st;
    if ((st = check_view(Z, *p, &out[0])) != TTT_OK) return st;
    // the bf16 kernel addresses a slice's K, V, Q and Z rows through 32-bit
    // buffer offsets, walking up to 512 tokens past either end
    const int64_t span_lim = (int64_t)1 << 31;
    for (const ttt_view* w : {&K, &Q, &V, &Z})
        if (p->dtype == TTT_BF16 && (int64_t)(p->N + 512) * std::max<int64_t>(w->stride_n, p->d) * 2 >= span_lim)
            return TTT_ERR_UNSUPPORTED;
    const size_t need = scan_ws_bytes(p->B, p->H, p->N, (int)p->mode);
    if ((st = check_ws(ws, ws_bytes, need, &out[1])) != TTT_OK) return st;
    if ((st = check_aliasing(in, 5, out, 2)) != TTT_OK) return st;

    ScanLaunch a{};
    a.K = v4(K); a.Q = v4(Q); a.V = v4(V); a.Z = v4(Z);
    if (p->N == 1) {
        // a one-token view may carry any stride_n; the kernel addresses the
        // empty slots of a mini-batch at multiples of stride_n, which must
        // then lie past the token's row (their loads return zeros and their
        // stores are dropped there)
        for (View4* w : {&a.K, &a.Q, &a.V, &a.Z}) w->sn = std::max<long long>(w->sn, p->d);
    }
    a.W0 = W0; a.eta = eta;
    a.B = p->B; a.H = p->H; a.N = p->N; a.b = p->minibatch; a.mode = (int)p->mode;
    a.bf16 = p->dtype == TTT_BF16;
    a.ws = ws;
    a.cus = device_cus();
    a.w0dir = p->w0_per_direction;
    // test switch: TTT_SCAN_SEGMENTS=n cuts every chain into n segments (at
    // most 8, and no more than its mini-batches) instead of the planned count
    const char* sg = getenv("TTT_SCAN_SEGMENTS");
    a.segs = sg ? atoi(sg) : 0;
    if (!a.bf16) return hip_status(launch_scan_f32(a, (hipStream_t)stream));
    return hip_status(launch_scan(a, (hipStream_t)stream));
}

ttt_status ttt_linear_minibatch_bidir_bwd(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                          const float* W0, const float* eta, ttt_view dZ, ttt_view dK,
                                          ttt_view dQ, ttt_view dV, float* dW0, float* deta, void* ws,
                                          size_t ws_bytes, ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if (p->minibatch < 1) return TTT_ERR_BAD_SHAPE;
    if (p->mode != TTT_BIDIR_AVG && p->mode != TTT_FORWARD_ONLY && p->mode != TTT_BACKWARD_ONLY)
        return TTT_ERR_UNSUPPORTED;
    if (!scan_bwd_supported(p->minibatch) || p->loss != TTT_LOSS_L2 || p->steps > 1) return TTT_ERR_UNSUPPORTED;
    if (noop) return TTT_OK;
    const size_t nw0 = p->w0_per_direction ? 2 : 1;
    Span in[6], out[6];
    if ((st = check_buf(dW0, nw0 * p->H * p->d * p->d * 4, 4, &out[3])) != TTT_OK) return st;
    if ((st = check_buf(deta, (size_t)p->H * 4, 4, &out[4])) != TTT_OK) return st;
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(Q, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[2])) != TTT_OK) return st;
    if ((st = check_buf(W0, nw0 * p->H * p->d * p->d * 4, 16, &in[3])) != TTT_OK) return st;
    if ((st = check_buf(eta, (size_t)p->H * 4, 4, &in[4])) != TTT_OK) return st;
    if ((st = check_view(dZ, *p, &in[5])) != TTT_OK) return st;
    if ((st = check_view(dK, *p, &out[0])) != TTT_OK) return st;
    if ((st = check_view(dQ, *p, &out[1])) != TTT_OK) return st;
    if ((st = check_view(dV, *p, &out[2])) != TTT_OK) return st;
    const size_t need = scan_bwd_ws_bytes(p->B, p->H, p->N, p->minibatch, (int)p->mode);
    if ((st = check_ws(ws, ws_bytes, need, &out[5])) != TTT_OK) return st;
    if ((st = check_aliasing(in, 6, out, 6)) != TTT_OK) return st;
    ScanBwdLaunch a{};
    a.K = v4(K); a.Q = v4(Q); a.V = v4(V); a.dZ = v4(dZ);
    a.dK = v4(dK); a.dQ = v4(dQ); a.dV = v4(dV);
    a.W0 = W0; a.eta = eta; a.dW0 = dW0; a.deta = deta;
    a.B = p->B; a.H = p->H; a.N = p->N; a.b = p->minibatch; a.mode = (int)p->mode;
    a.w0dir = p->w0_per_direction;
    a.bf16 = p->dtype == TTT_BF16;
    a.ws = ws;
    // the matrix-core walks address a slice's rows with 32-bit buffer
    // offsets, walking up to 176 tokens past either end (their prefetch);
    // TTT_SCAN_BWD_VECTOR_WALKS (a test switch) keeps the vector walks
    bool spans = true;
    for (const ttt_view* v : {&K, &Q, &V, &dZ})
        if ((int64_t)(p->N + 512) * std::max<int64_t>(v->stride_n, p->d) * 2 >= ((int64_t)1 << 31)) spans = false;
    a.walks = a.bf16 && p->minibatch <= 16 && spans && !getenv("TTT_SCAN_BWD_VECTOR_WALKS") ? 1 : 0;
    a.cus = device_cus();
    if (p->N == 1 && a.walks) {
        // one-token views may carry any stride_n (see the forward scan)
        for (View4* w : {&a.K, &a.Q, &a.V, &a.dZ}) w->sn = std::max<long long>(w->sn, p->d);
    }
    return hip_status(launch_scan_bwd(a, (hipStream_t)stream));
}

ttt_status ttt_mlp_fullbatch(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V, const float* W1,
                             const float* W2, const float* eta, ttt_view Z, void* ws, size_t ws_bytes,
                             ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if (p->hidden <= 0) return TTT_ERR_BAD_SHAPE;
    if (!mlp_hidden_supported(p->hidden) || p->dtype != TTT_BF16 || p->loss != TTT_LOSS_L2)
        return TTT_ERR_UNSUPPORTED;
    if ((st = check_single_step(p)) != TTT_OK) return st;
    if (noop) return TTT_OK;
    const int64_t slices = (int64_t)p->B * p->H;
    if (slices * ((p->N + 255) / 256) > INT32_MAX || slices * (2 * 64 * p->hidden / 256) > INT32_MAX)
        return TTT_ERR_UNSUPPORTED; // grid sizes
    const size_t nw = (size_t)p->H * p->hidden * p->d * 4;
    Span in[6], out[2];
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(Q, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[2])) != TTT_OK) return st;
    if ((st = check_buf(W1, nw, 4, &in[3])) != TTT_OK) return st;
    if ((st = check_buf(W2, nw, 4, &in[4])) != TTT_OK) return st;
    if ((st = check_buf(eta, (size_t)p->H * 4, 4, &in[5])) != TTT_OK) return st;
    if ((st = check_view(Z, *p, &out[0])) != TTT_OK) return st;
    const size_t need = mlp_ws_bytes(p->B, p->H, p->N, p->hidden);
    if ((st = check_ws(ws, ws_bytes, need, &out[1])) != TTT_OK) return st;
    if ((st = check_aliasing(in, 6, out, 2)) != TTT_OK) return st;
    MlpLaunch a{};
    a.K = v4(K); a.Q = v4(Q); a.V = v4(V); a.Z = v4(Z);
    a.W1 = W1; a.W2 = W2; a.eta = eta;
    a.B = p->B; a.H = p->H; a.N = p->N; a.hid = p->hidden;
    a.ws = ws;
    return hip_status(launch_mlp(a, (hipStream_t)stream));
}

ttt_status ttt_linear_gradient_magnitude(const ttt_problem* p, ttt_view K, ttt_view V, const float* W0,
                                         float* gmm, ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if ((st = check_single_step(p)) != TTT_OK) return st;
    if (noop) return TTT_OK;
    Span in[3], out[1];
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_buf(W0, (size_t)p->H * p->d * p->d * 4, 16, &in[2])) != TTT_OK) return st;
    if ((st = check_buf(gmm, (size_t)p->B * p->H * p->N * 4, 4, &out[0])) != TTT_OK) return st;
    if ((st = check_aliasing(in, 3, out, 1)) != TTT_OK) return st;
    LinGmmArgs a{v4(K), v4(V), W0, gmm, p->B, p->H, p->N, p->loss == TTT_LOSS_DOT ? 1 : 0};
    return hip_status(launch_lin_gmm(a, p->dtype == TTT_BF16, (hipStream_t)stream));
}

ttt_status ttt_linear_fullbatch_bwd(const ttt_problem* p, ttt_view K, ttt_view Q, ttt_view V,
                                    const float* W0, const float* eta, ttt_view dZ,
                                    const float* saved, ttt_view dK, ttt_view dQ, ttt_view dV,
                                    float* dW0, float* deta, void* ws, size_t ws_bytes,
                                    ttt_stream_t stream) {
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if ((st = check_single_step(p)) != TTT_OK) return st;
    if (noop) return TTT_OK;
    Span in[7], out[6];
    int nin = 6;
    if ((st = check_buf(dW0, (size_t)p->H * p->d * p->d * 4, 4, &out[3])) != TTT_OK) return st;
    if ((st = check_buf(deta, (size_t)p->H * 4, 4, &out[4])) != TTT_OK) return st;
    if ((st = check_view(K, *p, &in[0])) != TTT_OK) return st;
    if ((st = check_view(Q, *p, &in[1])) != TTT_OK) return st;
    if ((st = check_view(V, *p, &in[2])) != TTT_OK) return st;
    if ((st = check_buf(W0, (size_t)p->H * p->d * p->d * 4, 16, &in[3])) != TTT_OK) return st;
    if ((st = check_buf(eta, (size_t)p->H * 4, 4, &in[4])) != TTT_OK) return st;
    if ((st = check_view(dZ, *p, &in[5])) != TTT_OK) return st;
    if (saved) {
        if ((st = check_buf(saved, (size_t)p->B * p->H * 2 * p->d * p->d * 4, 4, &in[6])) != TTT_OK)
            return st;
        nin = 7;
    }
    if ((st = check_view(dK, *p, &out[0])) != TTT_OK) return st;
    if ((st = check_view(dQ, *p, &out[1])) != TTT_OK) return st;
    if ((st = check_view(dV, *p, &out[2])) != TTT_OK) return st;
    const size_t need = lin_bwd_ws_bytes(p->B, p->H, p->N);
    if ((st = check_ws(ws, ws_bytes, need, &out[5])) != TTT_OK) return st;
    if ((st = check_aliasing(in, nin, out, 6)) != TTT_OK) return st;

    LinBwdLaunch a{};
    a.K = v4(K); a.Q = v4(Q); a.V = v4(V); a.dZ = v4(dZ);
    a.dK = v4(dK); a.dQ = v4(dQ); a.dV = v4(dV);
    a.W0 = W0; a.eta = eta; a.saved = saved; a.dW0 = dW0; a.deta = deta;
    a.B = p->B; a.H = p->H; a.N = p->N;
    a.bf16 = p->dtype == TTT_BF16;
    a.ws = ws;
    a.dot = p->loss == TTT_LOSS_DOT ? 1 : 0;
    if (!saved) {
        // recompute A and G with the forward's Gram pass, into the workspace
        float* sv = lin_bwd_saved_region(ws, p->B, p->H, p->N);
        const View4 none{nullptr, 0, 0, 0};
        st = launch_fullbatch(p, a.K, a.K, a.V, none, W0, eta, sv, ws, (hipStream_t)stream);
        if (st != TTT_OK) return st;
        a.saved = sv;
    }
    return hip_status(launch_lin_bwd(a, (hipStream_t)stream));
}

ttt_status ttt_plan_query(ttt_op op, const ttt_problem* p, int with_saved, ttt_plan_info* out) {
    if (!out) return TTT_ERR_NULL_POINTER;
    *out = ttt_plan_info{0, 0, 0, 0};
    bool noop = false;
    ttt_status st = check_problem(p, &noop);
    if (st != TTT_OK) return st;
    if (noop) return TTT_OK;
    if (op == TTT_OP_LINEAR_FULLBATCH) {
        LinFwdLaunch a;
        int resident = 0;
        const View4 none{nullptr, 0, 0, 0}, zv{(void*)16, 0, 0, 0};
        static float dummy_saved;
        st = plan_fullbatch(p, none, none, none, zv, nullptr, nullptr, with_saved ? &dummy_saved : nullptr,
                            nullptr, a, resident);
        if (st != TTT_OK) return st;
        out->kernel = lin_fwd_kernel(a, resident);
        out->splits = a.S;
        out->xcd_local = a.xcd;
        // several steps: one launch when the G-exchange kernel runs them
        out->fused = p->steps > 1 && !with_saved && out->kernel == kLinResidentGx && !knobs().split_steps ? 1 : 0;
        return TTT_OK;
    }
    if (op == TTT_OP_DWCONV3X3_FULLBATCH) {
        if (p->grid_h <= 0 || p->grid_w <= 0 || (int64_t)p->grid_h * p->grid_w != p->N) return TTT_ERR_BAD_SHAPE;
        const View4 none{nullptr, 0, 0, 0};
        const ConvLaunch c = plan_conv_call(p, none, none, none, none, nullptr, nullptr, nullptr, nullptr);
        int S = 0, x = 0;
        conv_plan_info(c, &S, &x);
        out->kernel = TTT_KERNEL_DWCONV;
        out->splits = S;
        out->xcd_local = x;
        return TTT_OK;
    }
    return TTT_ERR_UNSUPPORTED;
}

ttt_status ttt_layer_plan_query(const ttt_problem* lin, const ttt_problem* conv, int32_t* fused) {
    if (!fused) return TTT_ERR_NULL_POINTER;
    *fused = 0;
    bool lnoop = false, cnoop = false;
    ttt_status st = check_problem(lin, &lnoop);
    if (st != TTT_OK) return st;
    if ((st = check_problem(conv, &cnoop)) != TTT_OK) return st;
    if (conv->grid_h <= 0 || conv->grid_w <= 0 || (int64_t)conv->grid_h * conv->grid_w != conv->N)
        return TTT_ERR_BAD_SHAPE;
    if (lnoop || cnoop) return TTT_OK;
    LinFwdLaunch l;
    int resident = 0;
    const View4 none{nullptr, 0, 0, 0}, zv{(void*)16, 0, 0, 0};
    if ((st = plan_fullbatch(lin, none, none, none, zv, nullptr, nullptr, nullptr, nullptr, l, resident)) != TTT_OK)
        return st;
    const ConvLaunch c = plan_conv_call(conv, none, none, none, zv, nullptr, nullptr, nullptr, nullptr);
    *fused = layer_would_fuse(l, resident, c) ? 1 : 0;
    return TTT_OK;
}

// Counter blocks of each workspace kind: linear, conv and backward
// workspaces start with one; the layer workspace holds the conv block at 0
// and the linear block right after it; the scan's has none.
static int counter_blocks(ttt_op op) {
    switch (op) {
    case TTT_OP_LINEAR_FULLBATCH:
    case TTT_OP_DWCONV3X3_FULLBATCH:
    case TTT_OP_LINEAR_FULLBATCH_BWD: return 1;
    case TTT_OP_LAYER_FULLBATCH: return 2;
    default: return 0;
    }
}

ttt_status ttt_workspace_exchange_failed(ttt_op op, const void* ws, size_t ws_bytes, int32_t* failed,
                                         ttt_stream_t stream) {
    if (!failed) return TTT_ERR_NULL_POINTER;
    *failed = 0;
    if (op < TTT_OP_LINEAR_FULLBATCH || op > TTT_OP_MLP_FULLBATCH) return TTT_ERR_UNSUPPORTED;
    const int nb = counter_blocks(op);
    if (nb == 0 || ws_bytes == 0) return TTT_OK;
    if (!ws) return TTT_ERR_NULL_POINTER;
    if ((uintptr_t)ws % 256) return TTT_ERR_MISALIGNED;
    // a workspace smaller than its counter blocks has never run a split slice
    const int lines = (int)std::min<size_t>((size_t)nb * kMaxBarrierSlices, ws_bytes / (kCounterStride * 4));
    unsigned words[2 * kMaxBarrierSlices];
    // the failure word of each counter line (4th word of its 256 bytes)
    const char* src = (const char*)ws + 4 * sizeof(unsigned);
    if (hipMemcpy2DAsync(words, sizeof(unsigned), src, kCounterStride * sizeof(unsigned), sizeof(unsigned), lines,
                         hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
        return TTT_ERR_HIP;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TTT_ERR_HIP;
    for (int i = 0; i < lines; ++i)
        if (words[i]) *failed = 1;
    return TTT_OK;
}

ttt_status ttt_workspace_reset(void* ws, size_t ws_bytes, ttt_stream_t stream) {
    if (ws_bytes == 0) return TTT_OK;
    if (!ws) return TTT_ERR_NULL_POINTER;
    return hip_status(hipMemsetAsync(ws, 0, ws_bytes, (hipStream_t)stream));
}

} // extern "C"
