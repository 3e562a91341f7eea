// common.hpp -- device helpers shared by the gfx950 TTT kernels: element
// types, bf16 conversion, matrix-core (MFMA) wrappers, the per-slice
// workgroup barrier and the XCD-aware slice mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

constexpr int kD = 64;        // head dimension handled by these kernels
constexpr int kThreads = 256; // 4 waves of 64 lanes per workgroup

typedef uint16_t bf16_t; // bf16 storage

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4))); // native 16-byte vector
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 --
__device__ __forceinline__ float bf2f(bf16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with the hardware packed conversion (v_cvt_pk_bf16_f32:
// round to nearest even, NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
__device__ __forceinline__ bf16_t f2bf(float f) { return (bf16_t)(pack_bf2(f, 0.f) & 0xffffu); }

// ----------------------------------------------------------------- MFMA --
// 16x16 output tile, fp32 accumulate.  Lane l of the wave holds
//   A[m = l%16][k],  B[k][n = l%16],  D[rows 4*(l/16)+i, i=0..3][col l%16].
// mfma32: k = 8*(l/16) + j, j = 0..7 (bf16 operands, 16x16x32).
__device__ __forceinline__ v4f mfma32(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// mfma16: k = 4*(l/16) + i, i = 0..3 (bf16 operands, 16x16x16).
__device__ __forceinline__ v4f mfma16(const v4s& a, const v4s& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// mfma4: k = l/16 (fp32 operands, 16x16x4).
__device__ __forceinline__ v4f mfma4(float a, float b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(const u32x4& u) {
    return __builtin_bit_cast(v8bf, u);
}
__device__ __forceinline__ v4s as_v4s(const u32x2& u) {
    return __builtin_bit_cast(v4s, u);
}

// ------------------------------------------------------- LDS barrier --
// Workgroup barrier that orders LDS accesses only.  Unlike __syncthreads()
// it does not wait for outstanding global loads, so register prefetches
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------ slice barrier --
// Workgroups that cooperate on one slice exchange small partial results
// through the workspace, meeting at a per-slice counter.  Two protocols:
//  * XCD-local: all workgroups of the slice run on one XCD (see map_block_xcc),
//    so its L2 is their coherence point.  Data moves with ordinary 16-byte
//    stores and loads.  A CU's L1 is not coherent with the other CUs' stores
//    and cannot be invalidated cheaply (a workgroup-scope invalidate leaves
//    it as it is, measured on MI355X), so the protocol keeps exchanged
//    lines out of the reader's L1 until they are final: every exchanged
//    line is read with plain loads only after the barrier that follows its
//    last store, by workgroups that have not loaded it earlier in the
//    launch (L1 starts clean at each launch); earlier touches, such as L2
//    prefetches, use device-scope loads, which do not fill L1.
//  * device-wide: data moves with device-scope relaxed atomics (xstore /
//    xload), performed at the device coherence point.
// Neither needs an L2-wide writeback or invalidate.
__device__ __forceinline__ void xstore(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float xload(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned xcc_id() {
    return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20); // HW_REG_XCC_ID[3:0]
}

// Every workspace starts with a fixed block of kMaxBarrierSlices counters,
// whatever the problem shape, so partial sums of one call can never land on
// the counters another call relies on being zero.  Each counter has a
// 256-byte line of its own: slices polling neighbouring counters would
// otherwise serialise on one line.  Slices only meet at barriers when
// S >= 2 workgroups share a slice, which the resident-grid limit (256
// workgroups) confines to at most 128 slices.
constexpr int kMaxBarrierSlices = 256;
constexpr int kCounterStride = 64; // unsigned ints
constexpr size_t kCounterBytes = (size_t)kMaxBarrierSlices * kCounterStride * sizeof(unsigned);
__device__ __forceinline__ unsigned* counter_at(unsigned* base, int slice) {
    return base + (size_t)slice * kCounterStride;
}

// Barrier of the S workgroups of one slice at its counter.  The counter
// only grows during a launch (targets S, 2S, ...); after the last barrier
// every workgroup adds one more and the one that brings it to
// (nbarriers+1)*S resets it to zero, so the next call on the same workspace
// starts from zero.  All workgroups of a slice must be co-resident: the
// host keeps the grid within the device's resident capacity.
// Each wave first drains its vector-memory counter, so its exchange stores
// have completed before lane 0 signals (a workgroup barrier alone does not
// wait for global stores); the __syncthreads() after the wait keeps later
// exchange loads behind it.
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The wait is bounded (kSpinLimit polls, about a second): a slice whose
// workgroups never all arrive -- co-residency broken by other work on the
// device, or a dispatch that placed two workgroups on one split (see
// map_block_xcc) -- marks its counter line as failed instead of hanging;
// every later check of that line (slice_bad) reports it, in this call and
// in every later call on the same workspace, until the host clears it
// (ttt_workspace_reset); the host can read it (ttt_workspace_exchange_failed).
// The poll limit and an offset added to every barrier target are kernel
// arguments, so the host can force the give-up path (a tiny limit and an
// unreachable target) with every kernel still ending normally.
constexpr unsigned kSpinLimit = 1u << 21;
// The slice's placement word (see placement_note) and the failure word
// share the counter's line.
__device__ __forceinline__ unsigned long long* placement_at(unsigned* cnt) {
    return reinterpret_cast<unsigned long long*>(cnt + 2);
}
__device__ __forceinline__ unsigned* failed_at(unsigned* cnt) { return cnt + 4; }

// Outcome of the exchange: thread 0 loads the slice's words after the
// slice's last waiting barrier (slice_words: the loads are issued at once,
// their values are needed only by slice_bad), and before the workgroup's
// release (the reset clears them once every workgroup has released).
// slice_bad is true when the line has failed or, for an XCD-local exchange
// (S > 0), when the splits that arrived are not exactly 0..S-1 once each.
struct SliceWords {
    unsigned long long placement;
    unsigned failed;
};
__device__ __forceinline__ SliceWords slice_words(unsigned* cnt) {
    SliceWords w;
    w.placement = __hip_atomic_load(placement_at(cnt), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w.failed = __hip_atomic_load(failed_at(cnt), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return w;
}
__device__ __forceinline__ bool slice_bad(const SliceWords& w, int S) {
    if (S <= 0) return w.failed != 0;
    return w.failed != 0 || w.placement != (0x5555555555555555ull >> (64 - 2 * S));
}

// A wave that made no exchange stores since the last barrier may pass
// drain = false, keeping its loads in flight.
__device__ __forceinline__ void slice_barrier(unsigned* cnt, unsigned target, bool drain, unsigned spin) {
    if (drain) drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned it = 0;
        while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++it >= spin) {
                __hip_atomic_store(failed_at(cnt), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
}

// Reset by the workgroup that completes the slice's count: counter and
// placement word start from zero at the next call (the failure word stays).
__device__ __forceinline__ void slice_reset(unsigned* cnt) {
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(placement_at(cnt), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slice_barrier_release(unsigned* cnt, unsigned total) {
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == total - 1) slice_reset(cnt);
    }
}

// ------------------------------------------------- placement check -------
// With map_block_xcc every workgroup of a slice runs on the slice's XCD by
// construction; what remains to check is that each split arrived exactly
// once.  Thread 0 of each workgroup adds one to its split's 2-bit field of
// the slice's placement word before its first barrier arrival (which
// drains its memory operations); after the last waiting barrier the word
// reads 0b01 in each of the S fields unless a split was missing or doubled
// (slice_bad).  S <= 32.
__device__ __forceinline__ void placement_note(unsigned* cnt, int split) {
    __hip_atomic_fetch_add(placement_at(cnt), 1ull << (2 * split), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------- direct-to-LDS load --
// Direct global->LDS 16-byte load per lane (lane l writes 16 bytes at
// lds_off + 16 l), written as inline assembly: the compiler neither sees it
// nor makes later LDS reads wait for it, so the kernel waits for exactly
// the loads it needs with vmcnt_at_most().  lds_off must be wave-uniform.
__device__ __forceinline__ void dma16(const void* src, const void* lds_dst) {
    const uint32_t off = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_dst);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(off)
                 : "memory", "m0");
}
// Wait until at most n of this wave's vector-memory operations are
// outstanding (they complete in issue order).  n of 63 and above (the
// counter's limit) waits for none; n <= 0 waits for all.
__device__ __forceinline__ void vmcnt_at_most(int n) {
    switch (__builtin_amdgcn_readfirstlane(n)) { // wave-uniform
#define TTT_VMCNT(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
#define TTT_VMCNT8(k) TTT_VMCNT(k) TTT_VMCNT(k + 1) TTT_VMCNT(k + 2) TTT_VMCNT(k + 3) \
    TTT_VMCNT(k + 4) TTT_VMCNT(k + 5) TTT_VMCNT(k + 6) TTT_VMCNT(k + 7)
        TTT_VMCNT(1) TTT_VMCNT(2) TTT_VMCNT(3) TTT_VMCNT(4) TTT_VMCNT(5) TTT_VMCNT(6) TTT_VMCNT(7)
        TTT_VMCNT8(8) TTT_VMCNT8(16) TTT_VMCNT8(24) TTT_VMCNT8(32) TTT_VMCNT8(40) TTT_VMCNT8(48)
        TTT_VMCNT(56) TTT_VMCNT(57) TTT_VMCNT(58) TTT_VMCNT(59) TTT_VMCNT(60) TTT_VMCNT(61) TTT_VMCNT(62)
#undef TTT_VMCNT8
#undef TTT_VMCNT
    default:
        if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        break;
    }
}

// ------------------------------------------ transposing LDS reads --
// Staged bf16 token rows (128 bytes) read with transposing loads:
// one half-wave of such a read covers rows 8g + e, 8(g+1) + e (e = 0..3,
// g even), 32 bytes each; the swizzle gives the four rows of each parity
// four different slot pairs, so the half-wave touches every LDS bank once.
__device__ __forceinline__ int swz_tr(int row) { return 2 * ((row >> 1) & 1) + 4 * ((row >> 3) & 1); }

// ------------------------------------------- Gram by tile ownership (bf16) --
// Wave w accumulates rows 16w..16w+15 of C = V^T K and of A = K^T K over
// every token of the split (16 + 16 tiles of which it owns 4 + 4), so the
// four waves never add partial sums.  Token-contracted operands come from
// the staged rows with ds_read_b64_tr_b16: in each 16-lane group, lane
// 4e + a points at token 8g + e (second read: + 4), channels 16 blk + 4a,
// and lane m of the group receives channel 16 blk + m of those four tokens,
// which is the MFMA operand layout (k = token).  Rows are XOR-swizzled by
// swz_tr (the same for the two reads of a pair).
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s;

__device__ __forceinline__ int tr_off(int lane, int blk) {
    const int g = lane >> 4, e = (lane & 15) >> 2, aa = lane & 3;
    return (8 * g + e) * 128 + (((2 * blk + (aa >> 1)) ^ swz_tr(8 * g + e)) << 4) + (aa & 1) * 8;
}
__device__ __forceinline__ v8bf tr_pair(const char* p) {
    const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
    const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * 128));
    return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// K, V: staged bf16 rows (128 bytes, swz_tr), rows past the data zeroed up
// to a multiple of 32.  Adds rows [r0, r1) (multiples of 32) of the
// products to rows 16W.. of C and A in accC / accA: lane (g, m) holds
// [16W + 4g + i][16cb + m].  W is the wave's block (compile time, so its
// own K block is one of the four it reads); DC / DA select the C and A
// parts.
template <int W, bool DC = true, bool DA = true>
__device__ __forceinline__ void gram_owned_bf(const char* Ks, const char* Vs, int r0, int r1, int lane, v4f* accC,
                                              v4f* accA) {
    int off[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) off[blk] = tr_off(lane, blk);
    if (r1 <= r0) return;
    // two operand sets in turn: the reads of one 32-token step are in
    // flight while the products of the previous one run (a re-read of the
    // last step of the range is in bounds and unused)
    struct Ops {
        v8bf k[4], vown;
    };
    auto fetch = [&](int r0, Ops& o) __attribute__((always_inline)) {
        const char* kp = Ks + r0 * 128;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) o.k[blk] = tr_pair(kp + off[blk]);
        if constexpr (DC) o.vown = tr_pair(Vs + r0 * 128 + off[W]);
    };
    auto products = [&](const Ops& o) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            if constexpr (DC) accC[cb] = mfma32(o.vown, o.k[cb], accC[cb]);
            if constexpr (DA) accA[cb] = mfma32(o.k[W], o.k[cb], accA[cb]);
        }
    };
    Ops A, B;
    fetch(r0, A);
    int r = r0;
    for (; r + 64 <= r1; r += 64) {
        fetch(r + 32, B);
        products(A);
        fetch(min(r + 64, r1 - 32), A);
        products(B);
    }
    if (r < r1) products(A);
}

// --------------------------------------------------- slice mapping ------
// Workgroup i runs on XCD i % 8 on MI355X (8 XCDs, round-robin dispatch).
// XCD-aware mapping: slice s lives on XCD s % 8 and its S workgroups are
// blocks {8*(S*(s/8) + j) + s%8 : j < S}; the grid is padded to
// 8 * ceil(slices/8) * S blocks and blocks of padding slices (>= slices)
// have no work.  Plain mapping: slice = block / S.
// Output-row permutation of the 16x16 apply products: MFMA row m of output
// block rb -> output channel, so that lane (g, .) owns the contiguous
// channels [8g, 8g+8) (blocks 0,1) and [32+8g, 32+8g+8) (blocks 2,3) and
// stores them as whole 16-byte (bf16) or 32-byte (fp32) runs.
__device__ __forceinline__ int perm_row(int rb, int m) {
    return 32 * (rb >> 1) + 8 * (m >> 2) + 4 * (rb & 1) + (m & 3);
}

struct SliceSplit {
    int slice, split;
};
// The same mapping for kernels whose splits exchange data through one XCD's
// L2, with the XCD taken from the hardware instead of assumed from the
// block index: dispatch is round-robin over the XCDs, but its starting XCD
// can change during a process (it did after a graph replay), so block i is
// treated as virtual block (i & ~7) | xcc -- every aligned group of eight
// consecutive blocks still covers each XCD once.  placement_note() checks
// the outcome.
__device__ __forceinline__ SliceSplit map_block_xcc(int blk, int S, unsigned xcc) {
    const int j = blk >> 3, x = (int)(xcc & 7);
    SliceSplit r;
    r.slice = (j / S) * 8 + x;
    r.split = j % S;
    return r;
}
__device__ __forceinline__ SliceSplit map_block(int blk, int S, int xcd_aware) {
    SliceSplit r;
    if (xcd_aware) {
        int x = blk & 7, j = blk >> 3;
        r.slice = (j / S) * 8 + x;
        r.split = j % S;
    } else {
        r.slice = blk / S;
        r.split = blk % S;
    }
    return r;
}

} // namespace ttt
