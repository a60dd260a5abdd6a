// lnr_prims.h -- device primitives for the row-reduction kernels on gfx950 (CDNA4, wave64).
//
// * Group all-reduce over G = 1..64 lanes of one wavefront with DPP lane permutations
//   (quad_perm, row_half_mirror, row_mirror), one ds_swizzle (xor 16 inside each 32-lane
//   half) and v_readlane for the two halves. Every lane of the group ends with the same,
//   bitwise identical value, and the combination order depends only on G. This is the
//   "one fewer synchronisation" idea of the L10 lecture ("Technique 2") expressed with
//   CDNA lane-crossing operations instead of warp shuffles.
// * Cross-wave reduction for rows that span several waves: one LDS slot per wave, a
//   workgroup barrier, then every lane sums the slots in wave order.
// * 128-bit global loads/stores of 8 fp16 or 4 fp32 values (global_load_dwordx4), the
//   counterpart of the float4 access the HW4 page asks for, with fp32 math in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lnr {

// ------------------------------------------------------------------------------------------
// Storage types and 16-byte vectors.
// ------------------------------------------------------------------------------------------
using f16 = _Float16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Vec16;
template <> struct Vec16<float> {
    using type = f32x4;
    static constexpr int N = 4;
};
template <> struct Vec16<f16> {
    using type = f16x8;
    static constexpr int N = 8;
};

// Two cache policies. Row data is streamed: every score, activation and gradient byte is
// read once and written once, so those accesses are non-temporal and do not evict lines
// that are reused. Small tensors that every row reads again (the key mask, gamma, beta)
// use ordinary cached loads.
template <typename T> using RawVec = typename Vec16<T>::type;

template <typename T>
__device__ __forceinline__ RawVec<T> load_stream_raw(const T *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const RawVec<T> *>(p));
}
template <typename T>
__device__ __forceinline__ RawVec<T> load_keep_raw(const T *p) {
    return *reinterpret_cast<const RawVec<T> *>(p);
}

// Widen a 16-byte vector to fp32.
template <typename T>
__device__ __forceinline__ void widen(const RawVec<T> &v, float (&out)[Vec16<T>::N]) {
#pragma unroll
    for (int e = 0; e < Vec16<T>::N; ++e) out[e] = static_cast<float>(v[e]);
}

template <typename T>
__device__ __forceinline__ void load_stream(const T *p, float (&out)[Vec16<T>::N]) {
    widen<T>(load_stream_raw<T>(p), out);
}
template <typename T>
__device__ __forceinline__ void load_keep(const T *p, float (&out)[Vec16<T>::N]) {
    widen<T>(load_keep_raw<T>(p), out);
}

// Round fp32 values to T (nearest even) and store them as one non-temporal 16-byte vector.
template <typename T>
__device__ __forceinline__ void store_stream(T *p, const float (&in)[Vec16<T>::N]) {
    RawVec<T> v;
#pragma unroll
    for (int e = 0; e < Vec16<T>::N; ++e) v[e] = static_cast<T>(in[e]);
    __builtin_nontemporal_store(v, reinterpret_cast<RawVec<T> *>(p));
}

// Branch-free stores. A row kernel whose stores sit behind a branch (a row past the end, a
// vector slot past the row) pays for it at every later wait: after the join, the compiler's
// wait counts must assume that the stores were skipped, so a wait for data loaded before them
// also waits for everything issued since. Stores through a buffer descriptor need no branch: a
// lane with nothing to store passes an offset beyond the descriptor's range and the hardware
// drops its store. `wave_base` must be the same for every lane of the wave; offsets are bytes.
constexpr uint32_t kDropOffset = 0xFFFFFFF0u;
constexpr int32_t kBufferRange = 0x7FFFFFFF;    // valid offsets stay below it
constexpr int32_t kBufferDword3 = 0x00020000;   // untyped 32-bit data (gfx9 family)
constexpr int kBufferNonTemporal = 2;           // cache policy bits of a streaming access
// Streaming stores at device scope (sc1 and nt). Measured on MI355X with one-shot 16-byte
// streams: read one tensor and write one at 512 MiB, 161.3 -> 159.1-159.6 us; read two and
// write one unchanged (243 us), and in the backward kernels 0.2-2.5% slower. So the forward
// kernels (one read stream, one write stream) store this way and the backward kernels do not.
constexpr int kBufferDeviceStream = 18;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void *wave_base, int32_t range = kBufferRange) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(wave_base), 0, range, kBufferDword3);
}
template <int POLICY = kBufferNonTemporal, typename RV>
__device__ __forceinline__ void store16_or_drop(const void *wave_base, uint32_t off, const RV &v) {
    static_assert(sizeof(RV) == 16, "16-byte vectors");
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), wave_rsrc(wave_base), off, 0, POLICY);
}
// A 16-byte vector through the same kind of descriptor, non-temporal: a lane whose offset is
// beyond the range (kDropOffset) reads zeros and touches no memory.
template <typename T>
__device__ __forceinline__ RawVec<T> load16_or_zero(const void *wave_base, uint32_t off) {
    return __builtin_bit_cast(RawVec<T>, __builtin_amdgcn_raw_buffer_load_b128(wave_rsrc(wave_base), off, 0,
                                                                               kBufferNonTemporal));
}
// A float through a descriptor of `range` bytes (0: every store dropped), cached.
__device__ __forceinline__ void store4_or_drop(const void *wave_base, int32_t range, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), wave_rsrc(wave_base, range), off, 0, 0);
}
// Round fp32 values to T (nearest even) as one 16-byte vector.
template <typename T>
__device__ __forceinline__ RawVec<T> pack16(const float (&in)[Vec16<T>::N]) {
    RawVec<T> v;
#pragma unroll
    for (int e = 0; e < Vec16<T>::N; ++e) v[e] = static_cast<T>(in[e]);
    return v;
}

template <typename T> __device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// ------------------------------------------------------------------------------------------
// Lane-crossing moves.
// ------------------------------------------------------------------------------------------
namespace dpp {
constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int kXor1 = quad_perm(1, 0, 3, 2);   // lane i <- lane i^1 within each quad
constexpr int kXor2 = quad_perm(2, 3, 0, 1);   // lane i <- lane i^2 within each quad
constexpr int kRowHalfMirror = 0x141;          // lane i <- lane 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;              // lane i <- lane 15-i within each 16 lanes
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    // All row/bank masks enabled; every source lane lies inside the same 16-lane row.
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// ds_swizzle in bit mode: and_mask = 0x1F, or_mask = 0, xor_mask = 0x10, i.e. lane i reads
// lane i ^ 16 inside each 32-lane half. Moves data through the LDS crossbar, no LDS storage.
__device__ __forceinline__ float swizzle_xor16(float v) {
    constexpr int kPattern = 0x1F | (0x10 << 10);
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kPattern));
}

__device__ __forceinline__ float read_lane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

struct OpSum {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// All-reduce across each aligned group of G consecutive lanes (G a power of two, <= 64).
// Every lane of the wave must execute this call (no divergent EXEC mask): lanes of groups
// with nothing to contribute pass the operation's identity.
// Each butterfly step leaves every lane of the next-larger aligned group with op(a, b) of
// the two halves; op is commutative, so both halves end bitwise equal, which is what lets
// the mirror permutations stand in for xor 4 and xor 8.
template <int G, class Op>
__device__ __forceinline__ float group_allreduce(float v, Op op) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64,
                  "group size must be a power of two up to a wavefront");
    if constexpr (G >= 2) v = op(v, dpp_move<dpp::kXor1>(v));
    if constexpr (G >= 4) v = op(v, dpp_move<dpp::kXor2>(v));
    if constexpr (G >= 8) v = op(v, dpp_move<dpp::kRowHalfMirror>(v));
    if constexpr (G >= 16) v = op(v, dpp_move<dpp::kRowMirror>(v));
    if constexpr (G >= 32) v = op(v, swizzle_xor16(v));
    if constexpr (G >= 64) v = op(read_lane(v, 0), read_lane(v, 32));
    return v;
}

// Two independent sums reduced together (interleaved so the lane moves overlap).
template <int G>
__device__ __forceinline__ void group_allreduce_sum2(float &a, float &b) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64,
                  "group size must be a power of two up to a wavefront");
    if constexpr (G >= 2) {
        const float ta = dpp_move<dpp::kXor1>(a), tb = dpp_move<dpp::kXor1>(b);
        a += ta; b += tb;
    }
    if constexpr (G >= 4) {
        const float ta = dpp_move<dpp::kXor2>(a), tb = dpp_move<dpp::kXor2>(b);
        a += ta; b += tb;
    }
    if constexpr (G >= 8) {
        const float ta = dpp_move<dpp::kRowHalfMirror>(a), tb = dpp_move<dpp::kRowHalfMirror>(b);
        a += ta; b += tb;
    }
    if constexpr (G >= 16) {
        const float ta = dpp_move<dpp::kRowMirror>(a), tb = dpp_move<dpp::kRowMirror>(b);
        a += ta; b += tb;
    }
    if constexpr (G >= 32) {
        const float ta = swizzle_xor16(a), tb = swizzle_xor16(b);
        a += ta; b += tb;
    }
    if constexpr (G >= 64) {
        a = read_lane(a, 0) + read_lane(a, 32);
        b = read_lane(b, 0) + read_lane(b, 32);
    }
}

// Reduction over a row held by G lanes, where G may exceed one wave (G = 64 * W).
// `lds` must hold 2 * (blockDim.x / 64) floats. Every thread of the workgroup must call it
// (it contains barriers). The wave partials are summed in wave order, so the result does
// not depend on timing.
template <int G>
__device__ __forceinline__ void row_allreduce_sum2(float &a, float &b, float *lds) {
    if constexpr (G <= 64) {
        group_allreduce_sum2<G>(a, b);
    } else {
        constexpr int W = G / 64;
        group_allreduce_sum2<64>(a, b);
        const int wave = threadIdx.x >> 6;
        const int first = wave - (wave % W);   // first wave of this row's group
        if ((threadIdx.x & 63) == 0) {
            lds[2 * wave] = a;
            lds[2 * wave + 1] = b;
        }
        __syncthreads();
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            sa += lds[2 * (first + w)];
            sb += lds[2 * (first + w) + 1];
        }
        __syncthreads();  // the slots may be rewritten by the next row
        a = sa;
        b = sb;
    }
}

// Sums of NV values at once over a row held by G lanes (G <= 64, or G = 64 * W with the
// wave partials crossing through LDS). `lds` must hold NV * (blockDim.x / 64) floats. Every
// thread of the workgroup must call it. Fixed order, as above.
template <int G, int NV>
__device__ __forceinline__ void row_allreduce_sumN(float (&v)[NV], float *lds) {
    static_assert(NV % 2 == 0, "values are reduced in pairs");
#pragma unroll
    for (int i = 0; i < NV; i += 2) group_allreduce_sum2<G < 64 ? G : 64>(v[i], v[i + 1]);
    if constexpr (G > 64) {
        constexpr int W = G / 64;
        const int wave = threadIdx.x >> 6;
        const int first = wave - (wave % W);
        if ((threadIdx.x & 63) == 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i) lds[NV * wave + i] = v[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) t += lds[NV * (first + w) + i];
            v[i] = t;
        }
        __syncthreads();
    }
}

template <int G, class Op>
__device__ __forceinline__ float row_allreduce(float v, Op op, float *lds) {
    if constexpr (G <= 64) {
        return group_allreduce<G>(v, op);
    } else {
        constexpr int W = G / 64;
        v = group_allreduce<64>(v, op);
        const int wave = threadIdx.x >> 6;
        const int first = wave - (wave % W);
        if ((threadIdx.x & 63) == 0) lds[wave] = v;
        __syncthreads();
        float s = lds[first];
#pragma unroll
        for (int w = 1; w < W; ++w) s = op(s, lds[first + w]);
        __syncthreads();
        return s;
    }
}

// exp(d) for d <= 0 (or -inf) with the hardware base-2 exponential: exp(d) = 2^(d*log2(e)).
// d is formed as (z - max) before scaling, so its rounding error is relative to |z - max|
// and not to the magnitude of the scores.
__device__ __forceinline__ float exp_nonpos(float d) {
    return __builtin_amdgcn_exp2f(d * 1.4426950408889634f);
}

}  // namespace lnr
