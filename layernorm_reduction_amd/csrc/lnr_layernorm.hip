// lnr_layernorm.hip -- LayerNorm forward and backward for gfx950.
//
// Method: "CMU 11-868 L10 ...", section "Technique 2: rewrite the formula, drop a
// synchronization": sigma = sqrt(mu(x^2) - mu(x)^2), so mu(x) and mu(x^2) come from ONE
// reduction; the backward input gradient is two row sums (of gamma*dy and gamma*dy*xhat)
// computed together; FP32 compute with FP16 storage. "CMU 11-868 HW4 ...", section "Problem
// structure and scoring": eps = 1e-8 inside the root; gamma/beta gradients summed across
// rows (the page stages them in shared memory and reduces along the row axis).
//
// Design on CDNA4:
//   * Row kernels hold a row in registers across G lanes (G <= 64: one wave, several rows
//     per wave for short rows; G = 128..1024: several waves per row, the two partial sums
//     crossing waves through LDS with one barrier pair). 128-bit loads and stores.
//   * Forward: one read of x, one write of y, per-row mean and rstd in fp32. The variance
//     from the one-pass sums is clamped at 0 before eps is added.
//   * Backward, fused: P workgroups (one per CU) sweep the rows in bands of P*NG consecutive
//     rows, each taking NG consecutive rows of every band (NG row groups per workgroup), with
//     one or two rows fetched ahead. Because a lane owns the same columns in every row, it
//     accumulates dgamma/dbeta column partials in registers while it computes dx, so x and
//     dy are read from HBM exactly once. The launch plan depends on the width (a plan may
//     also require a minimum row count). At the end the workgroup's row groups are combined in
//     group order (through LDS when there are several) into one partial row per workgroup,
//     written to the workspace as 16-byte vectors. A second small kernel sums the partials
//     in a fixed order. No atomics: results are bitwise reproducible.
//     Partials are fp32 for fp16 storage and fp64 for fp32 storage, so the long column sums
//     over tens of thousands of rows add no rounding beyond the per-element products.
//   * RMSNorm ("FastTransformer: Breaking the Compiler Ceiling via Architectural
//     Co-Design", section 5.4: the LayerNorm without the mean, y = x * rsqrt(mean(x^2) +
//     eps) * weight, no bias) is the same kernels with the RMS flag: no shift or mean, one
//     reduction (sum of x^2 forward, sum of gamma*dy*xhat backward), no beta and no dbeta.
#include <math.h>

#include <atomic>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "lnr_common.h"
#include "lnr_prims.h"

namespace lnr {

template <typename T> struct Accum;
template <> struct Accum<f16> { using type = float; };
template <> struct Accum<float> { using type = double; };

// Statistics from the one fused pass. The two sums are taken over d = x - K, with K the
// row's first element: mu(d^2) - mu(d)^2 equals the variance of x for any shift K, and a
// shift near the mean removes the cancellation that fp32 one-pass sums suffer when the
// variance is small next to mean^2. xhat is then formed as (d - mu(d)) * rstd, so no
// rounding of K + mu(d) enters it. No contraction here: a constant row (or C = 1) gives
// s1 = s2 = 0 and therefore a variance of exactly 0. invC = 1 / C (rounded once per kernel);
// the means are products with it and rstd is the hardware reciprocal square root (both
// within 1 ulp of the divisions they replace, at a fraction of their instructions: every
// lane of a row evaluates this once per row).
__device__ __forceinline__ float ln_stats(float s1, float s2, float invC, float eps, float &m1) {
#pragma clang fp contract(off)
    m1 = s1 * invC;
    const float var = fmaxf(s2 * invC - m1 * m1, 0.f);
    return __builtin_amdgcn_rsqf(var + eps);
}

// What the row kernels normalise.
enum NormMode : int {
    kLayerNorm = 0,     // y = LayerNorm(x)
    kRmsNorm = 1,       // y = RMSNorm(x)
    kBdrLayerNorm = 2,  // s = residual + keep * (x + bias) * keep_scale; y = LayerNorm(s)
};

// Keep bits of vector c of a row: mask bytes hold one bit per element, least significant
// bit first; a 16-byte vector covers 8 fp16 elements (one byte) or 4 fp32 elements (half a
// byte).
template <typename T>
__device__ __forceinline__ uint32_t keep_bits(const uint8_t *mrow, int c) {
    if constexpr (Vec16<T>::N == 8) {
        return mrow[c];
    } else {
        const uint32_t b = mrow[c >> 1];
        return (c & 1) ? (b >> 4) : (b & 15u);
    }
}

// RMSNorm statistic: rstd = 1 / sqrt(mean(x^2) + eps), from the one sum of squares (invC
// and the reciprocal square root as in ln_stats).
__device__ __forceinline__ float rms_stats(float s2, float invC, float eps) {
#pragma clang fp contract(off)
    return __builtin_amdgcn_rsqf(s2 * invC + eps);
}

// ------------------------------------------------------------------------------------------
// Forward, vector path. Workgroup b normalises rows [b*P, (b+1)*P) with P = rows_per_block =
// NG * R; group g of the workgroup takes rows b*P + g, b*P + g + NG, ... (R of them). gamma
// and beta are loaded once per workgroup. The next row's vectors (and its shift K) are
// fetched before the current row is reduced, so each wave keeps a row of loads in flight
// while it computes; the fetch is issued unconditionally (an idle lane reads a vector that
// always exists) so that no branch makes the compiler drain the loads early.
// At fp16 the kernel is bound by VALU issue as much as by HBM (a wave64 fp32 operation takes
// a SIMD 4 cycles), so the per-element work is kept small: idle lanes (only in plans wider
// than the row) take the value K, which makes d = x - K exactly 0 without a select per
// element; the widening and the subtraction of K are one mixed-precision fma (x * 1 - K,
// rounded once like the plain subtraction; the 1 is hidden from the compiler, which would
// otherwise fold it back into a conversion and a subtraction); and y = (d * rstd - mu(d) *
// rstd) * gamma + beta is two fmas.
// kBdrLayerNorm: the row is s = residual + keep * (x + bias) * keep_scale, formed in fp32 from
// x, residual and the row's mask bytes, written to s_out (the residual stream), and
// normalised in fp32.
// ------------------------------------------------------------------------------------------
template <typename T, int G, int IT, int WG, int MODE, int R>
__global__ __launch_bounds__(WG) void layernorm_fw_vec(T *y, float *__restrict__ mean,
                                                       float *__restrict__ rstd, const T *x,
                                                       const T *__restrict__ gamma,
                                                       const T *__restrict__ beta, int64_t N,
                                                       int32_t C, float eps,
                                                       int64_t rows_per_block, T *s_out,
                                                       const T *residual,
                                                       const T *__restrict__ bias,
                                                       const uint8_t *__restrict__ mask,
                                                       float keep_scale) {
    constexpr bool RMS = MODE == kRmsNorm;
    constexpr bool BDR = MODE == kBdrLayerNorm;
    using RV = RawVec<T>;
    constexpr int V = Vec16<T>::N;
    constexpr int NG = WG / G;
    __shared__ float red[2 * (WG / 64)];
    const int lane = threadIdx.x % G;
    const int grp = threadIdx.x / G;
    const int nvec = C / V;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_block;
    const int64_t r1 = (r0 + rows_per_block < N) ? r0 + rows_per_block : N;
    const RV zero = {};

    const int64_t mb = (C + 7) / 8;  // mask bytes per row
    float gm[IT][V], bt[IT][RMS ? 1 : V], bs[IT][BDR ? V : 1];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        const int cc = c < nvec ? c : 0;
        widen<T>(load_keep_raw<T>(gamma + cc * V), gm[k]);
        if constexpr (!RMS) widen<T>(load_keep_raw<T>(beta + cc * V), bt[k]);
        if constexpr (BDR) widen<T>(load_keep_raw<T>(bias + cc * V), bs[k]);
    }
    // The shift K of a kBdrLayerNorm row is its first s element, formed from the inputs. A row
    // inside one wave (G <= 64) has that element in its group's first lane (vector slot 0,
    // element 0), which forms it from its own registers; the group reads it with one
    // cross-lane read, so the shift waits on no load of its own. Measured on MI355X: loaded
    // separately, the compiler sank the loads of x[0] and bias[0] under the keep bit and the
    // row waited for both in turn (forward at [16384,1024] fp16 5% slower). Rows over several
    // waves load the first element's inputs with the row.
    constexpr bool kShiftFromLane = G <= 64;
    float b0 = 0.f;
    if constexpr (BDR && !kShiftFromLane) b0 = to_f32(bias[0]);

    // The row loop has R iterations, a compile-time count, but stays rolled: unrolled, the
    // compiler issues the loads of all R rows up front, and the extra registers cost more
    // than the copy of the prefetched row at the end of each iteration (2-5% on MI355X).
    // Variants measured against this structure and rejected (all on MI355X, fp16 and fp32):
    // fetching the first row before gamma and beta, and clamping a dead first row to a live
    // one so that no branch forms around its loads (both 3-6% slower at 4096-8192 columns);
    // masking dead prefetch addresses through inline asm (6% slower: the asm splits the
    // loop's scheduling region).
    const float invC = 1.0f / static_cast<float>(C);
    RV xn[IT], rn[BDR ? IT : 1];
    uint32_t kn[BDR ? IT : 1];
    float Kn;
    T Kraw = T(0);  // the shift as stored (not kBdrLayerNorm): what idle lanes hold
    // kBdrLayerNorm: the raw inputs of the row's shift (x, residual and mask of its first
    // element), loaded with the row and combined when it is reduced. Combined in the fetch,
    // the compiler sinks the x load under the mask bit and the fetch waits for that load.
    T x0n = T(0), r0n = T(0);
    uint32_t m0n = 0u;
    auto fetch = [&](int64_t row, bool live) {
        const int64_t rbase = (live ? row : r0) * static_cast<int64_t>(C);
        const uint8_t *mrow = BDR ? mask + (live ? row : r0) * mb : nullptr;
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int c = k * G + lane;
            const bool ok = live && c < nvec;
            const int64_t off = rbase + (ok ? static_cast<int64_t>(c) * V : 0);
            const RV l = load_stream_raw<T>(x + off);
            xn[k] = BDR ? (ok ? l : zero) : l;
            if constexpr (BDR) {
                const RV lr = load_stream_raw<T>(residual + off);
                const uint32_t kb = keep_bits<T>(mrow, ok ? c : 0);
                rn[k] = ok ? lr : zero;
                kn[k] = ok ? kb : 0u;
            }
        }
        if constexpr (BDR) {
            if constexpr (!kShiftFromLane) {
                x0n = x[rbase];
                r0n = residual[rbase];
                m0n = mrow[0];
            }
            Kn = 0.f;
        } else if constexpr (!RMS) {
            Kraw = x[rbase];  // the shift: one broadcast load per group
            Kn = to_f32(Kraw);
        } else {
            Kn = 0.f;
        }
    };
    float one = 1.0f;
    if constexpr (V == 8) asm("" : "+v"(one));
    // Stores are branch-free (store16_or_drop): offsets count from the row of the wave's first
    // row group; a lane of a row past the end, or of a vector slot past the row, is dropped.
    // Rows over eight or more waves (fp32 from 4096 columns) store under a branch instead:
    // measured in one process at [32768,4096] fp32, 169.5 us against 175.0 branch-free, while
    // the fp16 plans (up to four waves per row) run 0.5-1.2% faster branch-free.
    constexpr bool kBranchStores = G >= 512;
    const int grp0 = __builtin_amdgcn_readfirstlane(grp);
    const int32_t stat_range = rstd != nullptr ? kBufferRange : 0;  // statistics not wanted: dropped
    fetch(r0 + grp, r0 + grp < r1);
#pragma unroll 1
    for (int it = 0; it < R; ++it) {
        const int64_t row = r0 + static_cast<int64_t>(it) * NG + grp;
        const bool live = row < r1;
        RV xc[IT], rc[BDR ? IT : 1];
        uint32_t kc[BDR ? IT : 1];
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            xc[k] = xn[k];
            if constexpr (BDR) {
                rc[k] = rn[k];
                kc[k] = kn[k];
            }
        }
        float K = Kn;
        const T Kc = Kraw;
        if constexpr (BDR && kShiftFromLane) {
            const float r0f = to_f32(rc[0][0]);
            const float own = (kc[0] & 1u) ? __builtin_fmaf(to_f32(xc[0][0]) + bs[0][0], keep_scale, r0f) : r0f;
            const int src = static_cast<int>((threadIdx.x & 63u) & ~static_cast<unsigned>(G - 1)) << 2;
            K = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, own)));
        } else if constexpr (BDR) {
            K = (m0n & 1u) ? __builtin_fmaf(to_f32(x0n) + b0, keep_scale, to_f32(r0n)) : to_f32(r0n);
        }
        fetch(row + NG, it + 1 < R && row + NG < r1);
        const int64_t wrow_raw = r0 + static_cast<int64_t>(it) * NG + grp0;
        const int64_t wrow = wrow_raw < N ? wrow_raw : 0;      // the wave's row base (uniform)
        auto off_of = [&](int k) -> uint32_t {
            const int c = k * G + lane;
            return (live && c < nvec) ? static_cast<uint32_t>(((row - wrow) * C + static_cast<int64_t>(c) * V) *
                                                              static_cast<int64_t>(sizeof(T)))
                                      : kDropOffset;
        };

        float d[IT][V];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const bool ok = k * G + lane < nvec;
            if constexpr (!BDR) {
                if ((k + 1) * G > nvec) {  // uniform: this vector slot has idle lanes
                    RV kv;
#pragma unroll
                    for (int e = 0; e < V; ++e) kv[e] = Kc;
                    xc[k] = ok ? xc[k] : kv;
                }
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    d[k][e] = __builtin_fmaf(static_cast<float>(xc[k][e]), one, -K);
                    if constexpr (!RMS) s1 += d[k][e];
                    s2 = __builtin_fmaf(d[k][e], d[k][e], s2);
                }
                continue;
            }
            widen<T>(xc[k], d[k]);
            if constexpr (BDR) {
                float rf[V];
                widen<T>(rc[k], rf);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    // s = r + (x + b) * scale for a kept element (one fma: one rounding), r
                    // exactly for a dropped one; the element-wise kernel forms it the same way.
                    d[k][e] = ((kc[k] >> e) & 1u) ? __builtin_fmaf(d[k][e] + bs[k][e], keep_scale, rf[e]) : rf[e];
                store16_or_drop<kBufferDeviceStream>(s_out + wrow * static_cast<int64_t>(C), off_of(k), pack16<T>(d[k]));
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                d[k][e] = ok ? d[k][e] - K : 0.f;
                if constexpr (!RMS) s1 += d[k][e];
                s2 = __builtin_fmaf(d[k][e], d[k][e], s2);
            }
        }
        float m1 = 0.f, rs;
        if constexpr (RMS) {
            s2 = row_allreduce<G>(s2, OpSum(), red);
            rs = rms_stats(s2, invC, eps);
        } else {
            row_allreduce_sum2<G>(s1, s2, red);
            rs = ln_stats(s1, s2, invC, eps, m1);
        }
        const float nmr = -(m1 * rs);
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if constexpr (RMS)
                    o[e] = d[k][e] * rs * gm[k][e];
                else
                    o[e] = __builtin_fmaf(__builtin_fmaf(d[k][e], rs, nmr), gm[k][e], bt[k][e]);
            }
            if constexpr (kBranchStores) {
                const int c = k * G + lane;
                if (live && c < nvec)
                    store_stream<T>(y + row * static_cast<int64_t>(C) + static_cast<int64_t>(c) * V, o);
            } else {
                store16_or_drop<kBufferDeviceStream>(y + wrow * static_cast<int64_t>(C), off_of(k), pack16<T>(o));
            }
        }
        // One lane per row stores its statistics (RMSNorm: no mean).
        if constexpr (kBranchStores) {
            if (live && lane == 0 && rstd != nullptr) {
                if constexpr (!RMS) mean[row] = K + m1;
                rstd[row] = rs;
            }
        } else {
            const uint32_t soff = (live && lane == 0) ? static_cast<uint32_t>((row - wrow) * 4) : kDropOffset;
            if constexpr (!RMS) store4_or_drop(stat_range ? mean + wrow : rstd, stat_range, soff, K + m1);
            store4_or_drop(stat_range ? rstd + wrow : mean, stat_range, soff, rs);
        }
    }
}

// ------------------------------------------------------------------------------------------
// Backward, vector path: dx plus per-workgroup dgamma/dbeta column partials.
// part layout: [P][2][C] of Accum<T>; slot 0 = dgamma, slot 1 = dbeta (unused for RMSNorm).
// ------------------------------------------------------------------------------------------
// LDS budget of the backward's final column-tile reduction (gfx950 gives a workgroup up to
// 160 KiB; the backward grids run one workgroup per CU).
constexpr size_t kTileBytes = 96 * 1024;

// Four 16-byte vectors of zeros in global memory (never written): what a row past the end
// reads in the backward (x from the first, dy from the second, its mean and rstd from the
// third and fourth), so that it adds nothing to the column partials without a select per
// element or on its stats. Distinct addresses: loads the compiler can prove equal for a dead
// row are merged and branched around.
__device__ uint32_t kZero32[16] __attribute__((aligned(16))) = {};
template <typename T>
__device__ __forceinline__ const T *zero16(int which) {
    return reinterpret_cast<const T *>(kZero32 + 4 * which);
}

// V column partials of one lane written as whole 16-byte vectors (dst 16-byte aligned).
template <typename A, int V>
__device__ __forceinline__ void store_partials16(A *dst, const A (&v)[V]) {
    constexpr int CH = static_cast<int>(16 / sizeof(A));
    using P = A __attribute__((ext_vector_type(CH)));
#pragma unroll
    for (int j = 0; j < V / CH; ++j) {
        P p;
#pragma unroll
        for (int i = 0; i < CH; ++i) p[i] = v[j * CH + i];
        *reinterpret_cast<P *>(dst + j * CH) = p;
    }
}

template <typename T, int G, int IT, int WG, int DEPTH, int MODE, bool EXTRA>
__global__ __launch_bounds__(WG) void layernorm_bw_vec(T *dx, typename Accum<T>::type *part,
                                                       const T *dy, const T *x,
                                                       const T *__restrict__ gamma,
                                                       const float *__restrict__ mean,
                                                       const float *__restrict__ rstd,
                                                       int64_t N, int32_t C,
                                                       int64_t rows_per_block, T *dx2,
                                                       const T *ds_extra,
                                                       const uint8_t *__restrict__ mask,
                                                       float keep_scale) {
#pragma clang fp contract(off)
    static_assert(DEPTH == 1 || DEPTH == 2, "rows fetched ahead: 1 or 2");
    // kBdrLayerNorm: x is the saved s; dx receives ds = (LayerNorm input gradient) + ds_extra
    // (the residual gradient; EXTRA says it is given, and it is then fetched with the row),
    // dx2 = keep * ds * keep_scale (the gradient of x), and a third column partial accumulates
    // dbias = sum over rows of dx2.
    constexpr bool RMS = MODE == kRmsNorm;
    constexpr bool BDR = MODE == kBdrLayerNorm;
    constexpr int SLOTS = BDR ? 3 : 2;
    using A = typename Accum<T>::type;
    using RV = RawVec<T>;
    constexpr int V = Vec16<T>::N;
    constexpr int NG = WG / G;  // row groups per workgroup
    // Column partials staged per round of the final LDS reduction: (vector slot, partial)
    // pairs of G*V columns from each staged row group (with two groups only the second is
    // staged), as many as fit kTileBytes (all of them for 512-thread plans).
    constexpr int NSTAGE = NG > 2 ? NG : 1;
    constexpr int PAIRS = IT * (RMS ? 1 : SLOTS);
    constexpr int PER_FIT = static_cast<int>(kTileBytes / (static_cast<size_t>(NSTAGE) * G * V * sizeof(A)));
    constexpr int PER = PER_FIT < 1 ? 1 : (PER_FIT < PAIRS ? PER_FIT : PAIRS);
    __shared__ float red[2 * (WG / 64)];
    __shared__ A tile[NSTAGE][NG > 1 ? PER * G * V : 1];

    const int lane = threadIdx.x % G;
    const int grp = threadIdx.x / G;
    const int nvec = C / V;
    // Rows of this workgroup: row = (it*P + blockIdx.x)*NG + grp (P = gridDim.x). All P
    // workgroups sweep one band of NG*P consecutive rows at a time, and within the band each
    // workgroup takes NG consecutive rows, so every workgroup reads one contiguous stretch of
    // each tensor per step. Measured on MI355X with the access pattern alone (no arithmetic,
    // [32768, 1024] fp16): 34.3 us, against 39.0 us with the band's rows dealt round-robin over
    // the workgroups (row = (it*NG + grp)*P + blockIdx.x: a workgroup's rows 512 KB apart) and
    // slower still with one contiguous chunk of N/P rows per workgroup.
    // rows_per_block >= ceil(N / P), a multiple of NG, bounds the trip count.
    const int64_t P = gridDim.x;
    const int64_t first_row = blockIdx.x;
    const float invC = 1.0f / static_cast<float>(C);
    const RV zero = {};
    // 1 and -0 hidden from the compiler, which would otherwise fold x * 1 + y and x * y + -0
    // back into separate widenings and plain operations.
    float one = 1.0f, nzero = -0.0f;
    asm("" : "+v"(one), "+v"(nzero));

    RV gmr[IT];  // gamma, kept as stored (16 bytes per vector) to save registers
    A adg[IT][V], adb[IT][RMS ? 1 : V], adx[IT][BDR ? V : 1];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        const RV gl = load_keep_raw<T>(gamma + (c < nvec ? c : 0) * V);
        gmr[k] = c < nvec ? gl : zero;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            adg[k][e] = A(0);
            if constexpr (!RMS) adb[k][e] = A(0);
            if constexpr (BDR) adx[k][e] = A(0);
        }
    }
    const int64_t mb = (C + 7) / 8;  // mask bytes per row

    // A row buffer holds one row's x and dy vectors (as stored) plus its mean and rstd.
    // DEPTH rows are fetched ahead of the one being reduced, so every wave keeps DEPTH rows
    // of loads in flight while it computes. With DEPTH = 2 three buffers rotate through an
    // unrolled loop (no register copies). Fetches are issued unconditionally (an idle lane
    // reads the workgroup's first row, which always exists) and idle values are zeroed: with no
    // branch around the loads the compiler keeps them outstanding. Iterations past the last
    // row are idle rows of zeros, so every group runs the same trip count and multi-wave rows
    // can use barriers.
    static_assert(!EXTRA || BDR, "ds_extra belongs to the bias-dropout-residual mode");
    struct RowBuf {
        RV xv[IT], dv[IT], ev[EXTRA ? IT : 1];
        uint32_t kb[BDR ? IT : 1];
        float mu, rs;
    };
    // DEFER: a row's dx is stored after the next row's fetch has been issued. Memory
    // operations retire in issue order, so a store issued before a fetch holds up the wait for
    // that fetch's data by its own round trip. It pays off where a row sits inside one wave
    // with one or two vectors per lane (measured on MI355X: fp16 256 columns -4% backward time,
    // fp32 512 columns -9%). Rows spread over several waves (a barrier per row) ran 4-5% slower
    // with it and three vectors per lane ran out of registers (-14%): those plans store each
    // row as soon as it is formed.
    constexpr bool DEFER = DEPTH == 1 && G <= 64 && IT <= 2 && !BDR;
    const int64_t iters = (rows_per_block + NG - 1) / NG;
    auto row_of = [&](int64_t it) { return (it * P + first_row) * NG + grp; };
    // Statistics as scalar loads where a row covers whole waves and a row iteration carries
    // enough work to cover their latency, which the next LDS wait exposes (scalar loads and
    // LDS share one counter). Measured on MI355X, bitwise-equal outputs: fp32 8192 columns
    // -6%, 2048 -4%, 1024 -1%, fp16 1024-8192 -0.3 to -1.5%; with one vector per lane and
    // one row ahead (a plan of 16 waves per row at fp32 4096 columns) +2.5 to +4.5%.
    constexpr bool kScalarStats = G >= 64 && (IT >= 2 || DEPTH == 2);
    auto fetch = [&](RowBuf &b, int64_t it) {
        const int64_t row = row_of(it);
        const bool live = it < iters && row < N;
        const int64_t rbase = (live ? row : first_row) * static_cast<int64_t>(C);
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int c = k * G + lane;
            const bool ok = live && c < nvec;
            if constexpr (!BDR) {
                // No select per element: an idle lane (c >= nvec) reads its row's first vector
                // and adds nothing, since its gamma is zero and its column partials are never
                // written; a row past the end reads zeros from the sentinel.
                const int64_t off = rbase + (c < nvec ? static_cast<int64_t>(c) * V : 0);
                b.xv[k] = load_stream_raw<T>(live ? x + off : zero16<T>(0));
                b.dv[k] = load_stream_raw<T>(live ? dy + off : zero16<T>(1));
                continue;
            }
            // Bias-dropout-residual mode: a lane with nothing to load (a row past the end, or
            // a vector slot past the row) reads zeros from the sentinels, so that its row
            // adds nothing to any column partial.
            const int64_t off = rbase + (ok ? static_cast<int64_t>(c) * V : 0);
            b.xv[k] = load_stream_raw<T>(ok ? x + off : zero16<T>(0));
            b.dv[k] = load_stream_raw<T>(ok ? dy + off : zero16<T>(1));
            if constexpr (BDR)
                b.kb[k] = keep_bits<T>(ok ? mask + row * mb : reinterpret_cast<const uint8_t *>(zero16<T>(2)),
                                       ok ? c : 0);
            if constexpr (EXTRA) b.ev[k] = load_stream_raw<T>(ok ? ds_extra + off : zero16<T>(3));
        }
        // The stats come as loaded, with no select after the load: a select on a loaded value
        // makes the compiler wait for every memory operation in flight at that point. mean is
        // NULL in RMSNorm mode and is never dereferenced there.
        if constexpr (kScalarStats) {
            // A wave holds part of one row: its stats are read through the constant address
            // space at a wave-uniform address, i.e. as scalar loads, which neither queue
            // behind the row's vector loads nor hold its vector-memory waits.
            using CF = const __attribute__((address_space(4))) float;
            const int64_t urow = (it * P + first_row) * NG + __builtin_amdgcn_readfirstlane(grp);
            const bool ulive = it < iters && urow < N;
            const float *prs = ulive ? rstd + urow : reinterpret_cast<const float *>(zero16<T>(3));
            b.rs = *reinterpret_cast<CF *>(reinterpret_cast<uintptr_t>(prs));
            if constexpr (!RMS) {
                const float *pmu = ulive ? mean + urow : reinterpret_cast<const float *>(zero16<T>(2));
                b.mu = *reinterpret_cast<CF *>(reinterpret_cast<uintptr_t>(pmu));
            } else {
                b.mu = 0.f;
            }
        } else {
            b.rs = *(live ? rstd + row : reinterpret_cast<const float *>(zero16<T>(3)));
            if constexpr (!RMS)
                b.mu = *(live ? mean + row : reinterpret_cast<const float *>(zero16<T>(2)));
            else
                b.mu = 0.f;
        }
    };
    // Every store is branch-free (store16_or_drop): offsets count from the row of the wave's
    // first row group, and a lane with nothing to store (a row past the end, or a vector slot
    // past the row) is dropped. With a branch around the stores, the deferred plans waited, for
    // each row's data, also for the first loads of the next row (seen in the gfx950 ISA).
    // A row's dx as stored, held until the next row's fetch has been issued (DEFER only).
    struct RowOut {
        RV dv[IT];
        uint32_t off[IT];  // byte offset from the wave's row base, or kDropOffset
        int64_t row0;      // row of the wave's first row group (wave-uniform)
    };
    const int grp0 = __builtin_amdgcn_readfirstlane(grp);
    auto store_row = [&](const RowOut &o) {
#pragma unroll
        for (int k = 0; k < IT; ++k) store16_or_drop(dx + o.row0 * static_cast<int64_t>(C), o.off[k], o.dv[k]);
    };
    auto process = [&](const RowBuf &b, int64_t it, RowOut &out) {
        const int64_t row = row_of(it);
        const bool live = it < iters && row < N;
        const float mu = b.mu, rs = b.rs;
        // First pass: xhat, g = gamma*dy, the fused pair of row sums, and the column
        // partials. g is rounded once and that same value enters both the row sum and dx,
        // so a row whose exact gradient is zero (C = 1, or g constant with xhat = 0) gives
        // exactly zero even when rstd is as large as 1/sqrt(eps).
        float xh[IT][V], gv[IT][V];
        float sg = 0.f, sgx = 0.f;
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            if constexpr (!BDR && V == 8) {
                // fp16 storage: every operation that takes a stored value is one mixed-precision
                // fma, with no separate widening (the kernel is VALU-bound at fp16). x - mu and
                // gamma * dy round exactly as the plain operations do (the product of two
                // halves is exact in fp32); the dgamma partial rounds once (an fma).
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float xs = static_cast<float>(b.xv[k][e]);
                    const float ds = static_cast<float>(b.dv[k][e]);
                    if constexpr (RMS)
                        xh[k][e] = __builtin_fmaf(xs, rs, nzero);
                    else
                        xh[k][e] = __builtin_fmaf(xs, one, -mu) * rs;
                    gv[k][e] = __builtin_fmaf(static_cast<float>(gmr[k][e]), ds, nzero);
                    if constexpr (!RMS) sg += gv[k][e];
                    sgx = __builtin_fmaf(gv[k][e], xh[k][e], sgx);
                    adg[k][e] = __builtin_fmaf(ds, xh[k][e], adg[k][e]);
                    if constexpr (!RMS) adb[k][e] = __builtin_fmaf(ds, one, adb[k][e]);
                }
                continue;
            }
            float xf[V], df[V], gmf[V];
            widen<T>(b.xv[k], xf);
            widen<T>(b.dv[k], df);
            widen<T>(gmr[k], gmf);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if constexpr (RMS)
                    xh[k][e] = xf[e] * rs;
                else
                    xh[k][e] = (xf[e] - mu) * rs;
                gv[k][e] = gmf[e] * df[e];
                if constexpr (!RMS) sg += gv[k][e];
                sgx = __builtin_fmaf(gv[k][e], xh[k][e], sgx);
                if constexpr (std::is_same_v<A, double>) {
                    // fp32 storage: the column term dy * xhat is formed in double from the
                    // stored values and the fp32 statistics (x - mean and the product with rstd
                    // are exact in double, the fma rounds once at 2^-53), so a column sum over
                    // tens of thousands of rows carries no fp32 rounding of its terms.
                    const double xhd = RMS ? static_cast<double>(xf[e]) * static_cast<double>(rs)
                                           : (static_cast<double>(xf[e]) - static_cast<double>(mu)) *
                                                 static_cast<double>(rs);
                    adg[k][e] = __builtin_fma(static_cast<double>(df[e]), xhd, adg[k][e]);
                } else {
                    adg[k][e] += static_cast<A>(df[e] * xh[k][e]);
                }
                if constexpr (!RMS) adb[k][e] += static_cast<A>(df[e]);
            }
        }
        if constexpr (RMS)
            sgx = row_allreduce<G>(sgx, OpSum(), red);
        else
            row_allreduce_sum2<G>(sg, sgx, red);
        const float a = sg * invC, bb = sgx * invC;  // a = 0 for RMSNorm
        // the rows of one wave's groups are consecutive
        const int64_t wrow_raw = (it * P + first_row) * NG + grp0;
        const int64_t wrow = wrow_raw < N ? wrow_raw : 0;
        auto off_of = [&](int k) -> uint32_t {
            const int c = k * G + lane;
            return (live && c < nvec) ? static_cast<uint32_t>(((row - wrow) * C + static_cast<int64_t>(c) * V) *
                                                              static_cast<int64_t>(sizeof(T)))
                                      : kDropOffset;
        };
        if constexpr (DEFER) {
            out.row0 = wrow;
#pragma unroll
            for (int k = 0; k < IT; ++k) out.off[k] = off_of(k);
        }
        // Rows past the end and idle lanes compute finite values from zeros (their stores are
        // dropped); for the bias-dropout-residual mode their dbias terms are zero (keep bit 0).
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    if constexpr (RMS)
                        o[e] = rs * __builtin_fmaf(-xh[k][e], bb, gv[k][e]);
                    else
                        o[e] = rs * __builtin_fmaf(-xh[k][e], bb, gv[k][e] - a);
                }
                if constexpr (BDR) {
                    if constexpr (EXTRA) {
                        float ef[V];
                        widen<T>(b.ev[k], ef);
#pragma unroll
                        for (int e = 0; e < V; ++e) o[e] += ef[e];
                    }
                    float o2[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        o2[e] = ((b.kb[k] >> e) & 1u) ? o[e] * keep_scale : 0.f;
                        adx[k][e] += static_cast<A>(o2[e]);
                    }
                    store16_or_drop(dx2 + wrow * static_cast<int64_t>(C), off_of(k), pack16<T>(o2));
                }
                if constexpr (DEFER)
                    out.dv[k] = pack16<T>(o);
                else
                    store16_or_drop(dx + wrow * static_cast<int64_t>(C), off_of(k), pack16<T>(o));
            }
        }
    };

    if constexpr (DEFER) {
        // Two buffers alternate through a loop unrolled by two (a copy of the fetched row into
        // the one being reduced would wait for every memory operation in flight).
        RowBuf b0, b1;
        RowOut o;
        o.row0 = 0;
#pragma unroll
        for (int k = 0; k < IT; ++k) o.off[k] = kDropOffset;
        fetch(b0, 0);
        // Dropped stores (every offset is kDropOffset): the loop is entered with stores behind the
        // first row's loads, as on every later iteration, so the compiler's wait counts at the
        // loop head need not assume that the loads are the newest operations in flight.
        store_row(o);
        // With two vectors per lane the waves of a workgroup meet at a bare barrier (no wait on
        // memory) before each row is reduced, so that their fetches of the following rows leave
        // together and the workgroup streams one contiguous run of rows at a time. Measured on
        // MI355X (three runs, bitwise-equal outputs): fp16 1024 columns -0.5 to -1.7% backward
        // time, RMSNorm -2 to -3%, fp32 512 columns -1 to -2%; with one vector per lane the
        // barrier costs more than it aligns (+2.5 to +5%).
        constexpr bool ALIGN = IT == 2;
        for (int64_t it = 0; it < iters; it += 2) {
            fetch(b1, it + 1);
            store_row(o);
            if constexpr (ALIGN) __builtin_amdgcn_s_barrier();
            process(b0, it, o);
            fetch(b0, it + 2);
            store_row(o);
            if constexpr (ALIGN) __builtin_amdgcn_s_barrier();
            process(b1, it + 1, o);
        }
        store_row(o);
    } else if constexpr (DEPTH == 1) {
        RowBuf nb, cb;
        RowOut o;
        fetch(nb, 0);
        for (int64_t it = 0; it < iters; ++it) {
            cb = nb;
            fetch(nb, it + 1);
            process(cb, it, o);
        }
    } else {
        RowBuf b0, b1, b2;
        RowOut o;
        fetch(b0, 0);
        fetch(b1, 1);
        for (int64_t it = 0; it < iters; it += 3) {
            fetch(b2, it + 2);
            process(b0, it, o);
            fetch(b0, it + 3);
            process(b1, it + 1, o);
            fetch(b1, it + 4);
            process(b2, it + 2, o);
        }
    }

    // Partial rows start 16-byte aligned (the workspace is, and a row holds a multiple of V
    // values), so a lane writes its V columns of a partial as whole 16-byte vectors.
    A *pg = part + static_cast<int64_t>(blockIdx.x) * SLOTS * C;
    A *pb = pg + C;
    A *px = pg + 2 * static_cast<int64_t>(C);  // kBdrLayerNorm only
    constexpr int NSL = RMS ? 1 : SLOTS;
    auto value = [&](int k, int which, int e) -> A {
        if constexpr (RMS) return adg[k][e];
        else if constexpr (BDR) return which == 0 ? adg[k][e] : (which == 1 ? adb[k][e] : adx[k][e]);
        else return which == 0 ? adg[k][e] : adb[k][e];
    };
    if constexpr (NG == 1) {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int c = k * G + lane;
            if (c < nvec) {
                store_partials16<A, V>(pg + c * V, adg[k]);
                if constexpr (!RMS) store_partials16<A, V>(pb + c * V, adb[k]);
                if constexpr (BDR) store_partials16<A, V>(px + c * V, adx[k]);
            }
        }
    } else if constexpr (NG == 2) {
        // The second group stages PER (vector slot k, partial) pairs of its G*V columns per
        // round in 16-byte chunks (consecutive lanes on consecutive chunks); the first adds them
        // to its own partials (group order, as below) and stores whole vectors from registers.
        // Measured on MI355X against the all-thread sum below: 0.2-1.5% less backward time at
        // 2048-4096 fp16 columns and fp32 1024 columns, with 8192 fp16 columns' direct vector
        // stores (NG = 1) 3.8% less than single-value stores.
        constexpr int CH = static_cast<int>(16 / sizeof(A));  // partials per 16-byte chunk
        constexpr int NCH = V / CH;                            // chunks per lane and pair
        auto at = [&](int q, int e) { return ((q * NCH + e / CH) * G + lane) * CH + e % CH; };
#pragma unroll
        for (int p0 = 0; p0 < PAIRS; p0 += PER) {
            if (p0 > 0) __syncthreads();  // the first group has read the previous round's tile
            if (grp == 1) {
#pragma unroll
                for (int q = 0; q < PER; ++q) {
                    const int pr = p0 + q;
                    if (pr < PAIRS) {
#pragma unroll
                        for (int e = 0; e < V; ++e) tile[0][at(q, e)] = value(pr / NSL, pr % NSL, e);
                    }
                }
            }
            __syncthreads();
            if (grp == 0) {
#pragma unroll
                for (int q = 0; q < PER; ++q) {
                    const int pr = p0 + q;
                    if (pr < PAIRS) {
                        const int k = pr / NSL, which = pr % NSL;
                        A sum[V];
#pragma unroll
                        for (int e = 0; e < V; ++e) sum[e] = value(k, which, e) + tile[0][at(q, e)];
                        const int c = k * G + lane;
                        if (c < nvec) store_partials16<A, V>((which == 0 ? pg : (which == 1 ? pb : px)) + c * V, sum);
                    }
                }
            }
        }
    } else {
        // LDS column tile: each round, every group stages PER (vector slot k, partial) pairs of
        // its G*V columns; then the workgroup sums the NG groups of each column in group order,
        // one column per thread at a time (with eight one-wave groups this spreads the sums
        // over the whole workgroup; the first group alone would sum seven staged groups).
#pragma unroll
        for (int p0 = 0; p0 < PAIRS; p0 += PER) {
            if (p0 > 0) __syncthreads();  // the previous round's sums have read the tile
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int pr = p0 + q;
                if (pr < PAIRS) {
#pragma unroll
                    for (int e = 0; e < V; ++e) tile[grp][q * G * V + lane * V + e] = value(pr / NSL, pr % NSL, e);
                }
            }
            __syncthreads();
            for (int idx = threadIdx.x; idx < PER * G * V; idx += WG) {
                const int pr = p0 + idx / (G * V);
                if (pr >= PAIRS) break;
                A sum = tile[0][idx];
#pragma unroll
                for (int g = 1; g < NG; ++g) sum += tile[g][idx];
                const int which = pr % NSL;
                const int col = (pr / NSL) * G * V + idx % (G * V);
                if (col < C) (which == 0 ? pg : (which == 1 ? pb : px))[col] = sum;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Column finalize: dgamma/dbeta (and dbias) = fixed-order sums of the P partial rows; slot
// `which` = blockIdx.y of partial row p is at part[(p * stride + which) * C].
// Block = TILE columns x SLICES slices; slice s sums partials p = s, s+SLICES, s+2*SLICES, ...
// in that order (with BATCH > 1, BATCH loads in flight at a time, added in order), then slice 0 adds the
// slice sums in slice order. Two shapes, measured on MI355X: 16 x 16 up to 1024 columns
// (the kernel sits at its launch floor there), 32 x 32 with 8 loads in flight above (C=4096:
// 4.1 -> 3.3 us).
// ------------------------------------------------------------------------------------------
template <typename T, int TILE, int SLICES, int BATCH>
__global__ __launch_bounds__(TILE *SLICES) void layernorm_bw_colsum(
    T *__restrict__ dgamma, T *__restrict__ dbeta, T *__restrict__ dbias,
    const typename Accum<T>::type *__restrict__ part, int32_t P, int32_t C, int32_t stride) {
    using A = typename Accum<T>::type;
    __shared__ A slab[SLICES][TILE];
    const int cl = threadIdx.x % TILE;
    const int sl = threadIdx.x / TILE;
    const int which = blockIdx.y;
    const int col = blockIdx.x * TILE + cl;
    A s = A(0);
    if (col < C) {
        if constexpr (BATCH == 1) {
#pragma unroll 8
            for (int p = sl; p < P; p += SLICES)
                s += part[(static_cast<int64_t>(p) * stride + which) * C + col];
        } else {
            for (int p0 = sl; p0 < P; p0 += SLICES * BATCH) {
                A v[BATCH];
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    const int p = p0 + u * SLICES;
                    v[u] = p < P ? part[(static_cast<int64_t>(p) * stride + which) * C + col] : A(0);
                }
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    if (p0 + u * SLICES < P) s += v[u];
            }
        }
    }
    slab[sl][cl] = s;
    __syncthreads();
    if (sl == 0 && col < C) {
        A t = slab[0][cl];
#pragma unroll
        for (int k = 1; k < SLICES; ++k) t += slab[k][cl];
        (which == 0 ? dgamma : (which == 1 ? dbeta : dbias))[col] = from_f32<T>(static_cast<float>(t));
    }
}

// ------------------------------------------------------------------------------------------
// Element-wise fallback kernels (any C, any element alignment): one workgroup per row.
// ------------------------------------------------------------------------------------------
constexpr int kLnGenericWG = 256;

template <typename T, bool RMS>
__global__ __launch_bounds__(kLnGenericWG) void layernorm_fw_generic(
    T *y, float *__restrict__ mean, float *__restrict__ rstd, const T *x,
    const T *__restrict__ gamma, const T *__restrict__ beta, int64_t N, int32_t C, float eps) {
    __shared__ float red[2 * (kLnGenericWG / 64)];
    const int64_t row = blockIdx.x;
    const T *xr = x + row * static_cast<int64_t>(C);
    const float K = RMS ? 0.f : to_f32(xr[0]);
    float s1 = 0.f, s2 = 0.f;
    for (int j = threadIdx.x; j < C; j += kLnGenericWG) {
        const float d = to_f32(xr[j]) - K;
        s1 += d;
        s2 = __builtin_fmaf(d, d, s2);
    }
    float m1 = 0.f, rs;
    const float invC = 1.0f / static_cast<float>(C);
    if constexpr (RMS) {
        s2 = row_allreduce<kLnGenericWG>(s2, OpSum(), red);
        rs = rms_stats(s2, invC, eps);
    } else {
        row_allreduce_sum2<kLnGenericWG>(s1, s2, red);
        rs = ln_stats(s1, s2, invC, eps, m1);
    }
    T *yr = y + row * static_cast<int64_t>(C);
    for (int j = threadIdx.x; j < C; j += kLnGenericWG) {
        if constexpr (RMS)
            yr[j] = from_f32<T>(to_f32(xr[j]) * rs * to_f32(gamma[j]));
        else
            yr[j] = from_f32<T>(((to_f32(xr[j]) - K) - m1) * rs * to_f32(gamma[j]) + to_f32(beta[j]));
    }
    if (threadIdx.x == 0 && rstd != nullptr) {
        if constexpr (!RMS) mean[row] = K + m1;
        rstd[row] = rs;
    }
}

template <typename T, bool RMS>
__global__ __launch_bounds__(kLnGenericWG) void layernorm_bw_dx_generic(
    T *dx, const T *dy, const T *x, const T *__restrict__ gamma, const float *__restrict__ mean,
    const float *__restrict__ rstd, int64_t N, int32_t C) {
#pragma clang fp contract(off)
    __shared__ float red[2 * (kLnGenericWG / 64)];
    const int64_t row = blockIdx.x;
    const int64_t base = row * static_cast<int64_t>(C);
    const float mu = RMS ? 0.f : mean[row], rs = rstd[row];
    auto xhat = [&](int j) {
        const float xv = to_f32(x[base + j]);
        return RMS ? xv * rs : (xv - mu) * rs;
    };
    float sg = 0.f, sgx = 0.f;
    for (int j = threadIdx.x; j < C; j += kLnGenericWG) {
        const float g = to_f32(gamma[j]) * to_f32(dy[base + j]);
        sg += g;
        sgx = __builtin_fmaf(g, xhat(j), sgx);
    }
    if constexpr (RMS)
        sgx = row_allreduce<kLnGenericWG>(sgx, OpSum(), red);
    else
        row_allreduce_sum2<kLnGenericWG>(sg, sgx, red);
    const float invC = 1.0f / static_cast<float>(C);
    const float a = RMS ? 0.f : sg * invC, b = sgx * invC;
    for (int j = threadIdx.x; j < C; j += kLnGenericWG) {
        const float g = to_f32(gamma[j]) * to_f32(dy[base + j]);
        dx[base + j] = from_f32<T>(rs * __builtin_fmaf(-xhat(j), b, RMS ? g : g - a));
    }
}

template <typename T, bool RMS>
__global__ __launch_bounds__(kLnGenericWG) void layernorm_bw_colpart_generic(
    typename Accum<T>::type *part, const T *dy, const T *x, const float *__restrict__ mean,
    const float *__restrict__ rstd, int64_t N, int32_t C, int64_t rows_per_block) {
    using A = typename Accum<T>::type;
    const int col = blockIdx.x * kLnGenericWG + threadIdx.x;
    if (col >= C) return;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rows_per_block;
    const int64_t r1 = (r0 + rows_per_block < N) ? r0 + rows_per_block : N;
    A sg = A(0), sb = A(0);
    for (int64_t r = r0; r < r1; ++r) {
        const float d = to_f32(dy[r * C + col]);
        const float xv = to_f32(x[r * C + col]);
        if constexpr (std::is_same_v<A, double>) {
            // fp32 storage: the term formed in double, as in the vector kernel.
            const double rs = static_cast<double>(rstd[r]);
            const double xh = RMS ? static_cast<double>(xv) * rs
                                  : (static_cast<double>(xv) - static_cast<double>(mean[r])) * rs;
            sg = __builtin_fma(static_cast<double>(d), xh, sg);
        } else {
            const float xh = RMS ? xv * rstd[r] : (xv - mean[r]) * rstd[r];
            sg += static_cast<A>(d * xh);
        }
        sb += static_cast<A>(d);
    }
    part[(static_cast<int64_t>(blockIdx.y) * 2 + 0) * C + col] = sg;
    if constexpr (!RMS) part[(static_cast<int64_t>(blockIdx.y) * 2 + 1) * C + col] = sb;
}

// ------------------------------------------------------------------------------------------
// Bias + dropout + residual feeding LayerNorm, element-wise fallback (any C, any element
// alignment). Forward: one workgroup per row, s formed in fp32 as the vector kernel forms it,
// stored, and normalised in fp32 (s is formed again in the second pass from the same inputs,
// so the value normalised is the fp32 one, not the stored rounding). Backward: one workgroup
// per chunk of rows; every thread owns columns j = tid, tid + WG, ... in every row, so it
// accumulates its columns' dgamma, dbeta and dbias terms in the workgroup's own partial row
// of the workspace, in row order (no atomics), for layernorm_bw_colsum to sum.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ bool keep_bit_of(const uint8_t *mrow, int j) {
    return (mrow[j >> 3] >> (j & 7)) & 1u;
}

constexpr int kBdrGenericPer = LNR_LAYERNORM_MAX_C / kLnGenericWG;  // row elements per thread

template <typename T>
__global__ __launch_bounds__(kLnGenericWG) void bdr_layernorm_fw_generic(
    T *s_out, T *y, float *__restrict__ mean, float *__restrict__ rstd, const T *x,
    const T *residual, const T *__restrict__ bias, const uint8_t *__restrict__ mask,
    float keep_scale, const T *__restrict__ gamma, const T *__restrict__ beta, int64_t N,
    int32_t C, float eps) {
    __shared__ float red[2 * (kLnGenericWG / 64)];
    const int64_t row = blockIdx.x;
    const int64_t base = row * static_cast<int64_t>(C);
    const uint8_t *mrow = mask + row * static_cast<int64_t>((C + 7) / 8);
    auto s_of = [&](int j) {
        const float r = to_f32(residual[base + j]);
        return keep_bit_of(mrow, j) ? __builtin_fmaf(to_f32(x[base + j]) + to_f32(bias[j]), keep_scale, r) : r;
    };
    // The shift K is the row's first s element. s may replace residual in place, so every
    // thread reads element 0 before any thread stores, and the row's fp32 s stays in
    // registers (element j = tid + k * WG) for the second pass.
    const float K = s_of(0);
    __syncthreads();
    float sv[kBdrGenericPer];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int k = 0; k < kBdrGenericPer; ++k) {
        const int j = threadIdx.x + k * kLnGenericWG;
        if (j < C) {
            sv[k] = s_of(j);
            const float d = sv[k] - K;
            s1 += d;
            s2 = __builtin_fmaf(d, d, s2);
            s_out[base + j] = from_f32<T>(sv[k]);
        }
    }
    float m1;
    row_allreduce_sum2<kLnGenericWG>(s1, s2, red);
    const float rs = ln_stats(s1, s2, 1.0f / static_cast<float>(C), eps, m1);
#pragma unroll
    for (int k = 0; k < kBdrGenericPer; ++k) {
        const int j = threadIdx.x + k * kLnGenericWG;
        if (j < C) y[base + j] = from_f32<T>(((sv[k] - K) - m1) * rs * to_f32(gamma[j]) + to_f32(beta[j]));
    }
    if (threadIdx.x == 0 && rstd != nullptr) {
        mean[row] = K + m1;
        rstd[row] = rs;
    }
}

template <typename T>
__global__ __launch_bounds__(kLnGenericWG) void bdr_layernorm_bw_generic(
    T *dres, T *dx, typename Accum<T>::type *part, const T *dy, const T *ds_extra, const T *s,
    const uint8_t *__restrict__ mask, float keep_scale, const T *__restrict__ gamma,
    const float *__restrict__ mean, const float *__restrict__ rstd, int64_t N, int32_t C,
    int64_t rows_per_block) {
#pragma clang fp contract(off)
    using A = typename Accum<T>::type;
    __shared__ float red[2 * (kLnGenericWG / 64)];
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_block;
    const int64_t r1 = (r0 + rows_per_block < N) ? r0 + rows_per_block : N;
    A *pg = part + static_cast<int64_t>(blockIdx.x) * 3 * C;
    A *pb = pg + C;
    A *px = pg + 2 * static_cast<int64_t>(C);
    for (int j = threadIdx.x; j < C; j += kLnGenericWG) pg[j] = pb[j] = px[j] = A(0);
    const float invC = 1.0f / static_cast<float>(C);
    const int64_t mb = (C + 7) / 8;
    for (int64_t row = r0; row < r1; ++row) {
        const int64_t base = row * static_cast<int64_t>(C);
        const float mu = mean[row], rs = rstd[row];
        float sg = 0.f, sgx = 0.f;
        for (int j = threadIdx.x; j < C; j += kLnGenericWG) {
            const float g = to_f32(gamma[j]) * to_f32(dy[base + j]);
            sg += g;
            sgx = __builtin_fmaf(g, (to_f32(s[base + j]) - mu) * rs, sgx);
        }
        row_allreduce_sum2<kLnGenericWG>(sg, sgx, red);
        const float a = sg * invC, b = sgx * invC;
        const uint8_t *mrow = mask + row * mb;
        for (int j = threadIdx.x; j < C; j += kLnGenericWG) {
            const float d = to_f32(dy[base + j]);
            const float sv = to_f32(s[base + j]);
            const float sh = (sv - mu) * rs;
            const float g = to_f32(gamma[j]) * d;
            float ds = rs * __builtin_fmaf(-sh, b, g - a);
            if (ds_extra != nullptr) ds += to_f32(ds_extra[base + j]);
            const float o2 = keep_bit_of(mrow, j) ? ds * keep_scale : 0.f;
            // written after every read of this element: dres may replace dy or ds_extra
            dres[base + j] = from_f32<T>(ds);
            dx[base + j] = from_f32<T>(o2);
            if constexpr (std::is_same_v<A, double>) {
                const double shd = (static_cast<double>(sv) - static_cast<double>(mu)) * static_cast<double>(rs);
                pg[j] = __builtin_fma(static_cast<double>(d), shd, pg[j]);
            } else {
                pg[j] += static_cast<A>(d * sh);
            }
            pb[j] += static_cast<A>(d);
            px[j] += static_cast<A>(o2);
        }
    }
}

// ------------------------------------------------------------------------------------------
// Hidden-size buckets.
// ------------------------------------------------------------------------------------------
struct LnPlan {
    int bucket;  // widest row this instantiation takes
    int G;       // lanes per row (multiples of 64 above one wave)
    int IT;      // 16-byte vectors per lane
    int WG;      // workgroup size
    int R;       // forward: rows per row group per workgroup (1 = one row each);
                 // backward: rows fetched ahead of the row being reduced (1 or 2)
    int64_t min_rows = 0;  // taken only by launches of at least this many rows (a bucket's
                           // plans are listed longest-launch first)
};

// Measured on MI355X (fp16, N = 8192..32768): both LayerNorm kernels run best with one or
// two 16-byte vectors per lane and as many lanes per row as that gives (several waves per row
// from 2048 columns up). The forward takes one row per group (R = 1) up to 2048 columns and
// two rows per group above, where the prefetch of the second row pays (at 4096-8192 columns
// 6-12% faster than one row; at 1024 fp16 columns one row is 3-8% faster than two). fp32 at
// 1024 columns is a tie and keeps two. At 8192 fp16 columns the forward takes four vectors
// per lane over four waves. At 1024 fp16 columns four rows per 256-thread workgroup beat two
// per 128 threads by 1-2% (64, 512 and 1024 threads: tie, tie, 8% slower). At 4096 fp16
// columns, launches of 24576 rows and more take two rows side by side in 512-thread
// workgroups: same arithmetic per row (bitwise-equal outputs), LayerNorm 0.3-4.9% faster at
// 24576-65536 rows and RMSNorm up to 10% at 65536, the bias-dropout-residual forward unchanged;
// below 24576 rows it is 0.4-1.5% slower. The same doubling loses at 1024 and 8192 fp16
// columns (+1-18%) and in every fp32 bucket; two waves per row with four vectors per lane
// gains more for LayerNorm at 4096 but costs RMSNorm and the bias-dropout-residual forward
// 6-7%. The same plans serve RMSNorm and the bias-dropout-residual LayerNorm.
template <typename T> struct LnFwTable;
template <> struct LnFwTable<f16> {  // V = 8
    static constexpr LnPlan plans[] = {
        {64, 8, 1, 256, 1},     {128, 16, 1, 256, 1},   {256, 16, 2, 256, 1},
        {512, 32, 2, 256, 1},   {768, 32, 3, 64, 1},    {1024, 64, 2, 256, 1},
        {2048, 128, 2, 128, 1}, {4096, 256, 2, 512, 2, 24576}, {4096, 256, 2, 256, 2},
        {8192, 256, 4, 256, 2}};
};
template <> struct LnFwTable<float> {  // V = 4
    static constexpr LnPlan plans[] = {
        {64, 16, 1, 256, 1},    {128, 16, 2, 256, 1},   {256, 32, 2, 128, 1},
        {512, 64, 2, 256, 2},   {768, 64, 3, 256, 2},   {1024, 128, 2, 256, 2},
        {2048, 256, 2, 256, 2}, {4096, 512, 2, 512, 2}, {8192, 1024, 2, 1024, 2}};
};
// The backward row kernel runs within 2-11% of a read-two-write-one stream of the same size
// (N = 16384..32768). Up to 1024 columns (fp16) and 512 (fp32) a row sits inside one wave and
// its dx stores are deferred (DEFER in the kernel): with that, two vectors per lane over 512
// threads beat a row over two waves at fp16 1024 columns (-0.5 to -2.4% up to 16384 rows) and
// at fp32 512 columns (-9%). Four fp32 vectors per lane at 1024 columns spill and lose (+3%).
// A row over two waves with two rows ahead once won at 1024 fp16 columns from 24576 rows
// (-3.6 to -7.2%); since the one-wave rows fetch aligned (a bare barrier per row) and read
// their statistics as scalar loads, the one-wave plan is 1.1-1.4% faster at 24576-65536 rows
// too, and no backward plan depends on the row count. Rows of 4-8 KB
// over four or eight waves likewise take two rows ahead in 512-thread workgroups instead of
// one row ahead in 1024-thread ones: fp16 2048 columns -7 to -8%, fp32 1024 columns -4%,
// fp32 2048 columns -5 to -6% (16384 and 32768 rows); at fp32 512 columns two waves with two
// rows ahead lose (+4%) to the one-wave plan. fp32 4096 columns take two vectors per lane over
// eight waves with one row ahead (-4 to -6% against one vector over sixteen waves in 1024
// threads, -2 to -3% against two rows ahead); at 8192 two rows ahead spill (2.3x slower).
template <typename T> struct LnBwTable;
template <> struct LnBwTable<f16> {
    static constexpr LnPlan plans[] = {
        {64, 8, 1, 512, 1},      {128, 16, 1, 512, 1},    {256, 32, 1, 512, 1},
        {512, 64, 1, 512, 1},    {768, 32, 3, 512, 1},    {1024, 64, 2, 512, 1},
        {2048, 256, 1, 512, 2},  {4096, 256, 2, 512, 2},
        {8192, 512, 2, 512, 2}};
};
template <> struct LnBwTable<float> {
    static constexpr LnPlan plans[] = {
        {64, 16, 1, 512, 1},     {128, 32, 1, 512, 1},    {256, 64, 1, 512, 1},
        {512, 64, 2, 512, 1},    {768, 64, 3, 512, 1},    {1024, 256, 1, 512, 2},
        {2048, 512, 1, 512, 2},  {4096, 512, 2, 512, 1}, {8192, 1024, 2, 1024, 1}};
};

// Backward plans of the fused bias-dropout-residual LayerNorm. Its third column partial
// (dbias) and second output cost registers, and two rows fetched ahead no longer fit: with
// 1024 threads they spill. Measured on MI355X (fp16, N = 16384): from 512 columns up the
// best plan is two vectors per lane, 512 threads and one row ahead (about 180 VGPRs, two
// waves per SIMD); at C = 4096 it takes 98 us against 128 us for one vector per lane, at
// 1024-8192 columns 9-14% less. fp32 at 8192 columns keeps two vectors per lane at 1024
// threads and spills part of its fp64 partials to scratch.
template <typename T> struct BdrBwTable;
template <> struct BdrBwTable<f16> {
    static constexpr LnPlan plans[] = {
        {64, 8, 1, 512, 1},      {128, 16, 1, 512, 1},    {256, 32, 1, 512, 1},
        {512, 32, 2, 512, 1},    {768, 64, 2, 512, 1},    {1024, 64, 2, 512, 1},
        {2048, 128, 2, 512, 1},  {4096, 256, 2, 512, 1},  {8192, 512, 2, 512, 1}};
};
template <> struct BdrBwTable<float> {
    static constexpr LnPlan plans[] = {
        {64, 16, 1, 512, 1},     {128, 32, 1, 512, 1},    {256, 64, 1, 512, 1},
        {512, 128, 1, 512, 1},   {768, 64, 3, 512, 1},    {1024, 256, 1, 1024, 1},
        {2048, 512, 1, 1024, 1}, {4096, 1024, 1, 1024, 1}, {8192, 1024, 2, 1024, 1}};
};

constexpr int64_t kLnBwTargetBlocks = 256;  // one partial row per CU

template <typename Table>
static bool find_plan(int64_t C, int64_t N, LnPlan &out) {
    for (const LnPlan &p : Table::plans)
        if (C <= p.bucket && N >= p.min_rows) {
            out = p;
            return true;
        }
    return false;
}

// Rows per backward workgroup: about N / kLnBwTargetBlocks, rounded up to whole row groups.
static int64_t bw_rows_per_block(int64_t N, int64_t groups) {
    int64_t r = (N + kLnBwTargetBlocks - 1) / kLnBwTargetBlocks;
    if (r < 1) r = 1;
    return ((r + groups - 1) / groups) * groups;
}

static int64_t bw_blocks(int64_t N, int64_t rpb) { return N == 0 ? 0 : (N + rpb - 1) / rpb; }

// Workgroups (= partial rows) of each backward path for this shape (bdr: the fused
// bias-dropout-residual LayerNorm's plan table).
static void bw_partials(int64_t N, int64_t C, lnr_dtype dtype, int64_t &p_vec, int64_t &p_gen,
                        int64_t &rpb_vec, int64_t &rpb_gen, bool bdr = false) {
    LnPlan p{};
    bool ok;
    if (bdr)
        ok = dtype == LNR_F16 ? find_plan<BdrBwTable<f16>>(C, N, p) : find_plan<BdrBwTable<float>>(C, N, p);
    else
        ok = dtype == LNR_F16 ? find_plan<LnBwTable<f16>>(C, N, p) : find_plan<LnBwTable<float>>(C, N, p);
    const int64_t groups = ok ? p.WG / p.G : 1;
    rpb_vec = bw_rows_per_block(N, groups);
    p_vec = bw_blocks(N, rpb_vec);
    rpb_gen = bw_rows_per_block(N, 1);
    p_gen = bw_blocks(N, rpb_gen);
}

struct LnFwArgs {
    void *y;
    float *mean;  // NULL for RMSNorm
    float *rstd;
    const void *x, *gamma, *beta;  // beta NULL for RMSNorm
    int64_t N;
    int32_t C;
    float eps;
    // kBdrLayerNorm only
    void *s_out = nullptr;
    const void *residual = nullptr, *bias = nullptr;
    const uint8_t *mask = nullptr;
    float keep_scale = 1.f;
};
struct LnBwArgs {
    void *dx;
    void *dgamma, *dbeta;  // dbeta NULL for RMSNorm
    void *part;
    const void *dy, *x, *gamma;
    const float *mean, *rstd;  // mean NULL for RMSNorm
    int64_t N;
    int32_t C;
    int64_t rows_per_block;
    int64_t blocks;
    // kBdrLayerNorm only
    void *dx2 = nullptr, *dbias = nullptr;
    const void *ds_extra = nullptr;
    const uint8_t *mask = nullptr;
    float keep_scale = 1.f;
};

template <typename T, int MODE, int I>
static hipError_t dispatch_ln_fw(const LnFwArgs &a, hipStream_t st) {
    constexpr LnPlan p = LnFwTable<T>::plans[I];
    if (a.C <= p.bucket && a.N >= p.min_rows) {
        static_assert(p.WG % p.G == 0 && p.WG % 64 == 0 && p.R >= 1, "bad forward plan");
        constexpr int64_t RPB = static_cast<int64_t>(p.WG / p.G) * p.R;
        const int64_t blocks = (a.N + RPB - 1) / RPB;
        return launch(layernorm_fw_vec<T, p.G, p.IT, p.WG, MODE, p.R>, dim3(static_cast<uint32_t>(blocks)),
                      dim3(p.WG), st, static_cast<T *>(a.y), a.mean, a.rstd,
                      static_cast<const T *>(a.x), static_cast<const T *>(a.gamma),
                      static_cast<const T *>(a.beta), a.N, a.C, a.eps, RPB,
                      static_cast<T *>(a.s_out), static_cast<const T *>(a.residual),
                      static_cast<const T *>(a.bias), a.mask, a.keep_scale);
    }
    if constexpr (I + 1 < static_cast<int>(sizeof(LnFwTable<T>::plans) / sizeof(LnPlan)))
        return dispatch_ln_fw<T, MODE, I + 1>(a, st);
    return hipErrorInvalidValue;
}

// Column sums of the P partial rows into dgamma, dbeta, dbias: `slots` outputs (1 RMSNorm,
// 2 LayerNorm, 3 bias-dropout-residual LayerNorm), `stride` slots per partial row.
template <typename T>
static hipError_t launch_colsum(void *dgamma, void *dbeta, void *dbias, const void *part, int64_t P,
                                int32_t C, int slots, int stride, hipStream_t st) {
    using A = typename Accum<T>::type;
    if (C <= 1024) {
        const dim3 grid(static_cast<uint32_t>((C + 15) / 16), static_cast<uint32_t>(slots));
        return launch(layernorm_bw_colsum<T, 16, 16, 1>, grid, dim3(16 * 16), st,
                      static_cast<T *>(dgamma), static_cast<T *>(dbeta), static_cast<T *>(dbias),
                      static_cast<const A *>(part), static_cast<int32_t>(P), C, stride);
    }
    const dim3 grid(static_cast<uint32_t>((C + 31) / 32), static_cast<uint32_t>(slots));
    return launch(layernorm_bw_colsum<T, 32, 32, 8>, grid, dim3(32 * 32), st,
                  static_cast<T *>(dgamma), static_cast<T *>(dbeta), static_cast<T *>(dbias),
                  static_cast<const A *>(part), static_cast<int32_t>(P), C, stride);
}

constexpr int slots_of(int mode) { return mode == kRmsNorm ? 1 : (mode == kBdrLayerNorm ? 3 : 2); }
constexpr int stride_of(int mode) { return mode == kBdrLayerNorm ? 3 : 2; }

template <typename T, int G, int IT, int WG, int R, int MODE, bool EXTRA>
static hipError_t launch_bw_vec(const LnBwArgs &a, hipStream_t st) {
    return launch(layernorm_bw_vec<T, G, IT, WG, R, MODE, EXTRA>, dim3(static_cast<uint32_t>(a.blocks)),
                  dim3(WG), st, static_cast<T *>(a.dx), static_cast<typename Accum<T>::type *>(a.part),
                  static_cast<const T *>(a.dy), static_cast<const T *>(a.x),
                  static_cast<const T *>(a.gamma), a.mean, a.rstd, a.N, a.C, a.rows_per_block,
                  static_cast<T *>(a.dx2), static_cast<const T *>(a.ds_extra), a.mask, a.keep_scale);
}

template <typename T, int MODE, int I>
static hipError_t dispatch_ln_bw(const LnBwArgs &a, hipStream_t st) {
    using Table = std::conditional_t<MODE == kBdrLayerNorm, BdrBwTable<T>, LnBwTable<T>>;
    constexpr LnPlan p = Table::plans[I];
    if (a.C <= p.bucket && a.N >= p.min_rows) {
        static_assert(p.WG % p.G == 0 && p.WG % 64 == 0 && (p.R == 1 || p.R == 2), "bad backward plan");
        static_assert(2 * (p.WG / 64) >= 2, "reduction slots");
        hipError_t e;
        if constexpr (MODE == kBdrLayerNorm)
            e = a.ds_extra != nullptr ? launch_bw_vec<T, p.G, p.IT, p.WG, p.R, MODE, true>(a, st)
                                      : launch_bw_vec<T, p.G, p.IT, p.WG, p.R, MODE, false>(a, st);
        else
            e = launch_bw_vec<T, p.G, p.IT, p.WG, p.R, MODE, false>(a, st);
        if (e != hipSuccess) return e;
        return launch_colsum<T>(a.dgamma, a.dbeta, a.dbias, a.part, a.blocks, a.C, slots_of(MODE),
                                stride_of(MODE), st);
    }
    if constexpr (I + 1 < static_cast<int>(sizeof(Table::plans) / sizeof(LnPlan)))
        return dispatch_ln_bw<T, MODE, I + 1>(a, st);
    return hipErrorInvalidValue;
}

static size_t accum_size(lnr_dtype d) { return d == LNR_F16 ? sizeof(float) : sizeof(double); }

static size_t bw_workspace_bytes(int64_t N, int64_t C, lnr_dtype dtype) {
    if (!valid_dtype(dtype) || N < 0 || C < 1 || C > LNR_LAYERNORM_MAX_C) return 0;
    int64_t pv, pg, rv, rg;
    bw_partials(N, C, dtype, pv, pg, rv, rg);
    const int64_t P = pv > pg ? pv : pg;
    return static_cast<size_t>(P) * 2 * static_cast<size_t>(C) * accum_size(dtype);
}

// Forward of either norm. LayerNorm: beta required; mean and rstd both given or both NULL.
// RMSNorm (rms): beta and mean are NULL; rstd optional.
template <bool RMS>
static int norm_fw(void *y, float *mean, float *rstd, const void *x, const void *gamma,
                   const void *beta, int64_t N, int64_t C, float eps, lnr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (N < 0 || C < 1) return LNR_ERR_SHAPE;
    if (C > LNR_LAYERNORM_MAX_C) return LNR_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || !isfinite(eps)) return LNR_ERR_SHAPE;
    if (!RMS && (mean == nullptr) != (rstd == nullptr)) return LNR_ERR_NULL;
    if (N == 0) return LNR_OK;
    if (N > INT32_MAX) return LNR_ERR_UNSUPPORTED;
    if (y == nullptr || x == nullptr || gamma == nullptr || (!RMS && beta == nullptr)) return LNR_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned_to(y, es) || !aligned_to(x, es) || !aligned_to(gamma, es) ||
        (!RMS && !aligned_to(beta, es)) || !aligned_to(mean, 4) || !aligned_to(rstd, 4))
        return LNR_ERR_ALIGN;
    const size_t nbytes = static_cast<size_t>(N) * static_cast<size_t>(C) * es;
    const size_t cbytes = static_cast<size_t>(C) * es;
    if (bad_alias(y, x, nbytes) || overlap(y, nbytes, gamma, cbytes) ||
        overlap(y, nbytes, beta, cbytes) || overlap(y, nbytes, mean, N * 4) ||
        overlap(y, nbytes, rstd, N * 4) || overlap(mean, N * 4, rstd, N * 4))
        return LNR_ERR_ALIAS;

    LnFwArgs a{y, mean, rstd, x, gamma, beta, N, static_cast<int32_t>(C), eps};
    const bool vec = (static_cast<size_t>(C) * es) % 16 == 0 && aligned_to(y, 16) &&
                     aligned_to(x, 16) && aligned_to(gamma, 16) && (RMS || aligned_to(beta, 16));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (vec) {
        constexpr int MODE = RMS ? kRmsNorm : kLayerNorm;
        e = dtype == LNR_F16 ? dispatch_ln_fw<f16, MODE, 0>(a, s) : dispatch_ln_fw<float, MODE, 0>(a, s);
    } else if (dtype == LNR_F16) {
        e = launch(layernorm_fw_generic<f16, RMS>, dim3(static_cast<uint32_t>(N)), dim3(kLnGenericWG), s,
                   static_cast<f16 *>(y), mean, rstd, static_cast<const f16 *>(x),
                   static_cast<const f16 *>(gamma), static_cast<const f16 *>(beta), N, a.C, eps);
    } else {
        e = launch(layernorm_fw_generic<float, RMS>, dim3(static_cast<uint32_t>(N)), dim3(kLnGenericWG), s,
                   static_cast<float *>(y), mean, rstd, static_cast<const float *>(x),
                   static_cast<const float *>(gamma), static_cast<const float *>(beta), N, a.C, eps);
    }
    return status_of(e);
}

// Backward of either norm. RMSNorm (rms): dbeta and mean are NULL. With check_only, every
// check that does not involve the workspace runs and nothing is launched (the no-allocation
// entry point validates its arguments this way before it touches a device).
template <bool RMS>
static int norm_bw(void *dx, void *dgamma, void *dbeta, const void *dy, const void *x,
                   const void *gamma, const float *mean, const float *rstd, int64_t N, int64_t C,
                   lnr_dtype dtype, void *workspace, size_t workspace_bytes, void *stream,
                   bool check_only = false) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (N < 0 || C < 1) return LNR_ERR_SHAPE;
    if (C > LNR_LAYERNORM_MAX_C) return LNR_ERR_UNSUPPORTED;
    if (N > INT32_MAX) return LNR_ERR_UNSUPPORTED;
    if (dgamma == nullptr || (!RMS && dbeta == nullptr)) return LNR_ERR_NULL;
    if (N > 0 && (dx == nullptr || dy == nullptr || x == nullptr || gamma == nullptr ||
                  (!RMS && mean == nullptr) || rstd == nullptr))
        return LNR_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned_to(dx, es) || !aligned_to(dgamma, es) || !aligned_to(dbeta, es) ||
        !aligned_to(dy, es) || !aligned_to(x, es) || !aligned_to(gamma, es) ||
        !aligned_to(mean, 4) || !aligned_to(rstd, 4))
        return LNR_ERR_ALIGN;
    const size_t need = check_only ? 0 : bw_workspace_bytes(N, C, dtype);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LNR_ERR_WORKSPACE;
    if (need > 0 && !aligned_to(workspace, 16)) return LNR_ERR_ALIGN;
    const size_t nbytes = static_cast<size_t>(N) * static_cast<size_t>(C) * es;
    const size_t cbytes = static_cast<size_t>(C) * es;
    if (overlap(dx, nbytes, x, nbytes) || overlap(dx, nbytes, dy, nbytes) ||
        overlap(dx, nbytes, gamma, cbytes) || overlap(dx, nbytes, mean, N * 4) ||
        overlap(dx, nbytes, rstd, N * 4) || overlap(dgamma, cbytes, dbeta, cbytes) ||
        overlap(workspace, need, dx, nbytes) || overlap(workspace, need, x, nbytes) ||
        overlap(workspace, need, dy, nbytes) || overlap(workspace, need, dgamma, cbytes) ||
        overlap(workspace, need, dbeta, cbytes) || overlap(workspace, need, gamma, cbytes) ||
        overlap(workspace, need, mean, N * 4) || overlap(workspace, need, rstd, N * 4))
        return LNR_ERR_ALIAS;
    for (const void *out : {dgamma, dbeta})
        if (overlap(out, cbytes, x, nbytes) || overlap(out, cbytes, dy, nbytes) ||
            overlap(out, cbytes, dx, nbytes) || overlap(out, cbytes, gamma, cbytes))
            return LNR_ERR_ALIAS;
    if (check_only) return LNR_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int slots = RMS ? 1 : 2;
    int64_t pv, pg, rv, rg;
    bw_partials(N, C, dtype, pv, pg, rv, rg);
    const int32_t C32 = static_cast<int32_t>(C);
    hipError_t e = hipSuccess;
    if (N == 0) {
        // No rows: the column sums are empty, and the column-sum kernel writes zeros.
        e = dtype == LNR_F16 ? launch_colsum<f16>(dgamma, dbeta, nullptr, workspace, 0, C32, slots, 2, s)
                             : launch_colsum<float>(dgamma, dbeta, nullptr, workspace, 0, C32, slots, 2, s);
        return status_of(e);
    }
    const bool vec = (static_cast<size_t>(C) * es) % 16 == 0 && aligned_to(dx, 16) &&
                     aligned_to(dy, 16) && aligned_to(x, 16) && aligned_to(gamma, 16);
    if (vec) {
        LnBwArgs a{dx, dgamma, dbeta, workspace, dy, x, gamma, mean, rstd, N, C32, rv, pv};
        constexpr int MODE = RMS ? kRmsNorm : kLayerNorm;
        e = dtype == LNR_F16 ? dispatch_ln_bw<f16, MODE, 0>(a, s) : dispatch_ln_bw<float, MODE, 0>(a, s);
    } else if (dtype == LNR_F16) {
        e = launch(layernorm_bw_dx_generic<f16, RMS>, dim3(static_cast<uint32_t>(N)),
                   dim3(kLnGenericWG), s, static_cast<f16 *>(dx), static_cast<const f16 *>(dy),
                   static_cast<const f16 *>(x), static_cast<const f16 *>(gamma), mean, rstd, N, C32);
        if (e == hipSuccess)
            e = launch(layernorm_bw_colpart_generic<f16, RMS>,
                       dim3(static_cast<uint32_t>((C + kLnGenericWG - 1) / kLnGenericWG),
                            static_cast<uint32_t>(pg)),
                       dim3(kLnGenericWG), s, static_cast<float *>(workspace),
                       static_cast<const f16 *>(dy), static_cast<const f16 *>(x), mean, rstd, N, C32, rg);
        if (e == hipSuccess) e = launch_colsum<f16>(dgamma, dbeta, nullptr, workspace, pg, C32, slots, 2, s);
    } else {
        e = launch(layernorm_bw_dx_generic<float, RMS>, dim3(static_cast<uint32_t>(N)),
                   dim3(kLnGenericWG), s, static_cast<float *>(dx), static_cast<const float *>(dy),
                   static_cast<const float *>(x), static_cast<const float *>(gamma), mean, rstd, N, C32);
        if (e == hipSuccess)
            e = launch(layernorm_bw_colpart_generic<float, RMS>,
                       dim3(static_cast<uint32_t>((C + kLnGenericWG - 1) / kLnGenericWG),
                            static_cast<uint32_t>(pg)),
                       dim3(kLnGenericWG), s, static_cast<double *>(workspace),
                       static_cast<const float *>(dy), static_cast<const float *>(x), mean, rstd, N, C32, rg);
        if (e == hipSuccess) e = launch_colsum<float>(dgamma, dbeta, nullptr, workspace, pg, C32, slots, 2, s);
    }
    return status_of(e);
}

static size_t bdr_workspace_bytes(int64_t N, int64_t C, lnr_dtype dtype) {
    if (!valid_dtype(dtype) || N < 0 || C < 1 || C > LNR_LAYERNORM_MAX_C) return 0;
    int64_t pv, pg, rv, rg;
    bw_partials(N, C, dtype, pv, pg, rv, rg, true);
    const int64_t P = pv > pg ? pv : pg;
    return static_cast<size_t>(P) * 3 * static_cast<size_t>(C) * accum_size(dtype);
}

// The fused op's vector path: every [N, C] and [C] buffer 16-byte aligned and C * element
// size a multiple of 16 (C a multiple of 8 for fp16, of 4 for fp32). Anything else takes the
// element-wise kernels.
static bool bdr_vec_ok(int64_t C, size_t es, std::initializer_list<const void *> bufs) {
    if ((static_cast<size_t>(C) * es) % 16 != 0) return false;
    for (const void *b : bufs)
        if (b != nullptr && !aligned_to(b, 16)) return false;
    return true;
}

static int bdr_fw(void *s_out, void *y, float *mean, float *rstd, const void *x,
                  const void *residual, const void *bias, const uint8_t *mask, float p,
                  const void *gamma, const void *beta, int64_t N, int64_t C, float eps,
                  lnr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (N < 0 || C < 1) return LNR_ERR_SHAPE;
    if (C > LNR_LAYERNORM_MAX_C || N > INT32_MAX) return LNR_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || !isfinite(eps) || !(p >= 0.f) || !(p < 1.f)) return LNR_ERR_SHAPE;
    if ((mean == nullptr) != (rstd == nullptr)) return LNR_ERR_NULL;
    if (N == 0) return LNR_OK;
    if (s_out == nullptr || y == nullptr || x == nullptr || residual == nullptr ||
        bias == nullptr || mask == nullptr || gamma == nullptr || beta == nullptr)
        return LNR_ERR_NULL;
    const size_t es = dtype_size(dtype);
    for (const void *b : std::initializer_list<const void *>{s_out, y, x, residual, bias, gamma, beta})
        if (!aligned_to(b, es)) return LNR_ERR_ALIGN;
    if (!aligned_to(mean, 4) || !aligned_to(rstd, 4)) return LNR_ERR_ALIGN;
    const size_t nb = static_cast<size_t>(N) * static_cast<size_t>(C) * es;
    const size_t cb = static_cast<size_t>(C) * es;
    const size_t mbytes = static_cast<size_t>(N) * static_cast<size_t>((C + 7) / 8);
    // s may replace residual in place (elementwise); no other overlap.
    if (bad_alias(s_out, residual, nb) || overlap(s_out, nb, x, nb) || overlap(y, nb, s_out, nb) ||
        overlap(y, nb, x, nb) || overlap(y, nb, residual, nb) || overlap(x, nb, residual, nb))
        return LNR_ERR_ALIAS;
    for (const void *out : {s_out, y})
        if (overlap(out, nb, bias, cb) || overlap(out, nb, gamma, cb) || overlap(out, nb, beta, cb) ||
            overlap(out, nb, mask, mbytes) || overlap(out, nb, mean, N * 4) ||
            overlap(out, nb, rstd, N * 4))
            return LNR_ERR_ALIAS;
    if (overlap(mean, N * 4, rstd, N * 4)) return LNR_ERR_ALIAS;

    LnFwArgs a{y, mean, rstd, x, gamma, beta, N, static_cast<int32_t>(C), eps};
    a.s_out = s_out;
    a.residual = residual;
    a.bias = bias;
    a.mask = mask;
    a.keep_scale = static_cast<float>(1.0 / (1.0 - static_cast<double>(p)));
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (bdr_vec_ok(C, es, {s_out, y, x, residual, bias, gamma, beta})) {
        e = dtype == LNR_F16 ? dispatch_ln_fw<f16, kBdrLayerNorm, 0>(a, st)
                             : dispatch_ln_fw<float, kBdrLayerNorm, 0>(a, st);
    } else if (dtype == LNR_F16) {
        e = launch(bdr_layernorm_fw_generic<f16>, dim3(static_cast<uint32_t>(N)), dim3(kLnGenericWG), st,
                   static_cast<f16 *>(s_out), static_cast<f16 *>(y), mean, rstd,
                   static_cast<const f16 *>(x), static_cast<const f16 *>(residual),
                   static_cast<const f16 *>(bias), mask, a.keep_scale, static_cast<const f16 *>(gamma),
                   static_cast<const f16 *>(beta), N, a.C, eps);
    } else {
        e = launch(bdr_layernorm_fw_generic<float>, dim3(static_cast<uint32_t>(N)), dim3(kLnGenericWG), st,
                   static_cast<float *>(s_out), static_cast<float *>(y), mean, rstd,
                   static_cast<const float *>(x), static_cast<const float *>(residual),
                   static_cast<const float *>(bias), mask, a.keep_scale,
                   static_cast<const float *>(gamma), static_cast<const float *>(beta), N, a.C, eps);
    }
    return status_of(e);
}

static int bdr_bw(void *dres, void *dx, void *dgamma, void *dbeta, void *dbias, const void *dy,
                  const void *ds_extra, const void *s_in, const uint8_t *mask, float p,
                  const void *gamma, const float *mean, const float *rstd, int64_t N, int64_t C,
                  lnr_dtype dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (N < 0 || C < 1) return LNR_ERR_SHAPE;
    if (C > LNR_LAYERNORM_MAX_C || N > INT32_MAX) return LNR_ERR_UNSUPPORTED;
    if (!(p >= 0.f) || !(p < 1.f)) return LNR_ERR_SHAPE;
    if (dgamma == nullptr || dbeta == nullptr || dbias == nullptr) return LNR_ERR_NULL;
    if (N > 0 && (dres == nullptr || dx == nullptr || dy == nullptr || s_in == nullptr ||
                  mask == nullptr || gamma == nullptr || mean == nullptr || rstd == nullptr))
        return LNR_ERR_NULL;
    const size_t es = dtype_size(dtype);
    for (const void *b : std::initializer_list<const void *>{dres, dx, dy, ds_extra, s_in, gamma, dgamma, dbeta, dbias})
        if (!aligned_to(b, es)) return LNR_ERR_ALIGN;
    if (!aligned_to(mean, 4) || !aligned_to(rstd, 4)) return LNR_ERR_ALIGN;
    const size_t need = bdr_workspace_bytes(N, C, dtype);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LNR_ERR_WORKSPACE;
    if (need > 0 && !aligned_to(workspace, 16)) return LNR_ERR_ALIGN;
    const size_t nb = static_cast<size_t>(N) * static_cast<size_t>(C) * es;
    const size_t cb = static_cast<size_t>(C) * es;
    const size_t mbytes = static_cast<size_t>(N) * static_cast<size_t>((C + 7) / 8);
    // dresidual may replace dy or ds_extra in place; dx overlaps nothing.
    if (bad_alias(dres, dy, nb) || bad_alias(dres, ds_extra, nb) || overlap(dres, nb, s_in, nb) ||
        overlap(dx, nb, dres, nb) || overlap(dx, nb, dy, nb) || overlap(dx, nb, ds_extra, nb) ||
        overlap(dx, nb, s_in, nb))
        return LNR_ERR_ALIAS;
    for (const void *out : {dres, dx})
        if (overlap(out, nb, gamma, cb) || overlap(out, nb, mask, mbytes) ||
            overlap(out, nb, mean, N * 4) || overlap(out, nb, rstd, N * 4) ||
            overlap(out, nb, workspace, need))
            return LNR_ERR_ALIAS;
    for (const void *out : {dgamma, dbeta, dbias}) {
        if (overlap(out, cb, dres, nb) || overlap(out, cb, dx, nb) || overlap(out, cb, dy, nb) ||
            overlap(out, cb, s_in, nb) || overlap(out, cb, gamma, cb) || overlap(out, cb, workspace, need))
            return LNR_ERR_ALIAS;
    }
    if (overlap(dgamma, cb, dbeta, cb) || overlap(dgamma, cb, dbias, cb) || overlap(dbeta, cb, dbias, cb))
        return LNR_ERR_ALIAS;
    // Every workgroup writes its partial row while others still read the inputs.
    if (overlap(workspace, need, dy, nb) || overlap(workspace, need, s_in, nb) ||
        overlap(workspace, need, ds_extra, nb) || overlap(workspace, need, gamma, cb) ||
        overlap(workspace, need, mean, N * 4) || overlap(workspace, need, rstd, N * 4) ||
        overlap(workspace, need, mask, mbytes))
        return LNR_ERR_ALIAS;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int32_t C32 = static_cast<int32_t>(C);
    if (N == 0) {
        const hipError_t e =
            dtype == LNR_F16 ? launch_colsum<f16>(dgamma, dbeta, dbias, workspace, 0, C32, 3, 3, st)
                             : launch_colsum<float>(dgamma, dbeta, dbias, workspace, 0, C32, 3, 3, st);
        return status_of(e);
    }
    int64_t pv, pg, rv, rg;
    bw_partials(N, C, dtype, pv, pg, rv, rg, true);
    const float keep_scale = static_cast<float>(1.0 / (1.0 - static_cast<double>(p)));
    hipError_t e;
    if (bdr_vec_ok(C, es, {dres, dx, dy, ds_extra, s_in, gamma})) {
        LnBwArgs a{dres, dgamma, dbeta, workspace, dy, s_in, gamma, mean, rstd, N, C32, rv, pv};
        a.dx2 = dx;
        a.dbias = dbias;
        a.ds_extra = ds_extra;
        a.mask = mask;
        a.keep_scale = keep_scale;
        e = dtype == LNR_F16 ? dispatch_ln_bw<f16, kBdrLayerNorm, 0>(a, st)
                             : dispatch_ln_bw<float, kBdrLayerNorm, 0>(a, st);
    } else {
        if (dtype == LNR_F16)
            e = launch(bdr_layernorm_bw_generic<f16>, dim3(static_cast<uint32_t>(pg)), dim3(kLnGenericWG), st,
                       static_cast<f16 *>(dres), static_cast<f16 *>(dx), static_cast<float *>(workspace),
                       static_cast<const f16 *>(dy), static_cast<const f16 *>(ds_extra),
                       static_cast<const f16 *>(s_in), mask, keep_scale, static_cast<const f16 *>(gamma),
                       mean, rstd, N, C32, rg);
        else
            e = launch(bdr_layernorm_bw_generic<float>, dim3(static_cast<uint32_t>(pg)), dim3(kLnGenericWG), st,
                       static_cast<float *>(dres), static_cast<float *>(dx), static_cast<double *>(workspace),
                       static_cast<const float *>(dy), static_cast<const float *>(ds_extra),
                       static_cast<const float *>(s_in), mask, keep_scale,
                       static_cast<const float *>(gamma), mean, rstd, N, C32, rg);
        if (e == hipSuccess)
            e = dtype == LNR_F16 ? launch_colsum<f16>(dgamma, dbeta, dbias, workspace, pg, C32, 3, 3, st)
                                 : launch_colsum<float>(dgamma, dbeta, dbias, workspace, pg, C32, 3, 3, st);
    }
    return status_of(e);
}

// ------------------------------------------------------------------------------------------
// layernorm_bw without a caller workspace, for callers that cannot allocate. The column
// partials go to `scratch`, a file-scope device array: every GPU the library runs on holds its
// own copy until the process ends. Its address on a device is looked up once, with that device
// current, and kept per device; host code never passes the array's name itself to a kernel
// (on the host it names a stand-in, not device memory). Nothing in it needs clearing: the
// backward's row kernel writes every partial row the column sum reads.
// ------------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = LNR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void *> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// The device `stream` runs on (the current device for the default stream).
static hipError_t stream_device(hipStream_t stream, int &dev) {
    if (stream == nullptr) return hipGetDevice(&dev);
    hipDevice_t d = 0;
    const hipError_t e = hipStreamGetDevice(stream, &d);
    dev = static_cast<int>(d);
    return e;
}

// Address of `scratch` on device `dev`, looked up on the first call for that device.
static int scratch_on(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return LNR_ERR_UNSUPPORTED;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int prev = 0;
            if (hipGetDevice(&prev) != hipSuccess) return LNR_ERR_HIP;
            if (prev != dev && hipSetDevice(dev) != hipSuccess) return LNR_ERR_HIP;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (prev != dev && hipSetDevice(prev) != hipSuccess) return LNR_ERR_HIP;
            if (e != hipSuccess || p == nullptr) return LNR_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LNR_OK;
}

static int layernorm_bw_scratch(void *dx, void *dgamma, void *dbeta, const void *dy, const void *x,
                                const void *gamma, const float *mean, const float *rstd, int64_t N,
                                int64_t C, lnr_dtype dtype, void *stream) {
    int st = norm_bw<false>(dx, dgamma, dbeta, dy, x, gamma, mean, rstd, N, C, dtype, nullptr, 0,
                            stream, true);
    if (st != LNR_OK) return st;
    if (bw_workspace_bytes(N, C, dtype) > kScratchBytes) return LNR_ERR_SCRATCH;
    int dev = 0;
    if (stream_device(static_cast<hipStream_t>(stream), dev) != hipSuccess) return LNR_ERR_HIP;
    void *ws = nullptr;
    st = scratch_on(dev, &ws);
    if (st != LNR_OK) return st;
    return norm_bw<false>(dx, dgamma, dbeta, dy, x, gamma, mean, rstd, N, C, dtype, ws, kScratchBytes,
                          stream);
}

}  // namespace lnr

using namespace lnr;

extern "C" int layernorm_bw_noalloc(void *dx, void *dgamma, void *dbeta, const void *dy,
                                    const void *x, const void *gamma, const float *mean,
                                    const float *rstd, int64_t N, int64_t C, lnr_dtype dtype,
                                    void *stream) {
    return layernorm_bw_scratch(dx, dgamma, dbeta, dy, x, gamma, mean, rstd, N, C, dtype, stream);
}

extern "C" int bdr_layernorm_fw(void *s, void *y, float *mean, float *rstd, const void *x,
                                const void *residual, const void *bias, const uint8_t *keep_mask,
                                float p, const void *gamma, const void *beta, int64_t N, int64_t C,
                                float eps, lnr_dtype dtype, void *stream) {
    return bdr_fw(s, y, mean, rstd, x, residual, bias, keep_mask, p, gamma, beta, N, C, eps, dtype,
                  stream);
}

extern "C" size_t bdr_layernorm_bw_workspace_bytes(int64_t N, int64_t C, lnr_dtype dtype) {
    return bdr_workspace_bytes(N, C, dtype);
}

extern "C" int bdr_layernorm_bw(void *dresidual, void *dx, void *dgamma, void *dbeta, void *dbias,
                                const void *dy, const void *ds_extra, const void *s,
                                const uint8_t *keep_mask, float p, const void *gamma,
                                const float *mean, const float *rstd, int64_t N, int64_t C,
                                lnr_dtype dtype, void *workspace, size_t workspace_bytes,
                                void *stream) {
    return bdr_bw(dresidual, dx, dgamma, dbeta, dbias, dy, ds_extra, s, keep_mask, p, gamma, mean,
                  rstd, N, C, dtype, workspace, workspace_bytes, stream);
}

extern "C" int layernorm_fw(void *y, float *mean, float *rstd, const void *x, const void *gamma,
                            const void *beta, int64_t N, int64_t C, float eps, lnr_dtype dtype,
                            void *stream) {
    return norm_fw<false>(y, mean, rstd, x, gamma, beta, N, C, eps, dtype, stream);
}

extern "C" size_t layernorm_bw_workspace_bytes(int64_t N, int64_t C, lnr_dtype dtype) {
    return bw_workspace_bytes(N, C, dtype);
}

extern "C" int layernorm_bw(void *dx, void *dgamma, void *dbeta, const void *dy, const void *x,
                            const void *gamma, const float *mean, const float *rstd, int64_t N,
                            int64_t C, lnr_dtype dtype, void *workspace, size_t workspace_bytes,
                            void *stream) {
    return norm_bw<false>(dx, dgamma, dbeta, dy, x, gamma, mean, rstd, N, C, dtype, workspace,
                          workspace_bytes, stream);
}

extern "C" int rmsnorm_fw(void *y, float *rstd, const void *x, const void *gamma, int64_t N,
                          int64_t C, float eps, lnr_dtype dtype, void *stream) {
    return norm_fw<true>(y, nullptr, rstd, x, gamma, nullptr, N, C, eps, dtype, stream);
}

extern "C" size_t rmsnorm_bw_workspace_bytes(int64_t N, int64_t C, lnr_dtype dtype) {
    return bw_workspace_bytes(N, C, dtype);
}

extern "C" int rmsnorm_bw(void *dx, void *dgamma, const void *dy, const void *x, const void *gamma,
                          const float *rstd, int64_t N, int64_t C, lnr_dtype dtype, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return norm_bw<true>(dx, dgamma, nullptr, dy, x, gamma, nullptr, rstd, N, C, dtype, workspace,
                         workspace_bytes, stream);
}

// Introspection: the bucket, lanes per row, vectors per lane and workgroup size of the
// forward (which = 0) or backward (which = 1) vector kernel for (C, dtype); bucket 0 means
// the element-wise fallback. For the backward, *blocks gets the number of partial rows.
extern "C" int lnr_layernorm_plan(int64_t N, int64_t C, lnr_dtype dtype, int which, int *bucket,
                                  int *lanes_per_row, int *vectors_per_lane, int *workgroup,
                                  int64_t *blocks) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (N < 0 || C < 1) return LNR_ERR_SHAPE;
    if (C > LNR_LAYERNORM_MAX_C) return LNR_ERR_UNSUPPORTED;
    if (!bucket || !lanes_per_row || !vectors_per_lane || !workgroup || !blocks) return LNR_ERR_NULL;
    const bool vec = (static_cast<size_t>(C) * dtype_size(dtype)) % 16 == 0;
    LnPlan p{0, kLnGenericWG, 0, kLnGenericWG, 1};
    bool ok = false;
    if (vec) {
        if (which == 0)
            ok = dtype == LNR_F16 ? find_plan<LnFwTable<f16>>(C, N, p) : find_plan<LnFwTable<float>>(C, N, p);
        else
            ok = dtype == LNR_F16 ? find_plan<LnBwTable<f16>>(C, N, p) : find_plan<LnBwTable<float>>(C, N, p);
    }
    if (!ok) p = LnPlan{0, kLnGenericWG, 0, kLnGenericWG, 1};
    *bucket = p.bucket;
    *lanes_per_row = p.G;
    *vectors_per_lane = p.IT;
    int64_t pv, pg, rv, rg;
    bw_partials(N, C, dtype, pv, pg, rv, rg);
    if (which == 0) {
        *workgroup = ok ? p.WG : kLnGenericWG;
        const int64_t rpb = ok ? static_cast<int64_t>(p.WG / p.G) * p.R : 1;
        *blocks = (N + rpb - 1) / rpb;
    } else {
        *workgroup = ok ? p.WG : kLnGenericWG;
        *blocks = ok ? pv : pg;
    }
    return LNR_OK;
}
