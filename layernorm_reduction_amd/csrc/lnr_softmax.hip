// lnr_softmax.hip -- masked / causal attention softmax, forward and backward, for gfx950.
//
// Method: "CMU 11-868 HW4: Softmax and LayerNorm as fused CUDA kernels", section "Problem
// structure and scoring" (scores plus the attention mask, future tokens at -inf, a row max,
// then a sum of exponentials; the backward templated on row length from {32, ..., 2048})
// and "CMU 11-868 L10 ...", section "Technique 2" (two reductions per row; rows <= 32 on
// one warp; elements per thread and blocks fixed at compile time, picked at launch).
//
// Design on CDNA4:
//   * A row of Tk elements is held in registers by a group of G lanes of one wave64; each
//     lane owns IT vectors of 16 bytes. Vector k of lane l covers elements
//     [(k*G + l)*V, +V), so every load instruction of a group reads G*16 contiguous bytes.
//     Short rows use small G and put several rows in one wave (16 rows of 32 fp16 each at
//     G = 4); rows up to 2048 use the whole wave. (G, IT) per row-length bucket is a
//     compile-time choice, picked by the host from Tk.
//   * The two softmax reductions (max, then sum) are lane-crossing DPP/ds_swizzle
//     butterflies inside the group (lnr_prims.h): no LDS, no barrier.
//   * One pass over HBM: each row is read once and written once. Rows whose byte length is
//     not a multiple of 16, or unaligned buffers, go to an element-wise fallback kernel
//     (one wave per row, three passes over the row through the caches).
#include <math.h>

#include "lnr_common.h"
#include "lnr_fastdiv.h"
#include "lnr_prims.h"

namespace lnr {

// The forward vector kernel indexes rows in 32 bits (multiply-shift division for the batch and
// query indices); larger row counts take the element-wise kernel.
constexpr int64_t kVecMaxRows = int64_t{UINT32_MAX} - 4096;

// ------------------------------------------------------------------------------------------
// Vector kernels.
// ------------------------------------------------------------------------------------------
template <typename T, int G, int IT, int WG>
__global__ __launch_bounds__(WG) void softmax_fw_vec(T *out, const T *inp,
                                                     const T *__restrict__ mask, uint32_t rows,
                                                     int32_t Tk, DivU32 per_batch,
                                                     DivU32 per_query, int32_t causal) {
    constexpr int V = Vec16<T>::N;
    constexpr int RPB = WG / G;
    const int lane = threadIdx.x % G;
    // rows < 2^32 - 4096 (checked by the host), so the row index and the one past the last
    // workgroup fit in 32 bits, and the batch and query indices come from multiply-shift
    // division: short rows leave few elements per lane to amortise the index math over.
    const uint32_t row = blockIdx.x * static_cast<uint32_t>(RPB) + threadIdx.x / G;
    const bool live = row < rows;
    const int nvec = Tk / V;
    const int64_t base = static_cast<int64_t>(live ? row : 0u) * Tk;
    static_assert(G <= 64, "a wave holds whole rows");
    // The wave's first row (clamped to row 0 when the whole wave is past the end, where every
    // store is dropped): the base of the branch-free stores at the end.
    const uint32_t wave_row0 = row - (threadIdx.x % 64) / G;
    const uint32_t wrow = wave_row0 < rows ? wave_row0 : 0u;

    // Scores and mask are loaded as stored, every load unconditional (an idle lane reads its
    // row's first vector; a row past the end reads row 0), so no branch makes the compiler
    // wait between loads. Idle lanes then take -inf scores (a select only in buckets wider
    // than the row); their mask values come from the same row and change nothing. At fp16 the
    // widening and the mask add are one mixed-precision fma (x * 1 + m: both exact in fp32,
    // the sum rounded once, as the plain addition).
    using RV = RawVec<T>;
    RV xr[IT], mr[IT];
    const T *mrow = mask != nullptr
                        ? mask + static_cast<int64_t>(divu32(live ? row : 0u, per_batch)) * Tk
                        : nullptr;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        const int64_t off = c < nvec ? static_cast<int64_t>(c) * V : 0;
        xr[k] = load_stream_raw<T>(inp + base + off);
    }
    if (mrow != nullptr) {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int c = k * G + lane;
            mr[k] = load_keep_raw<T>(mrow + (c < nvec ? static_cast<int64_t>(c) * V : 0));
        }
    } else {
#pragma unroll
        for (int k = 0; k < IT; ++k)
#pragma unroll
            for (int e = 0; e < V; ++e) mr[k][e] = T(0);
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        if ((k + 1) * G > nvec) {  // uniform: this vector slot has idle lanes
            RV ninf;
#pragma unroll
            for (int e = 0; e < V; ++e) ninf[e] = static_cast<T>(-INFINITY);
            xr[k] = k * G + lane < nvec ? xr[k] : ninf;
        }
    }
    float one = 1.0f;
    if constexpr (V == 8) asm("" : "+v"(one));
    float z[IT][V];
#pragma unroll
    for (int k = 0; k < IT; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e)
            z[k][e] = __builtin_fmaf(static_cast<float>(xr[k][e]), one, static_cast<float>(mr[k][e]));
    if (causal) {
        const int qi = static_cast<int>(row - divu32(row, per_query) * per_query.d);
#pragma unroll
        for (int k = 0; k < IT; ++k) {
#pragma unroll
            for (int e = 0; e < V; ++e)
                if ((k * G + lane) * V + e > qi) z[k][e] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < IT; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) mx = fmaxf(mx, z[k][e]);
    mx = group_allreduce<G>(mx, OpMax());
    if (mx == -INFINITY) mx = 0.f;  // fully masked (or idle) row: every exponential is 0

    float s = 0.f;
#pragma unroll
    for (int k = 0; k < IT; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) {
            z[k][e] = exp_nonpos(z[k][e] - mx);
            s += z[k][e];
        }
    s = group_allreduce<G>(s, OpSum());
    // v_rcp_f32 (1 ulp) instead of the IEEE divide sequence: s >= 1 (the max term is 1), and
    // the result is far inside the tolerance.
    const float inv = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;

    // Branch-free stores at device scope, through a descriptor at the wave's first row: a lane
    // with nothing to store (a row past the end, a vector slot past the row) passes an offset
    // beyond the range and is dropped. Offsets stay below 64 rows of 2048 fp32 keys.
    T *wave_out = out + static_cast<int64_t>(wrow) * Tk;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        float y[V];
#pragma unroll
        for (int e = 0; e < V; ++e) y[e] = z[k][e] * inv;
        const uint32_t off = (live && c < nvec)
                                 ? ((row - wrow) * static_cast<uint32_t>(Tk) + static_cast<uint32_t>(c * V)) *
                                       static_cast<uint32_t>(sizeof(T))
                                 : kDropOffset;
        store16_or_drop<kBufferDeviceStream>(wave_out, off, pack16<T>(y));
    }
}

template <typename T, int G, int IT, int WG>
__global__ __launch_bounds__(WG) void softmax_bw_vec(T *dinp, const T *dout,
                                                     const T *__restrict__ y, int64_t rows,
                                                     int32_t Tk) {
    constexpr int V = Vec16<T>::N;
    constexpr int RPB = WG / G;
    const int lane = threadIdx.x % G;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / G;
    const bool live = row < rows;
    const int nvec = Tk / V;
    const int64_t base = (live ? row : 0) * static_cast<int64_t>(Tk);

    // Every load unconditional (an idle lane reads its row's first vector, a row past the end
    // row 0), so no branch makes the compiler wait between loads (with a branch per vector it
    // waited after every pair of loads: 5-10% slower at 2-4 vectors per lane). Idle lanes then
    // take y = 0 (a select only in buckets wider than the row), which removes them from the sum.
    using RV = RawVec<T>;
    RV yr[IT], gr[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        const int64_t off = base + (c < nvec ? static_cast<int64_t>(c) * V : 0);
        yr[k] = load_stream_raw<T>(y + off);
        gr[k] = load_stream_raw<T>(dout + off);
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        if ((k + 1) * G > nvec) {  // uniform: this vector slot has idle lanes
            const RV zero = {};
            yr[k] = k * G + lane < nvec ? yr[k] : zero;
        }
    }
    float yv[IT][V], gv[IT][V];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        widen<T>(yr[k], yv[k]);
        widen<T>(gr[k], gv[k]);
    }
    // The product sum is a chain of fused multiply-adds. With the fp16 widening next to the
    // multiply, the compiler would pair two products into a dot2 instruction, which rounds
    // differently; an empty register constraint hides the widened values from that combine
    // (it emits no instruction), so this kernel and the read-skipping one agree bit for bit.
    if constexpr (V == 8) {
#pragma unroll
        for (int k = 0; k < IT; ++k)
#pragma unroll
            for (int e = 0; e < V; ++e) asm("" : "+v"(yv[k][e]), "+v"(gv[k][e]));
    }
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < IT; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) t += yv[k][e] * gv[k][e];
    t = group_allreduce<G>(t, OpSum());

#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        if (live && c < nvec) {
            float d[V];
#pragma unroll
            for (int e = 0; e < V; ++e) d[e] = yv[k][e] * (gv[k][e] - t);
            store_stream<T>(dinp + base + static_cast<int64_t>(c) * V, d);
        }
    }
}


// ------------------------------------------------------------------------------------------
// Element-wise fallback kernels: one wave per row, any Tk, any element alignment.
// ------------------------------------------------------------------------------------------
constexpr int kGenericWG = 256;
constexpr int kGenericRowsPerBlock = kGenericWG / 64;

template <typename T>
__device__ __forceinline__ float masked_score(const T *x, const T *m, int j, int qi, int causal) {
    if (causal && j > qi) return -INFINITY;
    float z = to_f32(x[j]);
    if (m != nullptr) z += to_f32(m[j]);
    return z;
}

template <typename T>
__global__ __launch_bounds__(kGenericWG) void softmax_fw_generic(T *out, const T *inp,
                                                                 const T *__restrict__ mask,
                                                                 int64_t rows, int32_t Tq,
                                                                 int32_t Tk,
                                                                 int64_t rows_per_batch,
                                                                 int32_t causal) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kGenericRowsPerBlock + (threadIdx.x >> 6);
    const bool live = row < rows;  // uniform across the wave
    const int64_t base = (live ? row : 0) * static_cast<int64_t>(Tk);
    const T *x = inp + base;
    const T *m = mask != nullptr ? mask + (live ? row / rows_per_batch : 0) * static_cast<int64_t>(Tk)
                                 : nullptr;
    const int qi = static_cast<int>(row % Tq);

    float mx = -INFINITY;
    if (live)
        for (int j = lane; j < Tk; j += 64) mx = fmaxf(mx, masked_score(x, m, j, qi, causal));
    mx = group_allreduce<64>(mx, OpMax());
    if (mx == -INFINITY) mx = 0.f;
    float s = 0.f;
    if (live)
        for (int j = lane; j < Tk; j += 64) s += exp_nonpos(masked_score(x, m, j, qi, causal) - mx);
    s = group_allreduce<64>(s, OpSum());
    const float inv = s > 0.f ? 1.0f / s : 0.f;
    if (live)
        for (int j = lane; j < Tk; j += 64)
            out[base + j] = from_f32<T>(exp_nonpos(masked_score(x, m, j, qi, causal) - mx) * inv);
}

template <typename T>
__global__ __launch_bounds__(kGenericWG) void softmax_bw_generic(T *dinp, const T *dout,
                                                                 const T *__restrict__ y,
                                                                 int64_t rows, int32_t Tk) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kGenericRowsPerBlock + (threadIdx.x >> 6);
    const bool live = row < rows;
    const int64_t base = (live ? row : 0) * static_cast<int64_t>(Tk);
    float t = 0.f;
    if (live)
        for (int j = lane; j < Tk; j += 64) t += to_f32(y[base + j]) * to_f32(dout[base + j]);
    t = group_allreduce<64>(t, OpSum());
    if (live)
        for (int j = lane; j < Tk; j += 64) {
            const float yj = to_f32(y[base + j]);
            dinp[base + j] = from_f32<T>(yj * (to_f32(dout[base + j]) - t));
        }
}

// ------------------------------------------------------------------------------------------
// Row-length buckets: (G lanes per row, IT vectors per lane) for each storage type, one
// table for the forward and one for the backward. Capacity G * IT * V equals the bucket
// length; rows shorter than their bucket leave the trailing vectors idle. The bucket lengths
// are the HW4 page's template list. Measured on MI355X, each plan against its neighbours in
// one process (old and new library alternating, median of 7-9):
//  * Up to 512 fp16 keys (256 fp32) both directions run best with a row on as few vectors
//    per lane as fit a wave and one wave per workgroup: one 64-thread workgroup per row from
//    256 fp16 keys, several rows per wave below. Against the earlier plans (two to four
//    vectors per lane over 8-32 lanes, or 128-256-thread workgroups): forward -1 to -4% at
//    32-512 fp16 keys and -1 to -5% at 32-256 fp32 keys; backward -3 to -4% at 32-256 fp16
//    keys, -1 to -2% at 512 fp16 keys, -2 to -5% at 32-512 fp32 keys.
//  * The fp32 512-key forward takes one row per 64-thread workgroup with two vectors per
//    lane: with the branch-free device-scope stores it runs 2-4.5% faster than four vectors
//    over 32 lanes in 256-thread workgroups (before those stores the two tied).
//  * Longer rows keep two to four vectors per lane in 256-thread workgroups, except the
//    2048-key forwards, where 64-thread workgroups win (-1% fp16, -4% fp32); one wave per
//    workgroup loses 1-6% at 384-1024 fp16 keys and 384-768 fp32 keys (re-measured with the
//    device-scope stores: +2 to +4%), and up to 5% in the
//    fp32 backward from 1024 keys. fp16 1024 keys take four vectors over 32 lanes in the
//    backward (-4% against one vector per lane), fp16 2048 and fp32 1024 keys 256-thread
//    workgroups (-4%, -5%).
//  * fp32 512 keys over 32 lanes with four vectors in the backward was 1-4% faster but not
//    taken: at fp32 storage the cancellation in dy - sum makes two summation orders differ by
//    more than an ulp, and the read-skipping backward keeps two vectors over 64 lanes.
// The read-skipping kernels have tables of their own: their forward loads a row's mask before
// its scores, so one vector per lane exposes that latency (22% slower at 512 fp16 keys) and it
// keeps several vectors per lane. Where the two forwards (or backwards) differ in lanes per
// row or vectors per lane, they add a row's terms in different orders and agree to an ulp of
// the storage type; elsewhere they agree exactly.
// ------------------------------------------------------------------------------------------
struct Plan {
    int bucket;  // longest row this instantiation takes; 0 = element-wise fallback
    int G;       // lanes per row
    int IT;      // 16-byte vectors per lane
    int WG;      // workgroup size
};

template <typename T> struct SoftmaxFwTable;
template <> struct SoftmaxFwTable<f16> {   // V = 8
    static constexpr Plan plans[] = {{32, 4, 1, 64},   {64, 8, 1, 64},    {128, 16, 1, 64},
                                     {256, 32, 1, 64},  {384, 16, 3, 256}, {512, 64, 1, 64},
                                     {768, 32, 3, 256}, {1024, 32, 4, 256}, {2048, 64, 4, 64}};
};
template <> struct SoftmaxFwTable<float> { // V = 4
    static constexpr Plan plans[] = {{32, 8, 1, 64},   {64, 16, 1, 256},  {128, 32, 1, 64},
                                     {256, 64, 1, 64},  {384, 32, 3, 256}, {512, 64, 2, 64},
                                     {768, 64, 3, 256}, {1024, 64, 4, 256}, {2048, 64, 8, 64}};
};
template <typename T> struct SoftmaxBwTable;
template <> struct SoftmaxBwTable<f16> {
    static constexpr Plan plans[] = {{32, 4, 1, 64},   {64, 8, 1, 64},   {128, 16, 1, 64},
                                     {256, 32, 1, 64},  {384, 16, 3, 256}, {512, 64, 1, 64},
                                     {768, 32, 3, 256}, {1024, 32, 4, 256}, {2048, 64, 4, 256}};
};
template <> struct SoftmaxBwTable<float> {
    static constexpr Plan plans[] = {{32, 8, 1, 64},   {64, 16, 1, 64},  {128, 32, 1, 64},
                                     {256, 64, 1, 64},  {384, 32, 3, 256}, {512, 64, 2, 64},
                                     {768, 64, 3, 128}, {1024, 64, 4, 256}, {2048, 64, 8, 128}};
};

struct SoftmaxFwArgs {
    void *out;
    const void *inp;
    const void *mask;
    int64_t rows;
    int32_t Tq, Tk;
    int64_t rows_per_batch;
    int32_t causal;
};
struct SoftmaxBwArgs {
    void *dinp;
    const void *dout;
    const void *y;
    int64_t rows;
    int32_t Tk;
};

template <typename T, int G, int IT, int WG>
static hipError_t launch_fw_vec(const SoftmaxFwArgs &a, hipStream_t st) {
    constexpr int RPB = WG / G;
    const int64_t blocks = (a.rows + RPB - 1) / RPB;
    return launch(softmax_fw_vec<T, G, IT, WG>, dim3(static_cast<uint32_t>(blocks)),
                  dim3(WG), st, static_cast<T *>(a.out), static_cast<const T *>(a.inp),
                  static_cast<const T *>(a.mask), static_cast<uint32_t>(a.rows), a.Tk,
                  make_divu32(static_cast<uint32_t>(a.rows_per_batch)),
                  make_divu32(static_cast<uint32_t>(a.Tq)), a.causal);
}

template <typename T, int G, int IT, int WG>
static hipError_t launch_bw_vec(const SoftmaxBwArgs &a, hipStream_t st) {
    constexpr int RPB = WG / G;
    const int64_t blocks = (a.rows + RPB - 1) / RPB;
    return launch(softmax_bw_vec<T, G, IT, WG>, dim3(static_cast<uint32_t>(blocks)),
                  dim3(WG), st, static_cast<T *>(a.dinp), static_cast<const T *>(a.dout),
                  static_cast<const T *>(a.y), a.rows, a.Tk);
}

// Compile-time walk over the bucket table: instantiate every (G, IT) and pick the first
// bucket that holds Tk.
template <typename T, int I>
static hipError_t dispatch_fw(const SoftmaxFwArgs &a, hipStream_t st) {
    constexpr Plan p = SoftmaxFwTable<T>::plans[I];
    if (a.Tk <= p.bucket) return launch_fw_vec<T, p.G, p.IT, p.WG>(a, st);
    if constexpr (I + 1 < static_cast<int>(sizeof(SoftmaxFwTable<T>::plans) / sizeof(Plan)))
        return dispatch_fw<T, I + 1>(a, st);
    return hipErrorInvalidValue;
}

template <typename T, int I>
static hipError_t dispatch_bw(const SoftmaxBwArgs &a, hipStream_t st) {
    constexpr Plan p = SoftmaxBwTable<T>::plans[I];
    if (a.Tk <= p.bucket) return launch_bw_vec<T, p.G, p.IT, p.WG>(a, st);
    if constexpr (I + 1 < static_cast<int>(sizeof(SoftmaxBwTable<T>::plans) / sizeof(Plan)))
        return dispatch_bw<T, I + 1>(a, st);
    return hipErrorInvalidValue;
}

template <typename Table>
static Plan softmax_plan(int64_t Tk, bool vector_ok) {
    if (vector_ok)
        for (const Plan &p : Table::plans)
            if (Tk <= p.bucket) return p;
    return Plan{0, 64, 0, kGenericWG};
}

static int check_common(const void *a, const void *b, const void *c, int64_t B, int64_t H,
                        int64_t Tq, int64_t Tk, lnr_dtype dtype) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (B < 0 || H < 0 || Tq < 0 || Tk < 1) return LNR_ERR_SHAPE;
    if (Tk > LNR_SOFTMAX_MAX_TK) return LNR_ERR_UNSUPPORTED;
    if (Tq > INT32_MAX) return LNR_ERR_UNSUPPORTED;
    // B * H * Tq must not overflow (the grid limit below is far smaller than INT64_MAX).
    if (H > 0 && Tq > 0 && B > INT64_MAX / H / Tq) return LNR_ERR_UNSUPPORTED;
    const int64_t rows = B * H * Tq;
    if (rows == 0) return LNR_OK;
    if (a == nullptr || b == nullptr || c == nullptr) return LNR_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned_to(a, es) || !aligned_to(b, es) || !aligned_to(c, es)) return LNR_ERR_ALIGN;
    // Grid size limit of the fallback (4 rows per block) bounds every path.
    if ((rows + kGenericRowsPerBlock - 1) / kGenericRowsPerBlock > INT32_MAX)
        return LNR_ERR_UNSUPPORTED;
    return LNR_OK;
}

}  // namespace lnr

using namespace lnr;

extern "C" int attn_softmax_fw(void *out, const void *inp, const void *mask, int64_t B,
                               int64_t H, int64_t Tq, int64_t Tk, int causal, lnr_dtype dtype,
                               void *stream) {
    const void *mask_or_inp = mask != nullptr ? mask : inp;
    int st = check_common(out, inp, mask_or_inp, B, H, Tq, Tk, dtype);
    if (st != LNR_OK) return st;
    if (causal && Tq != Tk) return LNR_ERR_SHAPE;
    const int64_t rows = B * H * Tq;
    if (rows == 0) return LNR_OK;
    const size_t es = dtype_size(dtype);
    const size_t nbytes = static_cast<size_t>(rows) * static_cast<size_t>(Tk) * es;
    if (bad_alias(out, inp, nbytes)) return LNR_ERR_ALIAS;
    if (mask != nullptr && overlap(out, nbytes, mask, static_cast<size_t>(B * Tk) * es))
        return LNR_ERR_ALIAS;

    SoftmaxFwArgs a{out, inp, mask, rows, static_cast<int32_t>(Tq), static_cast<int32_t>(Tk),
                    H * Tq, causal ? 1 : 0};
    const bool vec = (static_cast<size_t>(Tk) * es) % 16 == 0 && aligned_to(out, 16) &&
                     aligned_to(inp, 16) && (mask == nullptr || aligned_to(mask, 16)) &&
                     rows <= kVecMaxRows;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (vec) {
        e = dtype == LNR_F16 ? dispatch_fw<f16, 0>(a, s) : dispatch_fw<float, 0>(a, s);
    } else {
        const dim3 grid(static_cast<uint32_t>((rows + kGenericRowsPerBlock - 1) / kGenericRowsPerBlock));
        if (dtype == LNR_F16)
            e = launch(softmax_fw_generic<f16>, grid, dim3(kGenericWG), s, static_cast<f16 *>(out),
                       static_cast<const f16 *>(inp), static_cast<const f16 *>(mask), rows, a.Tq,
                       a.Tk, a.rows_per_batch, a.causal);
        else
            e = launch(softmax_fw_generic<float>, grid, dim3(kGenericWG), s, static_cast<float *>(out),
                       static_cast<const float *>(inp), static_cast<const float *>(mask), rows, a.Tq,
                       a.Tk, a.rows_per_batch, a.causal);
    }
    return status_of(e);
}

extern "C" int attn_softmax_bw(void *dinp, const void *dout, const void *out_fw, int64_t B,
                               int64_t H, int64_t Tq, int64_t Tk, lnr_dtype dtype, void *stream) {
    int st = check_common(dinp, dout, out_fw, B, H, Tq, Tk, dtype);
    if (st != LNR_OK) return st;
    const int64_t rows = B * H * Tq;
    if (rows == 0) return LNR_OK;
    const size_t es = dtype_size(dtype);
    const size_t nbytes = static_cast<size_t>(rows) * static_cast<size_t>(Tk) * es;
    if (bad_alias(dinp, dout, nbytes) || overlap(dinp, nbytes, out_fw, nbytes)) return LNR_ERR_ALIAS;

    SoftmaxBwArgs a{dinp, dout, out_fw, rows, static_cast<int32_t>(Tk)};
    const bool vec = (static_cast<size_t>(Tk) * es) % 16 == 0 && aligned_to(dinp, 16) &&
                     aligned_to(dout, 16) && aligned_to(out_fw, 16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (vec) {
        e = dtype == LNR_F16 ? dispatch_bw<f16, 0>(a, s) : dispatch_bw<float, 0>(a, s);
    } else {
        const dim3 grid(static_cast<uint32_t>((rows + kGenericRowsPerBlock - 1) / kGenericRowsPerBlock));
        if (dtype == LNR_F16)
            e = launch(softmax_bw_generic<f16>, grid, dim3(kGenericWG), s, static_cast<f16 *>(dinp),
                       static_cast<const f16 *>(dout), static_cast<const f16 *>(out_fw), rows, a.Tk);
        else
            e = launch(softmax_bw_generic<float>, grid, dim3(kGenericWG), s, static_cast<float *>(dinp),
                       static_cast<const float *>(dout), static_cast<const float *>(out_fw), rows, a.Tk);
    }
    return status_of(e);
}

// The read-skipping kernels' plan for (Tk, dtype) (lnr_softmax_skip.hip).
void skip_plan_of(int64_t Tk, lnr_dtype dtype, bool backward, int &bucket, int &G, int &IT);

// Introspection for tests and benchmarks: the bucket, lanes per row and vectors per lane
// that attn_softmax_fw (which = 0), attn_softmax_bw (1), attn_softmax_fw_skip (2) or
// attn_softmax_bw_skip (3) use for (Tk, dtype) with aligned buffers; bucket 0 means the
// element-wise fallback (the skipping entry points then call the dense ones).
extern "C" int lnr_softmax_plan(int64_t Tk, lnr_dtype dtype, int which, int *bucket,
                                int *lanes_per_row, int *vectors_per_lane) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (Tk < 1) return LNR_ERR_SHAPE;
    if (Tk > LNR_SOFTMAX_MAX_TK) return LNR_ERR_UNSUPPORTED;
    if (which < 0 || which > 3) return LNR_ERR_SHAPE;
    if (bucket == nullptr || lanes_per_row == nullptr || vectors_per_lane == nullptr) return LNR_ERR_NULL;
    const bool vec = (static_cast<size_t>(Tk) * dtype_size(dtype)) % 16 == 0;
    if (which >= 2) {
        if (!vec) return lnr_softmax_plan(Tk, dtype, which - 2, bucket, lanes_per_row, vectors_per_lane);
        skip_plan_of(Tk, dtype, which == 3, *bucket, *lanes_per_row, *vectors_per_lane);
        return LNR_OK;
    }
    Plan p;
    if (dtype == LNR_F16)
        p = which == 0 ? softmax_plan<SoftmaxFwTable<f16>>(Tk, vec) : softmax_plan<SoftmaxBwTable<f16>>(Tk, vec);
    else
        p = which == 0 ? softmax_plan<SoftmaxFwTable<float>>(Tk, vec) : softmax_plan<SoftmaxBwTable<float>>(Tk, vec);
    *bucket = p.bucket;
    *lanes_per_row = p.G;
    *vectors_per_lane = p.IT;
    return LNR_OK;
}
