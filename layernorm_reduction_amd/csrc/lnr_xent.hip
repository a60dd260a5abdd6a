// lnr_xent.hip -- softmax cross-entropy over a vocabulary, forward and backward, for gfx950.
//
// Method: "CMU 11-868 L10 ...", section "Technique 1: kernel fusion, leaving only GEMMs to
// cuBLAS" (cross entropy is one of the custom reduce kernels) and the inference section (a
// softmax over the whole vocabulary). The pages print no formula; this is the textbook one:
//   forward   lse_i = log sum_j exp(z_ij),  loss_i = lse_i - z_i,t_i
//   backward  dz_ij = dloss_i * scale * (exp(z_ij - lse_i) - [j == t_i])
// Rows whose target is ignore_index give loss 0 and a zero gradient row; a target outside
// [0, V) otherwise gives NaN (a visible result; a kernel cannot raise).
//
// Design on CDNA4:
//   * Rows are long (10^4 - 10^5 logits, 20-400 KB): a workgroup streams one row, 16-byte
//     non-temporal loads, U vectors in flight per thread per iteration. With too few rows to
//     fill the chip, the backward streams chunks of a row in separate workgroups, and so
//     does the forward for rows above 256 KB.
//   * Forward, one pass: each thread keeps a running maximum m and a sum s of exp(z - m);
//     per iteration it takes the maximum of its U*VE new logits and rescales s once, so the
//     cost is one exp per logit plus one per U*VE. Then the workgroup reduces (m, s): the
//     block maximum first, then the sum of the rescaled s. Split rows write (m, s) partials
//     and a small kernel combines them in chunk order.
//   * Any V and any row alignment: a row is a scalar head up to the first 128-byte line
//     boundary, 16-byte vectors, and a scalar tail, so a vocabulary of odd size (every row
//     starting at a different phase) still streams at full width, and every wave-wide vector
//     access covers whole cache lines (a 1 KiB access that straddles lines touches 9 of them,
//     and the backward's stores then write partial lines: 7-9% slower at V = 50001).
//   * Backward, one pass: each logit is read once and its gradient written once.
#include <math.h>

#include "lnr_common.h"
#include "lnr_prims.h"

namespace lnr {

constexpr float kLog2e = 1.4426950408889634f;

// Elements [0, head) and [tail, V) one at a time, [head, tail) as nvec 16-byte vectors.
struct RowSplit {
    int32_t head, nvec, tail;
};

// Vector part of a row starting at the first `align`-byte boundary of `row` (align 16 or
// 128; 0: no vector part, every element scalar). The head is shorter than align bytes.
template <typename T>
__device__ __forceinline__ RowSplit split_row(const T *row, int32_t V, uint32_t align) {
    constexpr int VE = Vec16<T>::N;
    if (align == 0) return {V, 0, V};
    const uint32_t phase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row) & (align - 1));
    int32_t head = static_cast<int32_t>(((align - phase) & (align - 1)) / sizeof(T));
    if (head > V) head = V;
    const int32_t nvec = (V - head) / VE;
    return {head, nvec, head + nvec * VE};
}

// Vectors [v0, v1) of chunk c out of S (contiguous, in order). Inner chunk boundaries are
// rounded down to a multiple of align / 16 vectors, so every chunk starts on a line.
__device__ __forceinline__ int32_t chunk_bound(int32_t nvec, int32_t c, int32_t S, uint32_t align) {
    if (c >= S) return nvec;
    const int32_t b = static_cast<int32_t>(static_cast<int64_t>(nvec) * c / S);
    return align > 16 ? b & ~static_cast<int32_t>(align / 16 - 1) : b;
}
__device__ __forceinline__ void chunk_range(int32_t nvec, int32_t c, int32_t S, uint32_t align,
                                            int32_t &v0, int32_t &v1) {
    v0 = chunk_bound(nvec, c, S, align);
    v1 = chunk_bound(nvec, c + 1, S, align);
}

// Fold logits whose maximum is vm and whose exp-sum relative to that maximum is acc into
// the running (m, s).
__device__ __forceinline__ void ms_fold(float &m, float &s, float vm, float acc) {
    const float mn = fmaxf(m, vm);
    if (mn == -INFINITY) return;  // nothing finite yet
    const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * kLog2e);
    const float b = vm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((vm - mn) * kLog2e);
    s = s * a + acc * b;
    m = mn;
}

// ------------------------------------------------------------------------------------------
// Forward statistics of row blockIdx.x, chunk blockIdx.y of S: (m, s) with s = sum exp(z - m).
// S == 1: writes lse and loss. S > 1: writes the chunk's (m, s) to part[(row*S + chunk)*2].
// ------------------------------------------------------------------------------------------
// 16 bytes of -inf in each storage type: what idle lanes of the forward's row loop read
// (global memory like the logits, so one global load serves both; never written).
__device__ uint32_t kIdleF16[4] __attribute__((aligned(16))) = {0xFC00FC00u, 0xFC00FC00u,
                                                                         0xFC00FC00u, 0xFC00FC00u};
__device__ uint32_t kIdleF32[4] __attribute__((aligned(16))) = {0xFF800000u, 0xFF800000u,
                                                                         0xFF800000u, 0xFF800000u};
template <typename T>
__device__ __forceinline__ const RawVec<T> *idle_vec() {
    return reinterpret_cast<const RawVec<T> *>(Vec16<T>::N == 8 ? kIdleF16 : kIdleF32);
}

// Largest element of a 16-byte vector, compared in the storage type (exact), as fp32.
template <typename T>
__device__ __forceinline__ float vec_max(const RawVec<T> &v) {
    if constexpr (Vec16<T>::N == 8) {
        const auto h4 = __builtin_elementwise_max(__builtin_shufflevector(v, v, 0, 1, 2, 3),
                                                  __builtin_shufflevector(v, v, 4, 5, 6, 7));
        const auto h2 = __builtin_elementwise_max(__builtin_shufflevector(h4, h4, 0, 1),
                                                  __builtin_shufflevector(h4, h4, 2, 3));
        return static_cast<float>(h2[0] > h2[1] ? h2[0] : h2[1]);
    } else {
        return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    }
}

template <typename T, int WG, int U>
__global__ __launch_bounds__(WG) void xent_fw_kernel(float *__restrict__ loss,
                                                     float *__restrict__ lse,
                                                     float *__restrict__ part, const T *z,
                                                     const int64_t *__restrict__ target,
                                                     int32_t V, int64_t ignore_index,
                                                     int32_t S, uint32_t align) {
    using RV = RawVec<T>;
    constexpr int VE = Vec16<T>::N;
    __shared__ float red[WG / 64];
    const int64_t row = blockIdx.x;
    const int32_t chunk = blockIdx.y;
    const T *zr = z + row * static_cast<int64_t>(V);
    const RowSplit sp = split_row(zr, V, align);
    int32_t v0, v1;
    chunk_range(sp.nvec, chunk, S, align, v0, v1);
    const RV *zv = reinterpret_cast<const RV *>(zr + sp.head);

    float m = -INFINITY, s = 0.f;
    // Scalar edges: the head with chunk 0, the tail with the last chunk.
    if (chunk == 0)
        for (int32_t j = threadIdx.x; j < sp.head; j += WG) ms_fold(m, s, to_f32(zr[j]), 1.f);
    if (chunk == S - 1)
        for (int32_t j = sp.tail + threadIdx.x; j < V; j += WG) ms_fold(m, s, to_f32(zr[j]), 1.f);

    // The loop is bound by VALU issue at fp16 (one exponential and a few operations per 2-byte
    // element), so the per-element work is kept small: idle vectors are replaced as raw bits,
    // the maximum is taken exactly in the storage type, and for fp16 the widening and the
    // subtraction of the maximum are one mixed-precision fma (x * 1 - vm, rounded once like the
    // plain subtraction; the 1 is hidden from the compiler, which would otherwise fold the fma
    // back into a widening and a subtraction).
    float one = 1.0f;
    if constexpr (VE == 8) asm("" : "+v"(one));
    // The next U vectors are fetched before the current ones are reduced, so a wave keeps
    // loads in flight through its exponentials.
    auto fetch = [&](RV (&dst)[U], int32_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t v = base + u * WG + threadIdx.x;
            const bool ok = v < v1;
            // Idle lanes read a vector of -inf: every load is unconditional, so no branch makes
            // the compiler wait for all loads in flight before the current vectors are reduced.
            const RV *src = ok ? zv + v : idle_vec<T>();
            dst[u] = load_stream_raw<T>(reinterpret_cast<const T *>(src));
        }
    };
    RV cur[U], nxt[U];
    if (v0 < v1) fetch(cur, v0);
    for (int32_t base = v0; base < v1; base += WG * U) {
        const bool more = base + WG * U < v1;
        if (more) fetch(nxt, base + WG * U);
        RV mv = cur[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mv = __builtin_elementwise_max(mv, cur[u]);
        const float vm = vec_max<T>(mv);
        if (vm != -INFINITY) {
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    acc += __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(cur[u][e]), one, -vm) * kLog2e);
            ms_fold(m, s, vm, acc);
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
    }

    const float M = row_allreduce<WG>(m, OpMax(), red);
    const float sc = (m == -INFINITY || M == -INFINITY) ? 0.f
                                                        : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
    const float Ssum = row_allreduce<WG>(sc, OpSum(), red);
    if (threadIdx.x != 0) return;
    if (S > 1) {
        part[(row * S + chunk) * 2 + 0] = M;
        part[(row * S + chunk) * 2 + 1] = Ssum;
        return;
    }
    const float logS = logf(Ssum);
    lse[row] = M + logS;
    const int64_t t = target[row];
    // loss = (M - z_t) + log S rather than lse - z_t: M and z_t are exact inputs, so their
    // difference rounds once, where lse - z_t would cancel two large numbers (|z| ~ 1e4).
    if (t == ignore_index)
        loss[row] = 0.f;
    else if (t < 0 || t >= V)
        loss[row] = NAN;
    else
        loss[row] = (M - to_f32(zr[t])) + logS;
}

// Combine the S chunk partials of each row in chunk order: M = max M_c, S = sum S_c *
// exp(M_c - M); then lse and loss. One thread per row.
template <typename T>
__global__ __launch_bounds__(256) void xent_fw_finish(float *__restrict__ loss,
                                                      float *__restrict__ lse,
                                                      const float *__restrict__ part, const T *z,
                                                      const int64_t *__restrict__ target,
                                                      int64_t N, int32_t V, int64_t ignore_index,
                                                      int32_t S) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (row >= N) return;
    const float *pr = part + row * S * 2;
    float M = -INFINITY;
    for (int32_t c = 0; c < S; ++c) M = fmaxf(M, pr[2 * c]);
    float Ssum = 0.f;
    if (M != -INFINITY)
        for (int32_t c = 0; c < S; ++c)
            if (pr[2 * c] != -INFINITY)
                Ssum += pr[2 * c + 1] * __builtin_amdgcn_exp2f((pr[2 * c] - M) * kLog2e);
    const float logS = logf(Ssum);
    lse[row] = M + logS;
    const int64_t t = target[row];
    if (t == ignore_index)
        loss[row] = 0.f;
    else if (t < 0 || t >= V)
        loss[row] = NAN;
    else
        loss[row] = (M - to_f32(z[row * static_cast<int64_t>(V) + t])) + logS;
}

// ------------------------------------------------------------------------------------------
// Backward: dz = g * (exp(z - lse) - onehot), g = dloss[row] * scale (dloss NULL: 1).
// Row blockIdx.x, chunk blockIdx.y of S. The row split follows dz's phase; the host passes an
// align for which z and dz rows share their phase (128, else 16, else 0).
// ------------------------------------------------------------------------------------------
template <typename T, int WG, int U>
__global__ __launch_bounds__(WG) void xent_bw_kernel(T *dz, const T *z,
                                                     const int64_t *__restrict__ target,
                                                     const float *__restrict__ lse,
                                                     const float *__restrict__ dloss, float scale,
                                                     int32_t V, int64_t ignore_index, int32_t S,
                                                     uint32_t align) {
    using RV = RawVec<T>;
    constexpr int VE = Vec16<T>::N;
    const int64_t row = blockIdx.x;
    const int32_t chunk = blockIdx.y;
    const int64_t rbase = row * static_cast<int64_t>(V);
    const T *zr = z + rbase;
    T *dr = dz + rbase;
    const RowSplit sp = split_row(static_cast<const T *>(dr), V, align);
    int32_t v0, v1;
    chunk_range(sp.nvec, chunk, S, align, v0, v1);

    const int64_t t = target[row];
    const bool ignored = t == ignore_index;
    const bool invalid = !ignored && (t < 0 || t >= V);
    // Ignored rows: gradient 0; invalid target: NaN. Both as a factor on every element.
    const float g = ignored ? 0.f : (invalid ? NAN : (dloss != nullptr ? dloss[row] : 1.f) * scale);
    const float l = lse[row];
    const int32_t tt = (ignored || invalid) ? -1 : static_cast<int32_t>(t);
    auto grad = [&](float zv, int32_t j) {
        const float p = __builtin_amdgcn_exp2f((zv - l) * kLog2e);
        return g * (j == tt ? p - 1.f : p);
    };

    if (chunk == 0)
        for (int32_t j = threadIdx.x; j < sp.head; j += WG) dr[j] = from_f32<T>(grad(to_f32(zr[j]), j));
    if (chunk == S - 1)
        for (int32_t j = sp.tail + threadIdx.x; j < V; j += WG) dr[j] = from_f32<T>(grad(to_f32(zr[j]), j));

    const RV *zv = reinterpret_cast<const RV *>(zr + sp.head);
    T *dv = dr + sp.head;
    for (int32_t base = v0; base < v1; base += WG * U) {
        RV raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t v = base + u * WG + threadIdx.x;
            raw[u] = load_stream_raw<T>(reinterpret_cast<const T *>(zv + (v < v1 ? v : v0)));
        }
        // Branch-free stores at device scope (one read stream, one write stream) through a
        // descriptor at the block's first vector: offsets stay below WG * U vectors, and a
        // lane past the chunk is dropped. Measured on MI355X against plain streaming stores
        // under a branch: -3.5% at [8192,32000] and [8192,50001] fp16, -7% at fp32, -6% at
        // [1024,32000] fp16.
        T *blk = dv + static_cast<int64_t>(base) * VE;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t v = base + u * WG + threadIdx.x;
            float x[VE], o[VE];
            widen<T>(raw[u], x);
            const int32_t j0 = sp.head + v * VE;
#pragma unroll
            for (int e = 0; e < VE; ++e) o[e] = grad(x[e], j0 + e);
            const uint32_t off = v < v1 ? static_cast<uint32_t>(v - base) * 16u : kDropOffset;
            store16_or_drop<kBufferDeviceStream>(blk, off, pack16<T>(o));
        }
    }
}

// ------------------------------------------------------------------------------------------
// Launch geometry.
// ------------------------------------------------------------------------------------------
// Workgroup size and vectors in flight per thread, measured on MI355X ([8192, 32000] and
// [8192, 50001] fp16): the forward is within 2% from 256x4 to 512x4 (84 us, 6.2 TB/s of
// reads); the backward gains 14-22% from 256x4 to 1024x2 (204 -> 179 us at V = 32000) and
// 1-2% more from 1024x2 to 1024x4 on whole rows (line-aligned; fp16 and fp32). Split rows
// ([64, 50001]: chunks of about 1000 vectors) stay at 1024x2, 3-5% faster than 1024x4 there.
constexpr int kXentFwWG = 512;
constexpr int kXentFwU = 4;
constexpr int kXentBwWG = 1024;
constexpr int kXentBwU = 4;       // whole rows (S == 1)
constexpr int kXentBwSplitU = 2;  // split rows (S > 1)
constexpr uint32_t kXentLine = 128;  // bytes: the row split's alignment
constexpr int64_t kXentTargetBlocks = 1024;  // split rows until about this many workgroups
// The forward splits rows only above this size: a split row needs a second kernel to combine
// its chunks, and that launch costs more than one workgroup takes to stream a shorter row.
// Measured on MI355X: one workgroup per row is faster at [64, 32000] fp16 (5.2 against 8.4 us),
// [256, 32000] (6.2 / 10.6), [64, 32000] fp32 (6.0 / 11.0) and still at [8, 128256] fp16
// (256 KB rows: 10.8 / 12.5). The backward has no second kernel and keeps splitting.
constexpr int64_t kXentFwSplitRowBytes = 256 << 10;

// Chunks per row: 1 when there are enough rows, else enough to reach kXentTargetBlocks
// workgroups while every chunk keeps at least one vector per thread (min_vectors = WG).
static int32_t xent_chunks(int64_t N, int64_t V, size_t es, int min_vectors) {
    if (N <= 0) return 1;
    if (N >= kXentTargetBlocks / 2) return 1;
    const int64_t nvec = static_cast<int64_t>(V) * static_cast<int64_t>(es) / 16;
    int64_t S = (kXentTargetBlocks + N - 1) / N;
    const int64_t maxS = nvec / min_vectors;
    if (S > maxS) S = maxS;
    if (S < 1) S = 1;
    if (S > 1024) S = 1024;
    return static_cast<int32_t>(S);
}

static bool xent_shape_ok(int64_t N, int64_t V) {
    return N >= 0 && N <= INT32_MAX && V >= 1 && V <= INT32_MAX / 2;
}

}  // namespace lnr

using namespace lnr;

static int32_t xent_fw_chunks(int64_t N, int64_t V, size_t es) {
    if (V * static_cast<int64_t>(es) <= kXentFwSplitRowBytes) return 1;
    return xent_chunks(N, V, es, kXentFwWG);
}

extern "C" size_t cross_entropy_fw_workspace_bytes(int64_t N, int64_t V, lnr_dtype dtype) {
    if (!valid_dtype(dtype) || !xent_shape_ok(N, V)) return 0;
    const int32_t S = xent_fw_chunks(N, V, dtype_size(dtype));
    return S > 1 ? static_cast<size_t>(N) * static_cast<size_t>(S) * 2 * sizeof(float) : 0;
}

extern "C" int cross_entropy_fw(float *loss, float *lse, const void *logits, const int64_t *target,
                                int64_t N, int64_t V, int64_t ignore_index, lnr_dtype dtype,
                                void *workspace, size_t workspace_bytes, void *stream) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (N < 0 || V < 1) return LNR_ERR_SHAPE;
    if (!xent_shape_ok(N, V)) return LNR_ERR_UNSUPPORTED;
    if (N == 0) return LNR_OK;
    if (loss == nullptr || lse == nullptr || logits == nullptr || target == nullptr)
        return LNR_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned_to(logits, es) || !aligned_to(loss, 4) || !aligned_to(lse, 4) ||
        !aligned_to(target, 8))
        return LNR_ERR_ALIGN;
    const size_t need = cross_entropy_fw_workspace_bytes(N, V, dtype);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LNR_ERR_WORKSPACE;
    if (need > 0 && !aligned_to(workspace, 8)) return LNR_ERR_ALIGN;
    const size_t zb = static_cast<size_t>(N) * static_cast<size_t>(V) * es;
    const size_t nb = static_cast<size_t>(N) * 4;
    if (overlap(loss, nb, lse, nb) || overlap(loss, nb, logits, zb) || overlap(lse, nb, logits, zb) ||
        overlap(loss, nb, target, N * 8) || overlap(lse, nb, target, N * 8) ||
        overlap(workspace, need, logits, zb) || overlap(workspace, need, loss, nb) ||
        overlap(workspace, need, lse, nb) || overlap(workspace, need, target, N * 8))
        return LNR_ERR_ALIAS;

    const int32_t S = xent_fw_chunks(N, V, es);
    const int32_t V32 = static_cast<int32_t>(V);
    float *part = static_cast<float *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<uint32_t>(N), static_cast<uint32_t>(S));
    hipError_t e;
    if (dtype == LNR_F16)
        e = launch(xent_fw_kernel<f16, kXentFwWG, kXentFwU>, grid, dim3(kXentFwWG), s, loss, lse,
                   part, static_cast<const f16 *>(logits), target, V32, ignore_index, S, kXentLine);
    else
        e = launch(xent_fw_kernel<float, kXentFwWG, kXentFwU>, grid, dim3(kXentFwWG), s, loss, lse,
                   part, static_cast<const float *>(logits), target, V32, ignore_index, S, kXentLine);
    if (e == hipSuccess && S > 1) {
        const dim3 g2(static_cast<uint32_t>((N + 255) / 256));
        if (dtype == LNR_F16)
            e = launch(xent_fw_finish<f16>, g2, dim3(256), s, loss, lse,
                       static_cast<const float *>(part), static_cast<const f16 *>(logits), target, N,
                       V32, ignore_index, S);
        else
            e = launch(xent_fw_finish<float>, g2, dim3(256), s, loss, lse,
                       static_cast<const float *>(part), static_cast<const float *>(logits), target,
                       N, V32, ignore_index, S);
    }
    return status_of(e);
}

extern "C" int cross_entropy_bw(void *dlogits, const void *logits, const int64_t *target,
                                const float *lse, const float *dloss, float scale, int64_t N,
                                int64_t V, int64_t ignore_index, lnr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (N < 0 || V < 1) return LNR_ERR_SHAPE;
    if (!xent_shape_ok(N, V)) return LNR_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return LNR_ERR_SHAPE;
    if (N == 0) return LNR_OK;
    if (dlogits == nullptr || logits == nullptr || target == nullptr || lse == nullptr)
        return LNR_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned_to(dlogits, es) || !aligned_to(logits, es) || !aligned_to(lse, 4) ||
        !aligned_to(dloss, 4) || !aligned_to(target, 8))
        return LNR_ERR_ALIGN;
    const size_t zb = static_cast<size_t>(N) * static_cast<size_t>(V) * es;
    const size_t nb = static_cast<size_t>(N) * 4;
    if (bad_alias(dlogits, logits, zb) || overlap(dlogits, zb, target, N * 8) ||
        overlap(dlogits, zb, lse, nb) || overlap(dlogits, zb, dloss, nb))
        return LNR_ERR_ALIAS;

    // Bandwidth needs enough workgroups: split rows as the forward does.
    const int32_t S = xent_chunks(N, V, es, kXentBwWG);
    // Vector part aligned to dz's lines where z shares that phase, else to 16 bytes, else none.
    const uintptr_t dphase = reinterpret_cast<uintptr_t>(dlogits) - reinterpret_cast<uintptr_t>(logits);
    const uint32_t align = (dphase & (kXentLine - 1)) == 0 ? kXentLine : (dphase & 15u) == 0 ? 16u : 0u;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<uint32_t>(N), static_cast<uint32_t>(S));
    const int32_t V32 = static_cast<int32_t>(V);
    auto go = [&](auto kernel, auto *dz, const auto *z) {
        return launch(kernel, grid, dim3(kXentBwWG), s, dz, z, target, lse, dloss, scale, V32,
                      ignore_index, S, align);
    };
    f16 *dh = static_cast<f16 *>(dlogits);
    const f16 *zh = static_cast<const f16 *>(logits);
    float *df = static_cast<float *>(dlogits);
    const float *zf = static_cast<const float *>(logits);
    hipError_t e;
    if (dtype == LNR_F16)
        e = S == 1 ? go(xent_bw_kernel<f16, kXentBwWG, kXentBwU>, dh, zh)
                   : go(xent_bw_kernel<f16, kXentBwWG, kXentBwSplitU>, dh, zh);
    else
        e = S == 1 ? go(xent_bw_kernel<float, kXentBwWG, kXentBwU>, df, zf)
                   : go(xent_bw_kernel<float, kXentBwWG, kXentBwSplitU>, df, zf);
    return status_of(e);
}
