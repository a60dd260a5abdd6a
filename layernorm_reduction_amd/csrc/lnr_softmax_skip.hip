// lnr_softmax_skip.hip -- attention softmax forward and backward that read only the score
// vectors holding at least one key the row may attend to.
//
// Method: "CMU 11-868 HW4: Softmax and LayerNorm as fused CUDA kernels", section "Problem
// structure and scoring" (future tokens set to -inf, the attention mask added, then the row max
// and the sum of exponentials), and "FastTransformer: Breaking the Compiler Ceiling via
// Architectural Co-Design", section 3 "The Surprising Bottleneck" (the materialised
// probability tensor's HBM traffic is the attention cost). A key after the query (causal) or
// under a -inf mask entry contributes exp(-inf) = 0 to the row sum and has probability
// exactly 0. So a 16-byte vector whose keys are all such keys need not be read:
//   * forward: its scores are taken as -inf without a load, and its zeros are written;
//   * backward: y is 0 there, so dx = y * (dy - t) = 0 and neither y nor dy is read.
// Everything else is the dense kernels' arithmetic in the same order, so for finite scores
// (forward) and for y = 0 with finite dy at the skipped keys (backward) the results equal the
// dense entry points' (up to the sign of zero). Rows keep the dense layout: G lanes of one
// wave hold a row, vector k of lane l covers elements [(k*G + l)*V, +V). Skipping is per
// lane, and a row's skipped vectors form whole tails of 16-byte runs (causal) or the padded
// tail (key-padding masks), so whole cache lines are never fetched.
//
// The causal limit is an index test. The mask test needs the mask vector first: it is read
// through the caches (one [B, Tk] row serves all H*Tq rows of a batch), and the score load
// waits for it. The score loads are buffer loads through a descriptor based at the row of the
// wave's first row group: a skipped vector's lane passes an offset beyond the descriptor's
// range and reads zeros without touching memory. So every load of a row is issued at once,
// with no branch: with a branch around each load, the compiler waited for each load (or pair
// of loads) in turn.
#include <math.h>

#include <type_traits>

#include "lnr_common.h"
#include "lnr_fastdiv.h"
#include "lnr_prims.h"

namespace lnr {

constexpr int64_t kSkipMaxRows = int64_t{UINT32_MAX} - 4096;

// True when some element of the mask vector is not -inf (the vector has a key to read).
template <typename T>
__device__ __forceinline__ bool any_open(const RawVec<T> &m) {
    bool open = false;
#pragma unroll
    for (int e = 0; e < Vec16<T>::N; ++e) open |= static_cast<float>(m[e]) != -INFINITY;
    return open;
}

template <typename T>
__device__ __forceinline__ RawVec<T> splat(float v) {
    RawVec<T> r;
#pragma unroll
    for (int e = 0; e < Vec16<T>::N; ++e) r[e] = static_cast<T>(v);
    return r;
}

// need[k] &= the mask vector k of the row has an open key; the mask vectors come back in m.
// Mask reads hit the caches, so they are issued for every k (a lane with nothing to read
// loads the row's first vector, which always exists) and the result is selected afterwards.
template <typename T, int G, int IT>
__device__ __forceinline__ void mask_runs(const T *mrow, int lane, bool (&need)[IT],
                                          RawVec<T> (&m)[IT]) {
    constexpr int V = Vec16<T>::N;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const RawVec<T> l = load_keep_raw<T>(mrow + (need[k] ? static_cast<int64_t>(k * G + lane) * V : 0));
        m[k] = need[k] ? l : splat<T>(-INFINITY);
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) need[k] = need[k] && any_open<T>(m[k]);
}

template <typename T, int G, int IT, int WG>
__global__ __launch_bounds__(WG) void softmax_fw_skip(T *out, const T *inp,
                                                      const T *__restrict__ mask, uint32_t rows,
                                                      int32_t Tk, DivU32 per_batch,
                                                      DivU32 per_query, int32_t causal) {
    constexpr int V = Vec16<T>::N;
    constexpr int RPB = WG / G;
    const int lane = threadIdx.x % G;
    const uint32_t row = blockIdx.x * static_cast<uint32_t>(RPB) + threadIdx.x / G;
    const bool live = row < rows;
    const uint32_t r = live ? row : 0u;
    const int nvec = Tk / V;
    // Keys [0, kend) may be attended to: all of them, or 0..query index when causal (Tq = Tk).
    const int qi = static_cast<int>(r - divu32(r, per_query) * per_query.d);
    const int kend = causal ? qi + 1 : Tk;

    bool need[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        need[k] = live && c < nvec && c * V < kend;
    }
    RawVec<T> m[IT];
    if (mask != nullptr)
        mask_runs<T, G, IT>(mask + static_cast<int64_t>(divu32(r, per_batch)) * Tk, lane, need, m);
    else
#pragma unroll
        for (int k = 0; k < IT; ++k) m[k] = splat<T>(0.f);
    // The wave's row base (its first row group's row; rows of one wave are consecutive).
    const uint32_t wrow = __builtin_amdgcn_readfirstlane(r);
    RawVec<T> xr[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const uint32_t off = need[k] ? static_cast<uint32_t>(((r - wrow) * static_cast<int64_t>(Tk) +
                                                              static_cast<int64_t>(k * G + lane) * V) *
                                                             static_cast<int64_t>(sizeof(T)))
                                     : kDropOffset;
        xr[k] = load16_or_zero<T>(inp + static_cast<int64_t>(wrow) * Tk, off);
    }
    // Skipped vectors take -inf (they read zeros). At fp16 the widening and the mask add are
    // one mixed-precision fma, as in the dense kernel (x * 1 + m, both exact in fp32, rounded
    // once like the plain sum); the mask of a skipped vector is -inf or 0, so -inf stays.
    float one = 1.0f;
    if constexpr (V == 8) asm("" : "+v"(one));
    float z[IT][V];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        xr[k] = need[k] ? xr[k] : splat<T>(-INFINITY);
#pragma unroll
        for (int e = 0; e < V; ++e)
            z[k][e] = __builtin_fmaf(static_cast<float>(xr[k][e]), one, static_cast<float>(m[k][e]));
    }
    if (causal) {
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
    const float inv = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;

    // Every vector of the row is written (zeros at skipped keys), as in the dense forward:
    // branch-free stores at device scope from the wave's row base, idle lanes dropped.
    // Measured on MI355X against stores under a branch with the plain streaming policy:
    // -3% at 32-64 keys, -0.6% at [64,16,512,512], +0.3 to +0.8% on long causal rows (the
    // same branch-free stores without device scope were slower everywhere).
    T *wave_out = out + static_cast<int64_t>(wrow) * Tk;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        float y[V];
#pragma unroll
        for (int e = 0; e < V; ++e) y[e] = z[k][e] * inv;
        const uint32_t off = (live && c < nvec)
                                 ? ((r - wrow) * static_cast<uint32_t>(Tk) + static_cast<uint32_t>(c * V)) *
                                       static_cast<uint32_t>(sizeof(T))
                                 : kDropOffset;
        store16_or_drop<kBufferDeviceStream>(wave_out, off, pack16<T>(y));
    }
}

template <typename T, int G, int IT, int WG>
__global__ __launch_bounds__(WG) void softmax_bw_skip(T *dinp, const T *dout,
                                                      const T *__restrict__ y,
                                                      const T *__restrict__ mask, uint32_t rows,
                                                      int32_t Tk, DivU32 per_batch,
                                                      DivU32 per_query, int32_t causal) {
    constexpr int V = Vec16<T>::N;
    constexpr int RPB = WG / G;
    const int lane = threadIdx.x % G;
    const uint32_t row = blockIdx.x * static_cast<uint32_t>(RPB) + threadIdx.x / G;
    const bool live = row < rows;
    const uint32_t r = live ? row : 0u;
    const int nvec = Tk / V;
    const int64_t base = static_cast<int64_t>(r) * Tk;
    const int kend = causal ? static_cast<int>(r - divu32(r, per_query) * per_query.d) + 1 : Tk;

    bool need[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int c = k * G + lane;
        need[k] = live && c < nvec && c * V < kend;
    }
    if (mask != nullptr) {
        RawVec<T> m[IT];
        mask_runs<T, G, IT>(mask + static_cast<int64_t>(divu32(r, per_batch)) * Tk, lane, need, m);
    }
    // Skipped vectors read zeros (y = 0 and dy = 0 give dx = 0) without touching memory.
    const uint32_t wrow = __builtin_amdgcn_readfirstlane(r);
    RawVec<T> yr[IT], gr[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const uint32_t off = need[k] ? static_cast<uint32_t>(((r - wrow) * static_cast<int64_t>(Tk) +
                                                              static_cast<int64_t>(k * G + lane) * V) *
                                                             static_cast<int64_t>(sizeof(T)))
                                     : kDropOffset;
        yr[k] = load16_or_zero<T>(y + static_cast<int64_t>(wrow) * Tk, off);
        gr[k] = load16_or_zero<T>(dout + static_cast<int64_t>(wrow) * Tk, off);
    }
    float yv[IT][V], gv[IT][V];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        widen<T>(yr[k], yv[k]);
        widen<T>(gr[k], gv[k]);
    }
    // The dense kernel's product sum is a chain of fused multiply-adds. With the fp16 widening
    // next to the multiply, the compiler would pair two products of widened fp16 values into
    // a dot2 instruction, which rounds differently (measured: results then differ from the
    // dense kernel's in the last bit). An empty register constraint hides the widened values
    // from that combine; it emits no instruction.
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
// Row-length buckets (G lanes per row, IT vectors per lane), the HW4 page's template list.
// Measured on MI355X (old and new library alternating in one process): 64-thread workgroups
// at fp16 32-64 and 256-1024 keys in the forward and 32-512 in the backward (forward -2 to -6%,
// backward -2 to -13%, the most on the 32 MiB GPT-2 shape), fp32 128, 256 and 1024 keys in
// the forward (-2 to -6%) and 256 in the backward (-3%), and fp32 512 keys in the forward once
// its stores became branch-free at device scope (-1.2%); they lose or tie at 2048 keys
// (+2-5%) and in the fp16 1024-key backward (+3%).
// ------------------------------------------------------------------------------------------
struct SkipPlan {
    int bucket;
    int G;
    int IT;
    int WG;
};

template <typename T> struct SkipFwTable;
template <> struct SkipFwTable<f16> {
    static constexpr SkipPlan plans[] = {{32, 4, 1, 64},   {64, 8, 1, 64},   {128, 8, 2, 256},
                                         {256, 8, 4, 64},   {384, 16, 3, 256}, {512, 32, 2, 64},
                                         {768, 32, 3, 256}, {1024, 32, 4, 64}, {2048, 64, 4, 256}};
};
template <> struct SkipFwTable<float> {
    static constexpr SkipPlan plans[] = {{32, 8, 1, 256},   {64, 16, 1, 256},  {128, 8, 4, 64},
                                         {256, 16, 4, 64},  {384, 32, 3, 256}, {512, 32, 4, 64},
                                         {768, 64, 3, 256}, {1024, 64, 4, 64},  {2048, 64, 8, 256}};
};
template <typename T> struct SkipBwTable;
template <> struct SkipBwTable<f16> {
    static constexpr SkipPlan plans[] = {{32, 4, 1, 64},   {64, 8, 1, 64},   {128, 16, 1, 64},
                                         {256, 32, 1, 64},  {384, 16, 3, 256}, {512, 64, 1, 64},
                                         {768, 32, 3, 256}, {1024, 64, 2, 128}, {2048, 64, 4, 128}};
};
template <> struct SkipBwTable<float> {
    static constexpr SkipPlan plans[] = {{32, 8, 1, 256},   {64, 16, 1, 256},  {128, 32, 1, 256},
                                         {256, 64, 1, 64},  {384, 32, 3, 256}, {512, 64, 2, 128},
                                         {768, 64, 3, 128}, {1024, 64, 4, 128}, {2048, 64, 8, 128}};
};

struct SkipArgs {
    void *out;         // fw: y;    bw: dinp
    const void *a;     // fw: inp;  bw: dout
    const void *b;     // fw: -;    bw: y
    const void *mask;  // [B, Tk] or null
    int64_t rows;
    int32_t Tq, Tk;
    int64_t rows_per_batch;
    int32_t causal;
};

template <typename T, int I, bool BW>
static hipError_t dispatch_skip(const SkipArgs &a, hipStream_t st) {
    using Table = std::conditional_t<BW, SkipBwTable<T>, SkipFwTable<T>>;
    constexpr SkipPlan p = Table::plans[I];
    if (a.Tk <= p.bucket) {
        constexpr int RPB = p.WG / p.G;
        const dim3 grid(static_cast<uint32_t>((a.rows + RPB - 1) / RPB));
        const DivU32 pb = make_divu32(static_cast<uint32_t>(a.rows_per_batch));
        const DivU32 pq = make_divu32(static_cast<uint32_t>(a.Tq));
        if constexpr (BW)
            return launch(softmax_bw_skip<T, p.G, p.IT, p.WG>, grid, dim3(p.WG), st,
                          static_cast<T *>(a.out), static_cast<const T *>(a.a),
                          static_cast<const T *>(a.b), static_cast<const T *>(a.mask),
                          static_cast<uint32_t>(a.rows), a.Tk, pb, pq, a.causal);
        else
            return launch(softmax_fw_skip<T, p.G, p.IT, p.WG>, grid, dim3(p.WG), st,
                          static_cast<T *>(a.out), static_cast<const T *>(a.a),
                          static_cast<const T *>(a.mask), static_cast<uint32_t>(a.rows), a.Tk, pb,
                          pq, a.causal);
    }
    if constexpr (I + 1 < static_cast<int>(sizeof(Table::plans) / sizeof(SkipPlan)))
        return dispatch_skip<T, I + 1, BW>(a, st);
    return hipErrorInvalidValue;
}

// Shape, dtype, null, alignment and alias checks shared by both entry points (the same rules
// as attn_softmax_fw / attn_softmax_bw, plus the mask against the output). The forward passes
// b = a (its one input, which out may equal); the backward's out must not overlap b (y).
static int check_skip(void *out, const void *a, const void *b, const void *mask, int64_t B,
                      int64_t H, int64_t Tq, int64_t Tk, int causal, lnr_dtype dtype, bool bw) {
    if (!valid_dtype(dtype)) return LNR_ERR_DTYPE;
    if (B < 0 || H < 0 || Tq < 0 || Tk < 1) return LNR_ERR_SHAPE;
    if (Tk > LNR_SOFTMAX_MAX_TK || Tq > INT32_MAX) return LNR_ERR_UNSUPPORTED;
    if (H > 0 && Tq > 0 && B > INT64_MAX / H / Tq) return LNR_ERR_UNSUPPORTED;
    if (causal && Tq != Tk) return LNR_ERR_SHAPE;
    const int64_t rows = B * H * Tq;
    if (rows == 0) return LNR_OK;
    if (out == nullptr || a == nullptr || b == nullptr) return LNR_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned_to(out, es) || !aligned_to(a, es) || !aligned_to(b, es) ||
        (mask != nullptr && !aligned_to(mask, es)))
        return LNR_ERR_ALIGN;
    const size_t nbytes = static_cast<size_t>(rows) * static_cast<size_t>(Tk) * es;
    if (bad_alias(out, a, nbytes)) return LNR_ERR_ALIAS;
    if (bw && overlap(out, nbytes, b, nbytes)) return LNR_ERR_ALIAS;
    if (mask != nullptr && overlap(out, nbytes, mask, static_cast<size_t>(B * Tk) * es))
        return LNR_ERR_ALIAS;
    return LNR_OK;
}

static bool skip_vec_ok(const void *out, const void *a, const void *b, const void *mask,
                        int64_t rows, int64_t Tk, lnr_dtype dtype) {
    return (static_cast<size_t>(Tk) * dtype_size(dtype)) % 16 == 0 && aligned_to(out, 16) &&
           aligned_to(a, 16) && aligned_to(b, 16) && (mask == nullptr || aligned_to(mask, 16)) &&
           rows <= kSkipMaxRows;
}

}  // namespace lnr

using namespace lnr;

// Plan introspection for lnr_softmax_plan (which = 2 and 3); Tk of whole 16-byte vectors.
void skip_plan_of(int64_t Tk, lnr_dtype dtype, bool backward, int &bucket, int &G, int &IT) {
    SkipPlan p{0, 64, 0, 0};
    auto find = [&](const auto &plans) {
        for (const SkipPlan &q : plans)
            if (Tk <= q.bucket) {
                p = q;
                return;
            }
    };
    if (dtype == LNR_F16)
        backward ? find(SkipBwTable<f16>::plans) : find(SkipFwTable<f16>::plans);
    else
        backward ? find(SkipBwTable<float>::plans) : find(SkipFwTable<float>::plans);
    bucket = p.bucket;
    G = p.G;
    IT = p.IT;
}

extern "C" int attn_softmax_fw_skip(void *out, const void *inp, const void *mask, int64_t B,
                                    int64_t H, int64_t Tq, int64_t Tk, int causal,
                                    lnr_dtype dtype, void *stream) {
    const int st = check_skip(out, inp, inp, mask, B, H, Tq, Tk, causal, dtype, false);
    if (st != LNR_OK) return st;
    const int64_t rows = B * H * Tq;
    if (rows == 0) return LNR_OK;
    if (!skip_vec_ok(out, inp, inp, mask, rows, Tk, dtype))
        return attn_softmax_fw(out, inp, mask, B, H, Tq, Tk, causal, dtype, stream);
    const SkipArgs a{out, inp, nullptr, mask, rows, static_cast<int32_t>(Tq), static_cast<int32_t>(Tk),
                     H * Tq, causal ? 1 : 0};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return status_of(dtype == LNR_F16 ? dispatch_skip<f16, 0, false>(a, s)
                                      : dispatch_skip<float, 0, false>(a, s));
}

extern "C" int attn_softmax_bw_skip(void *dinp, const void *dout, const void *out_fw,
                                    const void *mask, int64_t B, int64_t H, int64_t Tq,
                                    int64_t Tk, int causal, lnr_dtype dtype, void *stream) {
    const int st = check_skip(dinp, dout, out_fw, mask, B, H, Tq, Tk, causal, dtype, true);
    if (st != LNR_OK) return st;
    const int64_t rows = B * H * Tq;
    if (rows == 0) return LNR_OK;
    if (!skip_vec_ok(dinp, dout, out_fw, mask, rows, Tk, dtype))
        return attn_softmax_bw(dinp, dout, out_fw, B, H, Tq, Tk, dtype, stream);
    const SkipArgs a{dinp, dout, out_fw, mask, rows, static_cast<int32_t>(Tq),
                     static_cast<int32_t>(Tk), H * Tq, causal ? 1 : 0};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return status_of(dtype == LNR_F16 ? dispatch_skip<f16, 0, true>(a, s)
                                      : dispatch_skip<float, 0, true>(a, s));
}
