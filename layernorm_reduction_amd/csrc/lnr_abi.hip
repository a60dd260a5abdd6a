// lnr_abi.hip -- status strings, build information and the streaming helpers (copy, and
// read-two-write-one) used to measure the achievable HBM ceiling that the row kernels are
// compared with.
#include "lnr_common.h"
#include "lnr_prims.h"

namespace lnr {

// Streaming copy with the same non-temporal 16-byte accesses as the row kernels. Shape: one
// vector per thread in 64-thread workgroups, the fastest of the shapes measured on MI355X (or
// within 1% of it) at every size from 4 MiB to 1 GiB, for the copy and the read-two-write-one
// stream alike: 4-25% less time than four vectors per thread in 256-thread workgroups, up to
// 8% less than one vector in 256-thread workgroups. The loops keep the shape a parameter.
constexpr int kCopyUnroll = 1;
constexpr int kCopyWG = 64;

__global__ __launch_bounds__(kCopyWG) void copy16(f32x4 *__restrict__ dst,
                                                   const f32x4 *__restrict__ src, int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyWG * kCopyUnroll + threadIdx.x;
    f32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kCopyWG;
        if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kCopyWG;
        if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Read two, write one (the access pattern of both backward kernels): dst = a XOR b, 16 bytes
// per access, the same one-shot grid and non-temporal policy as copy16.
__global__ __launch_bounds__(kCopyWG) void xor16(u32x4 *__restrict__ dst, const u32x4 *__restrict__ a,
                                                  const u32x4 *__restrict__ b, int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyWG * kCopyUnroll + threadIdx.x;
    u32x4 va[kCopyUnroll], vb[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kCopyWG;
        if (i < n) {
            va[u] = __builtin_nontemporal_load(a + i);
            vb[u] = __builtin_nontemporal_load(b + i);
        }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kCopyWG;
        if (i < n) __builtin_nontemporal_store(va[u] ^ vb[u], dst + i);
    }
}

}  // namespace lnr

using namespace lnr;

extern "C" int lnr_copy(void *dst, const void *src, size_t bytes, void *stream) {
    if (bytes == 0) return LNR_OK;
    if (dst == nullptr || src == nullptr) return LNR_ERR_NULL;
    if (bytes % 16 != 0) return LNR_ERR_SHAPE;
    if (!aligned_to(dst, 16) || !aligned_to(src, 16)) return LNR_ERR_ALIGN;
    if (overlap(dst, bytes, src, bytes)) return LNR_ERR_ALIAS;
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const int64_t per_block = static_cast<int64_t>(kCopyWG) * kCopyUnroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > INT32_MAX) return LNR_ERR_UNSUPPORTED;
    return status_of(launch(copy16, dim3(static_cast<uint32_t>(blocks)), dim3(kCopyWG),
                            static_cast<hipStream_t>(stream), static_cast<f32x4 *>(dst),
                            static_cast<const f32x4 *>(src), n));
}

extern "C" int lnr_xor2(void *dst, const void *a, const void *b, size_t bytes, void *stream) {
    if (bytes == 0) return LNR_OK;
    if (dst == nullptr || a == nullptr || b == nullptr) return LNR_ERR_NULL;
    if (bytes % 16 != 0) return LNR_ERR_SHAPE;
    if (!aligned_to(dst, 16) || !aligned_to(a, 16) || !aligned_to(b, 16)) return LNR_ERR_ALIGN;
    if (overlap(dst, bytes, a, bytes) || overlap(dst, bytes, b, bytes)) return LNR_ERR_ALIAS;
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const int64_t per_block = static_cast<int64_t>(kCopyWG) * kCopyUnroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > INT32_MAX) return LNR_ERR_UNSUPPORTED;
    return status_of(launch(xor16, dim3(static_cast<uint32_t>(blocks)), dim3(kCopyWG),
                            static_cast<hipStream_t>(stream), static_cast<u32x4 *>(dst),
                            static_cast<const u32x4 *>(a), static_cast<const u32x4 *>(b), n));
}

extern "C" int lnr_time_next_launch(void *start_event, void *stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return LNR_ERR_NULL;
    next_launch_events() = NextLaunchEvents{static_cast<hipEvent_t>(start_event),
                                            static_cast<hipEvent_t>(stop_event)};
    return LNR_OK;
}

extern "C" const char *lnr_strerror(int status) {
    switch (status) {
        case LNR_OK: return "success";
        case LNR_ERR_NULL: return "a required pointer is NULL";
        case LNR_ERR_SHAPE: return "invalid size (negative or zero where not allowed, or causal with Tq != Tk)";
        case LNR_ERR_UNSUPPORTED: return "row length or grid beyond the supported range";
        case LNR_ERR_DTYPE: return "dtype is not LNR_F32 or LNR_F16";
        case LNR_ERR_ALIGN: return "pointer not aligned to its element size, or workspace not to its stated alignment";
        case LNR_ERR_ALIAS: return "buffers overlap in a way the operation forbids";
        case LNR_ERR_WORKSPACE: return "workspace missing or smaller than the matching *_workspace_bytes()";
        case LNR_ERR_HIP: return "the HIP runtime rejected a kernel launch";
        case LNR_ERR_SCRATCH: return "the shape needs more than the library's fixed scratch array (LNR_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

extern "C" const char *lnr_build_info(void) {
    return "liblnr 0.1 gfx950 (wave64 DPP row reductions, 128-bit vector I/O)";
}
