// lnr_abi.hip -- status strings, build information and the streaming-copy helper used to
// measure the achievable HBM ceiling that the row kernels are compared with.
#include "lnr_common.h"
#include "lnr_prims.h"

namespace lnr {

// Grid-stride copy with the same 16-byte accesses as the row kernels.
__global__ __launch_bounds__(256) void copy16(f32x4 *__restrict__ dst,
                                               const f32x4 *__restrict__ src, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
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
    // 8 workgroups of 256 threads per CU on 256 CUs, each thread looping over the rest.
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    return status_of(launch(copy16, dim3(static_cast<uint32_t>(blocks)), dim3(256),
                            static_cast<hipStream_t>(stream), static_cast<f32x4 *>(dst),
                            static_cast<const f32x4 *>(src), n));
}

extern "C" const char *lnr_strerror(int status) {
    switch (status) {
        case LNR_OK: return "success";
        case LNR_ERR_NULL: return "a required pointer is NULL";
        case LNR_ERR_SHAPE: return "invalid size (negative or zero where not allowed, or causal with Tq != Tk)";
        case LNR_ERR_UNSUPPORTED: return "row length or grid beyond the supported range";
        case LNR_ERR_DTYPE: return "dtype is not LNR_F32 or LNR_F16";
        case LNR_ERR_ALIGN: return "pointer not aligned to its element size";
        case LNR_ERR_ALIAS: return "buffers overlap in a way the operation forbids";
        case LNR_ERR_WORKSPACE: return "workspace missing or smaller than layernorm_bw_workspace_bytes()";
        case LNR_ERR_HIP: return "the HIP runtime rejected a kernel launch";
        default: return "unknown status";
    }
}

extern "C" const char *lnr_build_info(void) {
    return "liblnr 0.1 gfx950 (wave64 DPP row reductions, 128-bit vector I/O)";
}
