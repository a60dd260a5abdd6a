// lnr_common.h -- host-side helpers shared by the C-ABI entry points: argument checks and a
// kernel launcher that returns the launch's own status (no reliance on hipGetLastError,
// which could report an unrelated earlier error of the caller).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "lnr.h"

namespace lnr {

inline bool valid_dtype(lnr_dtype d) { return d == LNR_F32 || d == LNR_F16; }
inline size_t dtype_size(lnr_dtype d) { return d == LNR_F16 ? 2 : 4; }

inline bool aligned_to(const void *p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Byte ranges [a, a+na) and [b, b+nb) share at least one byte.
inline bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (na == 0 || nb == 0 || a == nullptr || b == nullptr) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// A buffer may be used in place (same start, same length) but may not partially overlap.
inline bool bad_alias(const void *out, const void *in, size_t n) {
    return out != in && overlap(out, n, in, n);
}

// Measurement hook (lnr_time_next_launch): events that the next launch made by this thread
// records at its kernel's own start and end. Cleared by that launch.
struct NextLaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
inline NextLaunchEvents &next_launch_events() {
    static thread_local NextLaunchEvents ev;
    return ev;
}

// Launch `kernel` with argument values converted to its exact parameter types and return
// the status of this launch.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         Args &&...args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
    std::tuple<KArgs...> values(static_cast<KArgs>(std::forward<Args>(args))...);
    void *argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    std::apply([&](auto &...v) {
        int i = 0;
        ((argv[i++] = static_cast<void *>(&v)), ...);
    }, values);
    NextLaunchEvents &ev = next_launch_events();
    if (ev.start != nullptr) {
        const hipEvent_t a = ev.start, b = ev.stop;
        ev = NextLaunchEvents{};
        return hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, 0,
                                  stream, a, b, 0);
    }
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, 0, stream);
}

inline int status_of(hipError_t e) { return e == hipSuccess ? LNR_OK : LNR_ERR_HIP; }

}  // namespace lnr
