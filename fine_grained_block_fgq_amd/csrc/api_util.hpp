// api_util.hpp -- host-side argument checks shared by the C entry points of libfgq and of
// the measurement library libfgq_calib (internal; both map HIP launch errors the same way).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fgq.h"

namespace fgq_api {

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges, empty ranges never overlap)
inline bool overlap(const void* a, int64_t na, const void* b, int64_t nb)
{
    if (na <= 0 || nb <= 0)
        return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// a grid beyond the dispatch's 32-bit work-item count is refused before launch: a shape error
inline int launch_status(hipError_t e)
{
    return e == hipSuccess                      ? FGQ_OK
           : e == hipErrorInvalidConfiguration ? FGQ_ERR_SHAPE
                                                : FGQ_ERR_LAUNCH;
}

}  // namespace fgq_api
