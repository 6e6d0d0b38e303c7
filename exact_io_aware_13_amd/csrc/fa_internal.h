// fa_internal.h -- declarations shared by the library's sources (not part of the C ABI).
#ifndef FA_INTERNAL_H
#define FA_INTERNAL_H

#include <hip/hip_runtime_api.h>

namespace fa_internal {

// The calling thread's record of the last launch error, read by
// fa_hip_error_string().  Hidden: shared by the library's sources only.
__attribute__((visibility("hidden"))) void record_hip_error(hipError_t err);
__attribute__((visibility("hidden"))) void clear_hip_error();

}  // namespace fa_internal

#endif  // FA_INTERNAL_H
