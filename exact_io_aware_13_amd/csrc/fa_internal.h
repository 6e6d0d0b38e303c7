// fa_internal.h -- declarations shared by the library's sources (not part of the C ABI).
#ifndef FA_INTERNAL_H
#define FA_INTERNAL_H

#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace fa_internal {

// The calling thread's record of the last launch error, read by
// fa_hip_error_string().  Hidden: shared by the library's sources only.
__attribute__((visibility("hidden"))) void record_hip_error(hipError_t err);
__attribute__((visibility("hidden"))) void clear_hip_error();

// Enqueues the merge of n_split partial results (op: fp32 [n_split][rows][d],
// lp: fp32 [n_split][rows], each split's normalised output and log-sum-exp)
// into o (bf16 [rows][d]) and lse (fp32 [rows]) on `stream`; d is 64 or 128.
// Returns the launch status.  Used by every split forward of the library.
__attribute__((visibility("hidden"))) hipError_t launch_split_combine(const float* op, const float* lp, uint16_t* o,
                                                                      float* lse, long long rows, int n_split, int d,
                                                                      hipStream_t stream);

}  // namespace fa_internal

#endif  // FA_INTERNAL_H
