// status.h -- status helpers shared by the C ABI sources (api.hip,
// moe_api.hip).  The text of the last failure is per host thread and is what
// flint_last_error() returns.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/flint.h"

namespace flint::abi {

// Workspace parts start on this alignment.
constexpr size_t kWsAlign = 256;

// Record the formatted message as the last error and return st.
flint_status fail(flint_status st, const char* fmt, ...);
// Clear the last error and return FLINT_OK.
flint_status ok();
// FLINT_OK for hipSuccess, else FLINT_ERR_HIP with the HIP error text.
flint_status hip_status(hipError_t e, const char* what);
bool aligned(const void* p, size_t a);
size_t align_up(size_t x);  // to kWsAlign
// Do the byte ranges [a, a+na) and [b, b+nb) intersect?
bool overlap(const void* a, size_t na, const void* b, size_t nb);

}  // namespace flint::abi
