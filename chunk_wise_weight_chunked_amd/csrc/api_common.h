// api_common.h -- helpers shared by the C ABI's source files: the calling
// thread's error message, descriptor validation and buffer range checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ttt_mlp.h"
#include "layer.h"

namespace ttt {
namespace api {

// Records the message for ttt_last_error() and returns `code`.
ttt_status_t fail(ttt_status_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message and returns TTT_OK.
ttt_status_t ok();
// TTT_ERR_HIP with the HIP error's text.
ttt_status_t hip_fail(hipError_t e, const char* what);

// Validates a descriptor and derives the call's shapes.
ttt_status_t make_dims(const ttt_mlp_desc_t* desc, Dims* dm);

// A named byte range [lo, hi) of a buffer, for overlap checks.
struct Range {
  const char* name;
  uintptr_t lo, hi;
};
Range range(const char* name, const void* p, size_t bytes);
bool overlaps(const Range& x, const Range& y);
bool aligned(const void* p, size_t a);

}  // namespace api
}  // namespace ttt
