// Launcher of the reference streaming copy (copy_ref.hip), a measurement aid
// outside the attention path.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "../../include/wf_stream_copy.h"

namespace wf {
// Plain streaming copy of n16 16-byte vectors from src to dst (n16 > 0).
hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, hipStream_t s);
}  // namespace wf
