// Launch of the history-rotation kernel (rotate.hip), used by api.cpp.
#pragma once
#include <cstdint>

#include <hip/hip_runtime.h>

namespace wf {

// largest window the single-workgroup kernel rotates (entries held in LDS)
constexpr int kMaxRotatePages = 16384;

// rotate the n table entries from `first` left by `shift`, in place
// (0 < shift < n <= kMaxRotatePages), stream-ordered
hipError_t launch_rotate(int32_t* table, int first, int n, int shift, hipStream_t stream);

}  // namespace wf
