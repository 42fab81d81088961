// wf_history_rotate kernel: rotate a window of page-table entries left by
// one chunk, in place.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §3.1:
// the per-layer context keeps a bounded clean history (oldest first) and the
// live store after it.  When a round completes a chunk the store becomes the
// newest history chunk and the oldest one leaves.  With chunks on page
// boundaries that is a permutation of the logical pages of the window: the
// K/V pages stay where they are and only the table changes.
//
// The window is at most a few hundred entries in practice (a history of a
// few chunks of tens of pages), so one workgroup reads all of it into LDS,
// then writes it back rotated: every read precedes every write, which makes
// the in-place update safe without a second buffer.
#include "wf_rotate.h"

namespace wf {
namespace {

constexpr int kThreads = 1024;

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void rotate_kernel(int32_t* __restrict__ table, int first, int n, int shift) {
  __shared__ int32_t win[kMaxRotatePages];
  for (int i = threadIdx.x; i < n; i += kThreads) win[i] = table[first + i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kThreads) {
    int src = i + shift;
    if (src >= n) src -= n;
    table[first + i] = win[src];
  }
}

}  // namespace

hipError_t launch_rotate(int32_t* table, int first, int n, int shift, hipStream_t stream) {
  hipLaunchKernelGGL(rotate_kernel, dim3(1), dim3(kThreads), 0, stream, table, first, n, shift);
  return hipGetLastError();
}

}  // namespace wf
