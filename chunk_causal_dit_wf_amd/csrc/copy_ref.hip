// Reference copy for bandwidth measurement (not part of the attention path).
//
// A plain device-to-device copy in the shape that moves a few tens of MB
// fastest on gfx950: a persistent grid of 2048 blocks of 256 threads that
// strides over the buffer, each thread moving four 16-byte vectors per step
// with nontemporal loads and stores (every byte is touched once).  The append
// of one layer's chunk moves about that many bytes; this kernel's rate is
// what a single launch of that size can reach, launch and ramp included.
#include "copy_ref.h"

namespace wf {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyVec = 4;        // 16-byte vectors per thread per step
constexpr int kCopyBlocks = 2048;  // 8 per CU

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst, int64_t n16) {
  const int64_t step = (int64_t)gridDim.x * kCopyThreads * kCopyVec;
  for (int64_t b = (int64_t)blockIdx.x * kCopyThreads * kCopyVec + threadIdx.x; b < n16; b += step) {
    u32x4 r[kCopyVec];
#pragma unroll
    for (int i = 0; i < kCopyVec; ++i) {
      const int64_t j = b + (int64_t)kCopyThreads * i;
      if (j < n16) r[i] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int i = 0; i < kCopyVec; ++i) {
      const int64_t j = b + (int64_t)kCopyThreads * i;
      if (j < n16) __builtin_nontemporal_store(r[i], dst + j);
    }
  }
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, hipStream_t s) {
  const int64_t per_block = (int64_t)kCopyThreads * kCopyVec;
  const int64_t need = (n16 + per_block - 1) / per_block;
  const dim3 grid((uint32_t)(need < kCopyBlocks ? need : kCopyBlocks));
  hipLaunchKernelGGL(stream_copy_kernel, grid, dim3(kCopyThreads), 0, s, (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace wf
