// Read-only HBM streaming probe for the benchmark (not part of libhsv): the
// bandwidth a plain stream of 16-byte loads reaches, against which the
// verification step's KV rate is also quoted.
//
//   hsv_probe_read(src, bytes, sink, stream)
//     src   device buffer of `bytes` bytes (16-byte aligned; bytes % 16 == 0)
//     sink  device buffer of at least hsv_probe_blocks() uint32 words; a word
//           is written only when a block's XOR of everything it read equals
//           a fixed constant, so the loads cannot be optimised away while
//           the writes add no traffic in practice
//   returns 0, or the hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 256 * 8;  // eight workgroups per CU
constexpr uint32_t kMagic = 0x9e3779b9u;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4 *__restrict__ src,
                                                              int64_t n16,
                                                              uint32_t *__restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride],
                d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == kMagic) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int hsv_probe_blocks() { return kBlocks; }

extern "C" int hsv_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(read_probe_kernel, dim3(kBlocks), dim3(kThreads), 0, stream,
                     static_cast<const uint4 *>(src), bytes / 16, sink);
  return static_cast<int>(hipGetLastError());
}
