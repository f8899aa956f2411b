// Read-only streaming kernel: the measured HBM read ceiling that the decode
// path's bandwidth is reported against (a plain sequential read of a buffer
// far larger than the 256 MB Infinity Cache, every byte once).
//
// 2048 workgroups of 256 threads stride over the buffer in 16-byte
// non-temporal loads (the cache-streaming hint) and fold what they read into
// one word, which is stored only if it equals an arbitrary constant, so the
// loads cannot be removed and nothing is written in practice.
#include "hq_common.h"

namespace hq {
namespace {

constexpr int kStreamBlocks = 2048;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, uint64_t n16,
                                                           uint32_t *__restrict__ sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 *v = reinterpret_cast<const u32x4 *>(p);
  uint32_t acc = 0;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 256u;
#pragma unroll 4
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256u + threadIdx.x; i < n16; i += stride) {
    const u32x4 x = __builtin_nontemporal_load(v + i);
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace
}  // namespace hq

using namespace hq;

extern "C" size_t hq_stream_read_sink_bytes(void) { return static_cast<size_t>(kStreamBlocks) * 256 * 4; }

extern "C" hq_status hq_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
  if (!buf || !sink) return fail(HQ_ERR_INVALID_ARG, "hq_stream_read: null pointer");
  if (bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
    return fail(HQ_ERR_INVALID_ARG, "hq_stream_read: buffer and size must be 16-byte aligned");
  if (bytes == 0) { clear_error(); return HQ_OK; }
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamBlocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4 *>(buf), static_cast<uint64_t>(bytes / 16), sink);
  return check_launch("hq_stream_read");
}
