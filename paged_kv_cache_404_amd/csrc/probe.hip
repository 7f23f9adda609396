// Streaming-read probe: the HBM read bandwidth a plain kernel achieves on this GPU, the yardstick
// beside the 8 TB/s nameplate for the decode kernel (which is bound by reading the cache).
//
// Every lane reads 16-byte words with nontemporal loads (the decode kernel's load form), eight per
// iteration, over a grid-stride walk of the buffer, and folds them with XOR.  The fold is written
// only when it equals a value no sane input produces, so the loads cannot be dropped and the
// kernel writes (almost) nothing: the measured traffic is reads.
#include "device.h"

namespace pkv {
namespace {

constexpr uint32_t kNever = 0x9E3779B9u;
constexpr int kUnroll = 8;  // loads in flight per lane (8 read faster than 4 or 16 on the MI355X)

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
  const uint32_t f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (f == kNever) sink[0] = f;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                       pkv_stream_t stream) {
  if (bytes == 0) return PKV_OK;
  if (!buf || !sink) return fail(PKV_EINVAL, "paged_probe_stream_read: NULL pointer");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(PKV_EINVAL, "paged_probe_stream_read: buffer and size must be multiples of 16 bytes");
  if (workgroups <= 0 || workgroups > 65536)
    return fail(PKV_EINVAL, "paged_probe_stream_read: workgroups %d outside [1, 65536]", workgroups);
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, as_stream(stream),
                     static_cast<const u32x4*>(buf), static_cast<int64_t>(bytes / 16), sink);
  return check_launch("paged_probe_stream_read");
}
