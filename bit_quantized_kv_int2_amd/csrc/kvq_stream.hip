// Streaming-read reference kernel: reads a buffer once with 128-bit
// non-temporal loads (as the decode kernels stream their codes). It is the
// practical HBM read ceiling that the decode rates are compared against
// (same byte count, no arithmetic beyond an XOR per word).
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per thread per step: 32 KB per work-group

// Work-group g reads the contiguous range [g * per, (g + 1) * per) of 16-byte
// words, 32 KB per step, the way the decode kernels stream their splits.
__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const u4* __restrict__ p, size_t n16,
                                                                     size_t per, uint32_t* sink) {
  const size_t g = __builtin_amdgcn_workgroup_id_x();
  const int tid = __builtin_amdgcn_workitem_id_x();
  const size_t beg = g * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  size_t i = beg;
  for (; i + kStreamUnroll * kStreamThreads <= end; i += kStreamUnroll * kStreamThreads) {
    u4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kStreamThreads + tid);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (size_t j = i + tid; j < end; j += kStreamThreads) {
    const u4 v = p[j];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // keeps the loads alive; true only if the XOR hits this one value
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  // 4 work-groups per CU on 256 CUs (fewer for small buffers), each a
  // contiguous range of whole 32 KB steps
  const size_t step = (size_t)kStreamUnroll * kStreamThreads;
  size_t blocks = (n16 + step - 1) / step;
  if (blocks > 1024) blocks = 1024;
  const size_t per = ((n16 + blocks - 1) / blocks + step - 1) / step * step;
  blocks = (n16 + per - 1) / per;
  stream_read_kernel<<<dim3((unsigned)blocks), dim3(kStreamThreads), 0, s>>>((const u4*)data, n16, per, sink);
  return hipGetLastError();
}

}  // namespace kvq

