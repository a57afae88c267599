// mk_probe.hip -- the streaming-read probe: how fast this chip can read a
// large buffer once.  A decode step at batch 1 is a single pass over the
// weights, so this rate (not the 8 TB/s HBM figure) is the practical ceiling
// of the step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"

namespace {

typedef unsigned u4p __attribute__((ext_vector_type(4)));

#ifndef MK_PROBE_BLOCKS
#define MK_PROBE_BLOCKS 4096
#endif
#ifndef MK_PROBE_UNROLL
#define MK_PROBE_UNROLL 8
#endif
#ifndef MK_PROBE_NT
#define MK_PROBE_NT 1
#endif
constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = MK_PROBE_BLOCKS;  // 16 per CU on 256 CUs
constexpr int kUnroll = MK_PROBE_UNROLL;       // 128-bit loads in flight per thread

__device__ __forceinline__ u4p ld16(const u4p *p) {
#if MK_PROBE_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Grid-stride pass over n16 16-byte words: each thread keeps kUnroll loads
// in flight and folds what it read into one word, stored to its sink slot so
// that the loads stay.
__global__ void __launch_bounds__(kProbeThreads) stream_read(const u4p *__restrict__ p, size_t n16,
                                                             uint32_t *__restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u4p v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = ld16(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u4p v = ld16(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = acc;
}

}  // namespace

extern "C" {

size_t mk_stream_read_sink_words(void) { return (size_t)kProbeBlocks * kProbeThreads; }

int mk_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes == 0 || (bytes & 15) != 0 || ((uintptr_t)buf & 15) != 0) return MK_ERR_INVALID_ARG;
  hipLaunchKernelGGL(stream_read, dim3(kProbeBlocks), dim3(kProbeThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const u4p *>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_ERR_HIP;
}

}  // extern "C"
