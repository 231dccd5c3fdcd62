// Plain streaming read of a device buffer: the HBM read rate that any kernel
// reading the same bytes can reach on this part, measured beside the decode
// kernel.  Batch-1 decode is bound by reading every weight once per token
// ([QK] §9.1: the per-token time is at least the weight bytes over the memory
// bandwidth; [LQ] "带宽与算力：Roofline"), so the decode kernel is judged
// against the published peak and against this achieved read rate.
//
// Two access patterns (the faster one is the ceiling; which one wins depends
// on the size): mode 0, every thread reads 16-byte pieces at a grid stride
// (consecutive lanes read consecutive pieces, a wave one contiguous kilobyte
// per load); mode 1, every workgroup reads one contiguous chunk of
// bytes / workgroups in kilobyte-per-wave steps.  Either way each thread has
// kUnroll loads in flight before their values are used, and the loads are
// non-temporal (a streamed buffer is not worth keeping in the caches).  The
// values are folded with XOR and each wave writes one word, so the loads
// cannot be dropped and the writes are negligible.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t fold(const u32x4* p) {
  const u32x4 v = __builtin_nontemporal_load(p);
  return v.x ^ v.y ^ v.z ^ v.w;
}

// reads pieces [b, e) of src, thread `t` of `nt` starting at b + t with stride nt
__device__ inline uint32_t read_range(const u32x4* __restrict__ src, uint64_t b, uint64_t e, uint64_t t,
                                      uint64_t nt) {
  uint32_t acc = 0;
  uint64_t i = b + t;
  for (; i + (kUnroll - 1) * nt < e; i += kUnroll * nt) {
    uint32_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = fold(src + i + u * nt);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < e; i += nt) acc ^= fold(src + i);
  return acc;
}

// The arguments (with the grid's size, nwg = gridDim.x) are preloaded into
// scalar registers at wave launch, as for the decode kernel, so that both
// start streaming after the same latency.
template <bool CHUNK>
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                              uint32_t nwg, uint32_t* __restrict__ sink) {
  uint32_t acc;
  if constexpr (CHUNK) {
    const uint64_t per = (n16 + nwg - 1) / nwg;
    const uint64_t b = min((uint64_t)blockIdx.x * per, n16), e = min(b + per, n16);
    acc = read_range(src, b, e, threadIdx.x, kThreads);
  } else {
    acc = read_range(src, 0, n16, (uint64_t)blockIdx.x * kThreads + threadIdx.x, (uint64_t)nwg * kThreads);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

int read_probe_sink_words(int workgroups) { return workgroups * (kThreads / 64); }

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups, int mode,
                             hipStream_t st) {
  const u32x4* s = static_cast<const u32x4*>(src);
  if (mode == 1)
    hipLaunchKernelGGL(read_probe_kernel<true>, dim3(workgroups), dim3(kThreads), 0, st, s, (uint64_t)(bytes / 16),
                       (uint32_t)workgroups, sink);
  else
    hipLaunchKernelGGL(read_probe_kernel<false>, dim3(workgroups), dim3(kThreads), 0, st, s, (uint64_t)(bytes / 16),
                       (uint32_t)workgroups, sink);
  return hipGetLastError();
}

}  // namespace ql
