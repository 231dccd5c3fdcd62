// Act-order activations: Xp[m][j] = X[m][perm[j]].
//
// With act-order ([LQ] GPTQ section, "工程细节": channels quantized in
// decreasing activation energy, g_idx giving each input channel's group),
// the groups are no longer runs of K, so reading a channel's scale becomes a
// scattered access.  The packed blob is therefore stored in processing order
// (q4_pack_act_order), where every group is again a run of 128 channels, and
// the activations are brought into the same order once per call: then
// Y = Xp · Wpᵀ = X · Wᵀ, and both W4A16 kernels run unchanged.
//
// A thread writes 8 consecutive columns (one 16-byte store) gathered from the
// row; the row is read from the L2 / L1 after its first touch.  Indices are
// clamped into [0, K), so a malformed permutation gives wrong values, never an
// out-of-bounds read.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void permute_cols_kernel(const uint16_t* __restrict__ X,
                                                                const int32_t* __restrict__ perm, int K,
                                                                uint16_t* __restrict__ Xp) {
  const int m = blockIdx.y;
  const int j0 = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (j0 >= K) return;
  const uint16_t* x = X + (size_t)m * K;
  const int4 p0 = *reinterpret_cast<const int4*>(perm + j0);
  const int4 p1 = *reinterpret_cast<const int4*>(perm + j0 + 4);
  const int idx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = x[min(max(idx[2 * i], 0), K - 1)];
    const uint32_t hi = x[min(max(idx[2 * i + 1], 0), K - 1)];
    w[i] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(Xp + (size_t)m * K + j0) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

hipError_t launch_permute_cols(const void* X, int M, int K, const int32_t* perm, void* Xp, hipStream_t st) {
  const dim3 grid((K / 8 + kThreads - 1) / kThreads, M);
  hipLaunchKernelGGL(permute_cols_kernel, grid, dim3(kThreads), 0, st, static_cast<const uint16_t*>(X), perm, K,
                     static_cast<uint16_t*>(Xp));
  return hipGetLastError();
}

}  // namespace ql
