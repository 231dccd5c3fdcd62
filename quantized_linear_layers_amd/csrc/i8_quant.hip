// Dynamic per-token int8 (and FP8 E4M3) activation quantization: one
// workgroup per row.
//
// The row's range is found with one reduction ([LQ] "校准：静态与动态":
// per-token absmax/range at run time costs one extra reduction), then the
// scale, the int32 zero point and the codes follow the formulas in qlinear.h
// with IEEE fp32 division and round-half-to-even, so every code is decided
// exactly as a scalar CPU implementation of the same steps decides it.
// The row is read from HBM once: up to 8 pieces of 8 values per thread stay
// in registers between the reduction and the quantization.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int kThreads = 256;
constexpr int kRegPieces = 8;     // 8 x 8 values per thread kept in registers (K <= 16384)

__device__ inline float half_lo(uint32_t v, bool bf16) {
  return bf16 ? __builtin_bit_cast(float, v << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ inline float half_hi(uint32_t v, bool bf16) {
  return bf16 ? __builtin_bit_cast(float, v & 0xFFFF0000u) : (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// FP8: symmetric, s = max(absmax, 1e-5) / 448 and the code is the E4M3
// rounding of x / s (the largest code maps to the row absmax)
template <bool BF16, bool ASYM, bool FP8 = false>
__global__ __launch_bounds__(kThreads) void i8_quant_kernel(const uint16_t* __restrict__ X, int K,
                                                             int8_t* __restrict__ Aq, float* __restrict__ s_a,
                                                             int32_t* __restrict__ azp) {
  __shared__ float red[2][kThreads / 64];
  const int m = blockIdx.x, tid = threadIdx.x;
  const uint16_t* x = X + (size_t)m * K;
  const int pieces = K / 8;

  uint4 v[kRegPieces];
  float mn = 0.0f, mx = 0.0f;       // the range always contains 0
  auto fold = [&](uint4 p) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = half_lo(w[i], BF16), b = half_hi(w[i], BF16);
      if (ASYM) {
        mn = fminf(mn, fminf(a, b));
        mx = fmaxf(mx, fmaxf(a, b));
      } else {
        mx = fmaxf(mx, fmaxf(fabsf(a), fabsf(b)));
      }
    }
  };
#pragma unroll
  for (int r = 0; r < kRegPieces; ++r) {
    const int p = tid + r * kThreads;
    v[r] = p < pieces ? reinterpret_cast<const uint4*>(x)[p] : make_uint4(0, 0, 0, 0);
    if (p < pieces) fold(v[r]);
  }
  for (int p = tid + kRegPieces * kThreads; p < pieces; p += kThreads) fold(reinterpret_cast<const uint4*>(x)[p]);

  // ---- row reduction: wave shuffles, then across the four waves
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = mn;
    red[1][tid >> 6] = mx;
  }
  __syncthreads();
  mn = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
  mx = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));

  float s, z;
  if (ASYM) {
    s = fmaxf(mx - mn, 1e-5f) / 255.0f;
    z = -128.0f - rintf(mn / s);
  } else {
    s = fmaxf(mx, 1e-5f) / (FP8 ? 448.0f : 127.0f);
    z = 0.0f;
  }
  if (tid == 0) {
    s_a[m] = s;
    if (ASYM) azp[m] = (int32_t)z;
  }
  const float lo = ASYM ? -128.0f : -127.0f;

  auto quant = [&](uint4 p) -> uint2 {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (FP8) {
        const uint32_t qa = e4m3_code(half_lo(w[i], BF16) / s), qb = e4m3_code(half_hi(w[i], BF16) / s);
        out[i >> 1] |= (qa | (qb << 8)) << (16 * (i & 1));
        continue;
      }
      const float a = fminf(fmaxf(rintf(half_lo(w[i], BF16) / s) + z, lo), 127.0f);
      const float b = fminf(fmaxf(rintf(half_hi(w[i], BF16) / s) + z, lo), 127.0f);
      const uint32_t qa = (uint32_t)(int32_t)a & 0xFFu, qb = (uint32_t)(int32_t)b & 0xFFu;
      out[i >> 1] |= (qa | (qb << 8)) << (16 * (i & 1));
    }
    return make_uint2(out[0], out[1]);
  };
  uint2* q = reinterpret_cast<uint2*>(Aq + (size_t)m * K);
#pragma unroll
  for (int r = 0; r < kRegPieces; ++r) {
    const int p = tid + r * kThreads;
    if (p < pieces) q[p] = quant(v[r]);
  }
  for (int p = tid + kRegPieces * kThreads; p < pieces; p += kThreads) q[p] = quant(reinterpret_cast<const uint4*>(x)[p]);
}

// RMSNorm fused with the per-token quantization (one workgroup per row):
// the row is normalized and quantized in the same pass over it, so the
// normalized activations never leave the compute unit ([QK] §9.9: fuse the
// per-row reduction of the activation quantization with the operator that
// produces the activations; [LQ] "校准：静态与动态": the dynamic per-token
// reduction is folded into RMSNorm's kernel).  Per row, in this order:
//   ms  = fp32( (sum of x^2 in fp64) / K in fp64 )   (the squares are exact)
//   inv = 1 / sqrt(ms + eps)                          (two correctly rounded fp32 steps)
//   y   = (x * inv) * gamma                           (fp32, never rounded to 16 bits)
// then the range of y, its scale / zero point and codes exactly as above.
template <bool BF16, bool ASYM>
__global__ __launch_bounds__(kThreads) void rmsnorm_quant_kernel(const uint16_t* __restrict__ X,
                                                                  const uint16_t* __restrict__ gamma, float eps, int K,
                                                                  int8_t* __restrict__ Aq, float* __restrict__ s_a,
                                                                  int32_t* __restrict__ azp) {
  __shared__ double dred[kThreads / 64];
  __shared__ float red[2][kThreads / 64];
  const int m = blockIdx.x, tid = threadIdx.x;
  const uint16_t* x = X + (size_t)m * K;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const uint4* gv = reinterpret_cast<const uint4*>(gamma);
  const int pieces = K / 8;

  // ---- mean square: fp64 sum of the exact squares
  uint4 v[kRegPieces], g[kRegPieces];
  double ss = 0.0;
  auto sq = [&](uint4 p) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = half_lo(w[i], BF16), b = half_hi(w[i], BF16);
      ss += a * a;
      ss += b * b;
    }
  };
#pragma unroll
  for (int r = 0; r < kRegPieces; ++r) {
    const int p = tid + r * kThreads;
    v[r] = p < pieces ? xv[p] : make_uint4(0, 0, 0, 0);
    g[r] = p < pieces ? gv[p] : make_uint4(0, 0, 0, 0);
    if (p < pieces) sq(v[r]);
  }
  for (int p = tid + kRegPieces * kThreads; p < pieces; p += kThreads) sq(xv[p]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((tid & 63) == 0) dred[tid >> 6] = ss;
  __syncthreads();
  ss = (dred[0] + dred[1]) + (dred[2] + dred[3]);
  const float ms = (float)(ss / (double)K);
  const float inv = 1.0f / sqrtf(ms + eps);

  // ---- y and its range
  auto norm = [&](uint32_t xw, uint32_t gw, float& a, float& b) {
    a = (half_lo(xw, BF16) * inv) * half_lo(gw, BF16);
    b = (half_hi(xw, BF16) * inv) * half_hi(gw, BF16);
  };
  float mn = 0.0f, mx = 0.0f;       // the range always contains 0
  auto fold = [&](uint4 p, uint4 q) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w}, u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a, b;
      norm(w[i], u[i], a, b);
      if (ASYM) {
        mn = fminf(mn, fminf(a, b));
        mx = fmaxf(mx, fmaxf(a, b));
      } else {
        mx = fmaxf(mx, fmaxf(fabsf(a), fabsf(b)));
      }
    }
  };
#pragma unroll
  for (int r = 0; r < kRegPieces; ++r)
    if (tid + r * kThreads < pieces) fold(v[r], g[r]);
  for (int p = tid + kRegPieces * kThreads; p < pieces; p += kThreads) fold(xv[p], gv[p]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = mn;
    red[1][tid >> 6] = mx;
  }
  __syncthreads();
  mn = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
  mx = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));

  float s, z;
  if (ASYM) {
    s = fmaxf(mx - mn, 1e-5f) / 255.0f;
    z = -128.0f - rintf(mn / s);
  } else {
    s = fmaxf(mx, 1e-5f) / 127.0f;
    z = 0.0f;
  }
  if (tid == 0) {
    s_a[m] = s;
    if (ASYM) azp[m] = (int32_t)z;
  }
  const float lo = ASYM ? -128.0f : -127.0f;

  auto quant = [&](uint4 p, uint4 q) -> uint2 {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w}, u[4] = {q.x, q.y, q.z, q.w};
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float ya, yb;
      norm(w[i], u[i], ya, yb);
      const float a = fminf(fmaxf(rintf(ya / s) + z, lo), 127.0f);
      const float b = fminf(fmaxf(rintf(yb / s) + z, lo), 127.0f);
      const uint32_t qa = (uint32_t)(int32_t)a & 0xFFu, qb = (uint32_t)(int32_t)b & 0xFFu;
      out[i >> 1] |= (qa | (qb << 8)) << (16 * (i & 1));
    }
    return make_uint2(out[0], out[1]);
  };
  uint2* q = reinterpret_cast<uint2*>(Aq + (size_t)m * K);
#pragma unroll
  for (int r = 0; r < kRegPieces; ++r) {
    const int p = tid + r * kThreads;
    if (p < pieces) q[p] = quant(v[r], g[r]);
  }
  for (int p = tid + kRegPieces * kThreads; p < pieces; p += kThreads) q[p] = quant(xv[p], gv[p]);
}

}  // namespace

hipError_t launch_rmsnorm_quant(const void* X, bool bf16, int M, int K, const void* gamma, float eps, int8_t* Aq,
                                float* s_a, int32_t* azp, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* g = static_cast<const uint16_t*>(gamma);
  if (bf16) {
    if (azp)
      hipLaunchKernelGGL((rmsnorm_quant_kernel<true, true>), dim3(M), dim3(kThreads), 0, st, x, g, eps, K, Aq, s_a, azp);
    else
      hipLaunchKernelGGL((rmsnorm_quant_kernel<true, false>), dim3(M), dim3(kThreads), 0, st, x, g, eps, K, Aq, s_a, azp);
  } else {
    if (azp)
      hipLaunchKernelGGL((rmsnorm_quant_kernel<false, true>), dim3(M), dim3(kThreads), 0, st, x, g, eps, K, Aq, s_a, azp);
    else
      hipLaunchKernelGGL((rmsnorm_quant_kernel<false, false>), dim3(M), dim3(kThreads), 0, st, x, g, eps, K, Aq, s_a,
                         azp);
  }
  return hipGetLastError();
}

hipError_t launch_i8_quant(const void* X, bool bf16, int M, int K, int8_t* Aq, float* s_a, int32_t* azp,
                           hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (bf16) {
    if (azp) hipLaunchKernelGGL((i8_quant_kernel<true, true>), dim3(M), dim3(kThreads), 0, st, x, K, Aq, s_a, azp);
    else hipLaunchKernelGGL((i8_quant_kernel<true, false>), dim3(M), dim3(kThreads), 0, st, x, K, Aq, s_a, azp);
  } else {
    if (azp) hipLaunchKernelGGL((i8_quant_kernel<false, true>), dim3(M), dim3(kThreads), 0, st, x, K, Aq, s_a, azp);
    else hipLaunchKernelGGL((i8_quant_kernel<false, false>), dim3(M), dim3(kThreads), 0, st, x, K, Aq, s_a, azp);
  }
  return hipGetLastError();
}

hipError_t launch_f8_quant(const void* X, bool bf16, int M, int K, uint8_t* Aq, float* s_a, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  int8_t* q = reinterpret_cast<int8_t*>(Aq);
  if (bf16)
    hipLaunchKernelGGL((i8_quant_kernel<true, false, true>), dim3(M), dim3(kThreads), 0, st, x, K, q, s_a, nullptr);
  else
    hipLaunchKernelGGL((i8_quant_kernel<false, false, true>), dim3(M), dim3(kThreads), 0, st, x, K, q, s_a, nullptr);
  return hipGetLastError();
}

}  // namespace ql
