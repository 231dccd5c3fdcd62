// W8A8 GEMM: int8 x int8 -> int32 on v_mfma_i32_32x32x32_i8, with the scale
// and zero-point epilogue applied to the accumulators in registers before
// the single store of the output ([VE] "一、背景": fusing it into the GEMM's
// epilogue avoids writing and re-reading the int32 result; [VE] "2.4": the
// per-token zero point is a rank-1 correction azp[m] * azp_adj[n], applied
// element-wise with O(M + N) extra memory).
//
// Each workgroup owns a BM x BN tile; both operands are [rows][K] int8
// (Aq row-major, Bq one row per output channel), staged through LDS with the
// next k-block's global loads in flight during the current block's MFMAs.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int ROW = BK + 16;            // LDS row length in bytes (16 bytes of padding)
constexpr int TILE = BM * ROW;

struct I8Args {
  const int8_t* A;
  const int8_t* B;
  int M, N, K;
  I8Epi e;
};

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void i8_gemm_kernel(I8Args a) {
  __shared__ __align__(16) int8_t as[2][TILE];
  __shared__ __align__(16) int8_t bs[2][TILE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ntn = (a.N + BN - 1) / BN;
  const int m0 = (blockIdx.x / ntn) * BM, n0 = (blockIdx.x % ntn) * BN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nkb = (a.K + BK - 1) / BK;

  uint4 ra[2], rb[2];
  auto load_block = [&](int kb) {
    const int k0 = kb * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + i * 256;        // 0 .. 511: 128 rows x 4 pieces of 16 bytes
      const int r = idx >> 2, c = idx & 3;
      const int k = k0 + c * 16;
      const int m = m0 + r, n = n0 + r;
      ra[i] = (m < a.M && k < a.K) ? *reinterpret_cast<const uint4*>(a.A + (size_t)m * a.K + k) : make_uint4(0, 0, 0, 0);
      rb[i] = (n < a.N && k < a.K) ? *reinterpret_cast<const uint4*>(a.B + (size_t)n * a.K + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + i * 256;
      const int r = idx >> 2, c = idx & 3;
      *reinterpret_cast<uint4*>(&as[buf][r * ROW + c * 16]) = ra[i];
      *reinterpret_cast<uint4*>(&bs[buf][r * ROW + c * 16]) = rb[i];
    }
  };

  i32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  load_block(0);
  store_block(0);
  __syncthreads();
  const int half = lane >> 5, l32 = lane & 31;
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_block(kb + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      // operand layout of the 32x32x32 int8 MFMA: lane l supplies row/column l%32,
      // k = 16 * (l / 32) .. +16 of the 32-wide k step
      uint4 af[2], bf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const uint4*>(&as[buf][(wm + t * 32 + l32) * ROW + ks * 32 + half * 16]);
        bf[t] = *reinterpret_cast<const uint4*>(&bs[buf][(wn + t * 32 + l32) * ROW + ks * 32 + half * 16]);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, af[mt]),
                                                              __builtin_bit_cast(i32x4, bf[nt]), acc[mt][nt], 0, 0, 0);
    }
    __syncthreads();
    if (kb + 1 < nkb) {
      store_block(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- fused epilogue: C = Dq - azp*azp_adj (int32), out = s_a * (s_b * C) + bias
  const I8Epi& e = a.e;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = n0 + wn + nt * 32 + l32;
    if (n >= a.N) continue;
    const float sb = e.s_b[e.s_b_vec ? n : 0];
    const int32_t adj = e.azp_adj ? e.azp_adj[n] : 0;
    float bias = 0.0f;
    if (e.bias) {
      const uint16_t bb = static_cast<const uint16_t*>(e.bias)[n];
      bias = OUT_BF16 ? __builtin_bit_cast(float, (uint32_t)bb << 16) : (float)__builtin_bit_cast(_Float16, bb);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        const int m = m0 + wm + mt * 32 + 8 * (el >> 2) + 4 * half + (el & 3);
        if (m >= a.M) continue;
        int32_t c = acc[mt][nt][el];
        if (e.azp) c -= e.azp[m] * adj;
        else c -= adj;
        if (e.raw) e.raw[(size_t)m * a.N + n] = c;
        const float sa = e.s_a[e.s_a_vec ? m : 0];
        const float v = sa * (sb * (float)c) + bias;
        static_cast<uint16_t*>(e.out)[(size_t)m * a.N + n] =
            OUT_BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
  }
}

}  // namespace

hipError_t launch_i8_gemm(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e, hipStream_t st) {
  I8Args a{A, B, M, N, K, e};
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (e.out_bf16)
    hipLaunchKernelGGL(i8_gemm_kernel<true>, dim3(tiles), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(i8_gemm_kernel<false>, dim3(tiles), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ql
