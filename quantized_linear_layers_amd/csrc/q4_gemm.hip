// W4A16 GEMM for large M (prefill): Y = X · dequant(W)ᵀ on bf16/fp16 MFMA.
//
// Structure ([QK] §9.5 and the tiled pseudocode of [LQ]'s W4A16 section):
// each workgroup owns a BM x BN tile of Y and walks K one 128-wide group at
// a time; the X tile and the still-packed W tile are staged in LDS (double
// buffered, the next k-block's global loads in flight during the current
// block's MFMAs); each wave reads its packed codes from LDS, expands them to
// 16-bit floats in registers with the group's scale and zero point, and feeds
// v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation.  The scale and zero
// of a group are constant over a k-block, so they are loaded once per block.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int APAD = 8;                       // halves of padding per X row in LDS
constexpr int AROW = BK + APAD;               // LDS row length of the X tile (halves)
constexpr int A_TILE = BM * AROW;             // halves per X buffer
constexpr int B_TILE = (BK / kChunkK) * BN * 16;   // bytes per W buffer: [chunk][column] x 16 bytes

struct GemmArgs {
  const uint16_t* X;
  int M, K, N, Np, Kp;
  const uint4* W;
  const uint32_t* S;
  const uint8_t* Z;
  uint16_t* Y;
};

__device__ inline uint32_t pack2(float lo, float hi, bool bf16) {
  if (bf16) {
    const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)lo), b = __builtin_bit_cast(uint16_t, (__bf16)hi);
    return a | (b << 16);
  }
  const uint32_t a = __builtin_bit_cast(uint16_t, (_Float16)lo), b = __builtin_bit_cast(uint16_t, (_Float16)hi);
  return a | (b << 16);
}

// 8 codes of one word (k offsets 0..7, code of k = 2i at bits 4i, of k = 2i+1
// at bits 16 + 4i) -> 8 dequantized 16-bit values s * (q - z), as 4 pairs.
__device__ inline uint4 dequant8(uint32_t w, float s, float nzs, bool bf16) {
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = fmaf((float)((w >> (4 * i)) & 0xFu), s, nzs);
    const float hi = fmaf((float)((w >> (16 + 4 * i)) & 0xFu), s, nzs);
    r[i] = pack2(lo, hi, bf16);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

template <bool BF16>
__global__ __launch_bounds__(256) void q4_gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) uint16_t as[2][A_TILE];
  __shared__ __align__(16) uint8_t bs[2][B_TILE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ntn = (a.N + BN - 1) / BN;
  const int m0 = (blockIdx.x / ntn) * BM, n0 = (blockIdx.x % ntn) * BN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nkb = a.K / BK;

  // ---- global -> register staging of one k-block
  uint4 ra[8], rb[2];
  auto load_block = [&](int kb) {
    const int k0 = kb * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + i * 256;          // 0 .. 2047: 128 rows x 16 pieces of 8 halves
      const int r = idx >> 4, c = idx & 15;
      const int m = m0 + r;
      ra[i] = m < a.M ? *reinterpret_cast<const uint4*>(a.X + (size_t)m * a.K + k0 + c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + i * 256;          // 0 .. 511: 4 chunks x 128 columns
      const int c = idx >> 7, col = idx & 127;
      const int n = n0 + col;
      rb[i] = n < a.Np ? a.W[(size_t)(kb * 4 + c) * a.Np + n] : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + i * 256;
      const int r = idx >> 4, c = idx & 15;
      *reinterpret_cast<uint4*>(&as[buf][r * AROW + c * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(&bs[buf][(tid + i * 256) * 16]) = rb[i];
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  load_block(0);
  store_block(0);
  __syncthreads();

  const int half = lane >> 5, l32 = lane & 31;
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_block(kb + 1);

    // scale and zero of this group for the wave's two 32-column MFMA tiles
    float s[2], nzs[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n = n0 + wn + nt * 32 + l32;
      const int g = kb;
      float sv = 0.0f, zv = 0.0f;
      if (n < a.Np) {
        const uint32_t sp = a.S[(size_t)(g / 2) * a.Np + n];
        const uint32_t zp = a.Z[(size_t)(g / 2) * a.Np + n];
        sv = (float)__builtin_bit_cast(_Float16, (uint16_t)(sp >> (16 * (g & 1))));
        zv = (float)((zp >> (4 * (g & 1))) & 0xFu);
      }
      s[nt] = sv;
      nzs[nt] = -zv * sv;
    }

#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      uint4 af[2], bf[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[mt] = *reinterpret_cast<const uint4*>(&as[buf][(wm + mt * 32 + l32) * AROW + ks * 16 + half * 8]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int c = wn + nt * 32 + l32;            // column inside the workgroup tile
        const int chunk = ks >> 1, j = (ks & 1) * 2 + half;
        const uint32_t w = *reinterpret_cast<const uint32_t*>(&bs[buf][(chunk * BN + c) * 16 + j * 4]);
        bf[nt] = dequant8(w, s[nt], nzs[nt], BF16);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          if (BF16)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[mt]),
                                                                  __builtin_bit_cast(bf16x8, bf[nt]), acc[mt][nt], 0, 0, 0);
          else
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, af[mt]),
                                                                 __builtin_bit_cast(f16x8, bf[nt]), acc[mt][nt], 0, 0, 0);
        }
    }
    __syncthreads();
    if (kb + 1 < nkb) {
      store_block(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- store: acc element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n = n0 + wn + nt * 32 + l32;
      if (n >= a.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm + mt * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        if (m < a.M) {
          const float v = acc[mt][nt][e];
          a.Y[(size_t)m * a.N + n] =
              BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
        }
      }
    }
}

}  // namespace

hipError_t launch_q4_gemm(const void* X, bool bf16, int M, int K, int N, const uint8_t* blob, const Q4Layout& L,
                          void* Y, hipStream_t st) {
  GemmArgs a;
  a.X = static_cast<const uint16_t*>(X);
  a.M = M;
  a.K = K;
  a.N = N;
  a.Np = L.Np;
  a.Kp = L.Kp;
  a.W = reinterpret_cast<const uint4*>(blob + L.w_off);
  a.S = reinterpret_cast<const uint32_t*>(blob + L.s_off);
  a.Z = blob + L.z_off;
  a.Y = static_cast<uint16_t*>(Y);
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (bf16)
    hipLaunchKernelGGL(q4_gemm_kernel<true>, dim3(tiles), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(q4_gemm_kernel<false>, dim3(tiles), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ql
