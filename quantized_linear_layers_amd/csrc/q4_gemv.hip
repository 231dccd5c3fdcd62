// W4A16 decode kernel (M <= 16): Y[m][n] = sum_k X[m][k] * s * (q - z).
//
// The step that dominates decode is streaming the packed weights from HBM
// once per token ([QK] §9.1: batch-1 decode reads every weight once; [LQ]
// "带宽与算力：Roofline": at a few tokens the arithmetic intensity is about
// the token count, far below the ridge).  So this kernel is built around the
// weight stream:
//   * lane l of a wave owns output channel 64t + l of layout tile t and reads
//     its 32 consecutive k as one 16-byte load; 64 lanes read 1 KB
//     contiguous, and consecutive workgroups walk consecutive memory;
//   * the codes are expanded in registers ([QK] §9.5, §9.6): a nibble ORed
//     into the low mantissa bits of fp16 1024.0 (0x6400) or bf16 128.0
//     (0x4300) is the exact number 1024 + q (128 + q) with one AND-OR per
//     pair of weights; for fp16 the mask 0x00F000F0 gives 1024 + 16q for the
//     next pair without a shift;
//   * the offsets and the zero point are not subtracted per weight: per group
//     the kernel accumulates sum x*(off + q) with packed dot products and
//     removes (off + z) * sum x once per group (the zero-point expansion of
//     [LQ] W8A8 section / [VE] "二", applied per group), then applies the
//     group scale, so the inner loop is one AND-OR plus one dot2 per pair;
//   * X of the workgroup's K range is staged once in LDS and read as
//     broadcast (every lane reads the same address); per-(row, group) sums
//     of X are formed while staging;
//   * the four waves of a workgroup split the K range and reduce in LDS;
//     workgroups split K further and the last one to arrive on a column
//     tile adds the fp32 partials in split order (deterministic) and stores Y.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

struct GemvArgs {
  const uint16_t* X;
  int M, K, N, Np, Kp;
  const uint4* W;          // [Np/64][Kp/32][64] chunks
  const uint32_t* S;       // [Np/64][Kp/256][64] scale pairs
  const uint8_t* Z;        // [Np/64][Kp/256][64] zero pairs
  int kw;                  // K per wave (multiple of 256)
  int splits;              // workgroups along K per tile
  float* part;             // [splits][M][Np]
  unsigned* cnt;           // [Np/64]
  uint16_t* Y;             // [M][N]
};

__device__ inline float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
}
__device__ inline float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ inline float lo_f(uint32_t v, bool bf16) {
  return bf16 ? __builtin_bit_cast(float, v << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ inline float hi_f(uint32_t v, bool bf16) {
  return bf16 ? __builtin_bit_cast(float, v & 0xFFFF0000u) : (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ inline uint16_t to_out(float y, bool bf16) {
  return bf16 ? __builtin_bit_cast(uint16_t, (__bf16)y) : __builtin_bit_cast(uint16_t, (_Float16)y);
}

template <int MT, bool BF16>
__device__ inline void group_dot(const uint4 (&w)[4], const uint16_t* xs, int xstride, int xk, float (&acc_a)[MT],
                                 float (&acc_b)[MT]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t ww[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = ww[j];
      uint32_t p0, p1, p2, p3;
      if (BF16) {
        p0 = (v & 0x000F000Fu) | 0x43004300u;
        p1 = ((v >> 4) & 0x000F000Fu) | 0x43004300u;
        p2 = ((v >> 8) & 0x000F000Fu) | 0x43004300u;
        p3 = ((v >> 12) & 0x000F000Fu) | 0x43004300u;
      } else {
        const uint32_t v8 = v >> 8;
        p0 = (v & 0x000F000Fu) | 0x64006400u;    // k 0,1  -> 1024 + q
        p1 = (v & 0x00F000F0u) | 0x64006400u;    // k 2,3  -> 1024 + 16 q
        p2 = (v8 & 0x000F000Fu) | 0x64006400u;   // k 4,5  -> 1024 + q
        p3 = (v8 & 0x00F000F0u) | 0x64006400u;   // k 6,7  -> 1024 + 16 q
      }
      const int k = xk + c * 32 + j * 8;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4 x = *reinterpret_cast<const uint4*>(xs + m * xstride + k);
        if (BF16) {
          acc_a[m] = dot2_bf16(x.x, p0, acc_a[m]);
          acc_a[m] = dot2_bf16(x.y, p1, acc_a[m]);
          acc_a[m] = dot2_bf16(x.z, p2, acc_a[m]);
          acc_a[m] = dot2_bf16(x.w, p3, acc_a[m]);
        } else {
          acc_a[m] = dot2_f16(x.x, p0, acc_a[m]);
          acc_b[m] = dot2_f16(x.y, p1, acc_b[m]);
          acc_a[m] = dot2_f16(x.z, p2, acc_a[m]);
          acc_b[m] = dot2_f16(x.w, p3, acc_b[m]);
        }
      }
    }
  }
}

template <int MT, bool BF16>
__global__ __launch_bounds__(256) void q4_gemv_kernel(GemvArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int kwg = 4 * a.kw;                 // K range of the workgroup
  const int ngw = kwg / kGroup;             // groups of the workgroup
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                      // [MT][kwg]
  float* csum = reinterpret_cast<float*>(smem + (size_t)MT * kwg * 2);    // [MT][ngw][2]
  float* red = csum + MT * ngw * 2;                                        // [4][MT][64]

  const int tile = blockIdx.x / a.splits;
  const int split = blockIdx.x % a.splits;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kb = split * kwg;
  const int kend = min(kb + kwg, a.Kp);
  const int k0 = kb + wave * a.kw;
  const int npairs = max(0, (min(k0 + a.kw, kend) - k0) / kPairK);

  // ---- issue the first weight loads before anything else (latency hiding)
  const int ck = a.Kp / kChunkK, pk = a.Kp / kPairK;
  const uint4* wp = a.W + ((size_t)tile * ck + k0 / kChunkK) * kTileN + lane;
  const uint32_t* sp = a.S + ((size_t)tile * pk + k0 / kPairK) * kTileN + lane;
  const uint8_t* zp = a.Z + ((size_t)tile * pk + k0 / kPairK) * kTileN + lane;
  uint4 bufA[8], bufB[8];
  uint32_t sA = 0, sB = 0, zA = 0, zB = 0;
  if (npairs > 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c) bufA[c] = wp[c * kTileN];
    sA = sp[0];
    zA = zp[0];
  }

  // ---- stage X[0:MT][kb:kb+kwg] in LDS and form per-(row, group) sums
  {
    const int per_row = kwg / 8;                 // 16-byte pieces per row
    const int total = MT * per_row;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
      const int m = idx / per_row, kc = idx % per_row;
      const int k = kb + kc * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < a.M && k < a.K) v = *reinterpret_cast<const uint4*>(a.X + (size_t)m * a.K + k);
      *reinterpret_cast<uint4*>(xs + m * kwg + kc * 8) = v;
      // k offsets 0,1,4,5 of every 8 are the "1024 + q" pairs, 2,3,6,7 the "1024 + 16 q" pairs
      float sa = lo_f(v.x, BF16) + hi_f(v.x, BF16) + lo_f(v.z, BF16) + hi_f(v.z, BF16);
      float sb = lo_f(v.y, BF16) + hi_f(v.y, BF16) + lo_f(v.w, BF16) + hi_f(v.w, BF16);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        sa += __shfl_xor(sa, o, 16);
        sb += __shfl_xor(sb, o, 16);
      }
      if ((kc & 15) == 0) {
        const int gi = kc / 16;
        float c1, c2;
        if (BF16) {
          c2 = sa + sb;
          c1 = 128.0f * c2;
        } else {
          c1 = 1024.0f * sa + 64.0f * sb;
          c2 = sa + sb;
        }
        csum[(m * ngw + gi) * 2 + 0] = c1;
        csum[(m * ngw + gi) * 2 + 1] = c2;
      }
    }
  }
  __syncthreads();

  // ---- main loop: one pair of groups (8 chunks, 256 k) per step, next pair prefetched
  float y[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) y[m] = 0.0f;

  auto consume = [&](const uint4 (&buf)[8], uint32_t sdw, uint32_t zb, int p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float acc_a[MT], acc_b[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc_a[m] = acc_b[m] = 0.0f;
      const uint4 w4[4] = {buf[h * 4 + 0], buf[h * 4 + 1], buf[h * 4 + 2], buf[h * 4 + 3]};
      const int xk = wave * a.kw + p * kPairK + h * kGroup;     // offset in the staged X
      group_dot<MT, BF16>(w4, xs, kwg, xk, acc_a, acc_b);
      const float s = h2f(sdw >> (16 * h));
      const float z = (float)((zb >> (4 * h)) & 0xFu);
      const int gi = xk / kGroup;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float c1 = csum[(m * ngw + gi) * 2 + 0];
        const float c2 = csum[(m * ngw + gi) * 2 + 1];
        const float t = BF16 ? (acc_a[m] - c1 - z * c2) : (acc_a[m] + 0.0625f * acc_b[m] - c1 - z * c2);
        y[m] += s * t;
      }
    }
  };

  for (int p = 0; p < npairs; p += 2) {
    if (p + 1 < npairs) {
#pragma unroll
      for (int c = 0; c < 8; ++c) bufB[c] = wp[((p + 1) * 8 + c) * kTileN];
      sB = sp[(p + 1) * kTileN];
      zB = zp[(p + 1) * kTileN];
    }
    consume(bufA, sA, zA, p);
    if (p + 1 < npairs) {
      if (p + 2 < npairs) {
#pragma unroll
        for (int c = 0; c < 8; ++c) bufA[c] = wp[((p + 2) * 8 + c) * kTileN];
        sA = sp[(p + 2) * kTileN];
        zA = zp[(p + 2) * kTileN];
      }
      consume(bufB, sB, zB, p + 1);
    }
  }

  // ---- reduce the four waves
#pragma unroll
  for (int m = 0; m < MT; ++m) red[(wave * MT + m) * 64 + lane] = y[m];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MT; ++m)
    y[m] = ((red[(0 * MT + m) * 64 + lane] + red[(1 * MT + m) * 64 + lane]) + red[(2 * MT + m) * 64 + lane]) +
           red[(3 * MT + m) * 64 + lane];

  const int n = tile * kTileN + lane;
  if (a.splits == 1) {
    if (n < a.N)
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < a.M) a.Y[(size_t)m * a.N + n] = to_out(y[m], BF16);
    return;
  }

  // ---- split-K: publish the partial, the last workgroup of the tile combines
#pragma unroll
  for (int m = 0; m < MT; ++m)
    if (m < a.M) a.part[((size_t)split * a.M + m) * a.Np + n] = y[m];
  __threadfence();
  unsigned prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(a.cnt + tile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  if (prev != (unsigned)(a.splits - 1)) return;
  __threadfence();
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= a.M) break;
    float acc = 0.0f;
    for (int s = 0; s < a.splits; ++s) acc += a.part[((size_t)s * a.M + m) * a.Np + n];
    if (n < a.N) a.Y[(size_t)m * a.N + n] = to_out(acc, BF16);
  }
  if (lane == 0) a.cnt[tile] = 0u;
}

template <int MT, bool BF16>
hipError_t launch_mt(const GemvArgs& a, int ntiles, hipStream_t st) {
  const int kwg = 4 * a.kw;
  const size_t lds = (size_t)MT * kwg * 2 + (size_t)MT * (kwg / kGroup) * 2 * 4 + (size_t)4 * MT * 64 * 4;
  hipLaunchKernelGGL((q4_gemv_kernel<MT, BF16>), dim3(ntiles * a.splits), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const GemvArgs& a, int mt, int ntiles, hipStream_t st) {
  switch (mt) {
    case 1: return launch_mt<1, BF16>(a, ntiles, st);
    case 2: return launch_mt<2, BF16>(a, ntiles, st);
    case 4: return launch_mt<4, BF16>(a, ntiles, st);
    case 8: return launch_mt<8, BF16>(a, ntiles, st);
    default: return launch_mt<16, BF16>(a, ntiles, st);
  }
}

}  // namespace

GemvPlan plan_q4_gemv(int M, int N, int K) {
  GemvPlan P;
  P.mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
  const Q4Layout L = q4_layout(N, K);
  const int ntiles = L.Np / kTileN;
  // X staged per workgroup: MT * 4 * kw * 2 bytes, kept <= 32 KB
  int max_kw = (4096 / P.mt) / kPairK * kPairK;
  if (max_kw < kPairK) max_kw = kPairK;
  const int target_wgs = 1024;
  const int max_splits = (L.Kp + 4 * kPairK - 1) / (4 * kPairK);
  int splits = (target_wgs + ntiles - 1) / ntiles;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int kw = (L.Kp + 4 * splits - 1) / (4 * splits);
  kw = (kw + kPairK - 1) / kPairK * kPairK;
  if (kw > max_kw) kw = max_kw;
  splits = (L.Kp + 4 * kw - 1) / (4 * kw);
  P.kw = kw;
  P.splits = splits;
  P.ws_bytes = 0;
  if (splits > 1)
    P.ws_bytes = round_up((size_t)ntiles * 4, 256) + (size_t)splits * M * L.Np * 4;
  return P;
}

hipError_t launch_q4_gemv(const void* X, bool bf16, int M, int K, int N, const uint8_t* blob, const Q4Layout& L,
                          const GemvPlan& P, void* ws, void* Y, hipStream_t st) {
  GemvArgs a;
  a.X = static_cast<const uint16_t*>(X);
  a.M = M;
  a.K = K;
  a.N = N;
  a.Np = L.Np;
  a.Kp = L.Kp;
  a.W = reinterpret_cast<const uint4*>(blob + L.w_off);
  a.S = reinterpret_cast<const uint32_t*>(blob + L.s_off);
  a.Z = blob + L.z_off;
  a.kw = P.kw;
  a.splits = P.splits;
  const int ntiles = L.Np / kTileN;
  a.cnt = static_cast<unsigned*>(ws);
  a.part = P.splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + round_up((size_t)ntiles * 4, 256))
                        : nullptr;
  a.Y = static_cast<uint16_t*>(Y);
  return bf16 ? launch_dtype<true>(a, P.mt, ntiles, st) : launch_dtype<false>(a, P.mt, ntiles, st);
}

}  // namespace ql
