// W4A16 decode kernel (M <= 16): Y[m][n] = sum_k X[m][k] * s * (q - z).
//
// Decode is bound by streaming the packed weights from HBM once per token
// ([QK] §9.1: batch-1 decode reads every weight once per token; [LQ]
// "带宽与算力：Roofline": with a few tokens the arithmetic intensity is about
// the token count, far below the ridge point), so the kernel is organised
// around that stream and keeps everything else off the critical path:
//
//   * a workgroup owns 16 * NT output channels for the whole of K, so no
//     partial sums ever leave the workgroup (cross-workgroup reductions need
//     device-scope cache write-backs on this multi-XCD part, which cost far
//     more than the layer itself); NT (1, 2 or 4) is the largest that still
//     gives every compute unit a workgroup;
//   * lane l of a wave reads output channel l % 16 of each of its NT 16-column
//     slices, K-block l / 16: one 16-byte load per lane and slice covers 4
//     consecutive 32-channel chunks x 16 channels = one 128-wide group, four
//     256-byte runs of the chunk-major blob, where all channels at one K
//     position are contiguous, so the waves of all workgroups that are at the
//     same point of K read one contiguous window (what HBM streams best);
//   * the activation fragment of a group is loaded once and used for all NT
//     slices, which keeps activation loads from crowding out weight loads;
//   * the codes stay packed until they are in registers ([QK] §9.5): an AND
//     with 0x000F000F and an OR with the bit pattern of fp16 1024.0 (0x6400)
//     or bf16 128.0 (0x4300) turns a pair of nibbles into the exact pair
//     (off + q0, off + q1) ([QK] §9.6);
//   * the 16-bit products and their fp32 sums run on the matrix unit
//     (v_mfma_f32_16x16x32_{f16,bf16}, one row per token, up to 16 tokens),
//     which leaves the vector ALU to the unpacking; the same A operand times
//     a constant B = -(off + z) in a second accumulator chain removes the
//     offset and the zero point exactly (the zero-point expansion of [LQ]'s
//     W8A8 section and [VE] "二", applied per group), and the group scale is
//     applied once per group to the 4 accumulators of a lane;
//   * the waves of a workgroup split K and add their 16 x 16 tiles in LDS.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct GemvArgs {
  const uint16_t* X;
  int M, K, N, Np, Kp;
  const uint4* W;          // [Kp/32][Np] chunks
  const uint32_t* S;       // [Kp/256][Np] scale pairs
  const uint8_t* Z;        // [Kp/256][Np] zero pairs
  uint16_t* Y;             // [M][N]
};

template <bool BF16>
__device__ inline f32x4 mfma(const uint4& a, const uint4& b, const f32x4& c) {
  if (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// word of 8 codes (code of k = 2i at bits 4i, of k = 2i + 1 at bits 16 + 4i)
// -> 4 registers of 16-bit pairs (off + q_{2i}, off + q_{2i+1})
template <bool BF16>
__device__ inline uint4 unpack8(uint32_t w) {
  const uint32_t magic = BF16 ? 0x43004300u : 0x64006400u;
  return make_uint4((w & 0x000F000Fu) | magic, ((w >> 4) & 0x000F000Fu) | magic, ((w >> 8) & 0x000F000Fu) | magic,
                    ((w >> 12) & 0x000F000Fu) | magic);
}

template <bool BF16>
__device__ inline uint32_t neg_offset_pair(uint32_t z) {
  const float v = -((BF16 ? 128.0f : 1024.0f) + (float)z);   // exact in both 16-bit types
  const uint32_t h = BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
  return h | (h << 16);
}

// NT: 16-column slices per wave; U: groups per step (even, so a step covers
// whole pairs of groups and their shared scale / zero words)
template <int NT, int U>
struct StepBuf {
  uint4 w[U][NT];          // one 16-byte chunk per group and slice
  uint4 x[U][4];           // activation fragments of each group (shared by the slices)
  uint32_t s[U / 2][NT];   // fp16 scales of a pair of groups
  uint32_t z[U / 2][NT];   // zero points of a pair of groups (two nibbles)
};

template <bool BF16, int NT, int U>
__global__ __launch_bounds__(512) void q4_gemv_kernel(GemvArgs a) {
  __shared__ f32x4 red[8][NT][64];
  const int nw = blockDim.x >> 6;
  // the wave index is uniform; saying so keeps the K loop a scalar loop
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int cl = lane & 15, blk = lane >> 4;
  const int G = a.K / kGroup;
  const int gpw = ((G + nw - 1) / nw + U - 1) / U * U;          // groups per wave, whole steps
  const int g0 = min(G, wave * gpw), g1 = min(G, g0 + gpw);
  const int gl = max(G - 1, 0);

  const uint4* wp[NT];
  const uint32_t* sp[NT];
  const uint8_t* zp[NT];
  const size_t np = a.Np;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (blockIdx.x * NT + t) * 16 + cl;          // output channel of this lane in slice t
    wp[t] = a.W + (size_t)blk * np + n;                     // + 4*Np*g for group g
    sp[t] = a.S + n;                                        // + Np*(g/2)
    zp[t] = a.Z + n;
  }
  const bool row_ok = cl < a.M;                                           // A-operand row of this lane
  const uint32_t rmask = row_ok ? 0xFFFFFFFFu : 0u;
  const uint16_t* xp = a.X + (size_t)(row_ok ? cl : 0) * a.K + blk * kChunkK;   // + 128*g + 8*j

  // All loads are branch-free (indices clamped into the layer, values past the
  // wave's range discarded) and a whole step ahead of their use: a step first
  // issues every load of the next step, then computes on data issued one step
  // earlier, so the in-order vector-memory counter never waits on a prefetch.
  auto issue = [&](int gs, StepBuf<NT, U>& b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = min(gs + u, gl);
#pragma unroll
      for (int t = 0; t < NT; ++t) b.w[u][t] = wp[t][(size_t)g * 4 * np];
#pragma unroll
      for (int j = 0; j < 4; ++j) b.x[u][j] = *reinterpret_cast<const uint4*>(xp + (size_t)g * kGroup + 8 * j);
    }
#pragma unroll
    for (int p = 0; p < U / 2; ++p) {
      const int pr = min(gs + 2 * p, gl) >> 1;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        b.s[p][t] = sp[t][(size_t)pr * np];
        b.z[p][t] = zp[t][(size_t)pr * np];
      }
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int gs, const StepBuf<NT, U>& b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // straight-line for every u: a group past the wave's range gets scale 0;
      // masks are arithmetic, not selects (a select of a loaded value would
      // become a branch around the load)
      const float valid = gs + u < g1 ? 1.0f : 0.0f;
      uint4 xa[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xa[j] = make_uint4(b.x[u][j].x & rmask, b.x[u][j].y & rmask, b.x[u][j].z & rmask, b.x[u][j].w & rmask);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int h = u & 1;                                   // steps start on even groups
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(b.s[u >> 1][t] >> (16 * h))) * valid;
        const uint32_t nz = neg_offset_pair<BF16>((b.z[u >> 1][t] >> (4 * h)) & 0xFu);
        const uint4 bz = make_uint4(nz, nz, nz, nz);
        const uint32_t ww[4] = {b.w[u][t].x, b.w[u][t].y, b.w[u][t].z, b.w[u][t].w};
        f32x4 t0 = {0.0f, 0.0f, 0.0f, 0.0f}, t1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          t0 = mfma<BF16>(xa[j], unpack8<BF16>(ww[j]), t0);
          t1 = mfma<BF16>(xa[j], bz, t1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] += s * (t0[i] + t1[i]);
      }
    }
  };

  StepBuf<NT, U> ba, bb;
  issue(g0, ba);
  // two steps per iteration with the buffers swapping roles, so no register
  // copy ever waits on a prefetch
  for (int gs = g0; gs < g1;) {
    issue(gs + U, bb);
    __builtin_amdgcn_sched_barrier(0);    // keep the prefetch ahead of the arithmetic
    compute(gs, ba);
    gs += U;
    if (gs >= g1) break;
    issue(gs + U, ba);
    __builtin_amdgcn_sched_barrier(0);
    compute(gs, bb);
    gs += U;
  }

  // ---- add the waves' tiles; lane l holds rows 4*(l/16) + i of column l % 16
#pragma unroll
  for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < nw; ++w)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 o = red[w][t][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += o[i];
    }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (blockIdx.x * NT + t) * 16 + cl;
    if (n >= a.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * blk + i;
      if (m < a.M)
        a.Y[(size_t)m * a.N + n] = BF16 ? __builtin_bit_cast(uint16_t, (__bf16)acc[t][i])
                                        : __builtin_bit_cast(uint16_t, (_Float16)acc[t][i]);
    }
  }
}

template <bool BF16>
hipError_t launch_dtype(const GemvArgs& a, const GemvPlan& P, hipStream_t st) {
  const dim3 grid(a.Np / (16 * P.nt)), block(64 * P.waves);
  switch (P.nt) {
    case 4: hipLaunchKernelGGL((q4_gemv_kernel<BF16, 4, 2>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((q4_gemv_kernel<BF16, 2, 2>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((q4_gemv_kernel<BF16, 1, 2>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

GemvPlan plan_q4_gemv(int M, int N, int K) {
  (void)M;
  (void)K;
  GemvPlan P;
  const Q4Layout L = q4_layout(N, K);
  const int slices = L.Np / 16;
  // widest column block that still leaves a workgroup for every compute unit;
  // four waves per workgroup (measured on the Llama-2 7B / 70B layer shapes:
  // fewer concurrent weight streams per compute unit keep HBM busier than
  // more, as for a plain streaming read)
  P.nt = (slices / 4 >= 256) ? 4 : (slices / 2 >= 256) ? 2 : 1;
  P.waves = 4;
  return P;
}

hipError_t launch_q4_gemv(const void* X, bool bf16, int M, int K, int N, const uint8_t* blob, const Q4Layout& L,
                          const GemvPlan& P, void* Y, hipStream_t st) {
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
  a.Y = static_cast<uint16_t*>(Y);
  return bf16 ? launch_dtype<true>(a, P, st) : launch_dtype<false>(a, P, st);
}

}  // namespace ql
