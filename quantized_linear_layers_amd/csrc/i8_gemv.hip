// W8A8 decode kernel (few tokens: see i8_gemv_serves): the GEMM and fused
// epilogue of i8_gemm_scaled / f8_gemm_scaled for a few tokens,
//   C[m][n]   = sum_k Aq[m][k] Bq[n][k] - azp[m] azp_adj[n]      (int32, exact)
//   out[m][n] = s_a[m] (s_b[n] C[m][n]) + bias[n]
// ([LQ] W8A8 section; [VE] "2.4" for the zero-point term, [VE] "一、背景" for
// the epilogue applied before the single store), or the same with E4M3 codes
// and fp32 accumulation and no zero points.
//
// With a few tokens the product streams Bq (N K bytes) once and does little
// arithmetic per byte ([LQ] "带宽与算力：Roofline": the arithmetic intensity is
// about the token count), so the kernel is laid out like the W4A16 decode
// kernel rather than like the tiled GEMM, whose 128-row tiles would leave
// 7/8 of each tile and most compute units idle:
//   * a workgroup owns 16 NT output channels for the whole of K (no partial
//     sums leave it), NT = 1 up to N = 16384 (more, smaller workgroups
//     stream best), 2 or 4 beyond;
//   * its 4 waves split K in groups of 128 bytes (one 128-byte line per row);
//     each wave streams its groups through a ring of 3 LDS slots filled by
//     global_load_lds two groups ahead: per group the activation rows (8,
//     16, 32 or 64: the fewest that hold M) and the NT 16-channel weight
//     blocks, 1 KB per copy instruction, full lines, the weights marked
//     non-temporal;
//   * rows are stored with their 16-byte pieces XOR-swizzled by row bits 1..3,
//     so that the 16 rows one fragment read serves fall on distinct banks;
//   * products on v_mfma_i32_16x16x64_i8 (two per group, slice and block of
//     16 rows) or v_mfma_f32_16x16x128_f8f6f4 (one), one row per token;
//   * the waves' 16 x 16 tiles are added in LDS in wave order, and the first
//     wave applies the epilogue and stores.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ql_internal.h"

namespace ql {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGrp = 128;       // bytes of K per group

template <bool FP8>
using GvAcc = std::conditional_t<FP8, f32x4, i32x4>;

// slot layout: MX KB of activation rows (8 MX rows of 128 bytes), then the
// NT weight blocks (16 channels of 128 bytes each)
template <int NT, int MX>
struct GvSlot {
  static constexpr int kX = 0;
  static constexpr int kW = MX * 1024;
  static constexpr int kBytes = kW + NT * 2048;
  static constexpr int kLoads = MX + 2 * NT;     // 1 KB copies per group
};

__device__ inline int gv_key(int r) { return (r >> 1) & 7; }
// byte offset of logical 16-byte piece p of row r inside a block of 128-byte rows
__device__ inline uint32_t gv_swz(int r, int p) { return (uint32_t)(r * kGrp + ((p ^ gv_key(r)) << 4)); }

template <int CP>
__device__ inline void gv_copy(const int8_t* src, int8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), lds, 16, 0, CP);
#else
  (void)src;
  (void)lds;
#endif
}

template <int N>
__device__ inline void gv_wait_vm() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
#endif
}

// LDS read of one 16-byte fragment (inline assembly keeps the compiler's
// conservative wait for every outstanding LDS copy out of the loop; the copy
// wait before it and gv_lds_wait after it provide the ordering).  `fence` is
// a value read from the last accumulator the previous group's products wrote
// (v_readfirstlane, for which the compiler inserts the wait states the
// matrix unit's results need): taking it as an operand places the read after
// those products have completed, so that it can never overwrite a fragment
// register an MFMA still in flight is reading.
template <int OFF>
__device__ inline i32x4 gv_read16(uint32_t addr, int fence) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  i32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF), "s"(fence) : "memory");
#else
  (void)fence;
  v = i32x4{(int)addr, 0, 0, 0};   // host pass only (never executed)
#endif
  return v;
}
__device__ inline void gv_lds_wait() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
}
__device__ inline void gv_after_wait(i32x4& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
}

template <int I, int N, typename F>
__device__ inline void gv_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    gv_for<I + 1, N>(f);
  }
}

// LDS of one workgroup: W waves, each with a ring of D slots
constexpr int gv_lds_bytes(int NT, int MX, int W, int D) { return W * D * (MX * 1024 + NT * 2048); }

// NT: 16-channel slices per workgroup; MX: 1 KB activation copies per group,
// 8 MX rows (MX = 1: the 8 rows of M <= 8, whose products take one block of
// 16 rows; MX = 2, 4, 8: MX / 2 blocks of 16 rows); W: waves (they split K);
// D: ring slots per wave (D - 1 groups in flight while one is multiplied).
// Rows past M repeat row M - 1 and channels past N repeat channel N - 1
// (valid loads whose products only reach outputs that are never stored).
template <bool FP8, bool OUT_BF16, int NT, int MX, int W, int D>
__global__ __launch_bounds__(64 * W) void i8_gemv_kernel(const int8_t* A, const int8_t* B, int M, int N, int K,
                                                        I8Epi e) {
  using SL = GvSlot<NT, MX>;
  constexpr int L = SL::kLoads;
  static_assert(gv_lds_bytes(NT, MX, W, D) <= 160 * 1024, "LDS per workgroup");
  constexpr int kWaveBytes = D * SL::kBytes;
  static_assert(kWaveBytes >= NT * (MX == 1 ? 1 : MX / 2) * 64 * 16, "the reduction reuses a wave's ring");
  __shared__ __align__(1024) int8_t lds_all[W * kWaveBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int G = (K + kGrp - 1) / kGrp;
  const int gpw = (G + W - 1) / W;
  const int g0 = min(G, wave * gpw), g1 = min(G, g0 + gpw);
  int8_t* ring = lds_all + wave * kWaveBytes;
  const int n0 = blockIdx.x * NT * 16;

  // this lane's copies: row (lane / 8) + 8 j of each 1 KB block, logical
  // piece (lane % 8) ^ key(row) into stored piece lane % 8
  constexpr int MR = MX == 1 ? 1 : MX / 2;       // 16-row blocks of products
  const int crow = lane >> 3;
  const int8_t* xsrc[MX];
  int xp16[MX];
#pragma unroll
  for (int j = 0; j < MX; ++j) {
    const int r = crow + 8 * j;
    xsrc[j] = A + (size_t)min(r, M - 1) * K;
    xp16[j] = ((lane & 7) ^ gv_key(r)) * 16;
  }
  const int8_t* wsrc[NT][2];
  int wp16[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = crow + 8 * j;
    wp16[j] = ((lane & 7) ^ gv_key(r)) * 16;
#pragma unroll
    for (int t = 0; t < NT; ++t) wsrc[t][j] = B + (size_t)min(n0 + t * 16 + r, N - 1) * K;
  }
  auto issue = [&](int g, int slot) {
    int8_t* dst = ring + slot * SL::kBytes;
    const int kg = g * kGrp;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) gv_copy<2>(wsrc[t][j] + min(kg + wp16[j], K - 16), dst + SL::kW + t * 2048 + j * 1024);
#pragma unroll
    for (int j = 0; j < MX; ++j) gv_copy<0>(xsrc[j] + min(kg + xp16[j], K - 16), dst + SL::kX + j * 1024);
  };

  // fragment addresses (slot 0): lane l supplies row / channel l % 16 and the
  // 16-byte pieces of lane group l / 16 (int8: piece 4 s + l / 16 of k step s;
  // FP8: pieces 2 (l / 16) and 2 (l / 16) + 1)
  typedef __attribute__((address_space(3))) int8_t* lds_ptr;
  const uint32_t rbase = (uint32_t)(uintptr_t)(lds_ptr)ring;
  const int fr = lane & 15, lg = lane >> 4;
  const int xr = MX == 1 ? (fr & 7) : fr;
  uint32_t xa[MR][2], wa[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int p = FP8 ? 2 * lg + s : 4 * s + lg;
#pragma unroll
    for (int rb = 0; rb < MR; ++rb) xa[rb][s] = rbase + SL::kX + gv_swz(xr + 16 * rb, p);
    wa[s] = rbase + SL::kW + gv_swz(fr, p);
  }

  GvAcc<FP8> acc[NT][MR];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int rb = 0; rb < MR; ++rb) acc[t][rb] = GvAcc<FP8>{0, 0, 0, 0};

  auto compute = [&](int g, auto SLOT) {
    constexpr int so = decltype(SLOT)::value * SL::kBytes;
    const int fence = __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, acc[NT - 1][MR - 1][0]));
    i32x4 xf[MR][2], wf[NT][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int rb = 0; rb < MR; ++rb) xf[rb][s] = gv_read16<so>(xa[rb][s], fence);
      gv_for<0, NT>([&](auto T) { wf[T][s] = gv_read16<so + decltype(T)::value * 2048>(wa[s], fence); });
    }
    gv_lds_wait();
    // pieces at or past K (only in a ragged last group) hold clamped data:
    // zero the activation side
    const int kg = g * kGrp;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int p = FP8 ? 2 * lg + s : 4 * s + lg;
#pragma unroll
      for (int rb = 0; rb < MR; ++rb) {
        gv_after_wait(xf[rb][s]);
        if (kg + 16 * p >= K) xf[rb][s] = i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) gv_after_wait(wf[t][s]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int rb = 0; rb < MR; ++rb) {
        if constexpr (FP8) {
          const i32x8 a8 = __builtin_shufflevector(xf[rb][0], xf[rb][1], 0, 1, 2, 3, 4, 5, 6, 7);
          const i32x8 b8 = __builtin_shufflevector(wf[t][0], wf[t][1], 0, 1, 2, 3, 4, 5, 6, 7);
          // format codes 0, 0: both operands FP8 E4M3; no block scales
          acc[t][rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[t][rb], 0, 0, 0, 0, 0, 0);
        } else {
          acc[t][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[rb][0], wf[t][0], acc[t][rb], 0, 0, 0);
          acc[t][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[rb][1], wf[t][1], acc[t][rb], 0, 0, 0);
        }
      }
  };

  // prologue: groups g0 .. g0 + D - 2 in flight (those inside the range)
#pragma unroll
  for (int i = 0; i < D - 1; ++i)
    if (g0 + i < g1) issue(g0 + i, i);
  int g = g0;
  while (g < g1) {
    gv_for<0, D>([&](auto SLOT) {
      constexpr int slot = decltype(SLOT)::value;
      if (g < g1) {
        // refill the slot the previous group was read from with group
        // g + D - 1, then wait until group g's copies have landed
        if (g + D - 1 < g1) {
          issue(g + D - 1, slot == 0 ? D - 1 : slot - 1);
          gv_wait_vm<(D - 1) * L>();
        } else {
          gv_wait_vm<0>();
        }
        __builtin_amdgcn_sched_barrier(0);
        compute(g, SLOT);
        __builtin_amdgcn_sched_barrier(0);
        ++g;
      }
    });
  }
  gv_wait_vm<0>();                           // no copy may still target the ring

  // ---- add the waves' tiles (each in its own ring) in wave order
  GvAcc<FP8>* red = reinterpret_cast<GvAcc<FP8>*>(ring);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int rb = 0; rb < MR; ++rb) red[(t * MR + rb) * 64 + lane] = acc[t][rb];
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < W; ++w)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int rb = 0; rb < MR; ++rb)
        acc[t][rb] += reinterpret_cast<const GvAcc<FP8>*>(lds_all + w * kWaveBytes)[(t * MR + rb) * 64 + lane];

  // ---- epilogue: lane l holds column l % 16 of each slice, rows
  // 16 rb + 4 (l / 16) + i of each block rb
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n0 + t * 16 + fr;
    if (n >= N) continue;
    const float sb = e.s_b[e.s_b_vec ? n : 0];
    const int32_t adj = e.azp_adj ? e.azp_adj[n] : 0;
    float b = 0.0f;
    if (e.bias) {
      const uint16_t bb = static_cast<const uint16_t*>(e.bias)[n];
      b = OUT_BF16 ? __builtin_bit_cast(float, (uint32_t)bb << 16) : (float)__builtin_bit_cast(_Float16, bb);
    }
#pragma unroll
    for (int rb = 0; rb < MR; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * rb + 4 * lg + i;
        if (m >= M) continue;
        float c;
        if constexpr (FP8) {
          c = acc[t][rb][i];
        } else {
          const int32_t ci = acc[t][rb][i] - (e.azp ? e.azp[m] * adj : adj);
          if (e.raw) e.raw[(size_t)m * N + n] = ci;
          c = (float)ci;
        }
        const float v = e.s_a[e.s_a_vec ? m : 0] * (sb * c) + b;
        static_cast<uint16_t*>(e.out)[(size_t)m * N + n] =
            OUT_BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
      }
  }
}

// The plan: one 16-channel slice per workgroup up to 1024 slices (N up to
// 16384), then two, then four; four waves, three slots (48 KB of LDS for
// one slice: three workgroups per compute unit).  Measured against
// every (slices, waves, slots) combination on the 7B and 70B layer shapes at
// 1, 8 and 16 tokens (weights from HBM): more, smaller workgroups beat the
// W4A16 kernel's rule here (8192 x 8192: 16.4 -> 12.3 us for one token with
// one slice on four waves instead of two slices on eight), since a group's
// weight block is 2 KB per slice instead of 1 KB.
constexpr int kGvWaves = 4, kGvDepth = 3;
int plan_gv_slices(int N) {
  const int slices = (N + 15) / 16;
  return slices <= 1024 ? 1 : slices <= 2048 ? 2 : 4;
}

template <bool FP8, bool OUT_BF16, int NT, int MX>
hipError_t launch_mx(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e, hipStream_t st) {
  const dim3 grid((unsigned)((N + 16 * NT - 1) / (16 * NT)));
  hipLaunchKernelGGL((i8_gemv_kernel<FP8, OUT_BF16, NT, MX, kGvWaves, kGvDepth>), grid, dim3(64 * kGvWaves), 0, st, A,
                     B, M, N, K, e);
  return hipGetLastError();
}

template <bool FP8, bool OUT_BF16, int NT>
hipError_t launch_nt(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e, hipStream_t st) {
  if (M <= 8) return launch_mx<FP8, OUT_BF16, NT, 1>(A, B, M, N, K, e, st);
  if (M <= 16) return launch_mx<FP8, OUT_BF16, NT, 2>(A, B, M, N, K, e, st);
  if constexpr (NT < 4) {      // more than 16 tokens only with M N <= 2^19 (N < 32768: NT <= 2)
    if (M <= 32) return launch_mx<FP8, OUT_BF16, NT, 4>(A, B, M, N, K, e, st);
    if (M <= 64) return launch_mx<FP8, OUT_BF16, NT, 8>(A, B, M, N, K, e, st);
  }
  return hipErrorInvalidValue;
}

template <bool FP8, bool OUT_BF16>
hipError_t launch_out(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e, hipStream_t st) {
  switch (plan_gv_slices(N)) {
    case 4: return launch_nt<FP8, OUT_BF16, 4>(A, B, M, N, K, e, st);
    case 2: return launch_nt<FP8, OUT_BF16, 2>(A, B, M, N, K, e, st);
    default: return launch_nt<FP8, OUT_BF16, 1>(A, B, M, N, K, e, st);
  }
}

}  // namespace

hipError_t launch_i8_gemv(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e, bool fp8,
                          hipStream_t st) {
  if (fp8)
    return e.out_bf16 ? launch_out<true, true>(A, B, M, N, K, e, st) : launch_out<true, false>(A, B, M, N, K, e, st);
  return e.out_bf16 ? launch_out<false, true>(A, B, M, N, K, e, st) : launch_out<false, false>(A, B, M, N, K, e, st);
}

}  // namespace ql
