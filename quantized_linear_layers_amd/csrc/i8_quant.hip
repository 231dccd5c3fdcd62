// Dynamic per-token activation quantization (int8 asymmetric / symmetric and
// FP8 E4M3), optionally fused with the RMSNorm that produces the row: one
// workgroup of four waves per row.
//
// The row's range is found with one reduction ([LQ] "校准：静态与动态":
// per-token absmax/range at run time costs one extra reduction), then the
// scale, the int32 zero point and the codes follow the formulas in qlinear.h
// in IEEE fp32 with round-half-to-even, so every code is decided exactly as a
// scalar CPU implementation of the same steps decides it.
//
// A workgroup owns a row: its threads read 16-byte pieces of it (thread t:
// pieces t, t + 256, ...; a wave's 64 lanes read one contiguous kilobyte per
// load), up to kLanePieces of them stay in registers between the reduction
// and the quantization (so the row is read from HBM once for K <= 4096; the
// rest of a longer row is read again, mostly from the L2).  The reductions
// are wave shuffles followed by one exchange of the four wave totals through
// LDS.  Splitting a row over four waves, rather than giving each wave a row,
// keeps eight waves per SIMD in flight at a few thousand rows, so one row's
// arithmetic runs while another's loads are outstanding.
//
// x / s with a cheap exact rounding.  The codes are functions of the
// correctly rounded fp32 quotient x / s.  With r = 1 / s and t = x * r (both
// rounded), |t - x/s| <= (2^-23 + 2^-48) |x/s| and the rounded quotient is
// within 2^-24 |x/s| of x/s: t decides the code unless it lies next to a
// rounding boundary of the code (about one value in 10^5 does), and those
// values are recomputed with the IEEE division in a loop outside the
// unrolled fast path.
#include <hip/hip_runtime.h>

#include "ql_internal.h"

namespace ql {
namespace {

constexpr int kRowWaves = 4;                    // waves per row (one workgroup per row)
constexpr int kRowThreads = 64 * kRowWaves;
constexpr int kLanePieces = 2;                  // 8-value pieces per thread held in registers (K <= 4096)
constexpr float kCodeBias = 0x1.8p23f;          // integers of magnitude < 2^22 plus this keep their low bits

__device__ inline float half_lo(uint32_t v, bool bf16) {
  return bf16 ? __builtin_bit_cast(float, v << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ inline float half_hi(uint32_t v, bool bf16) {
  return bf16 ? __builtin_bit_cast(float, v & 0xFFFF0000u) : (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Fast code of y / s from t = y * r (r = 1 / s).  Sets `near` when t lies
// so close to a rounding boundary that the rounded quotient might fall on the
// other side; such values are redone with the IEEE division (code_exact).
// t is within 3 fp32 ulps (relative 1.5 * 2^-23) of the rounded quotient.
//   int8: |y / s| <= 256; both round alike unless t is within 2^-21 |t| of
//         a half-integer;
//   E4M3: both round alike unless t is within 8 ulps of an E4M3 midpoint (low
//         20 significand bits near 0x80000); t below 2^-6 (the subnormal
//         codes, a few values in 10^4) always takes the exact path.  On the
//         fast path 2^-6 <= |t| <= 448 (1 + 2^-21), where the code is the
//         fp32 significand rounded at bit 20 (ties to even), which stays at
//         or below the largest code 0x7E.
template <int MODE>
__device__ inline uint32_t code_fast(float t, float zm, float lom, bool& near) {
  if constexpr (MODE == 1) {
    const uint32_t b = __builtin_bit_cast(uint32_t, t);
    const uint32_t a = b & 0x7FFFFFFFu;
    const int d = (int)(a & 0xFFFFFu) - 0x80000;
    near = a < 0x3C800000u || (d <= 8 && d >= -8);
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return ((b >> 24) & 0x80u) | (((r >> 20) - (120u << 3)) & 0x7Fu);   // garbage below 2^-6 stays in its byte
  } else {
    // zm = z + 1.5 * 2^23 and lom = lo + 1.5 * 2^23: the clamped rint(t) + z
    // plus 1.5 * 2^23 is an integer in [2^23, 2^24), exact in fp32, whose low
    // byte is the two's-complement code
    const float c = rintf(t);
    near = fabsf(t - c) >= 0.5f - fabsf(t) * 0x1p-21f;
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(c + zm, lom, kCodeBias + 127.0f));
  }
}

template <int MODE>
__device__ inline uint32_t code_exact(float y, float s, float z, float lo) {
  if constexpr (MODE == 1)
    return e4m3_code(y / s);
  else
    return (uint32_t)(int32_t)fminf(fmaxf(rintf(y / s) + z, lo), 127.0f) & 0xFFu;
}

// the 8 values of a piece as fp32, optionally normalized: (x * inv) * gamma
template <bool BF16, bool NORM>
__device__ inline void piece_values(uint4 p, uint4 g, float inv, float (&y)[8]) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
  const uint32_t u[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = half_lo(w[i], BF16);
    y[2 * i + 1] = half_hi(w[i], BF16);
    if constexpr (NORM) {
      y[2 * i] = (y[2 * i] * inv) * half_lo(u[i], BF16);
      y[2 * i + 1] = (y[2 * i + 1] * inv) * half_hi(u[i], BF16);
    }
  }
}

// The exact path of the sum of squares (rows whose mean square sits next to
// an fp32 rounding boundary) keeps an unevaluated pair hi + lo of doubles:
// each addition is done with an error-free transformation (TwoSum: s + e
// equals a + b exactly, s the rounded sum), the errors are gathered in lo,
// and hi + lo is rounded once at the end.  The result is as accurate as a sum in
// twice the fp64 precision rounded once: the correctly rounded fp64 sum,
// whatever the order of the additions, unless the exact sum lies within
// about n^2 * 2^-106 (relative; 2^-82 for n = 4096) of an fp64 rounding
// boundary.  A plain fp64 sum depends on the order: a row whose mean square
// sits next to an fp32 rounding boundary could round either way.
struct DD {
  double hi, lo;
};
__device__ inline DD two_sum(double a, double b) {
  const double s = a + b;
  const double bp = s - a;
  return DD{s, (a - (s - bp)) + (b - bp)};
}
__device__ inline DD dd_add(DD a, double v) {
  const DD t = two_sum(a.hi, v);
  return DD{t.hi, a.lo + t.lo};
}
__device__ inline DD dd_add(DD a, DD b) {
  const DD t = two_sum(a.hi, b.hi);
  return DD{t.hi, (a.lo + b.lo) + t.lo};
}
// Sum over the workgroup of one pair per thread: wave shuffles, then the
// wave totals through LDS, added in wave order, so every thread gets the same
// result; returns hi + lo rounded once.
__device__ inline double block_sum(DD v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = dd_add(v, DD{__shfl_xor(v.hi, o), __shfl_xor(v.lo, o)});
  if ((threadIdx.x & 63) == 0) {
    red[2 * (threadIdx.x >> 6)] = v.hi;
    red[2 * (threadIdx.x >> 6) + 1] = v.lo;
  }
  __syncthreads();
  DD t{red[0], red[1]};
#pragma unroll
  for (int w = 1; w < kRowWaves; ++w) t = dd_add(t, DD{red[2 * w], red[2 * w + 1]});
  return t.hi + t.lo;
}
// The exact sum of the squares of a row (TwoSum), re-read from memory, two
// values at a time (few registers: the rare exact path must not lower the
// occupancy of the fast one).
template <bool BF16>
__device__ inline double exact_sum_of_squares(const uint4* __restrict__ xv, int pieces, double* red) {
  DD dd{0.0, 0.0};
  for (int p = threadIdx.x; p < pieces; p += kRowThreads) {
    const uint4 v = xv[p];
#pragma unroll 1
    for (int w = 0; w < 4; ++w) {
      const uint32_t word = w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
      const double a = half_lo(word, BF16), b = half_hi(word, BF16);
      dd = dd_add(dd, a * a);
      dd = dd_add(dd, b * b);
    }
  }
  return block_sum(dd, red);
}

// Cross-lane steps inside rows of 16 lanes as DPP operands (no LDS traffic,
// no lane-index arithmetic): a butterfly over the quad (lane ^ 1, lane ^ 2),
// then two rotations of the row by 4 and 8 lanes, after which every lane
// holds its row's total; the four row totals are then read as scalars.
constexpr int kDppQuad1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuad2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRor4 = 0x124;     // row_ror:4
constexpr int kDppRor8 = 0x128;     // row_ror:8
template <int CTRL>
__device__ inline int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ inline double dpp(double v) {
  const int lo = dpp<CTRL>(__double2loint(v)), hi = dpp<CTRL>(__double2hiint(v));
  return __hiloint2double(hi, lo);
}
// the row totals of lanes 0, 16, 32, 48 combined by op (wave-uniform result)
template <typename T, typename Op>
__device__ inline T wave_reduce(T v, Op op) {
  v = op(v, dpp<kDppQuad1>(v));
  v = op(v, dpp<kDppQuad2>(v));
  v = op(v, dpp<kDppRor4>(v));
  v = op(v, dpp<kDppRor8>(v));
  T r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 8)
      r[i] = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 16 * i),
                              __builtin_amdgcn_readlane(__double2loint(v), 16 * i));
    else
      r[i] = __builtin_amdgcn_readlane(v, 16 * i);
  }
  return op(op(r[0], r[1]), op(r[2], r[3]));
}

// The same sum of one plain double per thread (the fast path).
__device__ inline double block_sum_plain(double v, double* red) {
  v = wave_reduce(v, [](double x, double y) { return x + y; });
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int w = 1; w < kRowWaves; ++w) t += red[w];
  return t;
}

// A finite or infinite fp32 value as an int that orders like it (-0 below
// +0), so the range is reduced with integer min / max; the map is its own
// inverse.  (A NaN in a row gives that row an unspecified range.)
__device__ inline int order_key(float f) {
  const int b = __builtin_bit_cast(int, f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ inline float from_key(int k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF)); }

template <bool ASYM>
__device__ inline void block_range(float& mn, float& mx, int* red) {
  int kmn = 0, kmx = wave_reduce(order_key(mx), [](int x, int y) { return x > y ? x : y; });
  if constexpr (ASYM) kmn = wave_reduce(order_key(mn), [](int x, int y) { return x < y ? x : y; });
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = kmn;
    red[kRowWaves + (threadIdx.x >> 6)] = kmx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    kmn = min(kmn, red[w]);
    kmx = max(kmx, red[kRowWaves + w]);
  }
  mn = from_key(kmn);
  mx = from_key(kmx);
}

// MODE 0: int8 (ASYM selects the zero point); MODE 1: FP8 E4M3 (symmetric,
// s = max(absmax, 1e-5) / 448, code = E4M3 rounding of x / s).  NORM: the
// row is first normalized as y = (x * inv) * gamma with
// inv = 1 / sqrt(fp32(S / K) + eps), S the correctly rounded fp64 sum of the
// squares ([QK] §9.9: the per-row reduction of the activation quantization
// fused into the operator that produces the activations; [LQ]
// "QuaRot：把整个残差流旋转掉" for the form of RMSNorm).  One workgroup per row.
template <bool BF16, bool ASYM, int MODE, bool NORM>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(8))) void quant_rows_kernel(const uint16_t* __restrict__ X,
                                                                 const uint16_t* __restrict__ gamma, float eps,
                                                                 int M, int K, int8_t* __restrict__ Aq,
                                                                 float* __restrict__ s_a,
                                                                 int32_t* __restrict__ azp) {
  __shared__ double red_ss[2 * kRowWaves];
  __shared__ int red_range[2 * kRowWaves];
  const int tid = threadIdx.x;
  const int m = blockIdx.x;
  const uint4* xv = reinterpret_cast<const uint4*>(X + (size_t)m * K);
  const uint4* gv = reinterpret_cast<const uint4*>(gamma);
  const int pieces = K / 8;

  // the thread's register-resident pieces tid + kRowThreads * r, converted to
  // fp32 once (zero past the row)
  float y[kLanePieces][8];
  uint4 g[kLanePieces];
  // every load is issued before the first wait: indices past the row re-read
  // its last piece (a valid address) and the value is then replaced by zeros
  uint4 xp[kLanePieces];
#pragma unroll
  for (int r = 0; r < kLanePieces; ++r) {
    const int pc = min(tid + kRowThreads * r, pieces - 1);
    xp[r] = xv[pc];
    if constexpr (NORM) g[r] = gv[pc];
  }
#pragma unroll
  for (int r = 0; r < kLanePieces; ++r) {
    const uint32_t keep = tid + kRowThreads * r < pieces ? 0xFFFFFFFFu : 0u;
    xp[r] = make_uint4(xp[r].x & keep, xp[r].y & keep, xp[r].z & keep, xp[r].w & keep);
    if constexpr (NORM) g[r] = make_uint4(g[r].x & keep, g[r].y & keep, g[r].z & keep, g[r].w & keep);
    else g[r] = make_uint4(0, 0, 0, 0);
    piece_values<BF16, false>(xp[r], xp[r], 1.0f, y[r]);
  }
  constexpr int kHeld = kRowThreads * kLanePieces;           // pieces held in registers

  // ---- RMSNorm: mean square from the correctly rounded fp64 sum of the
  // exact squares (each square of a 16-bit value is exact in fp64).  A plain
  // fp64 sum of K nonnegative terms, in any order, lies within
  // (K - 1) * 2^-53 (relative, to first order) of the exact sum; when the
  // fp32 mean square is the same at both ends of that interval it is the one
  // the correctly rounded sum gives (division and rounding are monotone), and
  // only otherwise (a mean square next to an fp32 rounding boundary: about
  // K * 2^-29 of the rows) is the sum redone exactly with TwoSum.  The branch
  // depends only on the workgroup-wide sum, so the whole workgroup takes it.
  float inv = 1.0f;
  if constexpr (NORM) {
    double acc = 0.0;
#pragma unroll
    for (int r = 0; r < kLanePieces; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += (double)y[r][i] * (double)y[r][i];
    for (int p = tid + kHeld; p < pieces; p += kRowThreads) {
      float t[8];
      piece_values<BF16, false>(xv[p], xv[p], 1.0f, t);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += (double)t[i] * (double)t[i];
    }
    double ss = block_sum_plain(acc, red_ss);
    const double err = ss * ((double)K * 0x1p-53 * 1.001);
    if (__builtin_expect((float)((ss - err) / (double)K) != (float)((ss + err) / (double)K), 0)) {
      __syncthreads();                           // every thread has read red_ss
      ss = exact_sum_of_squares<BF16>(xv, pieces, red_ss);
    }
    const float ms = (float)(ss / (double)K);
    inv = 1.0f / sqrtf(ms + eps);
#pragma unroll
    for (int r = 0; r < kLanePieces; ++r) {
      const uint32_t u[4] = {g[r].x, g[r].y, g[r].z, g[r].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[r][2 * i] = (y[r][2 * i] * inv) * half_lo(u[i], BF16);
        y[r][2 * i + 1] = (y[r][2 * i + 1] * inv) * half_hi(u[i], BF16);
      }
    }
  }

  // ---- range of the (normalized) row
  float mn = 0.0f, mx = 0.0f;                    // the range always contains 0
  auto fold8 = [&](const float (&t)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (ASYM) {
        mn = fminf(mn, t[i]);
        mx = fmaxf(mx, t[i]);
      } else {
        mx = fmaxf(mx, fabsf(t[i]));
      }
    }
  };
#pragma unroll
  for (int r = 0; r < kLanePieces; ++r) fold8(y[r]);         // zero pieces are inside the range
  for (int p = tid + kHeld; p < pieces; p += kRowThreads) {
    float t[8];
    piece_values<BF16, NORM>(xv[p], NORM ? gv[p] : make_uint4(0, 0, 0, 0), inv, t);
    fold8(t);
  }
  block_range<ASYM>(mn, mx, red_range);

  float s, z;
  if constexpr (ASYM) {
    s = fmaxf(mx - mn, 1e-5f) / 255.0f;
    z = -128.0f - rintf(mn / s);
  } else {
    s = fmaxf(mx, 1e-5f) / (MODE == 1 ? 448.0f : 127.0f);
    z = 0.0f;
  }
  if (tid == 0) {
    s_a[m] = s;
    if constexpr (ASYM) azp[m] = (int32_t)z;
  }
  const float rs = 1.0f / s;
  const float lo = ASYM ? -128.0f : -127.0f;

  const float zm = z + kCodeBias, lom = lo + kCodeBias;

  // codes of 8 values, packed in order; the low byte of each code_fast /
  // code_exact result is the code
  auto quant = [&](const float (&t)[8]) -> uint2 {
    uint32_t c[8], fix = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bool near;
      c[i] = code_fast<MODE>(t[i] * rs, zm, lom, near);
      fix |= (uint32_t)near << i;
    }
    uint2 out = make_uint2(__builtin_amdgcn_perm(c[1], c[0], 0x0C0C0400u) | __builtin_amdgcn_perm(c[3], c[2], 0x04000C0Cu),
                           __builtin_amdgcn_perm(c[5], c[4], 0x0C0C0400u) | __builtin_amdgcn_perm(c[7], c[6], 0x04000C0Cu));
    // the rare values next to a rounding boundary: exact division, one at a
    // time, outside the unrolled fast path
#pragma nounroll
    for (; __builtin_expect(fix != 0, 0); fix &= fix - 1) {
      const int i = __builtin_ctz(fix);
      float yi = t[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) yi = i == j ? t[j] : yi;
      const uint32_t sh = 8 * (i & 3), v = (code_exact<MODE>(yi, s, z, lo) & 0xFFu) << sh, keep = ~(0xFFu << sh);
      if (i < 4)
        out.x = (out.x & keep) | v;
      else
        out.y = (out.y & keep) | v;
    }
    return out;
  };
  uint2* qo = reinterpret_cast<uint2*>(Aq + (size_t)m * K);
#pragma unroll
  for (int r = 0; r < kLanePieces; ++r) {
    const int p = tid + kRowThreads * r;
    if (p < pieces) qo[p] = quant(y[r]);
  }
  for (int p = tid + kHeld; p < pieces; p += kRowThreads) {
    float t[8];
    piece_values<BF16, NORM>(xv[p], NORM ? gv[p] : make_uint4(0, 0, 0, 0), inv, t);
    qo[p] = quant(t);
  }
}

template <int MODE, bool NORM>
hipError_t launch_rows(const void* X, bool bf16, int M, int K, const void* gamma, float eps, int8_t* Aq, float* s_a,
                       int32_t* azp, hipStream_t st) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* g = static_cast<const uint16_t*>(gamma);
  const dim3 grid(M), block(kRowThreads);
  if (bf16) {
    if (azp)
      hipLaunchKernelGGL((quant_rows_kernel<true, true, MODE, NORM>), grid, block, 0, st, x, g, eps, M, K, Aq, s_a, azp);
    else
      hipLaunchKernelGGL((quant_rows_kernel<true, false, MODE, NORM>), grid, block, 0, st, x, g, eps, M, K, Aq, s_a,
                         azp);
  } else {
    if (azp)
      hipLaunchKernelGGL((quant_rows_kernel<false, true, MODE, NORM>), grid, block, 0, st, x, g, eps, M, K, Aq, s_a,
                         azp);
    else
      hipLaunchKernelGGL((quant_rows_kernel<false, false, MODE, NORM>), grid, block, 0, st, x, g, eps, M, K, Aq, s_a,
                         azp);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_i8_quant(const void* X, bool bf16, int M, int K, int8_t* Aq, float* s_a, int32_t* azp,
                           hipStream_t st) {
  return launch_rows<0, false>(X, bf16, M, K, nullptr, 0.0f, Aq, s_a, azp, st);
}

hipError_t launch_rmsnorm_quant(const void* X, bool bf16, int M, int K, const void* gamma, float eps, int8_t* Aq,
                                float* s_a, int32_t* azp, hipStream_t st) {
  return launch_rows<0, true>(X, bf16, M, K, gamma, eps, Aq, s_a, azp, st);
}

hipError_t launch_f8_quant(const void* X, bool bf16, int M, int K, uint8_t* Aq, float* s_a, hipStream_t st) {
  return launch_rows<1, false>(X, bf16, M, K, nullptr, 0.0f, reinterpret_cast<int8_t*>(Aq), s_a, nullptr, st);
}

}  // namespace ql
