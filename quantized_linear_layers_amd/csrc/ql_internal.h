// Internal declarations shared by the ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ql {

// Records a printf-style message for ql_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...);

// ---------------------------------------------------------------- W4 device blob layout
// Chunk-major: K is cut in 32-channel chunks; row c holds, for every output
// channel n, the 16 bytes of its 32 codes of chunk c (so all channels at one K
// position are contiguous).  Scales and zero points are stored the same way,
// one row per pair of 128-channel groups.  N is padded to kTileN.
constexpr int kTileN = 64;
constexpr int kChunkK = 32;
constexpr int kGroup = 128;
constexpr int kPairK = 256;          // two groups: K granularity of the blob
constexpr uint32_t kMagic = 0x50344C51u;   // "QL4P"
constexpr uint32_t kVersion = 2;

struct Q4Layout {
  int N, K, Np, Kp;
  size_t w_off, s_off, z_off, bytes;
};

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline Q4Layout q4_layout(int N, int K) {
  Q4Layout L;
  L.N = N;
  L.K = K;
  L.Np = (int)round_up((size_t)N, kTileN);
  L.Kp = (int)round_up((size_t)K, kPairK);
  L.w_off = 256;
  size_t wbytes = (size_t)L.Np * L.Kp / 2;
  L.s_off = round_up(L.w_off + wbytes, 256);
  size_t sbytes = (size_t)L.Np * (L.Kp / kGroup) * 2;
  L.z_off = round_up(L.s_off + sbytes, 256);
  size_t zbytes = (size_t)L.Np * (L.Kp / kPairK);
  L.bytes = round_up(L.z_off + zbytes, 256);
  return L;
}

// nibble position of the code of k = 8j + i inside word j of a lane chunk:
// even i in the low half-word (positions 0..3), odd i in the high half-word
// (positions 4..7), so that (word >> 4p) & 0x000F000F yields the pair
// (k = 2p, k = 2p + 1) as two 16-bit lanes.
inline int nib_pos(int i) { return (i & 1) * 4 + (i >> 1); }

// ---------------------------------------------------------------- launch plans
struct GemvPlan {
  int nt;          // 16-column slices per workgroup (1, 2 or 4)
  int waves;       // waves per workgroup; they split K
};

GemvPlan plan_q4_gemv(int M, int N, int K);

hipError_t launch_q4_gemv(const void* X, bool bf16, int M, int K, int N,
                          const uint8_t* blob, const Q4Layout& L, const GemvPlan& P,
                          void* Y, hipStream_t st);

hipError_t launch_q4_gemm(const void* X, bool bf16, int M, int K, int N,
                          const uint8_t* blob, const Q4Layout& L, void* Y, hipStream_t st);

hipError_t launch_i8_quant(const void* X, bool bf16, int M, int K, int8_t* Aq, float* s_a,
                           int32_t* azp, hipStream_t st);

struct I8Epi {
  const float* s_a; int s_a_vec;
  const float* s_b; int s_b_vec;
  const int32_t* azp;
  const int32_t* azp_adj;
  const void* bias;
  void* out; bool out_bf16;
  int32_t* raw;
};

hipError_t launch_i8_gemm(const int8_t* A, const int8_t* B, int M, int N, int K,
                          const I8Epi& e, hipStream_t st);

}  // namespace ql
