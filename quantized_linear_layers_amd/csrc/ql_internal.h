// Internal declarations shared by the ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <cmath>

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

// ---------------------------------------------------------------- FP8 E4M3
// fp32 -> OCP FP8 E4M3 code ("FN": sign, 4 exponent bits with bias 7, 3
// mantissa bits, no infinities, S.1111.111 = NaN, largest finite 1.75 * 2^8 =
// 448): round to nearest, ties to even, saturating at +-448.  Normal results
// round the fp32 significand at its bit 20 (the carry moves into the
// exponent); below 2^-6 the grid is 2^-9 and v * 512 is rounded exactly.
// Written with selects only (both roundings are computed, the range picks
// one), so an unrolled loop of codes stays straight-line code.
__host__ __device__ inline uint32_t e4m3_code(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  const uint32_t normal = (r >> 20) - (120u << 3);
  const float sub = rintf(__builtin_bit_cast(float, a < 0x3C800000u ? a : 0u) * 512.0f);   // |v| < 2^-6
  uint32_t c = a < 0x3C800000u ? (uint32_t)sub : normal;
  c = a >= 0x43E00000u ? 0x7Eu : c;                          // |v| >= 448: saturate
  c = a > 0x7F800000u ? 0x7Fu : c;                           // NaN
  return sign | c;
}

// ---------------------------------------------------------------- launch plans
struct GemvPlan {
  int nt;          // 16-column slices per workgroup (1, 2 or 4)
  int waves;       // waves per workgroup; they split K
};

GemvPlan plan_q4_gemv(int M, int N, int K);

// plan of the large-M kernel for an M x N x K product: its workgroup tile
// (index into its table) and the split of K across workgroups (splits groups
// of kbs 64-wide K blocks; splits == 1: no split, no workspace)
struct GemmPlan {
  int tile, splits, kbs;
};
GemmPlan plan_q4_gemm(int M, int N, int K, int max_splits);
size_t gemm_workspace_bytes(const GemmPlan& p, int M, int N);
// elements between consecutive K-split slices of the workspace: M * N rounded
// up to a multiple of 4, so that every slice starts 16-byte aligned (the
// reduction reads four elements at a time)
__host__ __device__ inline size_t splitk_slice(size_t MN) { return (MN + 3) & ~(size_t)3; }
void gemm_tile_shape(const GemmPlan& p, int* rows, int* cols);
// token counts served by the decode-family kernel; larger M takes the GEMM
constexpr int kGemvMaxM = 16;
hipError_t launch_q4_gemv(const void* X, bool bf16, int M, int K, int N,
                          const uint8_t* blob, const Q4Layout& L, const GemvPlan& P,
                          void* Y, hipStream_t st);

// size of the library's static device scratch (q4_gemm_no_alloc), and its
// address on the current device (looked up on the first call per device)
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void** ptr);

// ws: the plan's workspace (gemm_workspace_bytes), or null when p.splits == 1
hipError_t launch_q4_gemm(const void* X, bool bf16, int M, int K, int N, const uint8_t* blob, const Q4Layout& L,
                          const GemmPlan& p, void* Y, float* ws, hipStream_t st);

hipError_t launch_permute_cols(const void* X, int M, int K, const int32_t* perm, void* Xp, hipStream_t st);
hipError_t launch_rmsnorm_quant(const void* X, bool bf16, int M, int K, const void* gamma, float eps, int8_t* Aq,
                                float* s_a, int32_t* azp, hipStream_t st);
hipError_t launch_i8_quant(const void* X, bool bf16, int M, int K, int8_t* Aq, float* s_a,
                           int32_t* azp, hipStream_t st);

hipError_t launch_f8_quant(const void* X, bool bf16, int M, int K, uint8_t* Aq, float* s_a, hipStream_t st);

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

// FP8 (E4M3) operands with the same tiling; e.azp, e.azp_adj and e.raw must be null
hipError_t launch_f8_gemm(const uint8_t* A, const uint8_t* B, int M, int N, int K,
                          const I8Epi& e, hipStream_t st);
// the same GEMMs on 128 x 128 tiles (two workgroups per compute unit), which
// launch_i8_gemm / launch_f8_gemm use when i8_small_grid(M, N)
hipError_t launch_i8_gemm_small(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e,
                                hipStream_t st);
hipError_t launch_f8_gemm_small(const uint8_t* A, const uint8_t* B, int M, int N, int K, const I8Epi& e,
                                hipStream_t st);
// the same products for few tokens: a workgroup streams 16, 32 or 64 output
// channels' weights for all of K (fp8: E4M3 codes, e.azp, e.azp_adj and
// e.raw null); launch_i8_gemm / launch_f8_gemm use it when i8_gemv_serves(M, N)
hipError_t launch_i8_gemv(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e, bool fp8,
                          hipStream_t st);
// up to 16 tokens always; up to 64 while M N <= 2^19, where the tiled GEMM's
// 128-column tiles would leave most compute units idle (measured on the 7B and
// 70B layer shapes: 2 - 2.8x faster there, slower beyond)
inline bool i8_gemv_serves(int M, int N) { return M <= 16 || (M <= 64 && (long)M * N <= (1L << 19)); }
// true when the 256 x 128 tiles of an M x N output would occupy at most half
// of the 256 compute units
inline bool i8_small_grid(int M, int N) {
  return 2 * (long)((M + 255) / 256) * ((N + 127) / 128) <= 256;
}

// plain streaming read of `bytes` bytes (a multiple of 16): the achievable
// HBM read rate; sink receives read_probe_sink_words(workgroups) words
int read_probe_sink_words(int workgroups);
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups, int mode,
                             hipStream_t st);

}  // namespace ql
