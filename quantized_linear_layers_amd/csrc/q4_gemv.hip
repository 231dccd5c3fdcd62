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
//     gives every compute unit a workgroup (one slice for one token on a
//     short K, where more, smaller workgroups overlap their fixed costs);
//   * lane l of a wave reads output channel l % 16 of each of its NT 16-column
//     slices, K-block l / 16: one 16-byte load per lane and slice covers 4
//     consecutive 32-channel chunks x 16 channels = one 128-wide group, four
//     256-byte runs of the chunk-major blob, where all channels at one K
//     position are contiguous, so the waves of all workgroups that are at the
//     same point of K read one contiguous window (what HBM streams best);
//   * every operand of a group (the NT weight chunks, their scale words and
//     zero-point bytes and the activation rows the tokens need: 1, 4, 8 or 16
//     of them) is copied straight from global memory into a per-wave ring of
//     D LDS slots (global_load_lds, no register staging), D - 1 groups ahead
//     of the group being multiplied; the scales, zero points and a single
//     token's row share one copy instruction; all copies are the same kind of
//     vector-memory operation, so one counter wait per group covers them and
//     nothing else waits on the prefetch; the activation rows of a group are
//     read from LDS once and used for all NT slices; the weight copies are
//     marked non-temporal (each weight is read once per token);
//   * the codes stay packed until they are in registers ([QK] §9.5): one
//     v_and_or_b32 per register (the mask 0x000F000F and the bit pattern of
//     fp16 1024.0 (0x6400) or bf16 128.0 (0x4300) held in registers, since a
//     three-operand instruction takes no 32-bit literal here) turns a pair of
//     nibbles into the exact pair (off + q0, off + q1) ([QK] §9.6);
//   * the 16-bit products and their fp32 sums run on the matrix unit
//     (v_mfma_f32_16x16x32_{f16,bf16}, one row per token, up to 16 tokens),
//     which leaves the vector ALU to the unpacking; the same A operand times
//     a constant B = -(off + z), accumulated into the same chain after each
//     code step, removes the offset and the zero point (the zero-point
//     expansion of [LQ]'s W8A8 section and [VE] "二", applied per group; the
//     interleaving keeps the running sum small), and the group scale is
//     applied once per group to the 4 accumulators of a lane;
//   * the vector ALU is what bounds the loop once the weights stream at HBM
//     rate, so the per-group instruction count is kept minimal: rows past M
//     are not masked (each output row depends only on its own activation row,
//     and rows past M are never stored);
//   * the waves of a workgroup split K and add their 16 x 16 tiles in LDS.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ql_internal.h"

namespace ql {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// A word of 8 codes (code of k = 2i at bits 4i, of k = 2i + 1 at bits
// 16 + 4i) -> 4 registers of 16-bit pairs (off + q_{2i}, off + q_{2i+1}):
// register i is ((w >> 4i) & mask) | magic, mask = 0x000F000F and magic =
// the offset's bit pattern in both halves, both passed in registers so that
// each register is one v_and_or_b32.  Two words w0, w1 are unpacked together:
// the pair is shifted as one 64-bit value, so one shift per count serves both
// words (the bits that the low word receives from the high one land outside
// the mask); measured on the Llama-2-70B decode step: 112.8 -> 110.9 us,
// outputs bit-identical.
__device__ inline void unpack16(uint32_t w0, uint32_t w1, uint32_t mask, uint32_t magic, uint4& a, uint4& b) {
  const uint64_t p = ((uint64_t)w1 << 32) | w0;
  uint64_t s4, s8, s12;
#if defined(__HIP_DEVICE_COMPILE__)
  // (written out: the compiler turns a 64-bit shift whose result is masked
  // like this back into two 32-bit shifts)
  asm("v_lshrrev_b64 %0, 4, %1" : "=v"(s4) : "v"(p));
  asm("v_lshrrev_b64 %0, 8, %1" : "=v"(s8) : "v"(p));
  asm("v_lshrrev_b64 %0, 12, %1" : "=v"(s12) : "v"(p));
#else
  s4 = p >> 4;
  s8 = p >> 8;
  s12 = p >> 12;
#endif
  a = make_uint4((w0 & mask) | magic, ((uint32_t)s4 & mask) | magic, ((uint32_t)s8 & mask) | magic,
                 ((uint32_t)s12 & mask) | magic);
  b = make_uint4((w1 & mask) | magic, ((uint32_t)(s4 >> 32) & mask) | magic, ((uint32_t)(s8 >> 32) & mask) | magic,
                 ((uint32_t)(s12 >> 32) & mask) | magic);
}

// the pair (-(off + z), -(off + z)) for a zero point z in 0..15: -(1024 + z)
// is 0xE400 + z in fp16 and -(128 + z) is 0xC300 + z in bf16 (exact: z only
// fills low mantissa bits)
template <bool BF16>
__device__ inline uint32_t neg_offset_pair(uint32_t z) {
  return z * 0x00010001u + (BF16 ? 0xC300C300u : 0xE400E400u);
}

// issues one 16-byte global -> LDS copy per lane (lane i writes lds + 16 i)
__device__ inline void load_lds16(const void* src, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#else
  (void)src;
  (void)lds;
#endif
}

// the same copy marked non-temporal (the instruction's `nt` cache-policy
// bit): the weights are read once per token and then not again until every
// other layer has streamed through, so they are not worth keeping in the
// caches (measured on the 70B decode step: 119-122 -> 113-114.5 us)
constexpr int kNonTemporal = 2;
__device__ inline void load_lds16_stream(const void* src, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, kNonTemporal);
#else
  (void)src;
  (void)lds;
#endif
}

// issues one 4-byte global -> LDS copy per lane (lane i writes lds + 4 i)
__device__ inline void load_lds4(const void* src, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
#else
  (void)src;
  (void)lds;
#endif
}

// A lane's fixed 32-bit offset from a uniform base, made opaque to the
// optimizer (in place, so no copy is made) so that it stays a separate operand
// of each copy (the scalar-base plus vector-offset form) instead of being
// folded into a 64-bit per-lane pointer advanced with vector instructions
// every group.
__device__ inline uint32_t lane_offset(uint32_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
  return v;
}

// waits until at most N of this wave's vector-memory operations are in flight
template <int N>
__device__ inline void wait_vm() {
#if defined(__HIP_DEVICE_COMPILE__)
  // gfx9 s_waitcnt: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maximum
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
#endif
}

// LDS read of one 16-byte activation fragment at byte address addr.
// Inline assembly keeps the compiler's conservative tracking of in-flight
// LDS copies (it would wait for every outstanding load, including the next
// step's prefetch) out of the loop; the ordering is enforced explicitly by
// wait_vm before the reads and lds_wait before the fragments are used.
// waits until at most k groups of L copies each are in flight (0 <= k < D)
template <int D, int L>
__device__ inline void wait_groups(int k) {
  static_assert(D <= 9, "ring depth");
  switch (k) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<L>(); break;
    case 2: if constexpr (D > 2) wait_vm<2 * L>(); break;
    case 3: if constexpr (D > 3) wait_vm<3 * L>(); break;
    case 4: if constexpr (D > 4) wait_vm<4 * L>(); break;
    case 5: if constexpr (D > 5) wait_vm<5 * L>(); break;
    case 6: if constexpr (D > 6) wait_vm<6 * L>(); break;
    case 7: if constexpr (D > 7) wait_vm<7 * L>(); break;
    default: wait_vm<0>(); break;
  }
}

// OFF: a byte offset known at compile time, carried in the instruction's
// offset field (so the ring slot and the slice cost no address arithmetic)
template <int OFF>
__device__ inline u32x4 lds_read16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  u32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
#else
  v = u32x4{addr, 0, 0, 0};   // host pass only (never executed)
#endif
  return v;
}
__device__ inline void lds_wait() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
}
// makes the value depend on the preceding lds_wait
__device__ inline void after_wait(u32x4& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
}

template <int OFF>
__device__ inline uint32_t lds_read4(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  uint32_t v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
#else
  v = addr;   // host pass only (never executed)
#endif
  return v;
}

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
__device__ inline void after_wait(uint32_t& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
}

// One step of one wave = one 128-wide group: the staging slot holds, in this
// order, the NT weight chunks (1 KB each, lane l's 16 bytes at 16 l), the
// activation rows of the group (4 * MB rows, 1 KB per 4 rows) and a 1 KB
// block copied by one 16-byte-per-lane copy: the scale-pair words of the
// workgroup's 16 * NT channels (64 NT bytes) and their zero-point bytes
// (16 NT bytes), preceded for MB = 0 by the single row of one token (256 B).
// One copy instead of three keeps the per-group copy count (each copy
// instruction costs the address unit the same whatever its width) at NT + 1
// for one token and NT + MB + 1 otherwise.
constexpr int slot_bytes(int NT, int MB) { return NT * 1024 + (MB == 0 ? 0 : MB * 1024) + 1024; }

template <int NT, int MB>
struct Slot {
  static constexpr int kW = 0;
  static constexpr int kX = NT * 1024;                          // activation rows
  static constexpr int kC = kX + (MB == 0 ? 0 : MB * 1024);    // the combined 1 KB copy
  static constexpr int kS = kC + (MB == 0 ? 256 : 0);          // scale words
  static constexpr int kZ = kS + 64 * NT;                      // zero-point bytes
  static constexpr int kBytes = slot_bytes(NT, MB);
  static constexpr int kLoads = NT + (MB == 0 ? 0 : MB) + 1;   // copies a wave issues per step
  static constexpr int kRows = MB == 0 ? 1 : 4 * MB;
  static_assert(kZ + 16 * NT <= kC + 1024, "the combined copy's block");
};

constexpr int kGemvLdsBudget = 60 * 1024;
// Depth of each wave's ring of staging slots: as deep as the workgroup's LDS
// budget allows (D - 1 groups of copies in flight while one group is
// multiplied), at least 2 and at most 9.  Measured on the Llama-2 7B / 70B
// decode layers with weights streamed from HBM: 8 waves per workgroup with
// 1 - 2 groups in flight each stream best; deeper rings (more copies in flight
// per compute unit, fewer workgroups per compute unit) are slower, as for a
// plain streaming read.  The one-token slot (MB = 0) takes the depth of the
// four-row slot: the depth is about copies in flight, not LDS space.
// (the depth keeps its calibration: the budget over NT + 1.5 + max(MB, 1) KB
// per slot, the slot size the depths were measured with)
constexpr int ring_depth_of(int NT, int MB, int NW) {
  const int d = kGemvLdsBudget / (NW * (NT * 1024 + 512 + (MB == 0 ? 1 : MB) * 1024));
  return d > 9 ? 9 : d < 2 ? 2 : d;
}
template <int NT, int MB, int NW>
constexpr int ring_depth() {
  return ring_depth_of(NT, MB, NW);
}
// LDS of one workgroup (its staging rings)
constexpr int gemv_lds_bytes(int NT, int MB, int NW) { return NW * ring_depth_of(NT, MB, NW) * slot_bytes(NT, MB); }

// NT: 16-column slices per workgroup; MB: blocks of 4 activation rows staged
// per group (4 * MB >= M; 0: the one row of M = 1); NW: waves per workgroup
// (they split K).
//
// The arguments are separate scalars, in the order the kernel first needs
// them, so that the leading ones can be preloaded into scalar registers at
// wave launch instead of read from the argument segment (two dependent
// memory round trips before the first copy); Y, needed only at the end, is
// read from memory as usual.
template <bool BF16, int NT, int MB, int NW>
__global__ __launch_bounds__(64 * NW) void q4_gemv_kernel(const uint4* W, const uint16_t* X, const uint32_t* S,
                                                          const uint8_t* Z, int K, int Np, int M, int N, uint16_t* Y) {
  GemvArgs a;
  a.X = X;
  a.M = M;
  a.K = K;
  a.N = N;
  a.Np = Np;
  a.Kp = 0;
  a.W = W;
  a.S = S;
  a.Z = Z;
  a.Y = Y;
  using SL = Slot<NT, MB>;
  constexpr int D = ring_depth<NT, MB, NW>();
  constexpr int kWaveBytes = D * SL::kBytes;
  static_assert(kWaveBytes >= NT * 64 * 16, "the reduction reuses a wave's staging area");
  static_assert(NW * kWaveBytes == gemv_lds_bytes(NT, MB, NW), "the plan's LDS figure");
  static_assert(NT == 1 || NT == 2 || NT == 4, "slices per workgroup");
  __shared__ __align__(1024) uint8_t lds_all[NW * kWaveBytes];

  // the wave index is uniform; saying so keeps the K loop a scalar loop
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int cl = lane & 15, blk = lane >> 4;
  const int G = a.K / kGroup;
  const int gpw = (G + NW - 1) / NW;                             // groups per wave
  const int g0 = min(G, wave * gpw), g1 = min(G, g0 + gpw);
  uint8_t* ring = lds_all + wave * kWaveBytes;
  // Column block of this workgroup.  Workgroups are dealt round-robin to the
  // 8 XCDs, each with its own L2; neighbouring blocks share the 128-byte lines
  // of the scale and zero-point rows, so consecutive blocks go to one XCD
  // (otherwise up to 8 L2s would each fetch the same line).
  const int full = (int)((uint32_t)Np / (16 * NT)) & ~7;       // of the grid's Np / (16 NT) workgroups
  const int cb = (int)blockIdx.x < full ? (blockIdx.x & 7) * (full >> 3) + (blockIdx.x >> 3) : blockIdx.x;

  // Global sources of this lane's copies.  The weight and activation copies
  // address a workgroup-uniform base (advanced per group in scalar registers)
  // plus a 32-bit lane offset that stays fixed, so advancing costs no vector
  // instructions.  Weights: lane l of slice t reads channel
  // (cb NT + t) 16 + l % 16 of K-block l / 16 (uint4 units: + 4 Np per group).
  const size_t np = a.Np;
  const char* wbase = reinterpret_cast<const char*>(a.W + (size_t)cb * NT * 16);
  uint32_t wlane[NT];                                       // < 64 Np bytes
#pragma unroll
  for (int t = 0; t < NT; ++t) wlane[t] = (uint32_t)(blk * np + cl) * 16u + t * 256u;
  // The combined copy: lane l copies 16 bytes.  For MB = 0, lanes 0..15 copy
  // the token's 16-byte pieces of the group, then (from lane c0 = 16 for
  // MB = 0, 0 otherwise) 4 NT lanes copy the scale words of the workgroup's
  // channels (4 each) and NT lanes their zero-point bytes (16 each); the
  // remaining lanes repeat lane c0's source.  Per group, a lane's source
  // moves by g * cg + (g / 2) * cp bytes.
  const int n0 = cb * NT * 16;                              // first channel of the workgroup
  constexpr int c0 = MB == 0 ? 16 : 0;
  const char* csrc;
  uint32_t cg = 0, cp = 0;
  {
    const int j = lane - c0;
    if (MB == 0 && lane < 16) {
      csrc = reinterpret_cast<const char*>(a.X) + 16 * lane;
      cg = 2 * kGroup;
    } else if (j >= 0 && j < 4 * NT) {
      csrc = reinterpret_cast<const char*>(a.S + n0) + 16 * j;
      cp = 4 * (uint32_t)np;
    } else if (j >= 4 * NT && j < 5 * NT) {
      csrc = reinterpret_cast<const char*>(a.Z + n0) + 16 * (j - 4 * NT);
      cp = (uint32_t)np;
    } else {
      csrc = reinterpret_cast<const char*>(a.S + n0);
      cp = 4 * (uint32_t)np;
    }
  }
  // the zero-point byte of a channel is read as the aligned word holding it
  const int zshift = 8 * (cl & 3);                          // channel bases are multiples of 16
  // Activation rows (MB >= 1): lane l copies row r = 4b + l/16 of block b
  // into stored piece l % 16, which holds the row's logical 16-byte piece
  // (l % 16) ^ r (rows at or past M repeat row M - 1: a valid load whose
  // products only reach output rows that are never stored).  The one row of
  // MB = 0 travels in the combined copy, unswizzled (row 0's key is 0).
  constexpr int kXB = MB == 0 ? 1 : MB;
  uint32_t xlane[kXB];                                      // bytes from a.X + 256 g
#pragma unroll
  for (int b = 0; b < kXB; ++b) {
    const int r = 4 * b + blk;
    xlane[b] = ((uint32_t)min(r, a.M - 1) * (uint32_t)a.K + ((cl ^ r) & 15) * 8) * 2u;
  }

  // LDS byte addresses of this lane's reads inside slot 0
  typedef __attribute__((address_space(3))) uint8_t* lds_ptr;
  const uint32_t rbase = (uint32_t)(uintptr_t)(lds_ptr)ring;
  const uint32_t w_rd = rbase + SL::kW + lane * 16;
  const uint32_t s_rd = rbase + SL::kS + cl * 4;          // + 64 * t for slice t
  const uint32_t z_rd = rbase + SL::kZ + (cl & ~3);       // + 16 * t for slice t
  // A operand of the 16x16x32 MFMA: lane l supplies row l % 16, k values
  // 8 * (l / 16) .. +8 of each 32-wide k step j, i.e. logical piece 4*blk + j
  const int rr = min(cl, SL::kRows - 1);
  uint32_t x_rd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x_rd[j] = rbase + SL::kX + rr * 256 + (((4 * blk + j) ^ rr) & 15) * 16;

  // the copies of group g (inside the wave's range) into ring slot `slot`;
  // groups are issued in increasing order, one after the other, and the
  // combined copy's source (a different array per lane) advances by cg per
  // group and cp per pair of groups
  const char* cnext = csrc + (size_t)g0 * cg + (size_t)(g0 >> 1) * cp;
  auto issue = [&](int g, int slot) {
    uint8_t* dst = ring + slot * SL::kBytes;
    const char* wg = wbase + (size_t)g * 64 * np;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      wlane[t] = lane_offset(wlane[t]);
      load_lds16_stream(wg + wlane[t], dst + SL::kW + t * 1024);
    }
    if constexpr (MB > 0) {
      const char* xg = reinterpret_cast<const char*>(a.X) + (size_t)g * 2 * kGroup;
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        xlane[b] = lane_offset(xlane[b]);
        load_lds16(xg + xlane[b], dst + SL::kX + b * 1024);
      }
    }
    load_lds16(cnext, dst + SL::kC);
    cnext += cg + ((g & 1) ? cp : 0u);
  };

  // the unpacking constants in registers (one v_and_or_b32 per register of
  // 2 codes; a three-operand instruction takes no 32-bit literal here)
  uint32_t umask, umagic;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(umask));
  asm volatile("s_mov_b32 %0, %1" : "=s"(umagic) : "i"(BF16 ? 0x43004300 : 0x64006400));
#else
  umask = 0x000F000Fu;
  umagic = BF16 ? 0x43004300u : 0x64006400u;
#endif

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int g, auto SLOT) {
    constexpr int so = decltype(SLOT)::value * SL::kBytes;
    u32x4 xa[4], wv[NT];
    uint32_t sv[NT], zv[NT];
#pragma unroll
    for (int j = 0; j < 4; ++j) xa[j] = lds_read16<so>(x_rd[j]);
    static_for<0, NT>([&](auto T) {
      constexpr int t = decltype(T)::value;
      wv[t] = lds_read16<so + t * 1024>(w_rd);
      sv[t] = lds_read4<so + t * 64>(s_rd);
      zv[t] = lds_read4<so + t * 16>(z_rd);
    });
    lds_wait();
#pragma unroll
    for (int j = 0; j < 4; ++j) after_wait(xa[j]);
    const int h = g & 1;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      after_wait(wv[t]);
      after_wait(sv[t]);
      after_wait(zv[t]);
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(sv[t] >> (16 * h)));
      const uint32_t nz = neg_offset_pair<BF16>(__builtin_amdgcn_ubfe(zv[t], zshift + 4 * h, 4));
      const uint4 bz = make_uint4(nz, nz, nz, nz);
      f32x4 t0 = {0.0f, 0.0f, 0.0f, 0.0f};
      uint4 wu[4];
      unpack16(wv[t][0], wv[t][1], umask, umagic, wu[0], wu[1]);
      unpack16(wv[t][2], wv[t][3], umask, umagic, wu[2], wu[3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 x = __builtin_bit_cast(uint4, xa[j]);
        t0 = mfma<BF16>(x, wu[j], t0);
        t0 = mfma<BF16>(x, bz, t0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += s * t0[i];
    }
  };

  // prologue: groups g0 .. g0 + D - 2 in flight (those inside the range)
#pragma unroll
  for (int i = 0; i < D - 1; ++i)
    if (g0 + i < g1) issue(g0 + i, i);
  // the loop is unrolled over the D ring slots, so that every slot offset is
  // a constant of the instructions that read it
  int g = g0;
  while (g < g1) {
    static_for<0, D>([&](auto SLOT) {
      constexpr int slot = decltype(SLOT)::value;
      if (g < g1) {
        // refill the slot the previous group was read from (its reads
        // finished before its arithmetic) with group g + D - 1, then wait
        // until group g's copies have landed: the groups issued after it may
        // stay in flight
        if (g + D - 1 < g1) {
          issue(g + D - 1, slot == 0 ? D - 1 : slot - 1);
          wait_vm<(D - 1) * SL::kLoads>();
        } else {
          wait_groups<D, SL::kLoads>(g1 - 1 - g);
        }
        __builtin_amdgcn_sched_barrier(0);
        compute(g, SLOT);
        __builtin_amdgcn_sched_barrier(0);
        ++g;
      }
    });
  }
  wait_vm<0>();                           // no copy may still target the staging area

  // ---- add the waves' tiles (each in its own staging area); lane l holds
  // rows 4*(l/16) + i of column l % 16
  f32x4* red = reinterpret_cast<f32x4*>(ring);
#pragma unroll
  for (int t = 0; t < NT; ++t) red[t * 64 + lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < NW; ++w)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 o = reinterpret_cast<const f32x4*>(lds_all + w * kWaveBytes)[t * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += o[i];
    }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (cb * NT + t) * 16 + cl;
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

template <bool BF16, int NT, int MB>
hipError_t launch_cfg(const GemvArgs& a, const GemvPlan& P, hipStream_t st) {
  const dim3 grid(a.Np / (16 * NT));
  if (P.waves == 8)
    hipLaunchKernelGGL((q4_gemv_kernel<BF16, NT, MB, 8>), grid, dim3(512), 0, st, a.W, a.X, a.S, a.Z, a.K, a.Np, a.M,
                       a.N, a.Y);
  else
    hipLaunchKernelGGL((q4_gemv_kernel<BF16, NT, MB, 4>), grid, dim3(256), 0, st, a.W, a.X, a.S, a.Z, a.K, a.Np, a.M,
                       a.N, a.Y);
  return hipGetLastError();
}

// activation-row blocks staged per group for M tokens: 0 (one row), 1, 2 or 4
inline int row_blocks(int M) { return M == 1 ? 0 : M <= 4 ? 1 : M <= 8 ? 2 : 4; }

template <bool BF16, int NT>
hipError_t launch_nt(const GemvArgs& a, const GemvPlan& P, hipStream_t st) {
  switch (row_blocks(a.M)) {
    case 0: return launch_cfg<BF16, NT, 0>(a, P, st);
    case 1: return launch_cfg<BF16, NT, 1>(a, P, st);
    case 2: return launch_cfg<BF16, NT, 2>(a, P, st);
    default: return launch_cfg<BF16, NT, 4>(a, P, st);
  }
}

template <bool BF16>
hipError_t launch_dtype(const GemvArgs& a, const GemvPlan& P, hipStream_t st) {
  switch (P.nt) {
    case 4: return launch_nt<BF16, 4>(a, P, st);
    case 2: return launch_nt<BF16, 2>(a, P, st);
    default: return launch_nt<BF16, 1>(a, P, st);
  }
}

}  // namespace

GemvPlan plan_q4_gemv(int M, int N, int K) {
  constexpr int kCUs = 256, kLdsPerCU = 160 * 1024;     // MI355X
  GemvPlan P;
  const Q4Layout L = q4_layout(N, K);
  const int slices = L.Np / 16;
  // widest column block that still leaves a workgroup for every compute unit;
  // except for one token and a short K (at most 4 groups a wave), where one
  // slice per workgroup (three resident per compute unit) overlaps the
  // workgroups' fixed start and finish
  const int gpw = (K / kGroup + 7) / 8;
  if (M == 1 && gpw <= 4)
    P.nt = 1;
  else
    P.nt = (slices / 4 >= kCUs) ? 4 : (slices / 2 >= kCUs) ? 2 : 1;
  // eight waves, except with four slices (the widest 70B layer), where four
  // waves measured 4-9% faster; and four when the eight-wave workgroups
  // would not all be resident at once (their rings take too much LDS for
  // the grid to fit on the compute units in one round: 16 tokens on the
  // 4096 x 11008 layer measured 13.2 us with eight waves in two rounds).
  // With 16 staged rows, whose copies then outweigh the weights', such a
  // grid also takes twice the slices (half the activation copies): 12 and
  // 16 tokens on the 4096 x 11008 layer 9.6 -> 8.8 and 10.1 -> 8.9 us.
  P.waves = P.nt == 4 ? 4 : 8;
  const int grid = slices / P.nt;
  if (P.waves == 8 && grid > kCUs * (kLdsPerCU / gemv_lds_bytes(P.nt, row_blocks(M), 8))) {
    P.waves = 4;
    if (row_blocks(M) == 4 && P.nt == 2) P.nt = 4;
  }
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
