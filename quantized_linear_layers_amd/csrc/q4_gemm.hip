// W4A16 GEMM for M > 16 (batched decode to prefill): Y = X · dequant(W)ᵀ on
// 16-bit MFMA.  Described here for the prefill tile; the tile configurations
// for fewer tokens (Cfg below) split K among the waves instead.
//
// With many tokens the layer is compute-bound ([LQ] "带宽与算力：Roofline":
// the arithmetic intensity grows with the token count), and the dequant is
// extra vector work competing with the matrix unit ([LQ] W4A16 section: at
// large batch a naive W4A16 kernel can lose to fp16).  The kernel therefore
// spends the vector ALU on nothing but the dequant and amortizes each
// dequantized weight over as many tokens as the register file allows:
//
//   * a workgroup owns a 256 x 256 tile of Y; each of its 8 waves (two per
//     SIMD, so one multiplies while the other waits) owns all 256 rows x 32
//     columns (8 tiles of v_mfma_f32_32x32x16_{bf16,f16}), so every weight a
//     wave dequantizes feeds 8 MFMAs and no weight is dequantized twice in a
//     workgroup;
//   * K advances in blocks of 64 through a ring of 3 LDS stages filled by
//     global_load_lds (no register staging), two blocks ahead: the X tile
//     (shared by the 8 waves; 16-byte pieces XOR-swizzled by row so the MFMA
//     operand reads spread over the banks), and per wave its still-packed
//     weight chunks and the group's scale and zero-point words;
//   * the codes stay packed until they are in registers ([QK] §9.5) and are
//     expanded there with the group's scale and zero point to
//     s * (q - z) (exact in fp32: both products are exact and so is their
//     difference), rounded once to the MFMA's 16-bit type ([LQ] W4A16
//     section: dequant of a K tile with the tile's group scale, then the
//     product);
//   * inside a 32-wide chunk the two MFMA k-steps take k values in the order
//     (lane half h, step s) -> 8 * (2h + s) .. +8, for X and W alike; a
//     consistent permutation of k leaves every dot product unchanged, and it
//     lets each lane read its 8 codes of both steps as one 8-byte word pair.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "ql_internal.h"


namespace ql {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;
constexpr int kNTW = 1;                         // 32-column MFMA tiles per wave

// Tile configuration.  A workgroup owns BM = 32 MT rows x BN = 32 WN columns
// of Y.  Its WN * WK waves form WK K-groups of WN waves: the K-groups take
// consecutive, equal runs of the K blocks (the workgroup's split of K), each
// with its own X tile in every LDS stage; the WN waves of a K-group share
// that X tile and own 32 columns each.  With WK > 1 the K-groups add their
// partial tiles in LDS at the end.  Prefill uses <8, 8, 1>: one K-group, all
// 256 rows per wave; fewer tokens use smaller square tiles with the K range
// split among the waves, so that a layer still yields hundreds of workgroups.
template <int MT_, int WN_, int WK_, int ST_>
struct Cfg {
  static constexpr int kMT = MT_;               // 32-row MFMA tiles per wave (every wave spans all BM rows)
  static constexpr int WN = WN_, WK = WK_;
  static constexpr int kStages = ST_;
  static constexpr int BM = 32 * kMT, BN = 32 * WN * kNTW;
  static constexpr int kWaves = WN * WK;
  static constexpr int kATile = BM * BK * 2;             // X tile of one K-group and stage: BM rows x 128 bytes
  static constexpr int kBWave = 2 * 32 * kNTW * 16;      // packed weights of one wave: 2 chunks x 32 columns x 16 B
  static constexpr int kSZWave = 2 * 32 * kNTW * 4;      // scale words, then zero-point words, of one wave
  static constexpr int kBOff = kATile;
  static constexpr int kSZOff = kBOff + WN * kBWave;
  static constexpr int kKGroup = kSZOff + WN * kSZWave;  // one K-group's part of a stage
  static constexpr int kStage = WK * kKGroup;
  static constexpr int kLds = kStages * kStage;
  static constexpr int kAFills = kATile / 1024 / WN;     // 1 KB X blocks per wave and stage
  static constexpr int kLoads = kAFills + 2 * kNTW;      // copies per wave and stage
  static constexpr int kXBuf = kWaves >= 8 ? 1 : 2;      // X fragment buffers per wave
  static constexpr int kRed = (WK - 1) * WN * kMT * 4096;  // partial tiles of K-groups 1 .. WK-1
  // refill copies spread over the k steps (small tiles), or all issued at
  // once after the barrier (the prefill tile: there the second wave of each
  // SIMD covers the issue, and spreading them measured 1.6% slower)
  static constexpr bool kSpread = kMT < 8;
  static_assert(kAFills >= 1 && kATile % (1024 * WN) == 0, "X blocks per wave");
  static_assert(kRed <= kLds, "the K-group reduction reuses the stages");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
using PrefillCfg = Cfg<8, 8, 1, 3>;

struct GemmArgs {
  const uint16_t* X;
  int M, K, N, Np;         // N, Np: this launch's columns (real, padded)
  int ldw, ldy;            // row strides in columns of the blob's rows and of Y
  const uint4* W;          // [Kp/32][ldw] chunks
  const uint32_t* S;       // [Kp/256][ldw] scale pairs
  const uint8_t* Z;        // [Kp/256][ldw] zero pairs
  uint16_t* Y;             // [M][ldy]
  int kbs;                 // K blocks per split: split s = blockIdx.y takes blocks s * kbs .. (s + 1) * kbs - 1
  float* P;                // split-K partial tiles [gridDim.y][M][ldy] (fp32), or null: store Y
};

// ---- global -> LDS copies and counter waits
__device__ inline void load_lds16(const void* src, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#else
  (void)src;
  (void)lds;
#endif
}
__device__ inline void load_lds4(const void* src, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
#else
  (void)src;
  (void)lds;
#endif
}
template <int N>
__device__ inline void wait_vm() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
#endif
}
// waits until at most N of this wave's LDS reads are in flight
template <int N>
__device__ inline void wait_lgkm() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4) | ((N & 0xF) << 8));
#endif
}

// LDS reads as inline assembly (the compiler would otherwise wait for every
// in-flight LDS copy before each read, including the prefetch of later
// stages); the order is enforced by wait_vm + s_barrier before a stage is
// read and wait_lgkm + after_wait before the values are used.
template <int OFF>
__device__ inline u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
#else
  v = u32x4{addr, OFF, 0, 0};
#endif
  return v;
}
template <int OFF>
__device__ inline u32x2 lds_read8(uint32_t addr) {
  u32x2 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
#else
  v = u32x2{addr, OFF};
#endif
  return v;
}
template <int OFF>
__device__ inline uint32_t lds_read4(uint32_t addr) {
  uint32_t v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
#else
  v = addr + OFF;
#endif
  return v;
}
template <typename T>
__device__ inline void after_wait(T& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#else
  (void)v;
#endif
}

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// two floats -> one register of two 16-bit values (round to nearest even)
template <bool BF16>
__device__ inline uint32_t pack2(float lo, float hi) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

// a constant materialized in a vector register, out of the optimizer's sight
__device__ inline uint32_t in_vgpr(uint32_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(v));
#endif
  return v;
}

// The 4-, 8- and 12-bit right shifts of a pair of code words, each as one
// 64-bit shift of the pair: one instruction per count serves both words (the
// bits that the low word receives from the high one land outside the mask
// dequant8 applies).  Measured on the 4096 x 4096 x 14336 prefill layer:
// 443.3 -> 438.2 us, 512 tokens on 4096 x 11008 59.6 -> 57.9 us, outputs
// bit-identical.
__device__ inline void shift_pair(u32x2 w, uint64_t& s4, uint64_t& s8, uint64_t& s12) {
  const uint64_t p = ((uint64_t)w[1] << 32) | w[0];
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
}

// One word of 8 codes (code i at nibble position (i & 1) * 4 + (i >> 1)),
// given as ws[r] = w >> 4r (r = 0..3), -> the MFMA B operand of 8 consecutive
// k: register r = (k 2r, k 2r + 1), each s * (q - z) rounded once to the
// 16-bit type.  Masking w >> 4r with 0x000F000F and setting the bits of fp16
// 1024.0 puts nibbles r and r + 4 (codes 2r and 2r + 1) into the two halves
// of a register as the exact fp16 values 1024 + q.  One fused multiply-add
// per value with its fp16 operand, (1024 + q) * s + noff, where
// noff = -(1024 + z) * s is exact in fp32 (an 11-bit integer times an fp16
// scale), yields s * (q - z) exactly (at most 15 significant bits), which is
// then rounded once to the 16-bit type.
//   mask, magic: 0x000F000F and 0x64006400 in registers (see in_vgpr), so
//   that each register takes one v_and_or_b32, which has no literal form
template <bool BF16>
__device__ inline u32x4 dequant8(const uint32_t (&ws)[4], float s, float noff, uint32_t mask, uint32_t magic) {
  u32x4 out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t h = (ws[r] & mask) | magic;
    const float lo = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu)), s, noff);
    const float hi = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16)), s, noff);
    out[r] = pack2<BF16>(lo, hi);
  }
  return out;
}

template <bool BF16>
__device__ inline f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
}

// Workgroup -> tile.  Workgroups are dealt round-robin to the 8 XCDs; when
// the tile count allows, each XCD gets a contiguous run of a grouped order
// (4 tile rows at a time), so the tiles an XCD works on at once share X rows
// and weight columns in its L2.
__device__ inline void tile_of(int bid, int tm, int tn, int& mt, int& nt) {
  const int T = tm * tn;
  const int t = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
  constexpr int GM = 4;
  const int gsize = GM * tn;
  const int first = (t / gsize) * GM;
  const int gm = min(tm - first, GM);
  mt = first + (t % gsize) % gm;
  nt = (t % gsize) / gm;
}

// Per-lane sources and LDS destinations of one wave's copies for a stage.
// Each wave copies its own weight chunks (kNTW copies of 1 KB: flat index
// f = 64 d + lane -> chunk f / (32 kNTW), column f % (32 kNTW)) and its
// scale and zero-point words (kNTW copies of 256 B: f < 32 kNTW -> scale word
// of column f, else the aligned word holding the zero byte of column
// f - 32 kNTW).  Sources are kept as 32-bit byte offsets from the (uniform)
// base pointers, one register each; every operand is below 4 GiB.
template <class C>
struct FillPlan {
  uint32_t x[C::kAFills];       // X row of each 1 KB block (+ the lane's logical piece)
  int xdst[C::kAFills];         // byte offset of the block inside the stage
  uint32_t w[kNTW];             // weight column of each chunk copy (chunk row added per block)
  int wc[kNTW];                 // chunk (0 or 1) of each chunk copy
  uint32_t sz[kNTW];            // scale word / aligned zero word of each scale copy
  bool isz[kNTW];               // the copy reads the zero-point array
  int wdst, szdst;              // byte offsets of the wave's weight and scale/zero areas
};

// copies B .. E - 1 of a wave's kLoads copies of k block kb into stage S, in
// the order: kAFills X blocks, kNTW weight chunks, kNTW scale/zero words
template <class C, int S, int B, int E>
__device__ __forceinline__ void fill_range(uint8_t* lds, const GemmArgs& a, const FillPlan<C>& f, int kb) {
  uint8_t* st = lds + S * C::kStage;
  const uint32_t pr = kb >> 2;                              // pair of groups of this k block
  const uint32_t np = a.ldw;
  static_for<B, E>([&](auto I) {
    constexpr int i = I;
    if constexpr (i < C::kAFills) {
      load_lds16(reinterpret_cast<const char*>(a.X) + f.x[i] + (uint32_t)kb * (BK * 2), st + f.xdst[i]);
    } else if constexpr (i < C::kAFills + kNTW) {
      constexpr int d = i - C::kAFills;
      load_lds16(reinterpret_cast<const char*>(a.W) + f.w[d] + (uint32_t)(2 * kb + f.wc[d]) * np * 16,
                 st + f.wdst + d * 1024);
    } else {
      constexpr int d = i - C::kAFills - kNTW;
      // scale rows hold one word per column, zero rows one byte per column
      const char* szb = f.isz[d] ? reinterpret_cast<const char*>(a.Z) : reinterpret_cast<const char*>(a.S);
      load_lds4(szb + f.sz[d] + pr * (f.isz[d] ? np : np * 4), st + f.szdst + d * 256);
    }
  });
}

template <class C, int S>
__device__ inline void fill(uint8_t* lds, const GemmArgs& a, const FillPlan<C>& f, int kb) {
  uint8_t* st = lds + S * C::kStage;
  const char* xb = reinterpret_cast<const char*>(a.X);
  const char* wb = reinterpret_cast<const char*>(a.W);
#pragma unroll
  for (int i = 0; i < C::kAFills; ++i) load_lds16(xb + f.x[i] + (uint32_t)kb * (BK * 2), st + f.xdst[i]);
  const uint32_t pr = kb >> 2;                              // pair of groups of this k block
  const uint32_t np = a.ldw;
#pragma unroll
  for (int d = 0; d < kNTW; ++d)
    load_lds16(wb + f.w[d] + (uint32_t)(2 * kb + f.wc[d]) * np * 16, st + f.wdst + d * 1024);
#pragma unroll
  for (int d = 0; d < kNTW; ++d) {
    // scale rows hold one word per column, zero rows one byte per column
    const char* szb = f.isz[d] ? reinterpret_cast<const char*>(a.Z) : reinterpret_cast<const char*>(a.S);
    load_lds4(szb + f.sz[d] + pr * (f.isz[d] ? np : np * 4), st + f.szdst + d * 256);
  }
}

template <class C>
struct Frag {
  f32x16 acc[C::kMT][kNTW];
};

// Multiplies stage S (k block kb) into the accumulators.
//   xrd[j]: LDS address (stage 0) of the lane's X piece for k step j of the
//           block (j = 2c + s); + 4096 per 32-row tile, + kStage per stage
//   wrd:    LDS address (stage 0) of the lane's 8-byte word pair of chunk 0,
//           column tile 0; + 32 kNTW * 16 per chunk, + 512 per column tile
//   szrd:   LDS address (stage 0) of the lane's scale word of column tile 0;
//           + 128 kNTW for its zero word, + 128 per column tile
//   share(j): issues the j-th share of the refill of another stage (j = 0..3,
//           at the start of k step j, after its LDS reads are issued)
template <class C, bool BF16, int S, typename Share>
__device__ __forceinline__ void compute(Frag<C>& fr, int kb, const uint32_t (&xrd)[4], uint32_t wrd, uint32_t szrd,
                               int zshift, Share&& share) {
  constexpr int kMT = C::kMT, kXBuf = C::kXBuf;
  constexpr int SO = S * C::kStage;
  const uint32_t wst = wrd + SO, szst = szrd + SO;
  // packed words (2 chunks x kNTW column tiles) and this group's scale / zero
  u32x2 wv[2][kNTW];
  uint32_t sv[kNTW], zv[kNTW];
  static_for<0, 2>([&](auto CH) {
    static_for<0, kNTW>([&](auto T) { wv[CH][T] = lds_read8<CH * 32 * kNTW * 16 + T * 512>(wst); });
  });
  static_for<0, kNTW>([&](auto T) {
    sv[T] = lds_read4<T * 128>(szst);
    zv[T] = lds_read4<128 * kNTW + T * 128>(szst);
  });
  u32x4 xa[kXBuf][kMT];
  static_for<0, kMT>([&](auto MT) { xa[0][MT] = lds_read16<MT * 4096>(xrd[0] + SO); });
  share(std::integral_constant<int, 0>{});
  wait_lgkm<0>();                                // words, scales, zeros and step 0's X landed
  const int h = (kb >> 1) & 1;                   // group of the block inside its pair
  float s[kNTW], nzs[kNTW];
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    after_wait(wv[0][t]);
    after_wait(wv[1][t]);
    after_wait(sv[t]);
    after_wait(zv[t]);
    s[t] = (float)__builtin_bit_cast(_Float16, (uint16_t)(sv[t] >> (16 * h)));
    nzs[t] = -(1024.0f + (float)((zv[t] >> (zshift + 4 * h)) & 0xFu)) * s[t];   // exact
  }
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) after_wait(xa[0][mt]);
  // B operands of step j: chunk j / 2, word j % 2 of the lane's pair
  u32x4 b[2][kNTW];
  const uint32_t mask = in_vgpr(0x000F000Fu), magic = in_vgpr(0x64006400u);
  // shifted code words: chunk c's pair now, chunk 1's when step 2 is dequantized
  uint64_t sh4[2][kNTW], sh8[2][kNTW], sh12[2][kNTW];
  auto shifted = [&](int c, int i, int t, uint32_t(&ws)[4]) {
    ws[0] = wv[c][t][i];
    ws[1] = (uint32_t)(sh4[c][t] >> (32 * i));
    ws[2] = (uint32_t)(sh8[c][t] >> (32 * i));
    ws[3] = (uint32_t)(sh12[c][t] >> (32 * i));
  };
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    shift_pair(wv[0][t], sh4[0][t], sh8[0][t], sh12[0][t]);
    uint32_t ws[4];
    shifted(0, 0, t, ws);
    b[0][t] = dequant8<BF16>(ws, s[t], nzs[t], mask, magic);
  }
  static_for<0, 4>([&](auto J) {
    constexpr int j = J;
    constexpr int cur = kXBuf == 2 ? (j & 1) : 0;
    if constexpr (kXBuf == 1 && j > 0) {
      // one X buffer (two waves per SIMD hide the read latency)
      static_for<0, kMT>([&](auto MT) { xa[0][MT] = lds_read16<MT * 4096>(xrd[j] + SO); });
      share(J);
      wait_lgkm<0>();
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) after_wait(xa[0][mt]);
    }
    if constexpr (kXBuf == 2 && j > 0) share(J);
    // X of step j + 1 in flight while step j multiplies
    if constexpr (kXBuf == 2 && j < 3)
      static_for<0, kMT>([&](auto MT) { xa[cur ^ 1][MT] = lds_read16<MT * 4096>(xrd[j + 1] + SO); });
    // one scheduling region: the MFMAs of step j interleaved with the dequant
    // of step j + 1 (vector ALU work in the shadow of the matrix unit)
    if constexpr (j < 3) {
#pragma unroll
      for (int t = 0; t < kNTW; ++t) {
        if constexpr (j == 1) shift_pair(wv[1][t], sh4[1][t], sh8[1][t], sh12[1][t]);
        uint32_t ws[4];
        shifted((j + 1) >> 1, (j + 1) & 1, t, ws);
        b[(j & 1) ^ 1][t] = dequant8<BF16>(ws, s[t], nzs[t], mask, magic);
      }
    }
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int t = 0; t < kNTW; ++t) fr.acc[mt][t] = mfma<BF16>(xa[cur][mt], b[j & 1][t], fr.acc[mt][t]);
    if constexpr (j < 3) {
#if defined(__HIP_DEVICE_COMPILE__)
      static_for<0, kMT * kNTW>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three VALU
      });
#endif
      if constexpr (kXBuf == 2) {
        wait_lgkm<0>();
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) after_wait(xa[cur ^ 1][mt]);
      }
    }
  });
}

// Step i of a K-group's run (the run's block kb0 + i, present if i < cnt):
// wait for its copies, refill the stage read one step earlier with the block
// kStages - 1 steps ahead (clamped to the layer's last block kblast: a valid
// copy that is never multiplied), then multiply.  Every wave of the workgroup
// takes the same number of steps, so the barriers match.
template <class C, bool BF16, int S>
__device__ __forceinline__ void kstep(uint8_t* lds, Frag<C>& fr, const GemmArgs& a, const FillPlan<C>& f, int i,
                                      int kb0, int cnt, int kblast, const uint32_t (&xrd)[4], uint32_t wrd,
                                      uint32_t szrd, int zshift) {
  // this wave's copies of step i have landed once only the later steps' remain
  wait_vm<(C::kStages - 2) * C::kLoads>();
  __builtin_amdgcn_s_barrier();   // every wave's copies of step i landed; step i - 1 fully read
  constexpr int F = (S + C::kStages - 1) % C::kStages;
  const int kbf = min(kb0 + i + C::kStages - 1, kblast);
  // with kSpread the refill's copies go out in four shares, one per k step:
  // a wave stalls on a copy until the address unit takes it, and issuing
  // them all at once after the barrier held a small tile's arithmetic back
  constexpr int kQ = C::kLoads / 4, kR = C::kLoads % 4;     // the first kR shares take one more
  auto share = [&](auto J) {
    constexpr int q = J;
    constexpr int b = q * kQ + (q < kR ? q : kR), e = b + kQ + (q < kR ? 1 : 0);
    fill_range<C, F, b, e>(lds, a, f, kbf);
  };
  if constexpr (!C::kSpread) {
    fill<C, F>(lds, a, f, kbf);
    if (i < cnt) compute<C, BF16, S>(fr, kb0 + i, xrd, wrd, szrd, zshift, [](auto) {});
  } else if (i < cnt) {
    compute<C, BF16, S>(fr, kb0 + i, xrd, wrd, szrd, zshift, share);
  } else {
    fill<C, F>(lds, a, f, kbf);
  }
}

// The arguments the K loop needs are separate scalars, first in the list, so
// that they are preloaded into scalar registers at wave launch; the output
// pointers and stride follow, read from memory as usual (needed at the end).
template <class C, bool BF16>
__global__ __launch_bounds__(64 * C::kWaves) void q4_gemm_kernel(const uint4* W, const uint16_t* X, const uint32_t* S,
                                                                 const uint8_t* Z, int M, int K, int N, int Np,
                                                                 int ldw, int kbs, uint16_t* Y, float* P, int ldy) {
  GemmArgs a;
  a.X = X;
  a.M = M;
  a.K = K;
  a.N = N;
  a.Np = Np;
  a.ldw = ldw;
  a.ldy = ldy;
  a.W = W;
  a.S = S;
  a.Z = Z;
  a.Y = Y;
  a.kbs = kbs;
  a.P = P;
  constexpr int kMT = C::kMT, kAFills = C::kAFills, kStages = C::kStages;
  __shared__ __align__(1024) uint8_t lds[C::kLds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % C::WN, wk = wave / C::WN;          // column slot and K-group of this wave
  int mtile, ntile;
  tile_of(blockIdx.x, (a.M + C::BM - 1) / C::BM, (a.N + C::BN - 1) / C::BN, mtile, ntile);
  const int m0 = mtile * C::BM, n0 = ntile * C::BN;
  const int nw0 = n0 + 32 * kNTW * wn;           // first column of this wave
  const int kblast = a.K / BK - 1;
  // this workgroup's split of K: blocks sb0 .. sb0 + nkb - 1 (possibly none)
  const int sb0 = min(kblast + 1, (int)blockIdx.y * a.kbs);
  const int nkb = min(kblast + 1, sb0 + a.kbs) - sb0;
  // this K-group's run of blocks: kb0 .. kb0 + cnt - 1 (every run takes `steps` steps)
  const int steps = (nkb + C::WK - 1) / C::WK;
  const int kb0 = sb0 + min(nkb, wk * steps), cnt = min(sb0 + nkb, kb0 + steps) - kb0;
  const int kgoff = wk * C::kKGroup;             // this K-group's part of every stage

  // ---- copy plan.  X: the stage's 32 blocks of 1 KB (8 rows x 128 bytes),
  // kAFills per wave; lane l writes row 8b + l / 8, stored piece l % 8,
  // which holds logical piece (l % 8) ^ ((row >> 1) & 7): the 16 rows one
  // operand read serves at a time then touch 16 different 16-byte bank groups
  // (two consecutive 128-byte rows span the 64 banks once).  Rows past M
  // repeat row M - 1 and columns past Np repeat column Np - 1 (valid loads
  // whose results only reach outputs that are never stored).
  FillPlan<C> f;
#pragma unroll
  for (int i = 0; i < kAFills; ++i) {
    const int blk = wn * kAFills + i;
    const int r = blk * 8 + (lane >> 3);
    const int m = min(m0 + r, a.M - 1);
    f.x[i] = ((uint32_t)m * a.K + ((lane & 7) ^ ((r >> 1) & 7)) * 8) * 2;
    f.xdst[i] = kgoff + blk * 1024;
  }
#pragma unroll
  for (int d = 0; d < kNTW; ++d) {
    const int fl = 64 * d + lane;
    const int cw = fl % (32 * kNTW);                          // column of the chunk copy
    f.w[d] = (uint32_t)min(nw0 + cw, a.Np - 1) * 16;
    f.wc[d] = fl / (32 * kNTW);
    const int cs = fl % (32 * kNTW);                          // column of the scale / zero copy
    const int ncs = min(nw0 + cs, a.Np - 1);
    f.isz[d] = fl >= 32 * kNTW;
    f.sz[d] = f.isz[d] ? (uint32_t)(ncs & ~3) : (uint32_t)ncs * 4;
  }
  f.wdst = kgoff + C::kBOff + wn * C::kBWave;
  f.szdst = kgoff + C::kSZOff + wn * C::kSZWave;

  // ---- read addresses (stage 0)
  typedef __attribute__((address_space(3))) uint8_t* lds_ptr;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_ptr)lds;
  const int half = lane >> 5, l32 = lane & 31;
  uint32_t xrd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // step j = 2c + s takes k 32c + 8 * (2 * half + s) .. +8: logical piece 4c + 2*half + s
    const int p = 4 * (j >> 1) + 2 * half + (j & 1);
    xrd[j] = base + kgoff + l32 * 128 + ((p ^ ((l32 >> 1) & 7)) * 16);
  }
  const uint32_t wrd = base + f.wdst + l32 * 16 + half * 8;      // + 512 per column tile, + 32 kNTW * 16 per chunk
  const uint32_t szrd = base + f.szdst + l32 * 4;                // + 128 per column tile, + 128 kNTW for zeros
  const int zshift = 8 * (l32 & 3);                              // the column's byte inside its word

  Frag<C> fr;
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int t = 0; t < kNTW; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) fr.acc[i][t][e] = 0.0f;

  // prologue: steps 0 .. kStages - 2 in flight (clamped to the last block)
  static_for<0, kStages - 1>([&](auto J) { fill<C, J>(lds, a, f, min(kb0 + (int)J, kblast)); });

  int i = 0;
  for (; i + kStages <= steps; i += kStages)
    static_for<0, kStages>(
        [&](auto S) { kstep<C, BF16, S>(lds, fr, a, f, i + S, kb0, cnt, kblast, xrd, wrd, szrd, zshift); });
  static_for<0, kStages - 1>([&](auto S) {
    if (i + S < steps) kstep<C, BF16, S>(lds, fr, a, f, i + S, kb0, cnt, kblast, xrd, wrd, szrd, zshift);
  });
  wait_vm<0>();                                  // no copy may still target LDS at exit

  if constexpr (C::WK > 1) {
    // K-groups 1 .. WK-1 leave their partial tiles in LDS (16 bytes per lane
    // and 4 accumulators); K-group 0 adds them and stores
    __syncthreads();                             // every stage fully read
    if (wk > 0) {
      uint8_t* red = lds + ((wk - 1) * C::WN + wn) * (kMT * 4096);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(red + mt * 4096 + q * 1024 + lane * 16) =
              f32x4{fr.acc[mt][0][4 * q], fr.acc[mt][0][4 * q + 1], fr.acc[mt][0][4 * q + 2], fr.acc[mt][0][4 * q + 3]};
    }
    __syncthreads();
    if (wk > 0) return;
    for (int w = 1; w < C::WK; ++w) {
      const uint8_t* red = lds + ((w - 1) * C::WN + wn) * (kMT * 4096);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(red + mt * 4096 + q * 1024 + lane * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) fr.acc[mt][0][4 * q + e] += v[e];
        }
    }
  }

  // ---- store: acc element e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32; with a K split the fp32 partial tile goes to the split's
  // slice of P instead (added and rounded by splitk_reduce_kernel)
  float* part = a.P ? a.P + (size_t)blockIdx.y * splitk_slice((size_t)a.M * a.ldy) : nullptr;
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    const int n = nw0 + 32 * t + l32;
    if (n >= a.N) continue;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * mt + 8 * (e >> 2) + 4 * half + (e & 3);
        if (m < a.M) {
          const float v = fr.acc[mt][t][e];
          if (part)
            part[(size_t)m * a.ldy + n] = v;
          else
            a.Y[(size_t)m * a.ldy + n] =
                BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
        }
      }
  }
}

// Y = the 16-bit rounding of the sum of the S fp32 partial results P[s]
// (split s of K, at P + s * splitk_slice(MN): every slice 16-byte aligned),
// added in split order: 4 consecutive elements per thread, the last partial
// group element by element.
// Adds the S partial tiles in split order and rounds once.  S is a template
// argument so that a thread issues all S loads of its four elements before
// the first addition (with S a loop bound, each addition waited for its
// load: S memory round trips in a row); the order of the additions is the
// same either way.
template <bool BF16, int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, size_t MN,
                                                            uint16_t* __restrict__ Y) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  const size_t slice = splitk_slice(MN);
  auto cvt = [](float v) {
    return BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
  };
  if (i + 4 <= MN) {
    float4 v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = *reinterpret_cast<const float4*>(P + (size_t)s * slice + i);
    float4 acc = v[0];
#pragma unroll
    for (int s = 1; s < S; ++s) {
      acc.x += v[s].x;
      acc.y += v[s].y;
      acc.z += v[s].z;
      acc.w += v[s].w;
    }
    const uint2 o = make_uint2(cvt(acc.x) | ((uint32_t)cvt(acc.y) << 16), cvt(acc.z) | ((uint32_t)cvt(acc.w) << 16));
    *reinterpret_cast<uint2*>(Y + i) = o;
  } else {
    for (size_t j = i; j < MN; ++j) {
      float acc = P[j];
      for (int s = 1; s < S; ++s) acc += P[(size_t)s * slice + j];
      Y[j] = cvt(acc);
    }
  }
}

template <class C>
hipError_t launch_cfg(const GemmArgs& a, bool bf16, hipStream_t st, int splits = 1) {
  const int tiles = ((a.M + C::BM - 1) / C::BM) * ((a.N + C::BN - 1) / C::BN);
  if (bf16)
    hipLaunchKernelGGL((q4_gemm_kernel<C, true>), dim3(tiles, splits), dim3(64 * C::kWaves), 0, st, a.W, a.X, a.S, a.Z,
                       a.M, a.K, a.N, a.Np, a.ldw, a.kbs, a.Y, a.P, a.ldy);
  else
    hipLaunchKernelGGL((q4_gemm_kernel<C, false>), dim3(tiles, splits), dim3(64 * C::kWaves), 0, st, a.W, a.X, a.S, a.Z,
                       a.M, a.K, a.N, a.Np, a.ldw, a.kbs, a.Y, a.P, a.ldy);
  return hipGetLastError();
}

template <bool BF16, int S>
hipError_t launch_reduce_s(const float* P, size_t MN, uint16_t* Y, hipStream_t st) {
  const dim3 grid((unsigned)((MN + 1023) / 1024));
  hipLaunchKernelGGL((splitk_reduce_kernel<BF16, S>), grid, dim3(256), 0, st, P, MN, Y);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_reduce_t(const float* P, int S, size_t MN, uint16_t* Y, hipStream_t st) {
  switch (S) {
    case 2: return launch_reduce_s<BF16, 2>(P, MN, Y, st);
    case 3: return launch_reduce_s<BF16, 3>(P, MN, Y, st);
    case 4: return launch_reduce_s<BF16, 4>(P, MN, Y, st);
    case 5: return launch_reduce_s<BF16, 5>(P, MN, Y, st);
    case 6: return launch_reduce_s<BF16, 6>(P, MN, Y, st);
    case 7: return launch_reduce_s<BF16, 7>(P, MN, Y, st);
    case 8: return launch_reduce_s<BF16, 8>(P, MN, Y, st);
    default: return hipErrorInvalidValue;      // plans split K at most 8 ways
  }
}

hipError_t launch_reduce(const float* P, int S, size_t MN, uint16_t* Y, bool bf16, hipStream_t st) {
  return bf16 ? launch_reduce_t<true>(P, S, MN, Y, st) : launch_reduce_t<false>(P, S, MN, Y, st);
}

}  // namespace

// Workgroup tiles of the large-M kernel.  Every configuration has 8 waves
// and about 126-130 KB of LDS stages, so one workgroup fills a compute unit,
// and with few tokens its K loop runs at a near-constant time per step
// (memory round trips, not arithmetic, set the pace) until the copies of all
// the running workgroups saturate (see plan_q4_gemm).  step: that time in us,
// fitted on the Llama-2 7B / 70B layers.  The non-square tiles spend fewer
// LDS bytes per stage on activations (64 x 128 and 32 x 64: half the columns'
// share of each stage instead of four fifths, so their rings hold five
// stages); the 128 x 256 tile (8 waves of 128 rows x 32 columns, also the
// prefill's last-round tile) pays off on the wide layers from about 192
// tokens; it is only planned for 129 to 512 tokens, where it was timed.
struct TileOpt {
  int bm, bn, wk;
  double step;
};
constexpr TileOpt kTiles[] = {
    {256, 256, 1, 1.38},   // Cfg<8, 8, 1, 3>
    {128, 128, 2, 0.92},   // Cfg<4, 4, 2, 3>
    {64, 128, 2, 0.67},    // Cfg<2, 4, 2, 5>
    {64, 64, 4, 0.71},     // Cfg<2, 2, 4, 3>
    {32, 64, 4, 0.62},     // Cfg<1, 2, 4, 5>
    {32, 32, 8, 0.72},     // Cfg<1, 1, 8, 3>
    {128, 256, 1, 0.80},   // Cfg<4, 8, 1, 3> (129 to 512 tokens only)
};
constexpr int kNumTiles = (int)(sizeof(kTiles) / sizeof(kTiles[0]));

// Plan of the large-M kernel for an M x N x K product: the tile (index into
// kTiles) and the number of splits of K across workgroups.  The estimate is
// rounds x (ramp + K steps of a K-group x step time), with 256 workgroups a
// round and a ramp of 2.5 us a round.  A step takes the tile's own time or,
// when longer, the time the workgroups of a round need to copy their step's
// operands (per K-group, 128 bytes of activations per row and 32 bytes of
// packed weights per column) into LDS at 13.2 TB/s in all.  With a split,
// the reduce pass adds a launch of about 2.7 us and the partials written and
// read back at about 3.3 TB/s.  Ties go to the earlier tile and to fewer
// splits.  A split is only considered with at most 512 tokens (with more,
// the tiles alone fill the compute units).  The constants are fitted to
// every plan timed on the 7B and 70B layer shapes at 17 to 512 tokens
// (weights from HBM): the chosen plans come within 0.7% of the fastest on
// average and within 8.4% in the worst case (the previous constant-step
// model: 3.0% and 21%).
GemmPlan plan_q4_gemm(int M, int N, int K, int max_splits) {
  const long nkb = K / BK;
  GemmPlan best{0, 1, (int)nkb};
  double best_cost = 0.0;
  static const int kSplits[] = {1, 2, 3, 4, 6, 8};
  constexpr double kRamp = 2.5, kCopyBytesPerUs = 13.2e6, kReduceUs = 2.7, kPartialBytesPerUs = 3.3e6;
  for (int t = 0; t < kNumTiles; ++t) {
    const TileOpt& o = kTiles[t];
    if (o.bm == 128 && o.bn == 256 && (M <= 128 || M > 512)) continue;   // outside the range it was timed on
    const long tiles = (long)((M + o.bm - 1) / o.bm) * ((N + o.bn - 1) / o.bn);
    for (int S : kSplits) {
      if (S > max_splits || (S > 1 && (M > 512 || t == 0))) continue;
      const long kbs = (nkb + S - 1) / S;
      const long splits = (nkb + kbs - 1) / kbs;             // no empty split
      if (S > 1 && splits < 2) continue;
      const long wgs = tiles * splits;
      const double copy = (double)(wgs < 256 ? wgs : 256) * o.wk * (o.bm * 128 + o.bn * 32) / kCopyBytesPerUs;
      const double step = o.step > copy ? o.step : copy;
      double cost = (double)((wgs + 255) / 256) * (kRamp + (double)((kbs + o.wk - 1) / o.wk) * step);
      if (splits > 1) cost += kReduceUs + (double)(2 * splits * 4 + 2) * M * N / kPartialBytesPerUs;
      if ((t == 0 && S == 1) || cost < best_cost) {
        best = GemmPlan{t, (int)splits, (int)kbs};
        best_cost = cost;
      }
    }
  }
  return best;
}

size_t gemm_workspace_bytes(const GemmPlan& p, int M, int N) {
  return p.splits > 1 ? (size_t)p.splits * splitk_slice((size_t)M * N) * sizeof(float) : 0;
}

void gemm_tile_shape(const GemmPlan& p, int* rows, int* cols) {
  *rows = kTiles[p.tile].bm;
  *cols = kTiles[p.tile].bn;
}

// ---- static scratch for callers that cannot allocate (q4_gemm_no_alloc).
// Each device that loads the library holds its own copy of this array until
// the process ends.  In host code `scratch` is only a stand-in symbol: its
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_q4_gemm(const void* X, bool bf16, int M, int K, int N, const uint8_t* blob, const Q4Layout& L,
                          const GemmPlan& p, void* Y, float* ws, hipStream_t st) {
  GemmArgs a;
  a.X = static_cast<const uint16_t*>(X);
  a.M = M;
  a.K = K;
  a.N = N;
  a.Np = L.Np;
  a.ldw = L.Np;
  a.ldy = N;
  a.W = reinterpret_cast<const uint4*>(blob + L.w_off);
  a.S = reinterpret_cast<const uint32_t*>(blob + L.s_off);
  a.Z = blob + L.z_off;
  a.Y = static_cast<uint16_t*>(Y);
  a.kbs = p.kbs;
  a.P = p.splits > 1 ? ws : nullptr;
  if (p.tile != 0) {
    hipError_t e;
    switch (p.tile) {
      case 1: e = launch_cfg<Cfg<4, 4, 2, 3>>(a, bf16, st, p.splits); break;
      case 2: e = launch_cfg<Cfg<2, 4, 2, 5>>(a, bf16, st, p.splits); break;
      case 3: e = launch_cfg<Cfg<2, 2, 4, 3>>(a, bf16, st, p.splits); break;
      case 4: e = launch_cfg<Cfg<1, 2, 4, 5>>(a, bf16, st, p.splits); break;
      case 5: e = launch_cfg<Cfg<1, 1, 8, 3>>(a, bf16, st, p.splits); break;
      default: e = launch_cfg<Cfg<4, 8, 1, 3>>(a, bf16, st, p.splits); break;
    }
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_reduce(ws, p.splits, (size_t)M * N, a.Y, bf16, st);
  }
  // 256 x 256 tiles, one workgroup per compute unit.  When their last round
  // would leave at least half the compute units idle (the Llama-3-8B MLP
  // layer: 896 tiles, 3.5 rounds), the columns of that round go to a second
  // launch of 128 x 256 tiles, which fill every compute unit for about half a
  // round's time.
  constexpr int kCUs = 256;                                // MI355X
  const int tm = (M + 255) / 256, tn = (N + 255) / 256;
  const long tiles = (long)tm * tn;
  const long rounds = (tiles + kCUs - 1) / kCUs;
  const long last = tiles - (rounds - 1) * kCUs;
  const int cm = tm > 0 ? (int)(((rounds - 1) * kCUs) / tm) : 0;   // column tiles of the main launch
  const int n_off = cm * 256;
  if (rounds >= 2 && 2 * last <= kCUs && cm >= 1 && cm < tn &&
      (long)((M + 127) / 128) * ((N - n_off + 255) / 256) <= kCUs) {
    GemmArgs main = a;
    main.N = n_off;
    main.Np = n_off;
    GemmArgs tail = a;
    tail.N = N - n_off;
    tail.Np = L.Np - n_off;
    tail.W += n_off;
    tail.S += n_off;
    tail.Z += n_off;
    tail.Y += n_off;
    const hipError_t e = launch_cfg<PrefillCfg>(main, bf16, st);
    if (e != hipSuccess) return e;
    return launch_cfg<Cfg<4, 8, 1, 3>>(tail, bf16, st);
  }
  return launch_cfg<PrefillCfg>(a, bf16, st);
}

}  // namespace ql
