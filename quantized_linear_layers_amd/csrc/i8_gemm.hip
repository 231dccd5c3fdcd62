// W8A8 GEMM: int8 x int8 -> int32 on v_mfma_i32_32x32x32_i8, with the scale
// and zero-point epilogue applied to the accumulators in registers before
// the single store of the output ([VE] "一、背景": fusing it into the GEMM's
// epilogue avoids writing and re-reading the int32 result; [VE] "2.4": the
// per-token zero point is a rank-1 correction azp[m] * azp_adj[n], applied
// element-wise with O(M + N) extra memory).
//
// Each workgroup (8 waves, 4 x 2 waves of 64 x 64: two waves per SIMD, so one
// multiplies while the other waits) owns a 256 x 128 tile and walks K in
// blocks of 128 bytes through a ring of 3 LDS slots of 48 KB (one workgroup
// per compute unit).  The slots are filled straight from global memory by
// global_load_lds_dwordx4 (no register staging), two blocks ahead of the
// block being multiplied.  A block of 128 bytes makes every row segment a
// whole 128-byte line: the copies of the A and B tiles (A is re-read by every
// tile column) are what bounds this kernel, and full-line requests halve the
// number of L2 requests of 64-byte blocks (measured 7-8% faster).  Per 32-byte
// k step a wave reads 2 + 2 operand fragments for 4 MFMAs.  The epilogue
// stages each wave's outputs in LDS and writes them as 16-byte row pieces
// (full cache lines per store instruction).  Rows of a slot are 128 bytes (8
// pieces of 16 bytes) stored with the piece index XORed by row bits 1..3, so
// the 16 rows one operand read serves at a time fall on 16 different 16-byte
// bank groups.
//
// Small grids: built a second time with QL_I8_SMALL_TILE (i8_gemm_small.hip),
// the same kernel takes 128 x 128 tiles of 4 waves of 64 x 64, walking K in
// 64-byte blocks through 4 slots of 16 KB (64 KB: two workgroups share a
// compute unit, each multiplying while the other waits at its own barrier).
// launch_i8_gemm / launch_f8_gemm take it when the 256 x 128 grid would fill
// at most half the compute units: there the extra tiles outweigh the larger
// tile's fewer copies per product (measured: 128 tokens on a 4096 x 4096
// layer 26.8 -> 14.8 us, 512 tokens 22.9 -> 18.5 us; a wash at 128 large
// tiles; slower beyond).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ql_internal.h"

namespace ql {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// accumulators: int32 for int8 operands, fp32 for FP8 (E4M3) operands
template <bool FP8>
using Acc = std::conditional_t<FP8, f32x16, i32x16>;

#ifdef QL_I8_SMALL_TILE
constexpr int BM = 128, BN = 128, BK = 64;       // BK in bytes (int8 elements)
constexpr int kWaves = 4;
constexpr int kStages = 4;                       // 64 KB of slots: two workgroups per compute unit
#else
constexpr int BM = 256, BN = 128, BK = 128;
constexpr int kWaves = 8;
constexpr int kStages = 3;                       // 144 KB of slots: one workgroup per compute unit
#endif
constexpr int kMT = BM / (16 * kWaves), kNT = 2; // (kWaves / 2) x 2 waves; wave (wm, wn) owns
                                                 //   32 kMT rows x 64 columns (32 x 32 MFMA tiles)
constexpr int kHalves = BK / 64;                 // 64-byte halves of a block (one mma_block each)
constexpr int kASlot = BM * BK;                  // 16 KB
constexpr int kBSlot = BN * BK;                  // 8 KB
constexpr int kSlot = kASlot + kBSlot;           // 24 KB
constexpr int kPieces = BK / 16;                 // 16-byte pieces per row
constexpr int kAFills = kASlot / 1024 / kWaves;  // 1 KB blocks of A per wave and slot
constexpr int kBFills = kBSlot / 1024 / kWaves;  // 1 KB blocks of B per wave and slot
constexpr int kLoads = kAFills + kBFills;        // copies per wave and slot

__shared__ __align__(1024) int8_t g_lds[kStages * kSlot];

struct I8Args {
  const int8_t* A;
  const int8_t* B;
  int M, N, K;
  I8Epi e;
  bool off32;              // M K and N K below 2^32: lane offsets fit 32 bits
};

// byte offset of logical 16-byte piece p of row r inside an operand tile: four
// 64-byte rows span the 64 banks once, and the piece index is XORed with bits
// 2..3 of the row
__device__ inline int swz_key(int r) { return BK == 64 ? (r >> 2) & 3 : (r >> 1) & 7; }
__device__ inline int swz(int r, int p) { return r * BK + ((p ^ swz_key(r)) << 4); }

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// issues one 16-byte global -> LDS load per lane (lane i writes lds + 16 i)
__device__ inline void load_lds16(const int8_t* src, int8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), lds, 16, 0, 0);
#else
  (void)src;
  (void)lds;
#endif
}

// One wave's share of filling a slot: 1 KB blocks of 16 rows x 64 bytes,
// kAFills of A and kBFills of B.  Lane l of a block writes LDS bytes
// 16 l .. 16 l + 15 of the block, i.e. row l / 4 and stored piece l % 4, which
// holds logical piece (l % 4) ^ ((row >> 2) & 3).  Rows past M or N are
// clamped to the last row (valid loads whose data only reaches outputs that
// are never stored).
struct FillPlan {
  const int8_t* src[kLoads];   // row of each block
  int p16[kLoads];             // byte offset of this lane's logical piece inside a K block
  int dst[kLoads];             // byte offset of the lane's 1 KB destination block inside a slot
  uint32_t off[kLoads];        // row * K + p16: the lane's offset from the operand's base (off32 only)
};

__device__ inline FillPlan make_fill_plan(const I8Args& a, int m0, int n0, int wave, int lane) {
  FillPlan f;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const bool is_a = i < kAFills;
    const int blk = is_a ? wave * kAFills + i : wave * kBFills + (i - kAFills);
    const int r = blk * (1024 / BK) + lane / kPieces;
    const int row = is_a ? min(m0 + r, a.M - 1) : min(n0 + r, a.N - 1);
    f.src[i] = (is_a ? a.A : a.B) + (size_t)row * a.K;
    f.p16[i] = ((lane % kPieces) ^ swz_key(r)) * 16;
    f.dst[i] = (is_a ? 0 : kASlot) + blk * 1024;
    f.off[i] = (uint32_t)row * (uint32_t)a.K + (uint32_t)f.p16[i];
  }
  return f;
}

// K offsets past the end of a row are clamped to the row's last 16 bytes
// (their data is zeroed before use: see mma_block)
template <int S>
__device__ inline void fill(const FillPlan& f, int kb, int K) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int k = min(kb * BK + f.p16[i], K - 16);
    load_lds16(f.src[i] + k, g_lds + S * kSlot + f.dst[i]);
  }
}

// A lane's fixed 32-bit offset from a uniform base, made opaque to the
// optimizer (in place) so that each copy keeps the scalar-base plus
// vector-offset form instead of a 64-bit per-lane address computed with
// vector instructions every block.
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

// LDS read of one 16-byte operand fragment.  Written as inline assembly so
// that the compiler's conservative tracking of in-flight LDS DMA (it would wait
// for every outstanding slot fill) stays out of the K loop; the ordering it
// would enforce is provided explicitly: wait_vm + s_barrier before a slot is
// read, and lds_wait + after_wait before the fragments are used.
__device__ inline i32x4 lds_read16(uint32_t addr) {
  i32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
#else
  v = i32x4{(int)addr, 0, 0, 0};   // host pass only (never executed)
#endif
  return v;
}
// waits until at most N of this wave's LDS reads are in flight
template <int N>
__device__ inline void lds_wait() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(%0)" : : "n"(N) : "memory");
#endif
}
// makes a fragment depend on the preceding lds_wait
__device__ inline void after_wait(i32x4& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
}

// kvalid: bytes of this K block inside the matrix (BK except in a ragged last
// block); pieces past it hold whatever the clamped loads fetched and are zeroed
// here.  Rows past M or N need no masking: they only reach outputs that are
// never stored.
//   ard[ks], brd[ks]: LDS addresses (slot 0, tile 0) of the lane's A and B
//   fragments of k step ks; + 32 * BK per 32-row tile, + kSlot per slot
// The byte of K a lane's fragment register holds is the same for A and B
// (both are read with the same piece pattern), so the products pair up
// whatever order the matrix unit sums them in.
//   int8: two 32-byte k steps; lane l supplies bytes 16 * (l / 32) .. +16 of
//         each (piece 2 ks + l / 32)
//   FP8:  one 64-byte k step of v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3,
//         fp32 accumulation); lane l supplies bytes 32 * (l / 32) .. +32
//         (pieces 2 (l / 32) + j, j = 0, 1)
__device__ inline int frag_piece(bool fp8, int j, int half) { return fp8 ? 2 * half + j : 2 * j + half; }

template <int S, bool FP8, bool FULL, typename Mid>
__device__ inline void mma_block(Acc<FP8> (&acc)[kMT][kNT], const uint32_t (&ard)[2], const uint32_t (&brd)[2],
                                 int half, int kvalid, Mid&& mid) {
  if constexpr (FP8) {
    i32x4 af[2][kMT], bf[2][kNT];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int t = 0; t < kMT; ++t) af[j][t] = lds_read16(ard[j] + S * kSlot + t * 32 * BK);
#pragma unroll
      for (int t = 0; t < kNT; ++t) bf[j][t] = lds_read16(brd[j] + S * kSlot + t * 32 * BK);
    }
    lds_wait<0>();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // pieces past kvalid (a ragged last block): zero the A side
      const bool live = FULL || frag_piece(true, j, half) * 16 < kvalid;
#pragma unroll
      for (int t = 0; t < kMT; ++t) {
        after_wait(af[j][t]);
        if (!FULL) af[j][t] = live ? af[j][t] : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int t = 0; t < kNT; ++t) after_wait(bf[j][t]);
    }
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const i32x8 a8 = __builtin_shufflevector(af[0][mt], af[1][mt], 0, 1, 2, 3, 4, 5, 6, 7);
        const i32x8 b8 = __builtin_shufflevector(bf[0][nt], bf[1][nt], 0, 1, 2, 3, 4, 5, 6, 7);
        // format codes 0, 0: both operands FP8 E4M3; no block scales
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[mt][nt], 0, 0, 0, 0, 0, 0);
      }
      if (mt == 0) mid();
    }
    return;
  } else {
  // operand layout of the 32x32x32 int8 MFMA: lane l supplies row/column l%32,
  // bytes 16 * (l / 32) .. +16 of the 32-byte k step.  Both k steps'
  // fragments are read at once; the second step's reads land while the first
  // multiplies.
  i32x4 af[2][kMT], bf[2][kNT];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int t = 0; t < kMT; ++t) af[ks][t] = lds_read16(ard[ks] + S * kSlot + t * 32 * BK);
#pragma unroll
    for (int t = 0; t < kNT; ++t) bf[ks][t] = lds_read16(brd[ks] + S * kSlot + t * 32 * BK);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks == 0)
      lds_wait<kMT + kNT>();
    else
      lds_wait<0>();
    // pieces past kvalid (a ragged last block): zero the A side
    const bool live = FULL || (ks * 2 + half) * 16 < kvalid;
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      after_wait(af[ks][t]);
      if (!FULL) af[ks][t] = live ? af[ks][t] : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < kNT; ++t) after_wait(bf[ks][t]);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks][mt], bf[ks][nt], acc[mt][nt], 0, 0, 0);
    if (ks == 0) mid();
  }
  }
}

// one k-block: wait for slot S, barrier, refill the slot freed by the previous
// block with block kb + kStages - 1 (clamped to the last block near the end, so
// that every wave always has the same number of loads in flight), multiply slot S
template <int S, bool FP8, bool FULL, bool PLAIN>
__device__ inline void kstep(const I8Args& a, FillPlan& f, Acc<FP8> (&acc)[kMT][kNT], int kb, int nkb,
                             const uint32_t (&ard)[kHalves][2], const uint32_t (&brd)[kHalves][2], int half) {
  // this wave's loads of block kb are done once at most (kStages - 2) blocks
  // of its loads remain in flight
  wait_vm<(kStages - 2) * kLoads>();
  __builtin_amdgcn_s_barrier();                  // every wave's loads of block kb landed,
                                                 // and every wave finished block kb - 1
  constexpr int F = (S + kStages - 1) % kStages;
  // the refill's copies are issued a share before each half's MFMAs: a wave
  // stalls on a copy until the address unit takes it, and issuing all of
  // them at once held the whole block's arithmetic back
  const int fb = min(kb + kStages - 1, nkb - 1);
  // PLAIN (the prefetched block lies wholly inside K and the operands' lane
  // offsets fit 32 bits): the copies address the operand's base plus the
  // block's offset (scalar) plus the lane's fixed offset; otherwise K offsets
  // past a row's end are clamped to its last 16 bytes (zeroed before use: see
  // mma_block)
  auto copies = [&](auto I0, auto I1) {
    static_for<I0, I1>([&](auto I) {
      if constexpr (PLAIN) {
        const int8_t* base = (I < kAFills ? a.A : a.B) + (size_t)fb * BK;
        f.off[I] = lane_offset(f.off[I]);
        load_lds16(base + f.off[I], g_lds + F * kSlot + f.dst[I]);
      } else {
        const int k = min(fb * BK + f.p16[I], a.K - 16);
        load_lds16(f.src[I] + k, g_lds + F * kSlot + f.dst[I]);
      }
    });
  };
  // four shares: before each half's fragment reads and after its first MFMAs
  constexpr int kQ = kLoads / (2 * kHalves), kR = kLoads - 2 * kHalves * kQ;   // kR shares get one more
  static_for<0, kHalves>([&](auto HH) {
    constexpr int hh = HH;
    constexpr int q0 = 2 * hh, q1 = 2 * hh + 1;
    constexpr int b0 = q0 * kQ + (q0 < kR ? q0 : kR), e0 = b0 + kQ + (q0 < kR ? 1 : 0);
    constexpr int b1 = e0, e1 = b1 + kQ + (q1 < kR ? 1 : 0);
    copies(std::integral_constant<int, b0>{}, std::integral_constant<int, e0>{});
    mma_block<S, FP8, FULL>(acc, ard[hh], brd[hh], half, a.K - kb * BK - 64 * hh,
                      [&] { copies(std::integral_constant<int, b1>{}, std::integral_constant<int, e1>{}); });
  });
}

// the blocks after the main loop (at most 2 kStages - 1 of them, the last
// possibly ragged), slots continuing in order
template <int S, bool FP8>
__device__ inline void kstep_tail(const I8Args& a, FillPlan& f, Acc<FP8> (&acc)[kMT][kNT], int kb, int nkb,
                                  const uint32_t (&ard)[kHalves][2], const uint32_t (&brd)[kHalves][2], int half) {
  if constexpr (S < 2 * kStages - 1) {
    if (kb < nkb) {
      if (a.K - kb * BK >= BK)
        kstep<S % kStages, FP8, true, false>(a, f, acc, kb, nkb, ard, brd, half);
      else
        kstep<S % kStages, FP8, false, false>(a, f, acc, kb, nkb, ard, brd, half);
      kstep_tail<S + 1, FP8>(a, f, acc, kb + 1, nkb, ard, brd, half);
    }
  }
}

// Workgroup -> tile.  Workgroups are dealt round-robin to the 8 XCDs, each
// with its own L2; when the tile count allows, consecutive tiles of a grouped
// order (4 tile rows at a time) go to one XCD, so an XCD works on a block of
// 4 tile rows and its L2 serves the A and B rows those tiles share.
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

// The operands and sizes are separate scalars, first in the list, so that
// they are preloaded into scalar registers at wave launch; the epilogue's
// arguments follow, read from memory as usual (needed at the end).
#ifdef QL_I8_SMALL_TILE
#define QL_I8_KERNEL_ATTR __attribute__((amdgpu_waves_per_eu(2)))
#else
#define QL_I8_KERNEL_ATTR
#endif
template <bool OUT_BF16, bool FP8>
__global__ __launch_bounds__(64 * kWaves) QL_I8_KERNEL_ATTR void i8_gemm_kernel(const int8_t* A, const int8_t* B, int M, int N, int K,
                                                              int off32, I8Epi epi) {
  I8Args a;
  a.A = A;
  a.B = B;
  a.M = M;
  a.N = N;
  a.K = K;
  a.e = epi;
  a.off32 = off32 != 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int mtile, ntile;
  tile_of(blockIdx.x, (a.M + BM - 1) / BM, (a.N + BN - 1) / BN, mtile, ntile);
  const int m0 = mtile * BM, n0 = ntile * BN;
  const int wm = (wave >> 1) * (kMT * 32), wn = (wave & 1) * (kNT * 32);
  static_assert((kWaves / 2) * kMT * 32 == BM && 2 * kNT * 32 == BN, "waves cover the tile");
  const int nkb = (a.K + BK - 1) / BK;
  const int half = lane >> 5, l32 = lane & 31;

  Acc<FP8> acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int j = 0; j < kNT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // LDS addresses of the lane's fragments in slot 0, tile 0 ((row + 32 t)
  // keeps bits 2..3 of the row, so tile t is + 32 * BK * t)
  typedef __attribute__((address_space(3))) int8_t* lds_ptr;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_ptr)g_lds;
  uint32_t ard[kHalves][2], brd[kHalves][2];
#pragma unroll
  for (int hh = 0; hh < kHalves; ++hh)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      ard[hh][ks] = base + swz(wm + l32, frag_piece(FP8, ks, half) + 4 * hh);
      brd[hh][ks] = base + kASlot + swz(wn + l32, frag_piece(FP8, ks, half) + 4 * hh);
    }

  // prologue: blocks 0 .. kStages - 2 in flight (clamped to the last block)
  FillPlan f = make_fill_plan(a, m0, n0, wave, lane);
  static_for<0, kStages - 1>([&](auto J) { fill<J>(f, min((int)J, nkb - 1), a.K); });

  int kb = 0;
  // whole rounds of kStages blocks that lie wholly inside K (no piece of
  // them to zero), and whose prefetched blocks (kStages - 1 ahead) do too
  // when the copies can take the scalar-base form; then the rest
  const int nfull = a.K / BK;
  if (a.off32) {
    for (; kb + 2 * kStages - 1 <= nfull; kb += kStages)
      static_for<0, kStages>([&](auto S) { kstep<S, FP8, true, true>(a, f, acc, kb + S, nkb, ard, brd, half); });
  } else {
    for (; kb + kStages <= nfull; kb += kStages)
      static_for<0, kStages>([&](auto S) { kstep<S, FP8, true, false>(a, f, acc, kb + S, nkb, ard, brd, half); });
  }
  kstep_tail<0, FP8>(a, f, acc, kb, nkb, ard, brd, half);
  wait_vm<0>();                                  // no load may still target LDS at exit

  // ---- fused epilogue: C = Dq - azp*azp_adj (int32), out = s_a * (s_b * C) + bias.
  // Every per-row and per-column parameter is read before the first store
  // (a load after a store the compiler cannot prove disjoint would wait for a
  // full memory round trip per element): the tile's row scales and zero points
  // go through LDS (the operand slots are free now), a lane's columns through
  // registers.
  const I8Epi& e = a.e;
  constexpr int kOutWave = (kMT * 32) * (kNT * 32) * 2;      // a wave's output tile in LDS
  constexpr int kRowParams = kWaves * kOutWave;              // row scales, then row zero points
  static_assert(kRowParams + BM * 8 <= kStages * kSlot, "epilogue staging fits in the slots");
  float* row_s = reinterpret_cast<float*>(g_lds + kRowParams);
  int32_t* row_z = reinterpret_cast<int32_t*>(g_lds + kRowParams + BM * 4);
  __syncthreads();                               // every wave is done with the slots
  // whether every zero point and column sum of the tile fits 24 bits, so that
  // their product is one v_mul_i32_i24 (exact) instead of a quarter-rate
  // 32-bit multiply; real zero points are 8-bit and |azp_adj| <= 128 K
  constexpr int kI24 = 1 << 23;
  bool wide = false;
  for (int r = tid; r < BM; r += 64 * kWaves) {
    const int m = min(m0 + r, a.M - 1);
    row_s[r] = e.s_a[e.s_a_vec ? m : 0];
    const int32_t z = e.azp ? e.azp[m] : 0;
    row_z[r] = z;
    wide |= z < -kI24 || z >= kI24;
  }
  float col_s[kNT], col_b[kNT];
  int32_t col_adj[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int n = min(n0 + wn + nt * 32 + l32, a.N - 1);
    col_s[nt] = e.s_b[e.s_b_vec ? n : 0];
    col_adj[nt] = e.azp_adj ? e.azp_adj[n] : 0;
    wide |= col_adj[nt] < -kI24 || col_adj[nt] >= kI24;
    float b = 0.0f;
    if (e.bias) {
      const uint16_t bb = static_cast<const uint16_t*>(e.bias)[n];
      b = OUT_BF16 ? __builtin_bit_cast(float, (uint32_t)bb << 16) : (float)__builtin_bit_cast(_Float16, bb);
    }
    col_b[nt] = b;
  }
  wide = __syncthreads_or(wide);
  const bool per_token_azp = e.azp != nullptr;
  auto value = [&](int mt, int nt, int el, int r) -> uint16_t {
    float c;
    if constexpr (FP8)
      c = acc[mt][nt][el];
    else
      c = (float)(acc[mt][nt][el] - (per_token_azp ? row_z[r] * col_adj[nt] : col_adj[nt]));
    const float v = row_s[r] * (col_s[nt] * c) + col_b[nt];
    return OUT_BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
  };
  // acc element el of lane l: row 8*(el/4) + 4*(l/32) + el%4, column l%32 of its 32 x 32 tile
  const bool full = m0 + BM <= a.M && n0 + BN <= a.N && (a.N & 7) == 0 && e.raw == nullptr;
  if (full) {
    // whole tile inside Y: stage the wave's 128 x 64 outputs in LDS (16-byte
    // pieces of a 128-byte row XOR-swizzled by row, conflict-free both ways)
    // and store them as 16-byte row pieces, 8 full lines per instruction
    uint8_t* region = reinterpret_cast<uint8_t*>(g_lds) + wave * kOutWave;
    // the lane's 4 * kMT runs of 4 consecutive rows: their scales and zero
    // points as 16-byte LDS reads
    float4 rs[kMT][4];
    int4 rz[kMT][4];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm + mt * 32 + 8 * q + 4 * half;
        rs[mt][q] = *reinterpret_cast<const float4*>(row_s + r);
        rz[mt][q] = *reinterpret_cast<const int4*>(row_z + r);
      }
    auto stage = [&](auto corr) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
          for (int el = 0; el < 16; ++el) {
            const int q = el >> 2, i = el & 3;
            const float sr = i == 0 ? rs[mt][q].x : i == 1 ? rs[mt][q].y : i == 2 ? rs[mt][q].z : rs[mt][q].w;
            const int zr = i == 0 ? rz[mt][q].x : i == 1 ? rz[mt][q].y : i == 2 ? rz[mt][q].z : rz[mt][q].w;
            float c;
            if constexpr (FP8)
              c = acc[mt][nt][el];
            else
              c = (float)(acc[mt][nt][el] - corr(zr, col_adj[nt]));
            const float v = sr * (col_s[nt] * c) + col_b[nt];
            const uint16_t h =
                OUT_BF16 ? __builtin_bit_cast(uint16_t, (__bf16)v) : __builtin_bit_cast(uint16_t, (_Float16)v);
            const int rl = mt * 32 + 8 * q + 4 * half + i;                  // row inside the wave tile
            const int cl = nt * 32 + l32;                                   // column inside the wave tile
            *reinterpret_cast<uint16_t*>(region + rl * 128 + (((cl >> 3) ^ (rl & 7)) << 4) + (cl & 7) * 2) = h;
          }
    };
    if (FP8 || !per_token_azp)
      stage([](int, int adj) { return adj; });
    else if (!wide)
      stage([](int z, int adj) { return __mul24(z, adj); });
    else
      stage([](int z, int adj) { return z * adj; });
    // the output is written once, all tiles at about the same moment: the
    // stores carry the non-temporal hint (measured 3-6% faster on
    // 2048 x 4096 x 4096, 4096^3 and 2048 x 11008 x 4096, int8 and FP8)
    uint16_t* out = static_cast<uint16_t*>(e.out);
#pragma unroll
    for (int i = 0; i < (kMT * 32) / 8; ++i) {
      const int rl = (lane >> 3) + 8 * i, piece = lane & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(region + rl * 128 + ((piece ^ (rl & 7)) << 4));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (size_t)(m0 + wm + rl) * a.N + n0 + wn + piece * 8));
    }
  } else {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int n = n0 + wn + nt * 32 + l32;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
        for (int el = 0; el < 16; ++el) {
          const int r = wm + mt * 32 + 8 * (el >> 2) + 4 * half + (el & 3);
          const int m = m0 + r;
          if (m >= a.M || n >= a.N) continue;
          if constexpr (!FP8)
            if (e.raw)
              e.raw[(size_t)m * a.N + n] = acc[mt][nt][el] - (per_token_azp ? row_z[r] * col_adj[nt] : col_adj[nt]);
          static_cast<uint16_t*>(e.out)[(size_t)m * a.N + n] = value(mt, nt, el, r);
        }
      }
    }
  }
}

}  // namespace

#ifdef QL_I8_SMALL_TILE
hipError_t launch_i8_gemm_small(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e,
                                hipStream_t st) {
#else
hipError_t launch_i8_gemm(const int8_t* A, const int8_t* B, int M, int N, int K, const I8Epi& e, hipStream_t st) {
  if (i8_gemv_serves(M, N)) return launch_i8_gemv(A, B, M, N, K, e, false, st);
  if (i8_small_grid(M, N)) return launch_i8_gemm_small(A, B, M, N, K, e, st);
#endif
  I8Args a{A, B, M, N, K, e, (size_t)M * K <= 0xFFFFFFFFu && (size_t)N * K <= 0xFFFFFFFFu};
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (e.out_bf16)
    hipLaunchKernelGGL((i8_gemm_kernel<true, false>), dim3(tiles), dim3(64 * kWaves), 0, st, a.A, a.B, a.M, a.N,
                       a.K, (int)a.off32, a.e);
  else
    hipLaunchKernelGGL((i8_gemm_kernel<false, false>), dim3(tiles), dim3(64 * kWaves), 0, st, a.A, a.B, a.M, a.N,
                       a.K, (int)a.off32, a.e);
  return hipGetLastError();
}

#ifdef QL_I8_SMALL_TILE
hipError_t launch_f8_gemm_small(const uint8_t* A, const uint8_t* B, int M, int N, int K, const I8Epi& e,
                                hipStream_t st) {
#else
hipError_t launch_f8_gemm(const uint8_t* A, const uint8_t* B, int M, int N, int K, const I8Epi& e, hipStream_t st) {
  if (i8_gemv_serves(M, N)) {
    I8Epi f = e;
    f.azp = nullptr;
    f.azp_adj = nullptr;
    f.raw = nullptr;
    return launch_i8_gemv(reinterpret_cast<const int8_t*>(A), reinterpret_cast<const int8_t*>(B), M, N, K, f, true,
                          st);
  }
  if (i8_small_grid(M, N)) return launch_f8_gemm_small(A, B, M, N, K, e, st);
#endif
  I8Args a{reinterpret_cast<const int8_t*>(A), reinterpret_cast<const int8_t*>(B), M, N, K, e,
            (size_t)M * K <= 0xFFFFFFFFu && (size_t)N * K <= 0xFFFFFFFFu};
  a.e.azp = nullptr;
  a.e.azp_adj = nullptr;
  a.e.raw = nullptr;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (e.out_bf16)
    hipLaunchKernelGGL((i8_gemm_kernel<true, true>), dim3(tiles), dim3(64 * kWaves), 0, st, a.A, a.B, a.M, a.N,
                       a.K, (int)a.off32, a.e);
  else
    hipLaunchKernelGGL((i8_gemm_kernel<false, true>), dim3(tiles), dim3(64 * kWaves), 0, st, a.A, a.B, a.M, a.N,
                       a.K, (int)a.off32, a.e);
  return hipGetLastError();
}

}  // namespace ql
